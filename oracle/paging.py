"""Paged K/V as the oracle reads it — TEST INFRASTRUCTURE ONLY.

Block tables ("DCP: Addressing Input Dynamism In Long-Context Training via
Dynamic Context Parallelism", Executor Design, the Blockwise Attention
instruction, which addresses data blocks that need not be contiguous through
a table of block locations; the blocks themselves are per-head runs of B
tokens, Block Generation).  A page store X holds physical pages of P rows;
a table lists the physical page of each virtual page.  Paging only moves
rows, so attention over paged K/V is attention over the virtual K/V that the
table describes: the oracle materialises that virtual K/V and calls the
plain forward.

Reading: the virtual row v of a table is physical row table[v // P] * P +
v % P (row-major pages of P rows, all heads of a row together, as in the
unpaged layout).
"""

import numpy as np

from .attention import forward


def virtual_rows(X, table, page_rows):
    """The virtual tensor of a block table: len(table) * page_rows rows, row v
    copied from X[table[v // page_rows] * page_rows + v % page_rows]."""
    P = int(page_rows)
    table = np.asarray(table, dtype=np.int64).reshape(-1)
    out = np.empty((len(table) * P,) + X.shape[1:], dtype=X.dtype)
    for vp, pp in enumerate(table):
        out[vp * P:(vp + 1) * P] = X[pp * P:(pp + 1) * P]
    return out


def forward_paged(tasks, Q, K_pages, V_pages, table, page_rows, scale, o_rows=None):
    """forward() with kv_off / kv_len of every task read in the virtual row
    space of the table."""
    K = virtual_rows(K_pages, table, page_rows)
    V = virtual_rows(V_pages, table, page_rows)
    return forward(tasks, Q, K, V, scale, o_rows=o_rows)
