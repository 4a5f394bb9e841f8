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


def backward_paged(tasks, Q, K_pages, V_pages, dO, table, page_rows, scale):
    """Gradients of L = sum(O * dO) for the paged forward: dQ, and dK, dV as
    page stores shaped like K_pages / V_pages.  The gradient of virtual row v
    is added to its physical row, so a page that several virtual pages name
    collects all their contributions; rows of pages no entry names are 0."""
    from .attention import backward
    P = int(page_rows)
    table = np.asarray(table, dtype=np.int64).reshape(-1)
    K = virtual_rows(K_pages, table, P)
    V = virtual_rows(V_pages, table, P)
    dQ, dKv, dVv = backward(tasks, Q, K, V, dO, scale)
    rows = (table[:, None] * P + np.arange(P)[None, :]).reshape(-1)
    dK = np.zeros(K_pages.shape)
    dV = np.zeros(V_pages.shape)
    np.add.at(dK, rows, dKv)
    np.add.at(dV, rows, dVv)
    return dQ, dK, dV
