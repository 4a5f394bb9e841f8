"""Unmasked-pair counts and the FLOP convention (oracle side; test
infrastructure only).

* Attention cost grows with the square of a document's length:
  FLOPs(l) = alpha l^2 + beta l (Core Attention Disaggregation, Section 3.4,
  "The Compute-Memory Imbalance Formalization").
* FLOPs = 4 T D (T + P) for T new tokens over T + P keys: two matrix products
  (Q K^T and P V), two FLOPs per multiply-add (Context Parallelism for
  Scalable Million-Token Inference, Section 3.4 "The Analytical Model", from
  its Table 3).  Counted per unmasked (query, key) pair and per query head of
  width d this is 4 d FLOPs.  The backward pass re-computes Q K^T and adds
  four more d-length products (dO V^T, P^T dO, dS K, dS^T Q): 10 d per pair
  (a reading; the pages only put the backward at roughly twice the forward).
"""

import numpy as np


def visible_pairs_task(q_len, kv_len, q_pos0, kv_pos0):
    """Number of (query, key) pairs with kv_pos0 + j <= q_pos0 + i, summed row
    by row (row i sees min(kv_len, max(0, q_pos0 + i - kv_pos0 + 1)) keys)."""
    i = np.arange(int(q_len), dtype=np.int64)
    per_row = np.clip(int(q_pos0) + i - int(kv_pos0) + 1, 0, int(kv_len))
    return int(per_row.sum())


def visible_pairs_masked(q_len, kv_len, q_pos0, kv_pos0, window, sink):
    """Pairs under the sink + sliding-window mask, row by row: the causal
    context of row i is positions [kv_pos0, kv_pos0 + c_i); of those it sees
    the ones above qp - window and the ones below sink (window 0: all)."""
    if int(window) <= 0:
        return visible_pairs_task(q_len, kv_len, q_pos0, kv_pos0)
    total = 0
    for i in range(int(q_len)):
        qp = int(q_pos0) + i
        hi = int(kv_pos0) + min(int(kv_len), max(0, qp - int(kv_pos0) + 1))   # end of the causal context
        lo = int(kv_pos0)
        win_lo = max(lo, qp - int(window) + 1)
        n_win = max(0, hi - win_lo)
        n_sink = max(0, min(int(sink), hi, win_lo) - lo)
        total += n_win + n_sink
    return total


def visible_pairs(tasks):
    """Unmasked pairs of a whole task table (columns as oracle.TASK_FIELDS,
    optionally followed by window and sink)."""
    t = np.asarray(tasks, dtype=np.int64)
    t = t.reshape(-1, t.shape[-1]) if t.size else t.reshape(0, 7)
    if t.shape[1] == 7:
        return int(sum(visible_pairs_task(r[3], r[4], r[5], r[6]) for r in t))
    return int(sum(visible_pairs_masked(r[3], r[4], r[5], r[6], r[7], r[8]) for r in t))


def forward_flops(pairs, hq, d):
    """4 d FLOPs per unmasked pair and query head."""
    return 4 * int(d) * int(pairs) * int(hq)


def backward_flops(pairs, hq, d, per_pair=10):
    """10 d FLOPs per unmasked pair and query head (8 d = "twice forward"
    is the alternative convention, selectable by ``per_pair``)."""
    return int(per_pair) * int(d) * int(pairs) * int(hq)
