"""Plain float64 core attention on the CPU — the oracle (test infrastructure).

Only the test suite, ``smoke()`` and the benchmark's ``cpu_baseline`` leg may
use this module.  It imports numpy only and shares no code with the HIP path.

What is computed, and where the pages define it
-----------------------------------------------
* Core attention is the parameter-free softmax(Q K^T) V that sits between the
  QKV and output projections (Efficient Long-context Language Model Training
  by Core Attention Disaggregation, Sections 1 and 3.2).
* A CA-task is a query shard q(t) plus its context kv(t): the keys and values
  of every token from the document start up to and including the last query
  token (same page, Section 3.4, "The CA-Task Abstraction").  The causal mask
  lets the query at document position p see keys at positions 0..p, itself
  included (Context Parallelism for Scalable Million-Token Inference,
  Section 3.4, "Load-Balanced Sharding").
* Packed documents never attend across a document boundary (Core Attention
  Disaggregation, Section 2 on document packing).
* Scores are scaled by 1/sqrt(d) before the exponential, and the per-query
  log-sum-exp LSE_s = log sum_i exp(q . k_i / sqrt(d)) together with the
  normalised output O_s is what each partial attention returns; partials
  combine by Equation 4 (Context Parallelism ..., Section 3.4 "Merge
  Attention" and Appendix B).
* Grouped-query attention: query head h reads KV head floor(h * Hkv / Hq),
  i.e. contiguous groups of Hq/Hkv query heads share one KV head
  (Context Parallelism ..., "The CP+TP Nesting Design": GPU i holds KV head
  i with query heads 16i..16i+15).

Task table
----------
An ``(n, 7)`` int64 array, one row per CA-task, columns ``TASK_FIELDS``:

  q_off   first row of the task's queries in Q (and dQ)
  kv_off  first row of its context in K and V (and dK, dV)
  o_off   first row of its outputs in O and LSE (and of O, dO in backward)
  q_len   number of query rows
  kv_len  number of context rows
  q_pos0  document position of the first query
  kv_pos0 document position of the first context row

Key j of a task is visible to its query i  iff  kv_pos0 + j <= q_pos0 + i.

Two optional columns after these, ``MASK_FIELDS`` (0 when absent), narrow the
causal mask to the lambda shape of the sparse masks ("Dynamic Context
Parallelism", Section 2.4 / Figure 6b): an attention sink plus a sliding
window.  With kp = kv_pos0 + j and qp = q_pos0 + i, the key is visible iff
kp <= qp and (window == 0 or kp > qp - window or kp < sink): every query sees
the first ``sink`` positions and its ``window`` latest positions (itself
included).

A query shard may attend to several contexts: consecutive tasks with the
same q_off, o_off, q_len and q_pos0 (and q_len > 0) are one shard whose rows
attend to the union of the tasks' visible keys, with one softmax over all of
them.  This is how the causal-blockwise and shared-question masks ("Dynamic
Context Parallelism", Section 2.4, Figure 6c / 6d) are written: every query
sees a sink block or the question plus its own causal window, i.e. a union of
key ranges (the DCP executor's blockwise attention takes lists of query and
key blocks).  A key listed by two tasks of one shard counts twice.

A row with no visible key has O = 0 and LSE = -inf (a reading: the pages do
not discuss empty rows; this is the value that gives the row zero weight in
Equation 4).

Tensors are float64: Q [Tq, Hq, d], K and V [Tk, Hkv, d], O [To, Hq, d],
LSE [To, Hq].  bf16 inputs are widened exactly by ``bf16_bits_to_f64``.
"""

import numpy as np

TASK_FIELDS = ("q_off", "kv_off", "o_off", "q_len", "kv_len", "q_pos0", "kv_pos0")
MASK_FIELDS = ("window", "sink")

# Row-chunk budget for materialised score blocks (elements of float64).
_CHUNK_ELEMS = 1 << 24


def bf16_bits_to_f64(bits):
    """Exact widening of bfloat16 bit patterns (uint16 / int16) to float64.

    A bfloat16 value is the upper half of the float32 with the same bits.
    Pinned by test (against torch's own bfloat16 -> float32 conversion).
    """
    b = np.ascontiguousarray(np.asarray(bits)).view(np.uint16)
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _as_tasks(tasks):
    """(n, 7) or (n, 9) int table -> (n, 9) with zero window / sink columns
    where absent."""
    t = np.asarray(tasks, dtype=np.int64)
    if t.ndim == 1:
        t = t.reshape(1, -1)
    if t.shape[1] == len(TASK_FIELDS):
        t = np.concatenate([t, np.zeros((len(t), len(MASK_FIELDS)), dtype=np.int64)], axis=1)
    if t.shape[1] != len(TASK_FIELDS) + len(MASK_FIELDS):
        raise ValueError("task table must have columns %s (+ %s)" % (TASK_FIELDS, MASK_FIELDS))
    return t


def _group_of(h, hq, hkv):
    """KV head read by query head h: contiguous groups of hq // hkv."""
    return (h * hkv) // hq


def visible_mask(task, rows, n_keys):
    """Boolean [len(rows), n_keys]: key j visible to task row i.

    The definition of the causal CA-task mask: document position of key j is
    kv_pos0 + j, of query i is q_pos0 + i; a key is visible iff its position
    does not exceed the query's (diagonal included).  With a window (column 8)
    it must also lie within the query's ``window`` latest positions or below
    ``sink`` (column 9).
    """
    t = _as_tasks(task)[0]
    q_pos0, kv_pos0, window, sink = int(t[5]), int(t[6]), int(t[7]), int(t[8])
    qpos = q_pos0 + np.asarray(rows, dtype=np.int64)
    kpos = kv_pos0 + np.arange(n_keys, dtype=np.int64)
    vis = kpos[None, :] <= qpos[:, None]
    if window > 0:
        vis &= (kpos[None, :] > qpos[:, None] - window) | (kpos[None, :] < sink)
    return vis


def _context_len(task, rows):
    """How many leading context rows any of ``rows`` can see (keys past this
    are invisible to every row in the set)."""
    q_off, kv_off, o_off, q_len, kv_len, q_pos0, kv_pos0 = (int(x) for x in task[:7])
    if len(rows) == 0:
        return 0
    last = q_pos0 + int(np.max(rows)) - kv_pos0 + 1
    return max(0, min(kv_len, last))


def _shards(tasks):
    """Split a task table into query shards: maximal runs of consecutive
    tasks with the same q_off, o_off, q_len and q_pos0 (q_len > 0); every
    other task is a shard of its own.  Yields (n_seg, 9) arrays."""
    t = _as_tasks(tasks)
    i = 0
    while i < len(t):
        j = i + 1
        if t[i, 3] > 0:
            while j < len(t) and all(t[j, c] == t[i, c] for c in (0, 2, 3, 5)):
                j += 1
        yield t[i:j]
        i = j


def _as_shard(task):
    """A single task or the segments of one shard, as an (n_seg, 9) array."""
    segs = _as_tasks(task)
    for c in (0, 2, 3, 5):
        if np.any(segs[:, c] != segs[0, c]):
            raise ValueError("the segments of a shard must share q_off, o_off, q_len and q_pos0")
    return segs


def _row_chunks(segs, rows):
    n = max(1, sum(_context_len(t, rows) for t in segs))
    step = max(1, _CHUNK_ELEMS // n)
    for s in range(0, len(rows), step):
        yield rows[s:s + step]


def _head_rows(segs, rows, h, Q, K, V, scale, hq, hkv):
    """Softmax attention of one query head over one shard, for selected rows.

    Returns (O [r, d], LSE [r], [(P_s [r, n_s], n_s) per segment]) where P_s
    is the materialised probability block over the first n_s context keys of
    segment s (the rest are masked for every selected row).  The plain
    definition over the union of the segments' visible keys: s = scale * q.k,
    m = max s, w = exp(s - m), l = sum w, O = sum w v / l, LSE = m + ln l.
    No online rescaling, no blocking of the key axis.
    """
    q_off = int(segs[0][0])
    g = _group_of(h, hq, hkv)
    d = Q.shape[2]
    r = len(rows)
    O = np.zeros((r, d))
    LSE = np.full(r, -np.inf)
    q = Q[q_off + rows, h, :]                          # [r, d]
    S, VIS, VV, ns = [], [], [], []
    for t in segs:
        kv_off = int(t[1])
        n = _context_len(t, rows) if r else 0
        ns.append(n)
        k = K[kv_off:kv_off + n, g, :]                 # [n, d]
        VV.append(V[kv_off:kv_off + n, g, :])
        S.append(scale * (q @ k.T))                    # [r, n]
        VIS.append(visible_mask(t, rows, n))
    if sum(ns) == 0 or r == 0:
        return O, LSE, [(np.zeros((r, n)), n) for n in ns]
    s = np.concatenate(S, axis=1)
    vis = np.concatenate(VIS, axis=1)
    v = np.concatenate(VV, axis=0)
    s = np.where(vis, s, -np.inf)
    has = vis.any(axis=1)
    m = np.where(has, np.max(np.where(vis, s, -np.inf), axis=1), 0.0)
    w = np.where(vis, np.exp(s - m[:, None]), 0.0)
    l = w.sum(axis=1)
    safe_l = np.where(has, l, 1.0)
    P = w / safe_l[:, None]
    O = P @ v
    LSE = np.where(has, m + np.log(safe_l), -np.inf)
    bounds = np.cumsum([0] + ns)
    return O, LSE, [(P[:, bounds[i]:bounds[i + 1]], ns[i]) for i in range(len(ns))]


def forward_rows(task, rows, Q, K, V, scale, hq=None, hkv=None):
    """O [r, Hq, d] and LSE [r, Hq] for the given rows (task-relative indices)
    of one CA-task, or of one query shard given as its segment tasks.  Used
    directly for sampled checks at full size."""
    segs = _as_shard(task)
    hq = Q.shape[1] if hq is None else hq
    hkv = K.shape[1] if hkv is None else hkv
    rows = np.asarray(rows, dtype=np.int64)
    d = Q.shape[2]
    O = np.zeros((len(rows), hq, d))
    LSE = np.full((len(rows), hq), -np.inf)
    pos = 0
    for chunk in _row_chunks(segs, rows):
        for h in range(hq):
            o, lse, _ = _head_rows(segs, chunk, h, Q, K, V, scale, hq, hkv)
            O[pos:pos + len(chunk), h, :] = o
            LSE[pos:pos + len(chunk), h] = lse
        pos += len(chunk)
    return O, LSE


def forward(tasks, Q, K, V, scale, o_rows=None):
    """Core attention over every query shard of the table.

    Returns O [o_rows, Hq, d] and LSE [o_rows, Hq] in float64.  Output rows
    that no task covers hold NaN so that a comparison cannot pass on them by
    accident.
    """
    tasks = _as_tasks(tasks)
    hq, d = Q.shape[1], Q.shape[2]
    if o_rows is None:
        o_rows = int(max([t[2] + t[3] for t in tasks] + [0]))
    O = np.full((o_rows, hq, d), np.nan)
    LSE = np.full((o_rows, hq), np.nan)
    for segs in _shards(tasks):
        q_len = int(segs[0][3])
        o_off = int(segs[0][2])
        o, lse = forward_rows(segs, np.arange(q_len), Q, K, V, scale)
        O[o_off:o_off + q_len] = o
        LSE[o_off:o_off + q_len] = lse
    return O, LSE


def merge(O_parts, LSE_parts):
    """Merge attention, Equation 4 of Context Parallelism for Scalable
    Million-Token Inference (Appendix B).

    O_parts [S, T, H, d] and LSE_parts [S, T, H] are S partial results of the
    same queries against disjoint key sets.  With M = max_s LSE_s:
        O   = sum_s O_s exp(LSE_s - M) / sum_s exp(LSE_s - M)
        LSE = M + ln sum_s exp(LSE_s - M)
    The merged LSE is not printed on the page; it follows from the LSE
    definition there (log of the full normaliser).  A partial with
    LSE = -inf weighs zero; if every partial is empty, O = 0 and LSE = -inf.
    """
    O_parts = np.asarray(O_parts, dtype=np.float64)
    LSE_parts = np.asarray(LSE_parts, dtype=np.float64)
    M = np.max(LSE_parts, axis=0)                       # [T, H]
    finite = np.isfinite(M)
    Ms = np.where(finite, M, 0.0)
    w = np.where(np.isfinite(LSE_parts), np.exp(LSE_parts - Ms[None]), 0.0)  # [S, T, H]
    den = w.sum(axis=0)
    num = np.einsum("sth,sthd->thd", w, np.where(np.isfinite(LSE_parts)[..., None], O_parts, 0.0))
    safe = np.where(finite, den, 1.0)
    O = np.where(finite[..., None], num / safe[..., None], 0.0)
    LSE = np.where(finite, Ms + np.log(safe), -np.inf)
    return O, LSE


def backward(tasks, Q, K, V, dO, scale, dq_rows=None, dkv_rows=None):
    """Gradients of L = sum(O * dO) with respect to Q, K and V.

    The pages only say that the backward recomputes the attention
    probabilities from the saved per-row statistics instead of storing them
    (Core Attention Disaggregation, Sections 3.2 and 3.4).  The oracle takes
    the plain gradient of the forward definition: with P the softmax
    probabilities of a row (over all the keys its shard sees), D_i =
    <dO_i, O_i>,
        dV_j = sum_i P_ij dO_i,    dP_ij = <dO_i, V_j>,
        dS_ij = P_ij (dP_ij - D_i),
        dQ_i = scale sum_j dS_ij K_j,    dK_j = scale sum_i dS_ij Q_i,
    with dK and dV summed over every query head of the KV head's group and
    over every task that reads the same context rows.  O and P come from the
    oracle's own float64 forward of the same rows.
    """
    tasks = _as_tasks(tasks)
    hq, d = Q.shape[1], Q.shape[2]
    hkv = K.shape[1]
    dq_rows = Q.shape[0] if dq_rows is None else dq_rows
    dkv_rows = K.shape[0] if dkv_rows is None else dkv_rows
    dQ = np.zeros((dq_rows, hq, d))
    dK = np.zeros((dkv_rows, hkv, d))
    dV = np.zeros((dkv_rows, hkv, d))
    for segs in _shards(tasks):
        q_off, o_off, q_len = int(segs[0][0]), int(segs[0][2]), int(segs[0][3])
        for chunk in _row_chunks(segs, np.arange(q_len)):
            for h in range(hq):
                g = _group_of(h, hq, hkv)
                o, _, parts = _head_rows(segs, chunk, h, Q, K, V, scale, hq, hkv)
                do = dO[o_off + chunk, h, :]           # [r, d]
                q = Q[q_off + chunk, h, :]
                D = np.sum(do * o, axis=1)             # [r]
                for t, (P, n) in zip(segs, parts):
                    if n == 0:
                        continue
                    kv_off = int(t[1])
                    k = K[kv_off:kv_off + n, g, :]
                    v = V[kv_off:kv_off + n, g, :]
                    dV[kv_off:kv_off + n, g, :] += P.T @ do
                    dP = do @ v.T                      # [r, n]
                    dS = P * (dP - D[:, None])
                    dQ[q_off + chunk, h, :] += scale * (dS @ k)
                    dK[kv_off:kv_off + n, g, :] += scale * (dS.T @ q)
    return dQ, dK, dV


def backward_dq_rows(task, rows, Q, K, V, dO, scale, heads=None):
    """dQ [len(rows), len(heads), d] of selected rows of one task (or of one
    query shard given as its segment tasks): the rows of ``backward``'s dQ,
    computed from those rows alone.

    dQ_i depends only on row i (its probabilities P_i over its visible keys,
    D_i = <dO_i, O_i> and dP_i = dO_i V^T), so the gradient of
    L = sum(O * dO) with respect to query row i is
        dQ_i = scale sum_j P_ij (dP_ij - D_i) K_j
    whichever other rows exist; this is how the full-size checks sample it.
    ``heads`` lists the query heads (default: all); O and P come from the
    oracle's own float64 forward of the rows.
    """
    segs = _as_shard(task)
    o_off = int(segs[0][2])
    hq, d = Q.shape[1], Q.shape[2]
    hkv = K.shape[1]
    heads = list(range(hq)) if heads is None else [int(h) for h in heads]
    rows = np.asarray(rows, dtype=np.int64)
    dQ = np.zeros((len(rows), len(heads), d))
    pos = 0
    for chunk in _row_chunks(segs, rows):
        for k, h in enumerate(heads):
            g = _group_of(h, hq, hkv)
            o, _, parts = _head_rows(segs, chunk, h, Q, K, V, scale, hq, hkv)
            do = dO[o_off + chunk, h, :]
            D = np.sum(do * o, axis=1)
            for t, (P, n) in zip(segs, parts):
                if n == 0:
                    continue
                kv_off = int(t[1])
                dP = do @ V[kv_off:kv_off + n, g, :].T
                dS = P * (dP - D[:, None])
                dQ[pos:pos + len(chunk), k, :] += scale * (dS @ K[kv_off:kv_off + n, g, :])
        pos += len(chunk)
    return dQ


def forward_listed(Q, K, V, scale, rows_keys):
    """O [R, Hq, d], LSE [R, Hq] where output row r is the softmax attention
    of query row r over exactly the key rows listed in rows_keys[r]: the
    definition with the mask given as an explicit key list, which is how the
    sparse masks of "Dynamic Context Parallelism" (Section 2.4, Figure 6) are
    described — every query sees a union of ranges.  An empty list gives
    O = 0, LSE = -inf.  One row at a time, float64."""
    hq, d = Q.shape[1], Q.shape[2]
    hkv = K.shape[1]
    R = len(rows_keys)
    O = np.zeros((R, hq, d))
    LSE = np.full((R, hq), -np.inf)
    for r, keys in enumerate(rows_keys):
        ks = np.asarray(keys, dtype=np.int64)
        if ks.size == 0:
            continue
        for h in range(hq):
            g = _group_of(h, hq, hkv)
            s = scale * (K[ks, g] @ Q[r, h])
            m = s.max()
            w = np.exp(s - m)
            l = w.sum()
            O[r, h] = (w @ V[ks, g]) / l
            LSE[r, h] = m + np.log(l)
    return O, LSE


def backward_listed(Q, K, V, dO, scale, rows_keys):
    """Gradients of L = sum(O * dO) for the O of ``forward_listed``: row r
    attends to the listed key rows only.  The plain chain rule, one row and
    head at a time: with p the row's probabilities and o its output,
        dV_k += p_k dO_r,   ds_k = p_k (<dO_r, V_k> - <dO_r, o>),
        dQ_r += scale sum_k ds_k K_k,   dK_k += scale ds_k Q_r,
    dK and dV summed over the query heads of the KV head's group and over
    every row that lists the key.  Returns (dQ, dK, dV) shaped like Q, K, V."""
    hq = Q.shape[1]
    hkv = K.shape[1]
    dQ, dK, dV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    for r, keys in enumerate(rows_keys):
        ks = np.asarray(keys, dtype=np.int64)
        if ks.size == 0:
            continue
        for h in range(hq):
            g = _group_of(h, hq, hkv)
            s = scale * (K[ks, g] @ Q[r, h])
            p = np.exp(s - s.max())
            p /= p.sum()
            o = p @ V[ks, g]
            dp = V[ks, g] @ dO[r, h]
            ds = p * (dp - dO[r, h] @ o)
            np.add.at(dV[:, g], ks, p[:, None] * dO[r, h][None])
            dQ[r, h] += scale * (ds @ K[ks, g])
            np.add.at(dK[:, g], ks, scale * ds[:, None] * Q[r, h][None])
    return dQ, dK, dV
