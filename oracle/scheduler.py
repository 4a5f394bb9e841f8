"""CA-task scheduler — oracle (TEST INFRASTRUCTURE ONLY).

A plain Python restatement of the profiler cost model and the
communication-aware greedy scheduler of "Efficient Long-context Language Model
Training by Core Attention Disaggregation" (Section 4.2, The Profiler and Cost
Model; The Communication-Aware Greedy Scheduler, Steps 1-4; Appendix B,
Optimal Shard Dimension Computation).  Only numpy-free float64 Python and the
math module; nothing here is shared with the library.

Readings where the pages leave a step open (listed with the design notes):

* Items.  Documents are packed in batch order and device j owns the j-th
  block of ceil(T / k) tokens; every maximal piece of a document on one device
  is an Item: the query range [a, b) of its document with context [0, b).
* Load.  An Item's load is the profiler's predicted time for (n_q, n_kv) =
  (b - a, b): queries are the last n_q tokens of an n_kv-token causal context.
* Communication.  n_q * s_q + n_kv * s_kv bytes with s_q = h_q * d * 2 and
  s_kv = h_kv * d * 2, so beta = s_kv / s_q = h_kv / h_q as the pages state.
* Split.  alpha = dF / F(t) is applied as the FLOPs fraction of Appendix B.
  The real optimum (or the cheaper feasible boundary when it is infeasible)
  is rounded to whole tokens: n_q to nearest (at least 1, at most L_q), then
  n_kv to nearest, clamped to [n_q + L_kv - L_q, L_kv].  The sub-Item is the
  query range [n_kv - n_q, n_kv); the rest of the Item stays on the source as
  up to two Items.  A split is a candidate only if n_q >= min_shard.
* Head-tail shards (head_tail=True).  A split of Item [a, b) moves its first m
  and its last m queries, [a, a + m) and [b - m, b), mirroring how a
  head-tail shard of a document pairs a leading stretch of its tokens with the
  matching trailing stretch; the middle [a + m, b - m) stays on the source.
  The pair of pieces holds m (a + b + 1) of the Item's (b - a)(a + b + 1) / 2
  visible pairs, so the
  FLOPs fraction alpha gives m = alpha (b - a) / 2, rounded to nearest and
  clamped to [1, (b - a) // 2]; the shard is a candidate if 2 m >= min_shard.
  Its communication is 2 m queries and the context [0, b) that the tail piece
  needs (the head's context is inside it).  Whole-Item moves are unchanged.
* Order and ties.  Deficit servers are taken once each, in descending order of
  their deficit at the start (ties: lower index).  For a deficit server, the
  best candidate over every Item on every server with load above the target is
  migrated, repeatedly, until its deficit is at most eps * target, no
  candidate has E > e_min, or max_moves migrations were made in total.
  Highest E wins; ties go to the lower source server, then to the older Item.
"""

import math

SQRT = math.sqrt


# ---------------------------------------------------------------------------
# FLOPs of a causal query block (diagonal included)
# ---------------------------------------------------------------------------

def block_pairs(n_q, n_kv):
    """Visible (query, key) pairs when the n_q queries are the last n_q
    positions of an n_kv-token causal context: query i (0-based within the
    block) sees n_kv - n_q + i + 1 keys."""
    return n_q * n_kv - n_q * (n_q - 1) // 2


# ---------------------------------------------------------------------------
# Profiler cost model (Section 4.2, The Profiler and Cost Model)
# ---------------------------------------------------------------------------

class CostModel:
    """Predicted time of a (n_q, n_kv) call from a measured grid.

    grid_q, grid_kv: ascending grid coordinates; times[i][j]: measured seconds
    at (grid_q[i], grid_kv[j]); flops_per_pair: FLOPs the profiled call counts
    per visible pair (all heads).  Inside the grid: bilinear interpolation of
    time over the bracketing cell.  Beyond the grid in both coordinates (the
    saturated region): FLOPs / the maximum measured throughput.  Beyond it in
    one coordinate only: FLOPs / the throughput interpolated at the point
    clamped into the grid.  FLOPs count min(n_q, n_kv) queries (a grid point
    with more queries than context stands for the full causal block)."""

    def __init__(self, grid_q, grid_kv, times, flops_per_pair):
        self.q = [float(x) for x in grid_q]
        self.kv = [float(x) for x in grid_kv]
        self.t = [[float(x) for x in row] for row in times]
        self.fpp = float(flops_per_pair)
        best = 0.0
        for i, qv in enumerate(self.q):
            for j, kvv in enumerate(self.kv):
                tp = self.flops(qv, kvv) / self.t[i][j]
                if tp > best:
                    best = tp
        self.peak = best

    def flops(self, n_q, n_kv):
        """FLOPs of the block; a query block longer than its context is read
        as one of n_kv queries (every query of a causal block has its key)."""
        m = min(n_q, n_kv)
        return self.fpp * (m * n_kv - m * (m - 1) / 2.0)

    @staticmethod
    def _bracket(axis, x):
        """Index i with axis[i] <= x <= axis[i + 1] (x inside the axis)."""
        i = 0
        while i + 2 < len(axis) and axis[i + 1] < x:
            i += 1
        return i

    def _interp(self, x, y):
        q, kv, t = self.q, self.kv, self.t
        if len(q) == 1 and len(kv) == 1:
            return t[0][0]
        if len(q) == 1:
            j = self._bracket(kv, y)
            v = (y - kv[j]) / (kv[j + 1] - kv[j])
            return t[0][j] * (1.0 - v) + t[0][j + 1] * v
        if len(kv) == 1:
            i = self._bracket(q, x)
            u = (x - q[i]) / (q[i + 1] - q[i])
            return t[i][0] * (1.0 - u) + t[i + 1][0] * u
        i = self._bracket(q, x)
        j = self._bracket(kv, y)
        u = (x - q[i]) / (q[i + 1] - q[i])
        v = (y - kv[j]) / (kv[j + 1] - kv[j])
        return (t[i][j] * (1.0 - u) * (1.0 - v) + t[i + 1][j] * u * (1.0 - v)
                + t[i][j + 1] * (1.0 - u) * v + t[i + 1][j + 1] * u * v)

    def time(self, n_q, n_kv):
        if n_q <= 0:
            return 0.0
        x, y = float(n_q), float(n_kv)
        inside_q = self.q[0] <= x <= self.q[-1]
        inside_kv = self.kv[0] <= y <= self.kv[-1]
        if inside_q and inside_kv:
            return self._interp(x, y)
        if x > self.q[-1] and y > self.kv[-1]:
            return self.flops(x, y) / self.peak
        cx = min(max(x, self.q[0]), self.q[-1])
        cy = min(max(y, self.kv[0]), self.kv[-1])
        if cy < cx:                  # keep the clamped block causal-feasible
            cy = cx
        tp = self.flops(cx, cy) / self._interp(cx, cy)
        return self.flops(x, y) / tp


# ---------------------------------------------------------------------------
# Appendix B: shard dimensions that move a FLOPs fraction alpha for the
# least communication
# ---------------------------------------------------------------------------

def optimal_shard(alpha, L_q, L_kv, beta):
    """Real (n_q, n_kv) with n_q (2 n_kv - n_q) = alpha L_q (2 L_kv - L_q),
    minimising n_q + beta n_kv over 0 < n_q <= L_q, n_q + L_kv - L_q <= n_kv
    <= L_kv.  Interior optimum n_q = sqrt(alpha beta L_q (2 L_kv - L_q) /
    (beta + 2)); when it is infeasible, the cheaper of the two boundary
    solutions (shard ending at L_kv, or shard starting at the Item's first
    query) that is feasible."""
    C = alpha * L_q * (2.0 * L_kv - L_q)
    lo_off = float(L_kv - L_q)

    def kv_of(nq):
        return (C / nq + nq) / 2.0

    def feasible(nq, nkv):
        tol = 1e-9 * max(1.0, L_kv)
        return 0.0 < nq <= L_q + tol and nq + lo_off - tol <= nkv <= L_kv + tol

    cands = []
    nq = SQRT(alpha * beta * L_q * (2.0 * L_kv - L_q) / (beta + 2.0))
    if nq > 0.0 and feasible(nq, kv_of(nq)):
        return nq, kv_of(nq)
    # shard ending at the Item's end: n_kv = L_kv
    nq_end = L_kv - SQRT(max(L_kv * L_kv - C, 0.0))
    if feasible(nq_end, L_kv):
        cands.append((nq_end + beta * L_kv, nq_end, float(L_kv)))
    # shard starting at the Item's first query: n_kv = n_q + L_kv - L_q
    nq_start = -lo_off + SQRT(lo_off * lo_off + C)
    if feasible(nq_start, nq_start + lo_off):
        cands.append((nq_start + beta * (nq_start + lo_off), nq_start, nq_start + lo_off))
    if not cands:
        return float(L_q), float(L_kv)
    cands.sort()
    return cands[0][1], cands[0][2]


def round_shard(nq, nkv, L_q, L_kv):
    """Whole-token shard from the real solution (see the module docstring)."""
    n_q = int(math.floor(nq + 0.5))
    n_q = min(max(n_q, 1), L_q)
    n_kv = int(math.floor(nkv + 0.5))
    n_kv = min(max(n_kv, n_q + L_kv - L_q), L_kv)
    return n_q, n_kv


# ---------------------------------------------------------------------------
# the greedy scheduler (Steps 1-4)
# ---------------------------------------------------------------------------

def initial_items(doc_lens, k):
    """Items (server, doc, a, b) of the token-count placement."""
    T = sum(doc_lens)
    per = -(-T // k) if T > 0 else 0
    items = []
    start = 0
    for doc, L in enumerate(doc_lens):
        a = 0
        while a < L:
            dev = min((start + a) // per, k - 1) if per > 0 else 0
            dev_end = (dev + 1) * per if dev < k - 1 else T
            b = min(L, dev_end - start)
            items.append([dev, doc, a, b])
            a = b
        start += L
    return items


def head_tail_pairs(a, b, m):
    """Visible pairs of the head-tail shard [a, a + m) + [b - m, b) of an Item
    with queries [a, b) and context [0, b): m (a + b + 1)."""
    return m * (a + b + 1)


def head_tail_shard(alpha, a, b):
    """Half-width m of the head-tail shard holding a FLOPs fraction alpha of
    Item [a, b)."""
    half = (b - a) // 2
    m = int(math.floor(alpha * (b - a) / 2.0 + 0.5))
    return min(max(m, 1), half)


def schedule(doc_lens, k, model, hq, hkv, d, eps=0.05, e_min=0.0, min_shard=128, max_moves=10000,
             head_tail=False):
    """Returns (items, loads_before, loads_after, comm_bytes, moves) where
    items is a list of [server, doc, a, b] (query range [a, b) of document doc,
    context [0, b)) in creation order."""
    s_q = float(hq * d * 2)
    s_kv = float(hkv * d * 2)
    beta = s_kv / s_q
    items = initial_items(doc_lens, k)

    def F(it):
        return model.time(it[3] - it[2], it[3])

    load = [0.0] * k
    for it in items:
        load[it[0]] += F(it)
    before = list(load)
    target = sum(load) / k
    deficits = sorted(range(k), key=lambda s: (-(target - load[s]), s))
    deficits = [s for s in deficits if load[s] < target]
    comm = 0.0
    moves = 0
    for dst in deficits:
        while moves < max_moves:
            D = target - load[dst]
            if D <= eps * target:
                break
            best = None          # (E, src, idx, dF, whole, n_q, n_kv, V)
            for idx, it in enumerate(items):
                src = it[0]
                S = load[src] - target
                if src == dst or S <= 0.0:
                    continue
                Ft = F(it)
                if Ft <= 0.0:
                    continue
                dF = min(Ft, S, D)
                L_q = it[3] - it[2]
                L_kv = it[3]
                if dF == Ft:
                    n_q, n_kv, whole = L_q, L_kv, True
                elif head_tail:
                    if L_q < 2:
                        continue
                    m = head_tail_shard(dF / Ft, it[2], it[3])
                    n_q, n_kv = 2 * m, L_kv
                    whole = (n_q == L_q)
                    if not whole and n_q < min_shard:
                        continue
                else:
                    nq, nkv = optimal_shard(dF / Ft, L_q, L_kv, beta)
                    n_q, n_kv = round_shard(nq, nkv, L_q, L_kv)
                    whole = (n_q == L_q)
                    if not whole and n_q < min_shard:
                        continue
                V = n_q * s_q + n_kv * s_kv
                E = dF / V
                if E <= e_min:
                    continue
                if best is None or E > best[0] or (E == best[0] and (src, idx) < (best[1], best[2])):
                    best = (E, src, idx, dF, whole, n_q, n_kv, V)
            if best is None:
                break
            _, src, idx, _, whole, n_q, n_kv, V = best
            it = items[idx]
            load[src] -= F(it)
            if whole:
                it[0] = dst
                load[dst] += F(it)
            elif head_tail:
                doc, a, b = it[1], it[2], it[3]
                m = n_q // 2
                del items[idx]
                if b - m > a + m:
                    mid = [src, doc, a + m, b - m]
                    load[src] += F(mid)
                    items.insert(idx, mid)
                for new in ([dst, doc, a, a + m], [dst, doc, b - m, b]):
                    items.append(new)
                    load[dst] += F(new)
            else:
                doc, a, b = it[1], it[2], it[3]
                sa, sb = n_kv - n_q, n_kv
                del items[idx]
                pieces = []
                if sa > a:
                    pieces.append([src, doc, a, sa])
                if b > sb:
                    pieces.append([src, doc, sb, b])
                for pc in pieces:
                    load[src] += F(pc)
                items[idx:idx] = pieces
                new = [dst, doc, sa, sb]
                items.append(new)
                load[dst] += F(new)
            comm += V
            moves += 1
    return items, before, load, comm, moves


def task_rows(items, doc_lens):
    """ca_task rows (q_off, kv_off, o_off, q_len, kv_len, q_pos0, kv_pos0) of
    the items over the packed batch, and the server of each row."""
    starts = [0]
    for L in doc_lens:
        starts.append(starts[-1] + L)
    rows, servers = [], []
    for srv, doc, a, b in items:
        base = starts[doc]
        rows.append((base + a, base, base + a, b - a, b, a, 0))
        servers.append(srv)
    return rows, servers
