"""Pins of the scheduler oracle (oracle/scheduler.py) against brute force,
closed forms and invariants — "Efficient Long-context Language Model Training
by Core Attention Disaggregation", Section 4.2 (profiler; greedy Steps 1-4)
and Appendix B."""

import math
import random

import pytest

from oracle import scheduler as S


def brute_pairs(n_q, n_kv):
    """Count visible pairs one by one: query position p sees keys 0..p."""
    return sum(1 for p in range(n_kv - n_q, n_kv) for key in range(n_kv) if key <= p)


@pytest.mark.parametrize("n_q,n_kv", [(1, 1), (1, 7), (3, 3), (5, 9), (17, 40), (64, 64)])
def test_block_pairs_brute_force(n_q, n_kv):
    assert S.block_pairs(n_q, n_kv) == brute_pairs(n_q, n_kv)


def bilinear_model(a, b, c, e, gq, gkv):
    times = [[a + b * x + c * y + e * x * y for y in gkv] for x in gq]
    return S.CostModel(gq, gkv, times, 1.0)


def test_cost_model_exact_on_bilinear_functions():
    """Bilinear interpolation reproduces any bilinear function exactly inside
    the grid, at the nodes and between them."""
    gq, gkv = [128, 512, 2048, 8192], [256, 1024, 4096, 16384, 65536]
    a, b, c, e = 3e-5, 2e-9, 5e-10, 1e-13
    m = bilinear_model(a, b, c, e, gq, gkv)
    rng = random.Random(3)
    pts = [(x, y) for x in gq for y in gkv]
    pts += [(rng.uniform(128, 8192), rng.uniform(256, 65536)) for _ in range(200)]
    for x, y in pts:
        want = a + b * x + c * y + e * x * y
        assert abs(m.time(x, y) - want) <= 1e-12 * want


def test_cost_model_single_point_is_a_flops_model():
    """A 1x1 grid makes every prediction FLOPs / (the one measured
    throughput): inside, in the saturated region and clamped."""
    m = S.CostModel([1024], [4096], [[2.0e-3]], 4 * 128 * 32)
    peak = m.flops(1024, 4096) / 2.0e-3
    for n_q, n_kv in [(1024, 4096), (64, 100), (5000, 9000), (100, 20000), (3000, 3000), (1, 1)]:
        want = m.flops(n_q, n_kv) / peak
        assert abs(m.time(n_q, n_kv) - want) <= 1e-12 * want


def test_cost_model_saturation_uses_the_best_grid_throughput():
    gq, gkv = [128, 1024], [1024, 8192]
    times = [[1e-4, 5e-4], [6e-4, 2e-3]]
    m = S.CostModel(gq, gkv, times, 1.0)
    tps = [m.flops(x, y) / times[i][j] for i, x in enumerate(gq) for j, y in enumerate(gkv)]
    assert m.peak == max(tps)
    assert abs(m.time(4096, 65536) - m.flops(4096, 65536) / max(tps)) <= 1e-15


def brute_optimal_shard(alpha, L_q, L_kv, beta, steps=200000):
    """Minimise n_q + beta n_kv on a fine grid of n_q, n_kv from the FLOPs
    constraint, keeping feasible points only."""
    C = alpha * L_q * (2.0 * L_kv - L_q)
    best = None
    for s in range(1, steps + 1):
        nq = L_q * s / steps
        nkv = (C / nq + nq) / 2.0
        if nq + L_kv - L_q - 1e-9 <= nkv <= L_kv + 1e-9:
            c = nq + beta * nkv
            if best is None or c < best[0]:
                best = (c, nq, nkv)
    return best


@pytest.mark.parametrize("alpha,L_q,L_kv,beta", [
    (0.333, 4096, 8192, 0.25), (0.05, 4096, 8192, 0.25), (0.9, 4096, 8192, 0.25),
    (0.5, 1000, 1000, 0.25), (0.2, 300, 50000, 0.125), (0.7, 20000, 30000, 1.0),
    (0.01, 8192, 8192, 0.25)])
def test_optimal_shard_meets_the_constraint_and_minimises_communication(alpha, L_q, L_kv, beta):
    nq, nkv = S.optimal_shard(alpha, L_q, L_kv, beta)
    C = alpha * L_q * (2.0 * L_kv - L_q)
    assert abs(nq * (2 * nkv - nq) - C) <= 1e-9 * C
    assert 0 < nq <= L_q + 1e-6 and nq + L_kv - L_q - 1e-6 <= nkv <= L_kv + 1e-6
    ref = brute_optimal_shard(alpha, L_q, L_kv, beta)
    assert nq + beta * nkv <= ref[0] + 1e-6 * ref[0]


def test_optimal_shard_interior_matches_the_pages_closed_form():
    """Where the optimum is interior it is sqrt(alpha beta L_q (2 L_kv - L_q) /
    (beta + 2)) — stated as a number here: alpha 0.25, beta 0.25, L_q 4096,
    L_kv 8192 give sqrt(0.0625 * 4096 * 12288 / 2.25) = sqrt(1398101.33) = 1182.413;
    checked against the brute-force minimiser, not the formula."""
    nq, _ = S.optimal_shard(0.25, 4096, 8192, 0.25)
    ref = brute_optimal_shard(0.25, 4096, 8192, 0.25, steps=400000)
    assert abs(nq - ref[1]) < 0.05
    assert abs(nq - 1182.413) < 0.001


def test_round_shard_stays_feasible():
    rng = random.Random(5)
    for _ in range(2000):
        L_kv = rng.randint(1, 100000)
        L_q = rng.randint(1, L_kv)
        nq = rng.uniform(0.0, L_q * 1.2)
        nkv = rng.uniform(0.0, L_kv * 1.2)
        n_q, n_kv = S.round_shard(nq, nkv, L_q, L_kv)
        assert 1 <= n_q <= L_q and n_q + L_kv - L_q <= n_kv <= L_kv


def check_partition(items, doc_lens):
    per_doc = {}
    for srv, doc, a, b in items:
        assert 0 <= a < b <= doc_lens[doc]
        per_doc.setdefault(doc, []).append((a, b))
    for doc, L in enumerate(doc_lens):
        rs = sorted(per_doc.get(doc, []))
        assert rs[0][0] == 0 and rs[-1][1] == L
        for (a0, b0), (a1, b1) in zip(rs, rs[1:]):
            assert b0 == a1


def test_initial_items_place_equal_token_blocks():
    docs = [5000, 100, 12000, 900, 30000]
    k = 4
    items = S.initial_items(docs, k)
    check_partition(items, docs)
    per = -(-sum(docs) // k)
    tok = [0] * k
    for srv, doc, a, b in items:
        tok[srv] += b - a
    assert tok[:-1] == [per] * (k - 1) and sum(tok) == sum(docs)
    # devices take the packed stream in order
    order = [(srv, doc, a) for srv, doc, a, b in items]
    assert order == sorted(order, key=lambda x: (x[1], x[2]))


def flops_model():
    return S.CostModel([1024], [4096], [[1.0e-3]], 4 * 128 * 32)


def test_two_servers_one_document_by_hand():
    """k = 2, one 8192-token document, FLOPs-proportional cost: device 0
    holds queries [0, 4096) (8,390,656 pairs), device 1 [4096, 8192)
    (25,167,872 pairs); the target is 16,779,264 pairs each.  One split of
    device 1's Item moves the surplus; the result is balanced to within one
    percent, with the whole query range still partitioned."""
    m = flops_model()
    docs = [8192]
    items, before, after, comm, moves = S.schedule(docs, 2, m, 32, 8, 128, eps=0.01)
    unit = m.flops(1, 1) / m.peak          # seconds per visible pair
    assert abs(before[0] / unit - 8390656) < 1e-3
    assert abs(before[1] / unit - 25167872) < 1e-3
    tgt = (before[0] + before[1]) / 2
    assert moves == 1 and all(abs(x - tgt) <= 0.01 * tgt for x in after)
    check_partition(items, docs)
    moved = [it for it in items if it[0] == 0 and it[2] >= 4096]
    assert len(moved) == 1
    _, _, a, b = moved[0]
    # the moved shard satisfies Appendix B's constraint for its alpha, rounded
    alpha = (tgt - before[0]) / before[1]
    C = alpha * 4096 * (2 * 8192 - 4096)
    n_q, n_kv = b - a, b
    assert abs(n_q * (2 * n_kv - n_q) - C) <= 2 * (2 * n_kv) + 2 * n_q
    # communication = n_q s_q + n_kv s_kv
    assert comm == n_q * 32 * 128 * 2 + n_kv * 8 * 128 * 2


def loads_of(items, k, m):
    load = [0.0] * k
    for srv, doc, a, b in items:
        load[srv] += m.time(b - a, b)
    return load


@pytest.mark.parametrize("seed", range(6))
def test_schedule_invariants(seed):
    rng = random.Random(seed)
    docs = [int(math.exp(rng.uniform(math.log(64), math.log(60000)))) for _ in range(rng.randint(3, 40))]
    k = rng.choice([2, 4, 8])
    gq = [64, 256, 1024, 4096, 16384]
    gkv = [64, 512, 4096, 32768, 65536]
    times = [[2e-5 + 4 * 128 * 32 * S.block_pairs(x, max(x, y)) / (8e14 * (1 - 0.5 * math.exp(-x / 300.0)))
              for y in gkv] for x in gq]
    m = S.CostModel(gq, gkv, times, 4 * 128 * 32)
    eps = 0.05
    items, before, after, comm, moves = S.schedule(docs, k, m, 32, 8, 128, eps=eps)
    check_partition(items, docs)
    # returned loads are the loads of the returned items
    for x, y in zip(after, loads_of(items, k, m)):
        assert abs(x - y) <= 1e-9 * max(1e-12, y)
    tgt = sum(before) / k
    # no server ends further below the target than it started (deficits only shrink)
    for s in range(k):
        if before[s] < tgt:
            assert after[s] >= before[s] - 1e-12
    assert max(after) <= max(before) + 1e-12
    # every migrated shard (other than whole Items) is at least min_shard queries
    init = {(d, a, b) for _, d, a, b in S.initial_items(docs, k)}
    for srv, d, a, b in items:
        if (d, a, b) not in init:
            assert b - a >= 1
    # communication is the sum over moves of n_q s_q + n_kv s_kv: nonnegative, zero iff no move
    assert (comm == 0) == (moves == 0)


def test_greedy_choice_is_the_best_candidate_by_brute_force():
    """The first migration equals the argmax of E over every (Item, split)
    candidate, recomputed here from its parts."""
    m = flops_model()
    docs = [3000, 20000, 500, 9000, 700, 15000]
    k = 3
    s_q, s_kv = 32 * 128 * 2, 8 * 128 * 2
    items0 = S.initial_items(docs, k)
    load = loads_of(items0, k, m)
    tgt = sum(load) / k
    dst = min(range(k), key=lambda s: (load[s] - tgt, s))
    D = tgt - load[dst]
    cands = []
    for idx, (srv, doc, a, b) in enumerate(items0):
        Ssur = load[srv] - tgt
        if srv == dst or Ssur <= 0:
            continue
        Ft = m.time(b - a, b)
        dF = min(Ft, Ssur, D)
        if dF == Ft:
            n_q, n_kv = b - a, b
        else:
            nq, nkv = S.optimal_shard(dF / Ft, b - a, b, 0.25)
            n_q, n_kv = S.round_shard(nq, nkv, b - a, b)
            if n_q < 128 and n_q != b - a:
                continue
        cands.append((dF / (n_q * s_q + n_kv * s_kv), -srv, -idx, doc, n_kv - n_q, n_kv))
    best = max(cands)
    items, before, after, comm, moves = S.schedule(docs, k, m, 32, 8, 128, eps=0.05, max_moves=1)
    moved = [it for it in items if it[0] == dst and tuple(it) not in {tuple(x) for x in items0}]
    assert moves == 1 and len(moved) == 1
    assert (moved[0][1], moved[0][2], moved[0][3]) == (best[3], best[4], best[5])


def brute_range_pairs(a, b):
    """Visible pairs of queries [a, b) of a causal document, one by one."""
    return sum(1 for p in range(a, b) for key in range(b) if key <= p)


@pytest.mark.parametrize("a,b,m", [(0, 2, 1), (0, 10, 3), (5, 17, 6), (100, 131, 7), (0, 64, 32), (3, 5, 1)])
def test_head_tail_pairs_brute_force(a, b, m):
    """The head [a, a + m) plus the tail [b - m, b) of an Item, counted key by
    key, equal m (a + b + 1) — the per-document balance of a head-tail shard."""
    assert S.head_tail_pairs(a, b, m) == brute_range_pairs(a, a + m) + brute_range_pairs(b - m, b)
    # and the middle holds the rest of the Item's pairs
    assert (brute_range_pairs(a, b) - S.head_tail_pairs(a, b, m)
            == (brute_range_pairs(a + m, b - m) if b - m > a + m else 0))


def test_head_tail_shard_holds_the_requested_fraction():
    """m from alpha rounds to the nearest integer, so the shard's share of the
    Item's pairs is within (a + b + 1) / 2 pairs of alpha times the Item, and
    the clamps hold at both ends."""
    rng = random.Random(11)
    for _ in range(3000):
        a = rng.randint(0, 50000)
        b = a + rng.randint(2, 50000)
        alpha = rng.uniform(0.0, 1.0)
        m = S.head_tail_shard(alpha, a, b)
        assert 1 <= m <= (b - a) // 2
        want = alpha * brute_pairs_closed(a, b)
        if 1 < m < (b - a) // 2:
            assert abs(S.head_tail_pairs(a, b, m) - want) <= (a + b + 1) / 2.0 + 1e-6 * want
    assert S.head_tail_shard(0.0, 0, 1000) == 1
    assert S.head_tail_shard(1.0, 0, 1001) == 500


def brute_pairs_closed(a, b):
    """(b - a)(a + b + 1) / 2: pairs of queries [a, b), context [0, b)."""
    return (b - a) * (a + b + 1) / 2.0


def test_two_servers_head_tail_by_hand():
    """k = 2, one 4000-token document, FLOPs-proportional cost, head-tail
    shards.  Device 0 holds [0, 2000) (2,001,000 pairs), device 1 [2000, 4000)
    (6,001,000 pairs); the target is 4,001,000.  alpha = 2,000,000 / 6,001,000
    gives m = round(333.28) = 333: device 1 sends [2000, 2333) and
    [3667, 4000), 333 * 6001 = 1,998,333 pairs, and keeps [2333, 3667).
    Device 0 ends at 3,999,333 pairs and device 1 at 4,002,667, within the
    one-percent tolerance, so there is no second move."""
    m = flops_model()
    unit = m.flops(1, 1) / m.peak
    items, before, after, comm, moves = S.schedule([4000], 2, m, 32, 8, 128, eps=0.01, head_tail=True)
    assert abs(before[0] / unit - 2001000) < 1e-3 and abs(before[1] / unit - 6001000) < 1e-3
    assert moves == 1
    assert abs(after[0] / unit - 3999333) < 1e-3 and abs(after[1] / unit - 4002667) < 1e-3
    assert items == [[0, 0, 0, 2000], [1, 0, 2333, 3667], [0, 0, 2000, 2333], [0, 0, 3667, 4000]]
    # the shard sends 666 queries and the 4000-row context
    assert comm == 666 * 32 * 128 * 2 + 4000 * 8 * 128 * 2


@pytest.mark.parametrize("seed", range(6))
def test_head_tail_schedule_invariants(seed):
    rng = random.Random(100 + seed)
    docs = [int(math.exp(rng.uniform(math.log(64), math.log(60000)))) for _ in range(rng.randint(3, 40))]
    k = rng.choice([2, 4, 8])
    m = flops_model()
    eps = 0.05
    items, before, after, comm, moves = S.schedule(docs, k, m, 32, 8, 128, eps=eps, head_tail=True)
    check_partition(items, docs)
    for x, y in zip(after, loads_of(items, k, m)):
        assert abs(x - y) <= 1e-9 * max(1e-12, y)
    tgt = sum(before) / k
    for s in range(k):
        if before[s] < tgt:
            assert after[s] >= before[s] - 1e-12
    assert max(after) <= max(before) + 1e-12
    assert (comm == 0) == (moves == 0)
    # every split left its pieces as head/tail pairs of equal width on one server
    init = {(d, a, b) for _, d, a, b in S.initial_items(docs, k)}
    new = [it for it in items if (it[1], it[2], it[3]) not in init]
    assert all(b - a >= 1 for _, _, a, b in new)


def test_head_tail_balances_a_long_document_better_than_contiguous_halves():
    """One 65536-token document on 4 servers: head-tail shards reach the
    tolerance, and each server's pair count is within eps of the target."""
    m = flops_model()
    items, before, after, comm, moves = S.schedule([65536], 4, m, 32, 8, 128, eps=0.02, head_tail=True)
    tgt = sum(before) / 4
    assert max(after) <= 1.02 * tgt + 1e-12 and min(after) >= 0.98 * tgt - 1e-12
    check_partition(items, [65536])
