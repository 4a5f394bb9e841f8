"""Pins of the ring-planning oracle (oracle/ring.py) against the values the
pages print and against algebra and brute force — "Context Parallelism for
Scalable Million-Token Inference", Section 3.4 (Equations 1-3, Algorithm 1),
Appendix C (Equation 5), Section 3.5.1 (load-balanced sharding), Section 3.5.2
(pass-KV ring), Section 3.6 (round-robin decode sharding), Tables 4-5."""

import random

import pytest

from oracle import ring as R


def llama405b(N=4, C=8.0e14, BW=5.0e10, e=2):
    return R.RingModel(N, 128, 8, e, 16384, C, BW)


def test_equation1_threshold_values_the_pages_print():
    """12.5 % for Llama3 405B (128 query heads, 8 KV heads); 50 % for a model
    with 32 query heads and 8 KV heads."""
    assert llama405b().miss_threshold() == 0.125
    assert R.RingModel(4, 32, 8, 2, 4096, 1e15, 1e11).miss_threshold() == 0.5


def test_table5_measured_comparison():
    """Table 5 at 2.5 % miss (T = 3200, 4 ranks): pass-KV exposes
    3 x (627 - 414) = 639 us, pass-Q only its 424 us All2All -> pass-Q.
    At 10 % miss (T = 12800): pass-KV exposes nothing, pass-Q 1023 us ->
    pass-KV."""
    c, k, q = R.select_measured(4, 627e-6, 166e-6, 414e-6, 424e-6)
    assert c == R.PASS_Q and abs(k - 639e-6) < 1e-12 and abs(q - 424e-6) < 1e-12
    c, k, q = R.select_measured(4, 631e-6, 544e-6, 1608e-6, 1023e-6)
    assert c == R.PASS_KV and k == 0.0 and abs(q - 1023e-6) < 1e-12


@pytest.mark.parametrize("seed", range(5))
def test_equation2_threshold_balances_a_pass_kv_step(seed):
    """At T equal to the Equation 2 threshold, a pass-KV step's attention time
    equals its SendRecv time for every P (the (T + P) factors cancel); below
    it the SendRecv is longer, above it shorter."""
    rng = random.Random(seed)
    m = R.RingModel(rng.choice([2, 4, 8, 16]), rng.choice([32, 64, 128]), rng.choice([1, 4, 8]),
                    rng.choice([1, 2]), rng.choice([4096, 8192, 16384]), rng.uniform(1e14, 3e15),
                    rng.uniform(2e10, 4e11))
    T = m.t_threshold()
    for P in (0.0, 1000.0, 123456.0, 1e6):
        a, s = m.attn_step(T, P), m.sendrecv_kv(T, P)
        assert abs(a - s) <= 1e-12 * s
        assert m.attn_step(0.5 * T, P) < m.sendrecv_kv(0.5 * T, P)
        assert m.attn_step(2.0 * T, P) > m.sendrecv_kv(2.0 * T, P)


def test_equation3_threshold_balances_a_pass_q_step():
    m = llama405b(N=8, C=1.1e15, BW=1.5e11)
    ctx = m.ctx_threshold()
    for T in (1.0, 100.0, 0.5 * ctx):
        P = ctx - T
        assert abs(m.attn_step(T, P) - m.sendrecv_q(T, P)) <= 1e-12 * m.sendrecv_q(T, P)


@pytest.mark.parametrize("seed", range(5))
def test_equation5_is_the_exposed_time_comparison(seed):
    """exposed pass-KV - All2All = (N - 1)(T + P) D e / BW x (rhs(T) -
    T/(T + P) (D + 1)/D): Equation 5 is the time comparison with (D + 1)/D
    taken as 1.  Checked as an identity, and the two selections agree
    wherever the miss rate is not within that factor of the boundary."""
    rng = random.Random(100 + seed)
    m = R.RingModel(rng.choice([2, 4, 8]), 128, 8, rng.choice([1, 2]), 16384, rng.uniform(2e14, 2e15),
                    rng.uniform(2e10, 2e11))
    for _ in range(500):
        T = rng.randint(1, 200000)
        P = rng.randint(0, 500000)
        lhs = m.exposed_kv(T, P) - m.all2all(T)
        miss = T / (T + P)
        rhs = (m.N - 1) * (T + P) * m.D * m.e / m.BW * (m.eq5_rhs(T) - miss * (m.D + 1) / m.D)
        assert abs(lhs - rhs) <= 1e-9 * max(abs(lhs), abs(rhs), 1e-12)
        if abs(m.eq5_rhs(T) - miss) > 2 * miss / m.D:
            assert R.select_eq5(m, T, P) == R.select_refined(m, T, P)


def test_decode_and_full_prefill_choices():
    """Decode (T = 1 over a long cache) is far below the miss-rate threshold
    and picks pass-Q in both heuristics; full prefill (P = 0) has miss rate 1
    and picks pass-KV."""
    m = llama405b()
    assert R.select_simple(m, 1, 131071) == R.PASS_Q and R.select_refined(m, 1, 131071) == R.PASS_Q
    assert R.select_simple(m, 128000, 0) == R.PASS_KV and R.select_refined(m, 128000, 0) == R.PASS_KV


def test_sharding_example_the_pages_print():
    """N = 4: rank 0 holds (C0, C7), rank 1 (C1, C6), rank 2 (C2, C5), rank 3
    (C3, C4)."""
    ch = R.shard([800], 4)
    owner = {k: rank for k, (rank, s, b, e) in enumerate(ch)}
    assert [sorted(k for k in owner if owner[k] == r) for r in range(4)] == [[0, 7], [1, 6], [2, 5], [3, 4]]
    assert [(b, e) for _, _, b, e in ch] == [(100 * k, 100 * k + 100) for k in range(8)]


@pytest.mark.parametrize("N,lens", [(2, [8, 20, 4]), (4, [64, 800, 8]), (8, [160, 1600]), (3, [60, 36])])
def test_sharding_balances_causal_pairs_exactly_when_lengths_divide(N, lens):
    """With every length a multiple of 2N, each rank holds L / N tokens of
    each sequence and exactly the same causal pairs, c (2 N c + 1) per
    sequence for chunk length c, counted here key by key."""
    load = [0] * N
    tokens = [0] * N
    for rank, s, b, e in R.shard(lens, N):
        load[rank] += sum(p + 1 for p in range(b, e))
        tokens[rank] += e - b
    assert len(set(load)) == 1 and len(set(tokens)) == 1
    c_terms = sum((L // (2 * N)) * (2 * N * (L // (2 * N)) + 1) for L in lens)
    assert load[0] == c_terms
    assert R.rank_pairs(lens, N) == load


@pytest.mark.parametrize("seed", range(6))
def test_sharding_partitions_padded_sequences(seed):
    """Any lengths: every position of every sequence lies in exactly one chunk,
    every rank holds two chunks per sequence, and token counts differ by at
    most the padding 2 c - 2 of one sequence per sequence."""
    rng = random.Random(seed)
    N = rng.choice([1, 2, 3, 4, 8])
    lens = [rng.randint(0, 3000) for _ in range(rng.randint(1, 6))]
    ch = R.shard(lens, N)
    assert len(ch) == 2 * N * len(lens)
    for s, L in enumerate(lens):
        cover = [0] * L
        per_rank = [0] * N
        for rank, ss, b, e in ch:
            if ss != s:
                continue
            per_rank[rank] += 1
            for p in range(b, e):
                cover[p] += 1
        assert all(x == 1 for x in cover) and per_rank == [2] * N
    tok = [0] * N
    for rank, s, b, e in ch:
        tok[rank] += e - b
    slack = sum(max(0, 2 * R.chunk_len(L, N) - 2) for L in lens)
    assert max(tok) - min(tok) <= slack


@pytest.mark.parametrize("N", [1, 2, 4, 8])
def test_pass_kv_ring_meets_every_source_once(N):
    for r in range(N):
        assert sorted(R.kv_step_source(r, s, N) for s in range(N)) == list(range(N))
        assert R.kv_step_source(r, 0, N) == r


@pytest.mark.parametrize("N,B", [(4, 32), (4, 6), (8, 3), (3, 7)])
def test_round_robin_decode_balances_over_iterations(N, B):
    """Over any N consecutive iterations every rank receives exactly one
    token of each batch entry; within one iteration the ranks receive
    floor(B / N) or ceil(B / N) tokens."""
    for t0 in (0, 5, 17):
        for b in range(B):
            assert sorted(R.decode_rank(b, t, N) for t in range(t0, t0 + N)) == list(range(N))
        counts = [0] * N
        for b in range(B):
            counts[R.decode_rank(b, t0, N)] += 1
        assert max(counts) - min(counts) <= 1
