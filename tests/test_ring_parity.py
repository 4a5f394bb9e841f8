"""The C-ABI ring planning calls (libca ca_ring_*) against the oracle
(oracle/ring.py): identical time-model terms, identical choices, identical
chunks and pass-KV task tables, on randomised models and batches.  Host code
only: runs without a GPU."""

import random

import numpy as np
import pytest

from oracle import ring as R
from long_context_core_amd import ca


def random_model(rng):
    args = (rng.choice([1, 2, 3, 4, 8, 16]), rng.choice([8, 32, 64, 128]), rng.choice([1, 2, 4, 8]),
            rng.choice([1, 2]), rng.choice([2048.0, 4096.0, 16384.0]), rng.uniform(1e14, 3e15),
            rng.uniform(1e10, 5e11))
    return R.RingModel(*args), ca.ring_model(*args)


@pytest.mark.parametrize("seed", range(10))
def test_time_model_and_choices_match_the_oracle_exactly(seed):
    rng = random.Random(seed)
    om, cm = random_model(rng)
    for _ in range(200):
        T = rng.randint(1, 300000)
        P = rng.choice([0, rng.randint(0, 1000), rng.randint(0, 2000000)])
        got = ca.ring_plan(cm, T, P)
        want = {"attn_step": om.attn_step(T, P), "sendrecv_kv": om.sendrecv_kv(T, P),
                "sendrecv_q": om.sendrecv_q(T, P), "all2all": om.all2all(T), "exposed_kv": om.exposed_kv(T, P),
                "miss_threshold": om.miss_threshold(), "t_threshold": om.t_threshold(),
                "ctx_threshold": om.ctx_threshold(), "eq5_rhs": om.eq5_rhs(T)}
        assert got == want
        assert ca.ring_select(cm, T, P, refined=False) == R.select_simple(om, T, P)
        assert ca.ring_select(cm, T, P, refined=True) == R.select_refined(om, T, P)


def test_measured_choice_matches_the_oracle():
    rng = random.Random(3)
    for _ in range(500):
        args = (rng.randint(1, 16), rng.uniform(0, 1e-3), rng.uniform(0, 1e-3), rng.uniform(0, 1e-3),
                rng.uniform(0, 1e-3))
        assert ca.ring_select_measured(*args) == R.select_measured(*args)
    # the pages' Table 5 through the C ABI
    c, k, q = ca.ring_select_measured(4, 627e-6, 166e-6, 414e-6, 424e-6)
    assert c == ca.RING_PASS_Q and abs(k - 639e-6) < 1e-12


@pytest.mark.parametrize("seed", range(6))
def test_shard_and_pass_kv_tables_match_the_oracle(seed):
    rng = random.Random(50 + seed)
    N = rng.choice([1, 2, 3, 4, 8])
    lens = [rng.choice([0, rng.randint(1, 50), rng.randint(1, 5000)]) for _ in range(rng.randint(1, 7))]
    got = ca.ring_shard(lens, N)
    assert [tuple(int(x) for x in r) for r in got] == R.shard(lens, N)
    starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    chunks = R.shard(lens, N)
    for step in range(N):
        for slot in (0, 1):
            want = []
            for r in range(N):
                src = R.kv_step_source(r, step, N)
                kc = src if slot == 0 else 2 * N - 1 - src
                for s in range(len(lens)):
                    _, _, kb, ke = chunks[s * 2 * N + kc]
                    for qc in (r, 2 * N - 1 - r):
                        _, _, qb, qe = chunks[s * 2 * N + qc]
                        if qe > qb:
                            want.append((starts[s] + qb, starts[s] + kb, starts[s] + qb, qe - qb, ke - kb, qb, kb))
            tasks = ca.ring_kv_step_tasks(lens, N, step, slot)
            assert [tuple(int(t[f]) for f in ca.TASK_DTYPE.names) for t in tasks] == want
            # every query row of the batch appears exactly once per (step, slot)
            cover = np.zeros(int(starts[-1]), dtype=np.int32)
            for t in tasks:
                cover[t["q_off"]:t["q_off"] + t["q_len"]] += 1
            assert (cover == 1).all()


def test_decode_rank_matches_the_oracle():
    for N in (1, 3, 4, 8):
        for t in (0, 1, 7, 12345):
            for b in range(20):
                assert ca.ring_decode_rank(N, t, b) == R.decode_rank(b, t, N)


def test_ring_errors():
    cm = ca.ring_model(4, 128, 8, 2, 16384.0, 1e15, 1e11)
    with pytest.raises(ca.CAError):
        ca.ring_select(cm, 0, 10)                                         # T < 1
    with pytest.raises(ca.CAError):
        ca.ring_plan(ca.ring_model(0, 128, 8, 2, 16384.0, 1e15, 1e11), 10, 10)   # no ranks
    with pytest.raises(ca.CAError):
        ca.ring_plan(ca.ring_model(4, 128, 8, 2, 16384.0, 0.0, 1e11), 10, 10)    # no compute
    with pytest.raises(ca.CAError):
        ca.ring_shard([10, -1], 4)
    with pytest.raises(ca.CAError):
        ca.ring_kv_step_tasks([100], 4, 4, 0)                               # step out of range
    with pytest.raises(ca.CAError):
        ca.ring_kv_step_tasks([100], 4, 0, 2)                               # slot out of range
    with pytest.raises(ca.CAError):
        ca.ring_decode_rank(0, 1, 1)


@pytest.mark.parametrize("seed", range(5))
def test_partial_prefill_tables_match_the_oracle_and_cover_every_pair_once(seed):
    """Partial prefill: the C tables equal a construction from the oracle's
    sharding (new tokens and cached tokens each sharded load-balanced), and
    over the 4N (step, slot) tables every new query meets each key of its
    sequence it may see (positions <= its own) exactly once, counted key by
    key on small sizes."""
    rng = random.Random(300 + seed)
    N = rng.choice([1, 2, 3, 4])
    n_seq = rng.randint(1, 4)
    new = [rng.choice([0, 1, rng.randint(1, 90)]) for _ in range(n_seq)]
    cached = [rng.choice([0, rng.randint(1, 120)]) for _ in range(n_seq)]
    q_start = np.concatenate([[0], np.cumsum(new)]).astype(np.int64)
    kv_start = np.concatenate([[0], np.cumsum(np.array(new) + np.array(cached))]).astype(np.int64)
    ch_new, ch_old = R.shard(new, N), R.shard(cached, N)
    seen = {}
    for step in range(N):
        for slot in range(4):
            want = []
            for r in range(N):
                src = R.kv_step_source(r, step, N)
                kc = src if slot % 2 == 0 else 2 * N - 1 - src
                for s in range(n_seq):
                    P = cached[s]
                    if slot < 2:
                        _, _, kb, ke = ch_old[s * 2 * N + kc]
                    else:
                        _, _, kb, ke = ch_new[s * 2 * N + kc]
                        kb, ke = P + kb, P + ke
                    for qc in (r, 2 * N - 1 - r):
                        _, _, qb, qe = ch_new[s * 2 * N + qc]
                        if qe > qb:
                            want.append((q_start[s] + qb, kv_start[s] + kb, q_start[s] + qb, qe - qb, ke - kb,
                                         P + qb, kb))
            tasks = ca.ring_prefill_step_tasks(new, cached, N, step, slot)
            got = [tuple(int(t[f]) for f in ca.TASK_DTYPE.names) for t in tasks]
            assert got == want
            for q_off, kv_off, _, q_len, kv_len, q_pos0, kv_pos0 in got:
                for i in range(q_len):
                    for j in range(kv_len):
                        if kv_pos0 + j <= q_pos0 + i:
                            key = (q_off + i, kv_off + j)
                            seen[key] = seen.get(key, 0) + 1
    assert all(v == 1 for v in seen.values())
    # every query row sees exactly the keys of its sequence at positions <= its own
    for s in range(n_seq):
        for i in range(new[s]):
            row = q_start[s] + i
            n_keys = sum(1 for (q, k) in seen if q == row)
            assert n_keys == cached[s] + i + 1
