"""The C-ABI scheduler (libca ca_schedule / ca_cost_time / ca_sched_tasks)
against the oracle (oracle/scheduler.py): identical decisions, identical
loads and bytes, on randomised batches and cost grids.  Host code only: runs
without a GPU."""

import math
import random

import numpy as np
import pytest

from oracle import scheduler as S
from long_context_core_amd import ca

FPP = 4 * 128 * 32          # forward FLOPs per visible pair, Llama-3-8B heads


def random_grid(rng):
    gq = sorted({rng.choice([1, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096, 8192, 16384])
                 for _ in range(rng.randint(1, 6))})
    gkv = sorted({rng.choice([1, 64, 256, 1024, 4096, 8192, 16384, 32768, 65536, 131072])
                  for _ in range(rng.randint(1, 6))})
    times = [[1e-5 + FPP * S.block_pairs(min(int(x), int(y)), int(y)) /
              (9e14 * (1.0 - 0.6 * math.exp(-x / rng.uniform(50, 500))) * rng.uniform(0.9, 1.1))
              for y in gkv] for x in gq]
    return gq, gkv, times


def test_cost_model_matches_oracle_exactly():
    rng = random.Random(11)
    for _ in range(30):
        gq, gkv, times = random_grid(rng)
        m = S.CostModel(gq, gkv, times, FPP)
        for _ in range(60):
            kv = rng.randint(1, 300000)
            q = rng.randint(1, kv)
            assert ca.cost_time(gq, gkv, times, FPP, q, kv) == m.time(q, kv)


def run_both(docs, k, gq, gkv, times, **kw):
    m = S.CostModel(gq, gkv, times, FPP)
    o_items, o_before, o_after, o_comm, o_moves = S.schedule(docs, k, m, 32, 8, 128, **kw)
    items, before, after, comm, moves = ca.schedule(docs, k, gq, gkv, times, FPP, 32, 8, 128, **kw)
    return (o_items, o_before, o_after, o_comm, o_moves), (items, before, after, comm, moves)


@pytest.mark.parametrize("head_tail", [False, True])
@pytest.mark.parametrize("seed", range(40))
def test_schedule_matches_oracle_exactly(seed, head_tail):
    rng = random.Random(1000 + seed)
    n = rng.randint(1, 60)
    docs = [int(math.exp(rng.uniform(math.log(1), math.log(200000)))) for _ in range(n)]
    if rng.random() < 0.2:
        docs[rng.randrange(n)] = 0                      # empty document
    k = rng.choice([1, 2, 3, 4, 8, 16])
    gq, gkv, times = random_grid(rng)
    kw = dict(eps=rng.choice([0.0, 0.01, 0.05, 0.2]), min_shard=rng.choice([1, 64, 128, 512]),
              max_moves=rng.choice([0, 1, 5, 10000]), head_tail=head_tail)
    o, c = run_both(docs, k, gq, gkv, times, **kw)
    o_items, o_before, o_after, o_comm, o_moves = o
    items, before, after, comm, moves = c
    assert [tuple(x) for x in o_items] == [(int(r["server"]), int(r["doc"]), int(r["q_begin"]), int(r["q_end"]))
                                           for r in items]
    assert list(before) == o_before and list(after) == o_after
    assert comm == o_comm and moves == o_moves


@pytest.mark.parametrize("head_tail", [False, True])
def test_prolong_like_batch_on_eight_servers(head_tail):
    """A 512K-token batch with the training mix on 8 servers: identical to the
    oracle, balanced to eps, and the query positions of every document are
    covered exactly once by the task records (contiguous or head-tail
    shards)."""
    from long_context_core_amd import inputs as I
    w = I.train_8b_prolong_512k()
    docs = [int(x) for x in w.doc_lens]
    gq = [128, 512, 2048, 8192, 32768]
    gkv = [128, 1024, 8192, 65536, 524288]
    times = [[2e-5 + FPP * S.block_pairs(min(x, y), y) / 1.0e15 for y in gkv] for x in gq]
    o, c = run_both(docs, 8, gq, gkv, times, eps=0.02, head_tail=head_tail)
    assert [tuple(x) for x in o[0]] == [tuple(int(v) for v in r) for r in c[0]]
    after = c[2]
    tgt = sum(c[1]) / 8
    assert max(after) <= (1 + 0.02) * tgt * 1.001 + 1e-12 or max(after) < max(c[1])
    tasks = ca.sched_tasks(c[0], docs)
    rows, _ = S.task_rows(o[0], docs)
    assert [tuple(int(r[f]) for f in ca.TASK_DTYPE.names) for r in tasks] == [tuple(r) for r in rows]
    cover = np.zeros(sum(docs), dtype=np.int32)
    for t in tasks:
        cover[t["q_off"]:t["q_off"] + t["q_len"]] += 1
    assert (cover == 1).all()
    assert ca.visible_pairs(tasks) == ca.visible_pairs(ca.task_array(I.varlen_tasks(docs)))


def test_schedule_errors():
    gq, gkv, times = [128, 1024], [1024, 8192], [[1e-4, 5e-4], [6e-4, 2e-3]]
    with pytest.raises(ca.CAError):
        ca.schedule([100, 200], 0, gq, gkv, times, FPP, 32, 8, 128)           # k < 1
    with pytest.raises(ca.CAError):
        _raw_schedule(head_tail=2)                                           # flag not 0 / 1
    with pytest.raises(ca.CAError):
        ca.schedule([100, -5], 2, gq, gkv, times, FPP, 32, 8, 128)           # negative length
    with pytest.raises(ca.CAError):
        ca.schedule([100], 2, [1024, 128], gkv, times, FPP, 32, 8, 128)      # grid not increasing
    with pytest.raises(ca.CAError):
        ca.schedule([100], 2, gq, gkv, [[1e-4, 0.0], [6e-4, 2e-3]], FPP, 32, 8, 128)   # time 0
    with pytest.raises(ca.CAError):
        ca.schedule([100], 2, gq, gkv, [[1e-4, float("nan")], [6e-4, 2e-3]], FPP, 32, 8, 128)
    assert math.isnan(ca.cost_time(gq, gkv, [[1e-4, float("inf")], [6e-4, 2e-3]], FPP, 10, 10))
    bad = np.zeros(1, dtype=ca.SCHED_ITEM_DTYPE)
    bad[0] = (0, 0, 10, 400)
    with pytest.raises(ca.CAError):
        ca.sched_tasks(bad, [300])                                            # past the document


def test_schedule_workspace_error_reports_the_count():
    """ca_schedule with too small an Item buffer fails cleanly and says how
    many Items it needed."""
    import ctypes
    L = ca.lib()
    docs = np.array([8192, 100, 5000], dtype=np.int64)
    g = np.array([1024.0]), np.array([4096.0]), np.array([1e-3])
    p = ca.SchedParams(2, 32, 8, 128, 0.01, 0.0, 128, 100, 0, float(FPP))
    items = np.zeros(1, dtype=ca.SCHED_ITEM_DTYPE)
    bf, af = np.zeros(2), np.zeros(2)
    n, comm, mv = ctypes.c_int32(0), ctypes.c_double(0), ctypes.c_int32(0)
    st = L.ca_schedule(ctypes.byref(p), docs.ctypes.data, 3, g[0].ctypes.data, 1, g[1].ctypes.data, 1,
                       g[2].ctypes.data, items.ctypes.data, 1, ctypes.byref(n), bf.ctypes.data, af.ctypes.data,
                       ctypes.byref(comm), ctypes.byref(mv))
    assert st == ca.CA_ERR_WORKSPACE and n.value > 1


def _raw_schedule(head_tail):
    import ctypes
    L = ca.lib()
    docs = np.array([8192, 100], dtype=np.int64)
    g = np.array([1024.0]), np.array([4096.0]), np.array([1e-3])
    p = ca.SchedParams(2, 32, 8, 128, 0.01, 0.0, 128, 100, head_tail, float(FPP))
    items = np.zeros(64, dtype=ca.SCHED_ITEM_DTYPE)
    bf, af = np.zeros(2), np.zeros(2)
    n, comm, mv = ctypes.c_int32(0), ctypes.c_double(0), ctypes.c_int32(0)
    st = L.ca_schedule(ctypes.byref(p), docs.ctypes.data, 2, g[0].ctypes.data, 1, g[1].ctypes.data, 1,
                       g[2].ctypes.data, items.ctypes.data, 64, ctypes.byref(n), bf.ctypes.data, af.ctypes.data,
                       ctypes.byref(comm), ctypes.byref(mv))
    if st != ca.CA_OK:
        raise ca.CAError(st, "ca_schedule")
    return items[:n.value]


def test_head_tail_flag_layout():
    """head_tail sits in the struct's former padding: 0 and 1 are accepted and
    flops_per_pair keeps its offset."""
    import ctypes
    assert ca.SchedParams.flops_per_pair.offset == 48 and ctypes.sizeof(ca.SchedParams) == 56
    assert len(_raw_schedule(0)) >= 2 and len(_raw_schedule(1)) >= 2
