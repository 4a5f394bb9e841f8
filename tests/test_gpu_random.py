"""Seeded random CA-task tables through the forward and the backward, against
the fp64 oracle element by element.  The tables mix what the fixed cases
cover one at a time: empty and single-row query shards (single rows go to
the split-KV decode kernel, the rest to the tiled kernel, in one call),
empty contexts, queries positioned before their first key (rows with no
visible key), contexts shorter or longer than the shard, K/V ranges shared
between tasks, and every GQA grouping at d = 64 and 128; each table also runs
with a random sink + sliding-window mask per task."""

import math

import numpy as np
import pytest

import oracle
from long_context_core_amd import ca
from long_context_core_amd import inputs as I
from tests.gpu_util import GRAD_REL_FRO, announce, check_forward, rel_fro, torch_cuda, widen

pytestmark = pytest.mark.gpu

GEOMETRIES = [(8, 2), (4, 4), (16, 1), (6, 2), (12, 4), (32, 8), (8, 4), (16, 2)]


def random_tables(seed):
    rng = np.random.default_rng(9000 + seed)
    hq, hkv = GEOMETRIES[seed % len(GEOMETRIES)]
    d = (64, 128)[(seed // len(GEOMETRIES)) % 2]
    kv_rows = int(rng.integers(200, 1500))
    rows, q0 = [], 0
    for _ in range(int(rng.integers(1, 7))):
        q_len = int(rng.choice([0, 1, 1, int(rng.integers(2, 40)), int(rng.integers(40, 400))]))
        kv_len = int(rng.choice([0, 1] + [int(rng.integers(2, kv_rows + 1))] * 4))
        kv_off = int(rng.integers(0, kv_rows - kv_len + 1))
        kv_pos0 = int(rng.integers(0, 600))
        # mostly inside the context; sometimes before its first position (rows
        # with no key) or past its end (every key visible)
        mode = rng.random()
        if mode < 0.7:
            shift = int(rng.integers(0, kv_len + 1))
        elif mode < 0.85:
            shift = -int(rng.integers(1, 200))
        else:
            shift = kv_len + int(rng.integers(0, 300))
        q_pos0 = max(0, kv_pos0 + shift)
        rows.append((q0, kv_off, q0, q_len, kv_len, q_pos0, kv_pos0))
        q0 += q_len
    return np.array(rows, dtype=np.int64), hq, hkv, d, max(q0, 1), kv_rows


def with_masks(tasks, seed):
    """Columns 8-9: a sliding window (0 = none, else 1-700 positions) and a
    sink (the first 0-150 positions of the document) per task."""
    rng = np.random.default_rng(9500 + seed)
    n = len(tasks)
    window = np.where(rng.random(n) < 0.2, 0, rng.integers(1, 701, n))
    sink = np.where(rng.random(n) < 0.3, 0, rng.integers(0, 151, n))
    return np.concatenate([tasks, window[:, None], sink[:, None]], axis=1).astype(np.int64)


@pytest.mark.parametrize("masked", [False, True])
@pytest.mark.parametrize("seed", range(16))
def test_random_task_tables_forward_and_backward(seed, masked):
    tasks, hq, hkv, d, q_rows, kv_rows = random_tables(seed)
    if masked:
        tasks = with_masks(tasks, seed)
    announce("random task table seed %d masked=%s: hq=%d hkv=%d d=%d tasks=%s"
             % (seed, masked, hq, hkv, d, tasks.tolist()))
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    Q = I.randn_bf16((q_rows, hq, d), 9100 + seed)
    K = I.randn_bf16((kv_rows, hkv, d), 9200 + seed)
    V = I.randn_bf16((kv_rows, hkv, d), 9300 + seed)
    dO = I.randn_bf16((q_rows, hq, d), 9400 + seed)
    Qd, Kd, Vd, dOd = Q.to(dev), K.to(dev), V.to(dev), dO.to(dev)
    shape = ca.make_shape(hq, hkv, d, q_rows, kv_rows, q_rows)
    O = torch.full((q_rows, hq, d), float("nan"), dtype=torch.bfloat16, device=dev)
    LSE = torch.full((q_rows, hq), float("nan"), device=dev)
    ca.forward(shape, tasks, Qd, Kd, Vd, O, LSE)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(d)
    O_ref, L_ref = oracle.forward(tasks, widen(Q), widen(K), widen(V), scale, o_rows=q_rows)
    if np.isnan(L_ref).all():
        return                                   # no query rows at all
    check_forward(O, LSE, O_ref, L_ref, "random-%d" % seed)
    # the persistent launch (resident workgroups claiming the items) equals
    # the default launch bit for bit
    Op = torch.full_like(O, float("nan"))
    Lp = torch.full_like(LSE, float("nan"))
    ca.forward(ca.make_shape(hq, hkv, d, q_rows, kv_rows, q_rows, launch="persistent"), tasks, Qd, Kd, Vd, Op, Lp)
    torch.cuda.synchronize()
    rows = torch.from_numpy(np.flatnonzero(~np.isnan(L_ref[:, 0])))
    assert torch.equal(Op.cpu()[rows].view(torch.int16), O.cpu()[rows].view(torch.int16))
    assert torch.equal(Lp.cpu()[rows], LSE.cpu()[rows])
    dQ = torch.full_like(Qd, float("nan"))
    dK = torch.full_like(Kd, float("nan"))
    dV = torch.full_like(Vd, float("nan"))
    ca.backward(shape, tasks, Qd, Kd, Vd, O, dOd, LSE, dQ, dK, dV)
    torch.cuda.synchronize()
    ref = oracle.backward(tasks, widen(Q), widen(K), widen(V), widen(dO), scale)
    covered = ~np.isnan(L_ref[:, 0])
    for name, g, r in zip(("dQ", "dK", "dV"), (dQ, dK, dV), ref):
        gw = widen(g)
        if name == "dQ":
            gw, r = gw[covered], r[covered]
        assert np.all(np.isfinite(gw)), "%s not finite" % name
        e = rel_fro(gw, r)
        print("random-%d %s relF=%.3e" % (seed, name, e), flush=True)
        assert e <= GRAD_REL_FRO, name


def paged_layout(tasks, seed):
    """The random table's contexts moved into a virtual row space where each
    starts on a 128-row boundary (a fifth of the tasks reuse the previous
    task's context start: a shared prefix); random page size."""
    rng = np.random.default_rng(9600 + seed)
    P = int(rng.choice([128, 256, 512]))
    t = tasks.copy()
    run, prev = 0, None
    for i in range(len(t)):
        kv_len = int(t[i, 4])
        if prev is not None and kv_len <= prev[1] and rng.random() < 0.2:
            t[i, 1] = prev[0]
            continue
        t[i, 1] = run
        prev = (run, kv_len)
        run += -(-max(kv_len, 1) // 128) * 128
    n_vp = max(1, -(-run // P))
    return t, P, n_vp


@pytest.mark.parametrize("masked", [False, True])
@pytest.mark.parametrize("seed", range(8))
def test_random_task_tables_paged(seed, masked):
    """The same random tables over paged K/V in a shuffled page store: the
    paged forward equals the unpaged one bit for bit and the oracle; the paged
    backward's page-store gradients match the oracle."""
    from tests.test_gpu_paged import check_grads, check_paged, run_paged, run_paged_backward

    tasks, hq, hkv, d, q_rows, _ = random_tables(seed)
    tasks, P, n_vp = paged_layout(tasks, seed)
    masks = with_masks(tasks, seed)[:, 7:9] if masked else None
    announce("random paged table seed %d masked=%s: P=%d n_vp=%d hq=%d hkv=%d d=%d tasks=%s"
             % (seed, masked, P, n_vp, hq, hkv, d, tasks.tolist()))
    outs, O_ref, L_ref = run_paged(tasks, masks, hq, hkv, d, q_rows, n_vp, P, 9700 + seed)
    if np.isnan(L_ref).all():
        return
    check_paged(outs, O_ref, L_ref, "random-paged-%d" % seed)
    n_phys = n_vp + 5
    table = I.page_table(n_vp, n_phys, 9800 + seed)
    got, ref, _ = run_paged_backward(tasks, table, P, n_phys, hq, hkv, d, q_rows, 9900 + seed, masks=masks)
    covered = ~np.isnan(L_ref[:, 0])
    got = (got[0][torch_cuda().from_numpy(np.flatnonzero(covered))], got[1], got[2])
    ref = (ref[0][covered], ref[1], ref[2])
    check_grads(got, ref, "random-paged-bwd-%d" % seed)


@pytest.mark.parametrize("seed", range(2))
def test_random_long_overlapping_contexts_split_and_pieced(seed):
    """A few query shards over long, overlapping key ranges of one K/V buffer
    (most keys visible, some ranges sharing rows, one windowed task): the
    long shards' items are split over key chunks (forward merge, dQ sum), the
    overlapping contexts are cut into shared pieces for dK/dV, and the
    persistent launch runs the forward; O, LSE, dQ, dK, dV vs the oracle."""
    rng = np.random.default_rng(9700 + seed)
    hq, hkv, d = 8, 2, 128
    kv_rows = 90000
    rows, masks, q0 = [], [], 0
    for k in range(5):
        q_len = int(rng.choice([1, 40, 64, 150]))
        kv_len = int(rng.integers(20000, 80000))
        kv_off = int(rng.integers(0, kv_rows - kv_len + 1))
        kv_pos0 = int(rng.integers(0, 1000))
        q_pos0 = kv_pos0 + kv_len - q_len + int(rng.integers(-2000, 500))
        rows.append((q0, kv_off, q0, q_len, kv_len, max(0, q_pos0), kv_pos0))
        masks.append((int(rng.integers(500, 3000)), 64) if k == 4 else (0, 0))
        q0 += q_len
    tasks = np.array(rows, dtype=np.int64)
    full = np.concatenate([tasks, np.array(masks, dtype=np.int64)], axis=1)
    q_rows = q0
    announce("random long overlapping contexts seed %d: tasks=%s" % (seed, full.tolist()))
    shape = ca.make_shape(hq, hkv, d, q_rows, kv_rows, q_rows)
    info = ca.forward_queue_info(shape, tasks, full[:, 7:9])
    print("queue:", info, flush=True)
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    Q = I.randn_bf16((q_rows, hq, d), 9710 + seed)
    K = I.randn_bf16((kv_rows, hkv, d), 9720 + seed)
    V = I.randn_bf16((kv_rows, hkv, d), 9730 + seed)
    dO = I.randn_bf16((q_rows, hq, d), 9740 + seed)
    Qd, Kd, Vd, dOd = Q.to(dev), K.to(dev), V.to(dev), dO.to(dev)
    O = torch.full((q_rows, hq, d), float("nan"), dtype=torch.bfloat16, device=dev)
    LSE = torch.full((q_rows, hq), float("nan"), device=dev)
    fshape = ca.make_shape(hq, hkv, d, q_rows, kv_rows, q_rows, launch="persistent")
    ca.forward(fshape, full, Qd, Kd, Vd, O, LSE)
    dQ, dK, dV = (torch.full_like(x, float("nan")) for x in (Qd, Kd, Vd))
    ca.backward(shape, full, Qd, Kd, Vd, O, dOd, LSE, dQ, dK, dV)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(d)
    O_ref, L_ref = oracle.forward(full, widen(Q), widen(K), widen(V), scale, o_rows=q_rows)
    check_forward(O, LSE, O_ref, L_ref, "long-overlap-%d" % seed)
    ref = oracle.backward(full, widen(Q), widen(K), widen(V), widen(dO), scale)
    covered = ~np.isnan(L_ref[:, 0])
    for name, g, r in zip(("dQ", "dK", "dV"), (dQ, dK, dV), ref):
        gw = widen(g)
        if name == "dQ":
            gw, r = gw[covered], r[covered]
        assert np.all(np.isfinite(gw)), "%s not finite" % name
        e = rel_fro(gw, r)
        print("long-overlap-%d %s relF=%.3e" % (seed, name, e), flush=True)
        assert e <= GRAD_REL_FRO, name
