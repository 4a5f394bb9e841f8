"""Parity at the full benchmark shapes, in the launch configuration the
benchmark times: the oracle on sampled rows (it cannot do the whole job in
seconds), and the mask probe (K = 0, V = (-1)^position) whose closed form
checks every row of every head at full size."""

import math

import numpy as np
import pytest

import oracle
from long_context_core_amd import ca
from long_context_core_amd import inputs as I
from tests.gpu_util import announce, check_forward, torch_cuda, widen

pytestmark = pytest.mark.gpu


def device_inputs(w, seed):
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    Q = I.randn_bf16((w.q_rows, w.hq, w.d), seed, device=dev)
    K = I.randn_bf16((w.kv_rows, w.hkv, w.d), seed + 1, device=dev)
    V = I.randn_bf16((w.kv_rows, w.hkv, w.d), seed + 2, device=dev)
    return Q, K, V


def run_forward(w, Q, K, V, out_f32=False):
    torch = torch_cuda()
    O = torch.empty((w.o_rows, w.hq, w.d), device=Q.device,
                    dtype=torch.float32 if out_f32 else torch.bfloat16)
    LSE = torch.full((w.o_rows, w.hq), -float("inf"), device=Q.device)
    shape = ca.make_shape(w.hq, w.hkv, w.d, w.q_rows, w.kv_rows, w.o_rows, out_f32=out_f32)
    ca.forward(shape, w.tasks, Q, K, V, O, LSE)
    torch.cuda.synchronize()
    return O, LSE


def sampled_check(w, task_rows, Q, K, V, O, LSE, heads=None, label=""):
    """task_rows: list of (task index, task-relative rows).  The oracle gets
    only the context slice of each task."""
    heads = list(range(w.hq)) if heads is None else heads
    got_o, got_l, ref_o, ref_l = [], [], [], []
    for ti, rows in task_rows:
        t = w.tasks[ti]
        q_off, kv_off, o_off, q_len, kv_len, q_pos0, kv_pos0 = (int(x) for x in t)
        rows = np.asarray(rows)
        n_ctx = int(np.clip(q_pos0 + rows.max() - kv_pos0 + 1, 0, kv_len))
        qs = widen(Q[q_off + rows])
        ks = widen(K[kv_off:kv_off + n_ctx])
        vs = widen(V[kv_off:kv_off + n_ctx])
        local = np.array([0, 0, 0, q_len, n_ctx, q_pos0, kv_pos0])
        # rows are indexed inside qs directly: shift positions accordingly
        o_r = np.zeros((len(rows), w.hq, w.d))
        l_r = np.zeros((len(rows), w.hq))
        for k, r in enumerate(rows):
            tk = local.copy()
            tk[0], tk[3], tk[5] = k, 1, q_pos0 + r
            o1, l1 = oracle.forward_rows(tk, np.array([0]), qs, ks, vs, w.scale)
            o_r[k], l_r[k] = o1[0], l1[0]
        got_o.append(widen(O[o_off + rows])[:, heads])
        got_l.append(widen(LSE[o_off + rows])[:, heads])
        ref_o.append(o_r[:, heads])
        ref_l.append(l_r[:, heads])
    return check_forward(np.concatenate(got_o), np.concatenate(got_l),
                         np.concatenate(ref_o), np.concatenate(ref_l), label)


def probe_tensors(w, positions_of_kv_rows):
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    Q = I.randn_bf16((w.q_rows, w.hq, w.d), 77, device=dev)
    K = torch.zeros((w.kv_rows, w.hkv, w.d), dtype=torch.bfloat16, device=dev)
    sign = torch.from_numpy(np.where(positions_of_kv_rows % 2 == 0, 1.0, -1.0).astype(np.float32)).to(dev)
    V = sign[:, None, None].expand(w.kv_rows, w.hkv, w.d).to(torch.bfloat16).contiguous()
    return Q, K, V


def probe_expect(w):
    """Per output row: (mean of (-1)^p over visible positions, count)."""
    exp_o = np.zeros(w.o_rows)
    cnt = np.zeros(w.o_rows)
    for t in w.tasks:
        q_off, kv_off, o_off, q_len, kv_len, q_pos0, kv_pos0 = (int(x) for x in t)
        i = np.arange(q_len)
        last = np.clip(q_pos0 + i, kv_pos0 - 1, kv_pos0 + kv_len - 1)
        n = last - kv_pos0 + 1
        s = np.where(n > 0, np.where(kv_pos0 % 2 == 0, 1.0, -1.0) * ((last - kv_pos0) % 2 == 0), 0.0)
        exp_o[o_off:o_off + q_len] = np.where(n > 0, s / np.maximum(n, 1), 0.0)
        cnt[o_off:o_off + q_len] = n
    return exp_o, cnt


def check_probe(w, O, LSE, label, rows=None):
    torch = torch_cuda()
    exp_o, cnt = probe_expect(w)
    sel = np.arange(w.o_rows) if rows is None else rows
    e = torch.from_numpy(exp_o[sel]).to(O.device)
    c = torch.from_numpy(cnt[sel]).to(O.device)
    o = O[torch.from_numpy(sel).to(O.device)].float()
    err = (o - e[:, None, None].float()).abs().amax(dim=(1, 2))
    tol = 0.25 / torch.clamp(c, min=1.0)
    bad = int((err >= tol.float()).sum())
    l = LSE[torch.from_numpy(sel).to(O.device)].double()
    lref = torch.where(c > 0, torch.log(torch.clamp(c, min=1.0)), torch.full_like(c, -float("inf")))
    fin = c > 0
    dl = float((l[fin] - lref[fin][:, None]).abs().max()) if bool(fin.any()) else 0.0
    inf_ok = bool(torch.isneginf(l[~fin]).all()) if bool((~fin).any()) else True
    print("%s probe: rows=%d bad_rows=%d max|dLSE|=%.2e" % (label, len(sel), bad, dl), flush=True)
    assert bad == 0 and dl < 1e-4 and inf_ok, label


def doc_positions(w):
    pos = np.zeros(w.kv_rows, dtype=np.int64)
    for t in w.tasks:
        kv_off, kv_len, kv_pos0 = int(t[1]), int(t[4]), int(t[6])
        pos[kv_off:kv_off + kv_len] = kv_pos0 + np.arange(kv_len)
    return pos


# --------------------------------------------------------------------------


# Length seed 102 is the benchmark's headline draw (10 documents, 2.41e9
# visible pairs per head, two documents over 40K tokens); seed 103 is the
# draw with the median pair count of seeds 100-107 (30 documents, median
# length 1,349, 1.26e9 pairs).
@pytest.mark.parametrize("length_seed", [102, 103])
def test_llama8b_131k_sampled(length_seed):
    announce("fullsize llama3-8b packed 131k sampled rows, length seed %d" % length_seed)
    w = I.llama8b_packed_131k(seed=length_seed)
    Q, K, V = device_inputs(w, 202)
    O, LSE = run_forward(w, Q, K, V)
    rng = np.random.default_rng(1)
    tr = []
    for ti, t in enumerate(w.tasks):
        L = int(t[3])
        rows = np.unique(np.concatenate([np.arange(min(L, 8)), np.arange(max(0, L - 8), L),
                                         rng.integers(0, L, size=min(L, 16))]))
        tr.append((ti, rows))
    sampled_check(w, tr, Q, K, V, O, LSE, label="131k-sampled")


@pytest.mark.parametrize("length_seed", [102, 103])
def test_llama8b_131k_probe_all_rows(length_seed):
    announce("fullsize llama3-8b packed 131k probe, length seed %d" % length_seed)
    w = I.llama8b_packed_131k(seed=length_seed)
    Q, K, V = probe_tensors(w, doc_positions(w))
    O, LSE = run_forward(w, Q, K, V)
    check_probe(w, O, LSE, "131k")


def test_ca_tasks_34b_sampled_and_probe():
    announce("fullsize llama-34b CA-tasks 262k sampled + probe")
    torch = torch_cuda()
    w = I.ca_tasks_34b()
    Q, K, V = device_inputs(w, 203)
    O, LSE = run_forward(w, Q, K, V)
    tr = [(ti, np.array([0, int(t[3]) // 2, int(t[3]) - 1])) for ti, t in enumerate(w.tasks)]
    sampled_check(w, tr, Q, K, V, O, LSE, label="ca-tasks-sampled")      # all 64 heads
    del Q, K, V, O, LSE
    torch.cuda.empty_cache()
    Q, K, V = probe_tensors(w, doc_positions(w))
    O, LSE = run_forward(w, Q, K, V)
    check_probe(w, O, LSE, "ca-tasks")


def test_ring_prefill_405b_partials_merge():
    announce("fullsize llama3-405b tp8 ring prefill 8x8 partials + merge")
    torch = torch_cuda()
    w = I.ring_prefill_405b_tp8()
    Q, K, V = device_inputs(w, 204)
    O, LSE = run_forward(w, Q, K, V, out_f32=True)       # LSE pre-filled with -inf
    T = w.merged_rows
    Om = torch.empty((T, w.hq, w.d), dtype=torch.bfloat16, device=Q.device)
    Lm = torch.empty((T, w.hq), device=Q.device)
    ca.merge(ca.make_shape(w.hq, w.hkv, w.d, T, T, T), O.view(w.n_parts, T, w.hq, w.d),
             LSE.view(w.n_parts, T, w.hq), Om, Lm)
    torch.cuda.synchronize()
    whole = I.Workload("whole", w.hq, w.hkv, w.d, np.array([[0, 0, 0, T, T, 0, 0]]), T, T, T)
    rows = np.unique(np.concatenate([np.arange(4), [16383, 16384, 16385, 65535, 65536], np.arange(T - 4, T),
                                     np.random.default_rng(2).integers(0, T, 24)]))
    sampled_check(whole, [(0, rows)], Q, K, V, Om, Lm, label="ring-merged-sampled")


def test_ring_prefill_405b_probe():
    announce("fullsize ring prefill probe (partials and merged)")
    torch = torch_cuda()
    w = I.ring_prefill_405b_tp8()
    Q, K, V = probe_tensors(w, np.arange(w.kv_rows))
    O, LSE = run_forward(w, Q, K, V, out_f32=True)
    written = np.concatenate([np.arange(t[2], t[2] + t[3]) for t in w.tasks])
    check_probe(w, O, LSE, "ring-partials", rows=written)
    T = w.merged_rows
    Om = torch.empty((T, w.hq, w.d), dtype=torch.bfloat16, device=Q.device)
    Lm = torch.empty((T, w.hq), device=Q.device)
    ca.merge(ca.make_shape(w.hq, w.hkv, w.d, T, T, T), O.view(w.n_parts, T, w.hq, w.d),
             LSE.view(w.n_parts, T, w.hq), Om, Lm)
    torch.cuda.synchronize()
    whole = I.Workload("whole", w.hq, w.hkv, w.d, np.array([[0, 0, 0, T, T, 0, 0]]), T, T, T)
    check_probe(whole, Om, Lm, "ring-merged")


def test_ring_decode_405b_full():
    announce("fullsize llama3-405b tp8 pass-Q decode b32 x 128k")
    torch = torch_cuda()
    w = I.ring_decode_405b_tp8()
    Q, K, V = device_inputs(w, 205)
    O, LSE = run_forward(w, Q, K, V, out_f32=True)
    B = w.merged_rows
    Om = torch.empty((B, w.hq, w.d), dtype=torch.bfloat16, device=Q.device)
    Lm = torch.empty((B, w.hq), device=Q.device)
    ca.merge(ca.make_shape(w.hq, w.hkv, w.d, B, B, B), O.view(w.n_parts, B, w.hq, w.d),
             LSE.view(w.n_parts, B, w.hq), Om, Lm)
    torch.cuda.synchronize()
    ctx = 131072
    # the oracle over each sequence's whole cache (the unsplit definition)
    tasks = np.array([(b, b * ctx, b, 1, ctx, ctx - 1, 0) for b in range(B)])
    Or = np.zeros((B, w.hq, w.d))
    Lr = np.zeros((B, w.hq))
    qs = widen(Q)
    for b in range(B):
        ks = widen(K[b * ctx:(b + 1) * ctx])
        vs = widen(V[b * ctx:(b + 1) * ctx])
        o1, l1 = oracle.forward_rows(np.array([b, 0, 0, 1, ctx, ctx - 1, 0]), np.array([0]), qs, ks, vs, w.scale)
        Or[b], Lr[b] = o1[0], l1[0]
    check_forward(Om, Lm, Or, Lr, "decode-merged")


def test_ring_decode_405b_paged_full():
    """The bench's paged decode step at full size: the 32 caches in shuffled
    256-row pages (the paged kernel keeps two tiles in flight).  Same work
    items and arithmetic as the contiguous step, so the partials must match it
    bit for bit; the merged output is checked against the oracle on a few
    sequences."""
    announce("fullsize llama3-405b tp8 pass-Q decode b32 x 128k, shuffled 256-row pages")
    torch = torch_cuda()
    w = I.ring_decode_405b_tp8()
    Q, K, V = device_inputs(w, 205)
    O, LSE = run_forward(w, Q, K, V, out_f32=True)
    P = 256
    n_vp = w.kv_rows // P
    table = I.page_table(n_vp, n_vp, 206)
    idx = torch.from_numpy(table.astype(np.int64)).to(Q.device)
    Ks, Vs = torch.empty_like(K), torch.empty_like(V)
    Ks.view(n_vp, -1)[idx] = K.view(n_vp, -1)
    Vs.view(n_vp, -1)[idx] = V.view(n_vp, -1)
    Op = torch.empty_like(O)
    Lp = torch.full_like(LSE, -float("inf"))
    shape = ca.make_shape(w.hq, w.hkv, w.d, w.q_rows, w.kv_rows, w.o_rows, out_f32=True)
    ca.forward(shape, w.tasks, Q, Ks, Vs, Op, Lp, pages=ca.kv_pages(table, P))
    torch.cuda.synchronize()
    assert torch.equal(Op.view(torch.int32), O.view(torch.int32))
    assert torch.equal(Lp.view(torch.int32), LSE.view(torch.int32))
    del Ks, Vs
    B = w.merged_rows
    Om = torch.empty((B, w.hq, w.d), dtype=torch.bfloat16, device=Q.device)
    Lm = torch.empty((B, w.hq), device=Q.device)
    ca.merge(ca.make_shape(w.hq, w.hkv, w.d, B, B, B), Op.view(w.n_parts, B, w.hq, w.d),
             Lp.view(w.n_parts, B, w.hq), Om, Lm)
    torch.cuda.synchronize()
    ctx = 131072
    qs = widen(Q)
    for b in (0, 17, B - 1):
        ks = widen(K[b * ctx:(b + 1) * ctx])
        vs = widen(V[b * ctx:(b + 1) * ctx])
        o1, l1 = oracle.forward_rows(np.array([b, 0, 0, 1, ctx, ctx - 1, 0]), np.array([0]), qs, ks, vs, w.scale)
        check_forward(Om[b:b + 1], Lm[b:b + 1], o1, l1, "paged decode seq %d" % b)


def ring_load_balanced(Q, K, V, T, hq, hkv, d, N=8):
    """The 2N partials of a load-balanced pass-KV ring over one T-token
    document, one launch per step as the bench times them (all ranks' shares
    and both source chunks of a step fused; slot 1 writes the second block of
    the step's stacked partial buffer), merged by Equation 4."""
    torch = torch_cuda()
    dev = Q.device
    Op = torch.empty((2 * N, T, hq, d), device=dev)
    Lp = torch.empty((2 * N, T, hq), device=dev)
    shape = ca.make_shape(hq, hkv, d, T, T, 2 * T, out_f32=True)
    for step in range(N):
        tables = []
        for slot in (0, 1):
            t = ca.ring_kv_step_tasks([T], N, step, slot)
            t["o_off"] += slot * T
            tables.append(t)
        ca.forward(shape, np.concatenate(tables), Q, K, V, Op[2 * step:2 * step + 2], Lp[2 * step:2 * step + 2])
    Om = torch.empty((T, hq, d), dtype=torch.bfloat16, device=dev)
    Lm = torch.empty((T, hq), device=dev)
    ca.merge(ca.make_shape(hq, hkv, d, T, T, T), Op, Lp, Om, Lm)
    torch.cuda.synchronize()
    del Op, Lp
    return Om, Lm


def test_ring_prefill_405b_load_balanced_sampled_and_probe():
    announce("fullsize llama3-405b tp8 ring prefill, load-balanced pass-KV over 8 ranks")
    w = I.ring_prefill_405b_tp8()
    T = w.merged_rows
    whole = I.Workload("whole", w.hq, w.hkv, w.d, np.array([[0, 0, 0, T, T, 0, 0]]), T, T, T)
    Q, K, V = device_inputs(whole, 214)
    Om, Lm = ring_load_balanced(Q, K, V, T, w.hq, w.hkv, w.d)
    c = T // 16
    rows = np.unique(np.concatenate([np.arange(3), [c - 1, c, 7 * c, 8 * c - 1, 8 * c, 15 * c], np.arange(T - 3, T),
                                     np.random.default_rng(4).integers(0, T, 20)]))
    sampled_check(whole, [(0, rows)], Q, K, V, Om, Lm, label="ring-load-balanced-sampled")
    Q, K, V = probe_tensors(whole, np.arange(T))
    Om, Lm = ring_load_balanced(Q, K, V, T, w.hq, w.hkv, w.d)
    check_probe(whole, Om, Lm, "ring-load-balanced-merged")


def ring_partial_prefill(Q, K, V, new, cached, hq, hkv, d, N=4):
    """Partial prefill over a KV cache as the bench times it: per ring step
    one launch holding the four chunk pairs of every rank (each pair's
    outputs in its own block of the stacked fp32 partials), then the merge."""
    torch = torch_cuda()
    dev = Q.device
    Tq = sum(new)
    Tk = Tq + sum(cached)
    Op = torch.empty((4 * N, Tq, hq, d), device=dev)
    Lp = torch.empty((4 * N, Tq, hq), device=dev)
    shape = ca.make_shape(hq, hkv, d, Tq, Tk, 4 * Tq, out_f32=True)
    for step in range(N):
        tables = []
        for slot in range(4):
            t = ca.ring_prefill_step_tasks(new, cached, N, step, slot)
            t["o_off"] += slot * Tq
            tables.append(t)
        ca.forward(shape, np.concatenate(tables), Q, K, V, Op[4 * step:4 * step + 4], Lp[4 * step:4 * step + 4])
    Om = torch.empty((Tq, hq, d), dtype=torch.bfloat16, device=dev)
    Lm = torch.empty((Tq, hq), device=dev)
    ca.merge(ca.make_shape(hq, hkv, d, Tq, Tq, Tq), Op, Lp, Om, Lm)
    torch.cuda.synchronize()
    del Op, Lp
    return Om, Lm


def test_ring_partial_prefill_405b_miss10_sampled_and_probe():
    """12,800 new tokens over a 115,200-token cache (10 % miss), Llama3-405B
    TP8 share, 4 ranks: sampled rows against the oracle of one query block
    over the whole cache, and the mask probe on every new row."""
    announce("fullsize ring partial prefill 405b tp8, 12800 new over 115200 cached, 4 ranks")
    w0 = I.ring_prefill_405b_tp8()
    hq, hkv, d = w0.hq, w0.hkv, w0.d
    T_new, P_c = 12800, 115200
    whole = I.Workload("whole", hq, hkv, d, np.array([[0, 0, 0, T_new, T_new + P_c, P_c, 0]]),
                       T_new, T_new + P_c, T_new)
    Q, K, V = device_inputs(whole, 215)
    Om, Lm = ring_partial_prefill(Q, K, V, [T_new], [P_c], hq, hkv, d)
    c = T_new // 8
    rows = np.unique(np.concatenate([np.arange(3), [c - 1, c, 4 * c - 1, 4 * c, 7 * c], np.arange(T_new - 3, T_new),
                                     np.random.default_rng(6).integers(0, T_new, 16)]))
    sampled_check(whole, [(0, rows)], Q, K, V, Om, Lm, label="ring-partial-prefill-sampled")
    Q, K, V = probe_tensors(whole, np.arange(T_new + P_c))
    Om, Lm = ring_partial_prefill(Q, K, V, [T_new], [P_c], hq, hkv, d)
    check_probe(whole, Om, Lm, "ring-partial-prefill-merged")
