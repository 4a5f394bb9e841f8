"""Prepared forward calls captured in a HIP graph (the captured decode step of
"Context Parallelism for Scalable Million-Token Inference", Section 3.6):
ca_forward_prepare once, then ca_forward_prepared (+ ca_merge) recorded by
torch's graph capture.  Each replay follows eager work that changes Q and
runs the direct calls; every replay must equal the direct calls bit for bit,
and the last one the fp64 oracle."""

import math

import numpy as np
import pytest

import oracle
from long_context_core_amd import ca
from long_context_core_amd import inputs as I
from tests.gpu_util import announce, check_forward, torch_cuda, widen

pytestmark = pytest.mark.gpu

HQ, HKV, D = 16, 1, 128


def decode_blocks(B, ctx, n):
    """B single-token queries, each over its own ctx-entry cache in n
    stationary blocks; block s writes partial slot s."""
    S = ctx // n
    t = [(b, b * ctx + s * S, s * B + b, 1, S, ctx - 1, s * S) for b in range(B) for s in range(n)]
    return np.array(t, dtype=np.int64)


def decode_whole(B, ctx):
    return np.array([(b, b * ctx, b, 1, ctx, ctx - 1, 0) for b in range(B)], dtype=np.int64)


CASES = {
    # name: (tasks, q_rows, kv_rows, o_rows, n_parts merged after the call)
    "decode-4-blocks-merged": (decode_blocks(8, 16384, 4), 8, 8 * 16384, 4 * 8, 4),
    "decode-whole-cache": (decode_whole(8, 20000), 8, 8 * 20000, 8, 0),
    "prefill-causal-docs": (I.varlen_tasks([700, 128, 1, 1500]), 2329, 2329, 2329, 0),
}
# persistent launch (claim counters reset by a kernel inside the graph): many
# short documents, far more work items than resident workgroups
_LENS = [int(x) for x in np.random.default_rng(2733).integers(1, 300, size=300)]
CASES["prefill-many-docs-persistent"] = (I.varlen_tasks(_LENS), sum(_LENS), sum(_LENS), sum(_LENS), 0)


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_equal_direct_calls(name):
    announce("graph-captured prepared forward: %s" % name)
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    tasks, q_rows, kv_rows, o_rows, n_parts = CASES[name]
    merged = n_parts > 0
    launch = "persistent" if name.endswith("persistent") else None
    shape = ca.make_shape(HQ, HKV, D, q_rows, kv_rows, o_rows, out_f32=merged, launch=launch)
    if launch:
        assert ca.forward_queue_info(shape, tasks)["persistent_workgroups"] == 256
    K = I.randn_bf16((kv_rows, HKV, D), 2701, device=dev)
    V = I.randn_bf16((kv_rows, HKV, D), 2702, device=dev)
    Q = I.randn_bf16((q_rows, HQ, D), 2700, device=dev)
    odt = torch.float32 if merged else torch.bfloat16
    O = torch.empty((o_rows, HQ, D), dtype=odt, device=dev)
    LSE = torch.empty((o_rows, HQ), device=dev)
    O2, LSE2 = torch.empty_like(O), torch.empty_like(LSE)
    if merged:
        B = o_rows // n_parts
        mshape = ca.make_shape(HQ, HKV, D, B, B, B)
        Om = torch.empty((B, HQ, D), dtype=torch.bfloat16, device=dev)
        Lm = torch.empty((B, HQ), device=dev)
        Om2, Lm2 = torch.empty_like(Om), torch.empty_like(Lm)
    ws = ca.workspace_tensor(ca.forward_workspace(shape, tasks), dev)
    ws2 = ca.workspace_tensor(ca.forward_workspace(shape, tasks), dev)
    side = torch.cuda.Stream()
    plan = ca.forward_prepare(shape, tasks, ws, stream=side)
    side.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = torch.cuda.current_stream()
        ca.forward_prepared(plan, Q, K, V, O, LSE, stream=st)
        if merged:
            ca.merge(mshape, O.view(n_parts, B, HQ, D), LSE.view(n_parts, B, HQ), Om, Lm, stream=st)
    for rep in range(4):
        Q.copy_(I.randn_bf16((q_rows, HQ, D), 2710 + rep, device=dev))
        O.fill_(float("nan"))   # a replay that skipped work would leave NaN
        ca.forward(shape, tasks, Q, K, V, O2, LSE2, ws=ws2)
        if merged:
            ca.merge(mshape, O2.view(n_parts, B, HQ, D), LSE2.view(n_parts, B, HQ), Om2, Lm2)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_o, got_l, ref_o, ref_l = (Om, Lm, Om2, Lm2) if merged else (O, LSE, O2, LSE2)
        same = torch.equal(got_o.view(torch.int16) if got_o.dtype == torch.bfloat16 else got_o,
                           ref_o.view(torch.int16) if ref_o.dtype == torch.bfloat16 else ref_o)
        print("%s replay %d: identical to the direct calls: %s" % (name, rep, same), flush=True)
        assert same and torch.equal(got_l, ref_l)
    # the last replay against the oracle
    if merged:
        whole = np.array([(b, b * (kv_rows // B), b, 1, kv_rows // B, kv_rows // B - 1, 0) for b in range(B)],
                         dtype=np.int64)
        O_ref, L_ref = oracle.forward(whole, widen(Q), widen(K), widen(V), 1 / math.sqrt(D))
        check_forward(Om, Lm, O_ref, L_ref, name)
    else:
        O_ref, L_ref = oracle.forward(tasks, widen(Q), widen(K), widen(V), 1 / math.sqrt(D))
        check_forward(O, LSE, O_ref, L_ref, name)


def test_prepared_call_rejects_a_foreign_plan():
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    with pytest.raises(ca.CAError):
        t = torch.zeros(16, device=dev)
        ca.forward_prepared(ca.ForwardPlan(), t, t, t, t, t)


def test_graph_replays_masked_and_paged_calls():
    """A lambda-masked prefill and a paged decode, each prepared once, captured
    together and replayed: every replay equals the direct calls bit for bit."""
    announce("graph-captured prepared forward: lambda mask + paged decode")
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    lens = [1500, 300, 2200]
    mt = I.lambda_tasks(lens, window=512, sink=16)
    T = sum(lens)
    m_shape = ca.make_shape(HQ, HKV, D, T, T, T)
    Qm = I.randn_bf16((T, HQ, D), 2720, device=dev)
    Km = I.randn_bf16((T, HKV, D), 2721, device=dev)
    Vm = I.randn_bf16((T, HKV, D), 2722, device=dev)
    Om, Lm = torch.empty((T, HQ, D), dtype=torch.bfloat16, device=dev), torch.empty((T, HQ), device=dev)
    Om2, Lm2 = torch.empty_like(Om), torch.empty_like(Lm)
    # paged decode: 4 queries over 4096-token caches in shuffled 256-row pages
    P, B, ctx = 256, 4, 4096
    dt = decode_whole(B, ctx)
    n_vp = B * ctx // P
    table = I.page_table(n_vp, n_vp + 8, 2723)
    pages = ca.kv_pages(table, P)
    d_shape = ca.make_shape(HQ, HKV, D, B, (n_vp + 8) * P, B)
    Qd = I.randn_bf16((B, HQ, D), 2724, device=dev)
    Ks = I.randn_bf16(((n_vp + 8) * P, HKV, D), 2725, device=dev)
    Vs = I.randn_bf16(((n_vp + 8) * P, HKV, D), 2726, device=dev)
    Od, Ld = torch.empty((B, HQ, D), dtype=torch.bfloat16, device=dev), torch.empty((B, HQ), device=dev)
    Od2, Ld2 = torch.empty_like(Od), torch.empty_like(Ld)
    ws_m = ca.workspace_tensor(ca.forward_workspace(m_shape, mt), dev)
    ws_d = ca.workspace_tensor(ca.forward_workspace(d_shape, dt, pages=pages), dev)
    side = torch.cuda.Stream()
    plan_m = ca.forward_prepare(m_shape, mt, ws_m, stream=side)
    plan_d = ca.forward_prepare(d_shape, dt, ws_d, stream=side, pages=pages)
    side.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = torch.cuda.current_stream()
        ca.forward_prepared(plan_m, Qm, Km, Vm, Om, Lm, stream=st)
        ca.forward_prepared(plan_d, Qd, Ks, Vs, Od, Ld, stream=st)
    for rep in range(3):
        Qm.copy_(I.randn_bf16((T, HQ, D), 2730 + rep, device=dev))
        Qd.copy_(I.randn_bf16((B, HQ, D), 2740 + rep, device=dev))
        ca.forward(m_shape, mt, Qm, Km, Vm, Om2, Lm2)
        ca.forward(d_shape, dt, Qd, Ks, Vs, Od2, Ld2, pages=pages)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = (torch.equal(Om.view(torch.int16), Om2.view(torch.int16)) and torch.equal(Lm, Lm2)
                and torch.equal(Od.view(torch.int16), Od2.view(torch.int16)) and torch.equal(Ld, Ld2))
        print("masked + paged replay %d: identical to the direct calls: %s" % (rep, same), flush=True)
        assert same
    # the paged decode against the oracle over the virtual caches
    Kv = oracle.virtual_rows(widen(Ks), table, P)
    Vv = oracle.virtual_rows(widen(Vs), table, P)
    O_ref, L_ref = oracle.forward(dt, widen(Qd), Kv, Vv, 1 / math.sqrt(D))
    check_forward(Od, Ld, O_ref, L_ref, "paged-decode-replayed")


def test_prepared_call_rejects_a_plan_from_another_device():
    """A plan records the device current at preparation (its queue lives in
    that device's workspace); a launch with another device current is
    rejected.  With one GPU the recorded device is edited instead: it is the
    third 8-byte word of the plan (after the tag and the workspace pointer),
    a layout private to this test and the library."""
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    tasks = I.varlen_tasks([300])
    s = ca.make_shape(8, 2, 128, 300, 300, 300)
    Q = I.randn_bf16((300, 8, 128), 2750, device=dev)
    K = I.randn_bf16((300, 2, 128), 2751, device=dev)
    O = torch.full((300, 8, 128), 3.0, dtype=torch.bfloat16, device=dev)
    L = torch.full((300, 8), 3.0, device=dev)
    ws = ca.workspace_tensor(ca.forward_workspace(s, tasks), dev)
    plan = ca.forward_prepare(s, tasks, ws)
    assert plan.opaque[2] & 0xffffffff == torch.cuda.current_device()
    saved = plan.opaque[2]
    plan.opaque[2] = 7
    with pytest.raises(ca.CAError, match="prepared on device 7"):
        ca.forward_prepared(plan, Q, K, K, O, L)
    torch.cuda.synchronize()
    assert bool((O == 3.0).all())
    plan.opaque[2] = saved
    ca.forward_prepared(plan, Q, K, K, O, L)
    O2, L2 = torch.empty_like(O), torch.empty_like(L)
    ca.forward(s, tasks, Q, K, K, O2, L2)
    torch.cuda.synchronize()
    assert torch.equal(O.view(torch.int16), O2.view(torch.int16)) and torch.equal(L, L2)


def test_graph_replays_a_partial_prefill_ring():
    """The partial-prefill ring's per-step launches (each step's four chunk
    pairs fused into one table, one prepared plan per step) and the merge,
    captured in one graph: every replay equals the direct calls bit for bit
    and the last one the oracle of the whole query block over the cache."""
    announce("graph-captured partial prefill ring: N=4")
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    N, hq, hkv, d = 4, 8, 2, 128
    new, cached = [700, 1, 333], [1500, 0, 64]
    Tq, Tk = sum(new), sum(new) + sum(cached)
    K = I.randn_bf16((Tk, hkv, d), 2761, device=dev)
    V = I.randn_bf16((Tk, hkv, d), 2762, device=dev)
    Q = I.randn_bf16((Tq, hq, d), 2760, device=dev)
    fshape = ca.make_shape(hq, hkv, d, Tq, Tk, 4 * Tq, out_f32=True)
    mshape = ca.make_shape(hq, hkv, d, Tq, Tq, Tq)
    tables = []
    for step in range(N):
        parts = []
        for slot in range(4):
            t = ca.ring_prefill_step_tasks(new, cached, N, step, slot)
            t["o_off"] += slot * Tq
            parts.append(t)
        tables.append(np.concatenate(parts))
    bufs = [(torch.empty((4 * N, Tq, hq, d), device=dev), torch.empty((4 * N, Tq, hq), device=dev),
             torch.empty((Tq, hq, d), dtype=torch.bfloat16, device=dev), torch.empty((Tq, hq), device=dev))
            for _ in range(2)]
    side = torch.cuda.Stream()
    ws = [ca.workspace_tensor(ca.forward_workspace(fshape, t), dev) for t in tables]
    plans = [ca.forward_prepare(fshape, t, w, stream=side) for t, w in zip(tables, ws)]
    side.synchronize()
    Op, Lp, Om, Lm = bufs[0]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = torch.cuda.current_stream()
        for step, plan in enumerate(plans):
            ca.forward_prepared(plan, Q, K, V, Op[4 * step:4 * step + 4], Lp[4 * step:4 * step + 4], stream=st)
        ca.merge(mshape, Op, Lp, Om, Lm, stream=st)
    Op2, Lp2, Om2, Lm2 = bufs[1]
    for rep in range(3):
        Q.copy_(I.randn_bf16((Tq, hq, d), 2770 + rep, device=dev))
        for step, t in enumerate(tables):
            ca.forward(fshape, t, Q, K, V, Op2[4 * step:4 * step + 4], Lp2[4 * step:4 * step + 4])
        ca.merge(mshape, Op2, Lp2, Om2, Lm2)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = torch.equal(Om.view(torch.int16), Om2.view(torch.int16)) and torch.equal(Lm, Lm2)
        print("partial prefill ring replay %d: identical to the direct calls: %s" % (rep, same), flush=True)
        assert same
    q0 = np.concatenate([[0], np.cumsum(new)])
    k0 = np.concatenate([[0], np.cumsum(np.array(new) + np.array(cached))])
    whole = np.array([(q0[s], k0[s], q0[s], new[s], new[s] + cached[s], cached[s], 0) for s in range(len(new))],
                     dtype=np.int64)
    O_ref, L_ref = oracle.forward(whole, widen(Q), widen(K), widen(V), 1 / math.sqrt(d))
    check_forward(Om, Lm, O_ref, L_ref, "partial-prefill-ring-replayed")


def test_direct_calls_refuse_a_capturing_stream():
    """ca_forward and ca_backward copy a host-built work queue into the
    workspace; a captured copy would replay stale host memory, so both refuse
    a stream under capture before enqueuing anything: the outputs stay
    untouched."""
    announce("direct forward / backward refused under graph capture")
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    tasks = I.varlen_tasks([300, 77])
    T = 377
    shape = ca.make_shape(HQ, HKV, D, T, T, T)
    Q = I.randn_bf16((T, HQ, D), 2750, device=dev)
    K = I.randn_bf16((T, HKV, D), 2751, device=dev)
    V = I.randn_bf16((T, HKV, D), 2752, device=dev)
    O = torch.full((T, HQ, D), 7.0, dtype=torch.bfloat16, device=dev)
    LSE = torch.full((T, HQ), 7.0, device=dev)
    dQ, dK, dV = torch.full_like(Q, 7.0), torch.full_like(K, 7.0), torch.full_like(V, 7.0)
    ws = ca.workspace_tensor(ca.forward_workspace(shape, tasks), dev)
    bws = ca.workspace_tensor(ca.backward_workspace(shape, tasks), dev)
    torch.cuda.synchronize()
    errors = []
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = torch.cuda.current_stream()
        for call in (lambda: ca.forward(shape, tasks, Q, K, V, O, LSE, ws=ws, stream=st),
                     lambda: ca.backward(shape, tasks, Q, K, V, O, Q, LSE, dQ, dK, dV, ws=bws, stream=st)):
            try:
                call()
            except ca.CAError as e:
                errors.append(e)
    assert len(errors) == 2, errors
    assert all(e.status == ca.CA_ERR_INVALID and "capturing" in str(e) for e in errors), errors
    torch.cuda.synchronize()
    for x in (O, LSE, dQ, dK, dV):
        assert bool((x.float() == 7.0).all())
    # the same calls outside capture run normally
    ca.forward(shape, tasks, Q, K, V, O, LSE, ws=ws)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(LSE).all()) and not bool((LSE == 7.0).any())


def test_temporary_workspace_on_a_side_stream_is_not_reused_early():
    """A workspace the binding allocates for a call on a non-current stream
    is tied to that stream (record_stream): while the stream still has work
    queued, freeing it must not hand its block to the next allocation on the
    current stream.  Then a side-stream call without a workspace, followed at
    once by allocations that write on the current stream, still matches the
    same call on the current stream."""
    announce("temporary workspace on a side stream")
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    side = torch.cuda.Stream()
    nbytes = 3 << 20
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        torch.cuda._sleep(100_000_000)          # keeps the side stream busy (bounded spin)
    ws = ca.workspace_tensor(nbytes, dev, stream=side)
    p = ws.data_ptr()
    del ws
    x = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    assert x.data_ptr() != p
    torch.cuda.synchronize()
    del x
    tasks = I.varlen_tasks([2000, 513, 1])
    T = 2514
    shape = ca.make_shape(HQ, HKV, D, T, T, T)
    Q = I.randn_bf16((T, HQ, D), 2760, device=dev)
    K = I.randn_bf16((T, HKV, D), 2761, device=dev)
    V = I.randn_bf16((T, HKV, D), 2762, device=dev)
    O, LSE = torch.empty((T, HQ, D), dtype=torch.bfloat16, device=dev), torch.empty((T, HQ), device=dev)
    O2, LSE2 = torch.empty_like(O), torch.empty_like(LSE)
    ca.forward(shape, tasks, Q, K, V, O2, LSE2)
    torch.cuda.synchronize()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        torch.cuda._sleep(20_000_000)
    ca.forward(shape, tasks, Q, K, V, O, LSE, stream=side)
    junk = [torch.zeros(ca.forward_workspace(shape, tasks), dtype=torch.uint8, device=dev) for _ in range(4)]
    torch.cuda.synchronize()
    del junk
    assert torch.equal(O.view(torch.int16), O2.view(torch.int16)) and torch.equal(LSE, LSE2)
