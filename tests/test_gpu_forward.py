"""GPU parity of ca_forward / ca_forward_varlen / ca_merge against the fp64
oracle, element by element, at sizes the oracle finishes in seconds (several
tiles, ragged tails, empty and fully masked rows, every GQA grouping)."""

import math

import numpy as np
import pytest

import oracle
from long_context_core_amd import ca
from long_context_core_amd import inputs as I
from tests.gpu_util import announce, check_forward, torch_cuda, widen

pytestmark = pytest.mark.gpu


def run_case(tasks, hq, hkv, d, q_rows, kv_rows, o_rows, seed, out_f32=False, varlen=None, qkv=None):
    torch = torch_cuda()
    if qkv is None:
        Q = I.randn_bf16((q_rows, hq, d), seed)
        K = I.randn_bf16((kv_rows, hkv, d), seed + 1)
        V = I.randn_bf16((kv_rows, hkv, d), seed + 2)
    else:
        Q, K, V = qkv
    dev = torch.device("cuda:0")
    Qd, Kd, Vd = Q.to(dev), K.to(dev), V.to(dev)
    O = torch.full((o_rows, hq, d), float("nan"), device=dev,
                   dtype=torch.float32 if out_f32 else torch.bfloat16)
    LSE = torch.full((o_rows, hq), float("nan"), device=dev, dtype=torch.float32)
    shape = ca.make_shape(hq, hkv, d, q_rows, kv_rows, o_rows, out_f32=out_f32)
    if varlen is not None:
        ca.forward_varlen(shape, varlen, Qd, Kd, Vd, O, LSE)
    else:
        ca.forward(shape, tasks, Qd, Kd, Vd, O, LSE)
    torch.cuda.synchronize()
    O_ref, LSE_ref = oracle.forward(tasks, widen(Q), widen(K), widen(V), 1 / math.sqrt(d), o_rows=o_rows)
    return O, LSE, O_ref, LSE_ref


def test_tiny_config_full():
    announce("forward tiny 1k docs [512,256,128,128] hq4 hkv1 d64")
    w = I.tiny_forward()
    O, LSE, Or, Lr = run_case(w.tasks, w.hq, w.hkv, w.d, w.q_rows, w.kv_rows, w.o_rows, 201)
    check_forward(O, LSE, Or, Lr, "tiny")


def test_tiny_config_varlen_entry():
    announce("forward_varlen tiny")
    w = I.tiny_forward()
    cu = np.cumsum([0] + w.doc_lens)
    O, LSE, Or, Lr = run_case(w.tasks, w.hq, w.hkv, w.d, w.q_rows, w.kv_rows, w.o_rows, 201, varlen=cu)
    check_forward(O, LSE, Or, Lr, "tiny-varlen")


@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 4), (6, 2), (8, 2), (16, 2), (16, 1)])
@pytest.mark.parametrize("d", [64, 128])
def test_ragged_varlen_gqa(hq, hkv, d):
    announce("forward ragged varlen hq%d hkv%d d%d" % (hq, hkv, d))
    lens = [1, 31, 33, 64, 65, 127, 129, 200]
    tasks = I.varlen_tasks(lens)
    T = sum(lens)
    O, LSE, Or, Lr = run_case(tasks, hq, hkv, d, T, T, T, 300 + hq + hkv + d)
    check_forward(O, LSE, Or, Lr, "ragged hq%d hkv%d d%d" % (hq, hkv, d))


def test_ca_tasks_unaligned_offsets():
    announce("forward CA-tasks unaligned")
    rng = np.random.default_rng(7)
    tasks = []
    qo = ko = 0
    for _ in range(9):
        doc = int(rng.integers(200, 1500))
        ql = int(rng.integers(1, 300))
        end = int(rng.integers(ql, doc + 1))
        tasks.append((qo, ko, qo, ql, end, end - ql, 0))
        qo += ql
        ko += end
    tasks = np.array(tasks)
    O, LSE, Or, Lr = run_case(tasks, 16, 2, 128, qo, ko, qo, 400)
    check_forward(O, LSE, Or, Lr, "ca-tasks")


def test_ring_partials_fp32_with_empty_and_masked_tasks():
    announce("forward ring partials fp32 + merge")
    torch = torch_cuda()
    T, n = 768, 4
    S = T // n
    hq, hkv, d = 16, 1, 128
    tasks = [(i * S, j * S, j * T + i * S, S, S, i * S, j * S) for i in range(n) for j in range(i + 1)]
    # one fully masked task (block after the shard) and one empty context
    tasks.append((0, 3 * S, 3 * T + 0, S, S, 0, 3 * S))
    tasks.append((S, 0, 2 * T + S, S, 0, S, 0))
    tasks = np.array(tasks)
    O, LSE, Or, Lr = run_case(tasks, hq, hkv, d, T, T, n * T, 500, out_f32=True)
    check_forward(O, LSE, Or, Lr, "ring-partials")
    # merge the GPU partials (unwritten slots: LSE = -inf) and compare to the
    # unsplit oracle forward of the whole document
    LSE_p = torch.where(torch.isnan(LSE), torch.full_like(LSE, -float("inf")), LSE)
    O_p = torch.nan_to_num(O, nan=0.0)
    Om = torch.empty((T, hq, d), device=O.device, dtype=torch.bfloat16)
    Lm = torch.empty((T, hq), device=O.device, dtype=torch.float32)
    ca.merge(ca.make_shape(hq, hkv, d, T, T, T), O_p.view(n, T, hq, d), LSE_p.view(n, T, hq), Om, Lm)
    torch.cuda.synchronize()
    Q = I.randn_bf16((T, hq, d), 500)
    K = I.randn_bf16((T, hkv, d), 501)
    V = I.randn_bf16((T, hkv, d), 502)
    Ou, Lu = oracle.forward(np.array([(0, 0, 0, T, T, 0, 0)]), widen(Q), widen(K), widen(V), 1 / math.sqrt(d))
    check_forward(Om, Lm, Ou, Lu, "ring-merged-vs-unsplit")


def test_merge_alone_against_equation_4():
    announce("merge alone")
    torch = torch_cuda()
    S, T, hq, d = 5, 300, 4, 128
    g = torch.Generator().manual_seed(9)
    Op = torch.randn(S, T, hq, d, generator=g)
    Lp = torch.randn(S, T, hq, generator=g) * 5
    Lp[1, :50] = -float("inf")            # empty partials
    Lp[:, 60:70] = -float("inf")          # rows with no partial at all
    Op[1, :50] = float("nan")             # never read
    for out_f32 in (False, True):
        Om = torch.empty(T, hq, d, device="cuda", dtype=torch.float32 if out_f32 else torch.bfloat16)
        Lm = torch.empty(T, hq, device="cuda")
        ca.merge(ca.make_shape(hq, 1, d, T, T, T, out_f32=out_f32), Op.cuda(), Lp.cuda(), Om, Lm)
        torch.cuda.synchronize()
        Oref, Lref = oracle.merge(np.nan_to_num(Op.double().numpy(), nan=0.0), Lp.double().numpy())
        got_o, got_l = widen(Om), widen(Lm)
        assert np.array_equal(np.isneginf(got_l), np.isneginf(Lref))
        fin = np.isfinite(Lref)
        assert np.max(np.abs(got_l[fin] - Lref[fin])) < 1e-5
        tol = 1e-5 if out_f32 else 2e-2
        assert np.max(np.abs(got_o - Oref)) < tol
        assert np.all(got_o[60:70] == 0)


def test_decode_rows():
    announce("forward decode rows q_len=1")
    batch, ctx, n = 4, 3000, 3
    S = ctx // n
    tasks = np.array([(b, b * ctx + s * S, s * batch + b, 1, S, ctx - 1, s * S)
                      for b in range(batch) for s in range(n)])
    O, LSE, Or, Lr = run_case(tasks, 16, 1, 128, batch, batch * ctx, n * batch, 600, out_f32=True)
    check_forward(O, LSE, Or, Lr, "decode-partials")


def climbing_qkv(pos, hq, hkv, d, seed, rise_log2, period):
    """Q and K with a shared positive component whose size in K grows with the
    key's in-document position pos (a sawtooth of the given period): every
    64-key tile of a period scores about rise_log2 (log2 units) above the one
    before, so the kernels' running row maximum moves past their lazy-rescale
    threshold (2^8) again and again, and drops back at each period's end."""
    torch = torch_cuda()
    T = len(pos)
    Q = I.randn_bf16((T, hq, d), seed).float() + 1.0
    K = I.randn_bf16((T, hkv, d), seed + 1).float()
    # q . k grows by about d * gamma per unit of gamma; scaled by 1/sqrt(d), in log2 units
    per_key = rise_log2 / 64 / (math.sqrt(d) * math.log2(math.e))
    gamma = torch.from_numpy((np.asarray(pos) % period) * per_key).float()
    K = K + gamma[:, None, None]
    V = I.randn_bf16((T, hkv, d), seed + 2)
    return Q.to(torch.bfloat16), K.to(torch.bfloat16), V


def climb_natural(rise_log2, period, longest):
    """Natural-log height of the climb over the longest run of keys."""
    return rise_log2 * min(period, longest) / 64 * math.log(2)


@pytest.mark.parametrize("hq,hkv,d,rise,period", [(8, 2, 128, 12.0, 1 << 30), (16, 1, 128, 20.0, 512),
                                                  (4, 4, 64, 12.0, 256)])
def test_running_max_rescales(hq, hkv, d, rise, period):
    """Scores climbing tile after tile (and falling back at each sawtooth
    period): the online softmax rescales its accumulators mid-row, which
    N(0, 1) inputs almost never make it do after the first tile."""
    announce("forward climbing scores hq%d hkv%d d%d rise%.0f period%d" % (hq, hkv, d, rise, period))
    lens = [1, 70, 300, 1000, 2100]
    tasks = I.varlen_tasks(lens)
    T = sum(lens)
    pos = np.concatenate([np.arange(l) for l in lens])
    O, LSE, Or, Lr = run_case(tasks, hq, hkv, d, T, T, T, 0, qkv=climbing_qkv(pos, hq, hkv, d, 760 + d, rise, period))
    fin = np.isfinite(Lr)
    # the scores did climb far past the first tile
    assert np.max(Lr[fin]) > 0.5 * climb_natural(rise, period, max(lens))
    check_forward(O, LSE, Or, Lr, "climbing scores")


def test_decode_running_max_rescales():
    """Single-token rows over caches whose scores climb along the cache (the
    split-KV decode kernel's lazy rescale), whole caches and key chunks."""
    announce("decode climbing scores")
    batch, ctx = 3, 3000
    hq, hkv, d = 16, 1, 128
    pos = np.tile(np.arange(ctx), batch)
    Qa, K, V = climbing_qkv(pos, hq, hkv, d, 780, 10.0, 1 << 30)
    Q = Qa[:batch].contiguous()
    # whole caches, then the same caches in 3 key blocks (partials)
    tasks = np.array([(b, b * ctx, b, 1, ctx, ctx - 1, 0) for b in range(batch)] +
                     [(b, b * ctx + s * (ctx // 3), batch + s * batch + b, 1, ctx // 3, ctx - 1, s * (ctx // 3))
                      for b in range(batch) for s in range(3)], dtype=np.int64)
    O, LSE, Or, Lr = run_case(tasks, hq, hkv, d, batch, batch * ctx, 4 * batch, 0, out_f32=True, qkv=(Q, K, V))
    assert np.max(Lr[np.isfinite(Lr)]) > 0.5 * climb_natural(10.0, 1 << 30, ctx)
    check_forward(O, LSE, Or, Lr, "decode climbing scores")


def test_probe_mask_parity_small():
    """K = 0, V = (-1)^position: a leaked or dropped key moves a row by 1/(p+1)."""
    announce("forward probe small")
    torch = torch_cuda()
    lens = [5, 64, 65, 130, 257]
    tasks = I.varlen_tasks(lens)
    T = sum(lens)
    hq, hkv, d = 8, 2, 128
    Q = I.randn_bf16((T, hq, d), 700)
    K = torch.zeros((T, hkv, d), dtype=torch.bfloat16)
    pos = np.concatenate([np.arange(l) for l in lens])
    V = torch.from_numpy(np.where(pos % 2 == 0, 1.0, -1.0)).float()[:, None, None].expand(T, hkv, d).contiguous().to(torch.bfloat16)
    O, LSE, Or, Lr = run_case(tasks, hq, hkv, d, T, T, T, 0, qkv=(Q, K, V))
    o = widen(O)
    expect = np.where(pos % 2 == 0, 1.0 / (pos + 1), 0.0)
    err = np.abs(o - expect[:, None, None]).max(axis=(1, 2))
    assert np.all(err < 0.25 / (pos + 1))
    assert np.allclose(widen(LSE), np.log(pos + 1.0)[:, None], atol=1e-5)


@pytest.mark.parametrize("hq,hkv,d,out_f32", [(16, 2, 128, False), (8, 1, 64, True), (64, 2, 128, False)])
def test_decode_gqa_variants(hq, hkv, d, out_f32):
    """Single-token tasks: G <= 16 uses the split-KV decode kernel (chunked
    and unchunked), G = 32 falls back to the tiled kernel; one row sees no
    key and one sees a prefix only."""
    announce("decode variants hq%d hkv%d d%d f32=%s" % (hq, hkv, d, out_f32))
    ctx = [5000, 700, 1, 300, 64]
    tasks, off = [], 0
    for b, c in enumerate(ctx):
        tasks.append((b, off, b, 1, c, c - 1, 0))
        off += c
    tasks.append((len(ctx), 0, len(ctx), 1, 100, 10, 50))       # sees no key (q_pos0 < kv_pos0)
    tasks.append((len(ctx) + 1, 0, len(ctx) + 1, 1, 900, 400, 0))  # sees keys 0..400 only
    tasks = np.array(tasks)
    n = len(tasks)
    O, LSE, Or, Lr = run_case(tasks, hq, hkv, d, n, off, n, 650 + hq + d, out_f32=out_f32)
    check_forward(O, LSE, Or, Lr, "decode hq%d hkv%d d%d" % (hq, hkv, d))


@pytest.mark.parametrize("d", [64, 128])
def test_rows_without_keys_next_to_rows_with_keys(d):
    """Context blocks that start after the first queries (kv_pos0 > q_pos0):
    in one 32-row block some rows see no key while others do, so the
    running-max update must leave the empty rows at O = 0, LSE = -inf."""
    announce("forward partially empty row blocks d%d" % d)
    tasks = np.array([(0, 0, 0, 40, 50, 0, 30), (40, 50, 40, 70, 100, 5, 60), (110, 150, 110, 33, 64, 0, 31)])
    O, LSE, Or, Lr = run_case(tasks, 16, 2, d, 143, 214, 143, 660 + d)
    check_forward(O, LSE, Or, Lr, "partially-empty d%d" % d)


def test_calls_from_short_lived_threads():
    """Calls made from threads that then exit (each thread's ring of pinned
    staging buffers is released at its end, after its queued copies): every
    thread's results equal the main thread's bit for bit, concurrent threads
    included, and the library keeps working afterwards."""
    import threading

    announce("forward from short-lived threads")
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    hq, hkv, d = 8, 2, 128
    lens = [300, 1, 777, 64]
    tasks = I.varlen_tasks(lens)
    T = sum(lens)
    Q = I.randn_bf16((T, hq, d), 3100, device=dev)
    K = I.randn_bf16((T, hkv, d), 3101, device=dev)
    V = I.randn_bf16((T, hkv, d), 3102, device=dev)
    shape = ca.make_shape(hq, hkv, d, T, T, T)
    O0 = torch.empty((T, hq, d), dtype=torch.bfloat16, device=dev)
    L0 = torch.empty((T, hq), device=dev)
    ca.forward(shape, tasks, Q, K, V, O0, L0)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.forward(tasks, widen(Q), widen(K), widen(V), 1 / math.sqrt(d))
    check_forward(O0, L0, O_ref, L_ref, "main thread")
    n_threads, calls = 4, 12
    outs = [[torch.empty_like(O0) for _ in range(calls)] for _ in range(n_threads)]
    lses = [[torch.empty_like(L0) for _ in range(calls)] for _ in range(n_threads)]
    errors = []

    def work(i):
        try:
            torch.cuda.set_device(dev)
            for c in range(calls):
                ca.forward(shape, tasks, Q, K, V, outs[i][c], lses[i][c])
            # the thread ends with its last copies possibly still queued
        except Exception as e:  # reported by the main thread
            errors.append(repr(e))

    # two rounds of threads one after another, then all at once
    for group in ([0], [1], [2, 3]):
        th = [threading.Thread(target=work, args=(i,)) for i in group]
        for x in th:
            x.start()
        for x in th:
            x.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(n_threads):
        for c in range(calls):
            assert torch.equal(outs[i][c].view(torch.int16), O0.view(torch.int16)) and torch.equal(lses[i][c], L0)
    O1, L1 = torch.empty_like(O0), torch.empty_like(L0)
    ca.forward(shape, tasks, Q, K, V, O1, L1)
    torch.cuda.synchronize()
    assert torch.equal(O1.view(torch.int16), O0.view(torch.int16)) and torch.equal(L1, L0)
    print("short-lived threads: %d x %d calls identical to the main thread's" % (n_threads, calls), flush=True)


def test_binding_rejects_wrong_device_tensors_before_any_launch():
    """Wrong dtype, too few elements, a non-contiguous view or a workspace
    that is not bytes raise CAError in the binding; the outputs keep their
    sentinel values (nothing was launched) and a correct call still works."""
    announce("binding tensor checks")
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    hq, hkv, d, T = 8, 2, 64, 200
    tasks = I.varlen_tasks([T])
    s = ca.make_shape(hq, hkv, d, T, T, T)
    Q = I.randn_bf16((T, hq, d), 3200, device=dev)
    K = I.randn_bf16((T, hkv, d), 3201, device=dev)
    V = I.randn_bf16((T, hkv, d), 3202, device=dev)
    O = torch.full((T, hq, d), 7.0, dtype=torch.bfloat16, device=dev)
    L = torch.full((T, hq), 7.0, device=dev)
    bad = [
        ("dtype", dict(Q=Q.float())),
        ("elements", dict(O=O[:T - 1])),
        ("elements", dict(K=K[:T - 1])),
        ("dtype", dict(O=torch.empty((T, hq, d), device=dev))),          # fp32 O without out_f32
        ("contiguous", dict(Q=Q.transpose(0, 1))),
        ("dtype", dict(L=torch.empty((T, hq), dtype=torch.bfloat16, device=dev))),
    ]
    for why, kw in bad:
        args = dict(Q=Q, K=K, V=V, O=O, L=L)
        args.update(kw)
        with pytest.raises(ca.CAError, match=why):
            ca.forward(s, tasks, args["Q"], args["K"], args["V"], args["O"], args["L"])
    with pytest.raises(ca.CAError, match="workspace"):
        ca.forward(s, tasks, Q, K, V, O, L, ws=torch.empty(1 << 16, dtype=torch.float32, device=dev))
    ws = ca.workspace_tensor(ca.forward_workspace(s, tasks), dev)
    plan = ca.forward_prepare(s, tasks, ws)
    with pytest.raises(ca.CAError, match="elements"):
        ca.forward_prepared(plan, Q, K, V, O[:10], L)
    torch.cuda.synchronize()
    assert bool((O == 7.0).all()) and bool((L == 7.0).all()), "a rejected call wrote its outputs"
    ca.forward_prepared(plan, Q, K, V, O, L)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.forward(tasks, widen(Q), widen(K), widen(V), 1 / math.sqrt(d))
    check_forward(O, L, O_ref, L_ref, "after rejected calls")


@pytest.mark.parametrize("seed", range(8))
def test_merge_random_part_counts_and_ranges(seed):
    """Equation 4 over random part counts (1 to 40, past the kernel's eight
    partials in flight), row counts and head geometries, with LSEs spread over
    hundreds of units around large offsets and random empty (-inf) partials."""
    torch = torch_cuda()
    rng = np.random.default_rng(7000 + seed)
    S = int(rng.choice([1, 2, 3, 7, 8, 9, 16, 36, 40]))
    T = int(rng.integers(1, 700))
    hq = int(rng.choice([1, 4, 16, 32]))
    d = int(rng.choice([64, 128]))
    announce("merge random seed %d: S=%d T=%d hq=%d d=%d" % (seed, S, T, hq, d))
    g = torch.Generator().manual_seed(7100 + seed)
    Op = torch.randn(S, T, hq, d, generator=g)
    spread = float(rng.choice([1.0, 20.0, 300.0]))
    offset = float(rng.choice([0.0, 1e4, -1e4]))
    Lp = torch.randn(S, T, hq, generator=g) * spread + offset
    empty = torch.from_numpy(rng.random((S, T, hq)) < 0.3)
    Lp[empty] = -float("inf")
    Op[empty.unsqueeze(-1).expand_as(Op)] = float("nan")      # never read
    out_f32 = bool(seed % 2)
    Om = torch.empty(T, hq, d, device="cuda", dtype=torch.float32 if out_f32 else torch.bfloat16)
    Lm = torch.empty(T, hq, device="cuda")
    ca.merge(ca.make_shape(hq, 1, d, T, T, T, out_f32=out_f32), Op.cuda(), Lp.cuda(), Om, Lm)
    torch.cuda.synchronize()
    Oref, Lref = oracle.merge(np.nan_to_num(Op.double().numpy(), nan=0.0), Lp.double().numpy())
    got_o, got_l = widen(Om), widen(Lm)
    assert np.array_equal(np.isneginf(got_l), np.isneginf(Lref))
    fin = np.isfinite(Lref)
    # fp32 LSE around |offset| = 1e4 carries ~1e-3 of absolute rounding
    ltol = 1e-5 * max(1.0, abs(offset) + spread)
    assert np.max(np.abs(got_l[fin] - Lref[fin]), initial=0.0) <= ltol
    assert np.all(np.isfinite(got_o))
    assert np.max(np.abs(got_o - Oref)) < (2e-5 if out_f32 else 2e-2)
    assert np.all(got_o[~fin] == 0)


@pytest.mark.parametrize("hq,hkv,d,blockwise", [(8, 4, 64, False), (16, 2, 128, False), (8, 2, 128, True)])
def test_persistent_launch_claims_items_bit_identical(hq, hkv, d, blockwise):
    """Thousands of work items, far more than the resident workgroups of the
    persistent launch, so that most are claimed from the queue one after
    another by workgroups that already ran items of other KV heads, head
    groups, documents and (blockwise) multi-context shards.  The persistent
    launch equals the one-workgroup-per-item launch bit for bit, and both
    equal the oracle on every row and head."""
    announce("forward persistent vs per-item hq%d hkv%d d%d blockwise=%s" % (hq, hkv, d, blockwise))
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(4242 + hq + d)
    lens = [int(x) for x in rng.integers(1, 300, size=400)]
    tasks = I.blockwise_shards(lens, 64, 2) if blockwise else I.varlen_tasks(lens)
    T = sum(lens)
    Q = I.randn_bf16((T, hq, d), 5150 + hq + d)
    K = I.randn_bf16((T, hkv, d), 5151 + hq + d)
    V = I.randn_bf16((T, hkv, d), 5152 + hq + d)
    Qd, Kd, Vd = Q.to(dev), K.to(dev), V.to(dev)
    outs = []
    for launch in ("persistent", "per_item"):
        O = torch.full((T, hq, d), float("nan"), dtype=torch.bfloat16, device=dev)
        LSE = torch.full((T, hq), float("nan"), device=dev)
        ca.forward(ca.make_shape(hq, hkv, d, T, T, T, launch=launch), tasks, Qd, Kd, Vd, O, LSE)
        outs.append((O, LSE))
    torch.cuda.synchronize()
    (Op, Lp), (Oi, Li) = outs
    assert torch.equal(Op.view(torch.int16), Oi.view(torch.int16))
    assert torch.equal(Lp, Li)
    O_ref, LSE_ref = oracle.forward(tasks, widen(Q), widen(K), widen(V), 1 / math.sqrt(d), o_rows=T)
    check_forward(Op, Lp, O_ref, LSE_ref, "persistent hq%d hkv%d d%d" % (hq, hkv, d))


def test_persistent_launch_paged_and_masked_bit_identical():
    """The paged and sink/window-masked instantiations of the persistent
    launch: bit-identical to one workgroup per item over many claimed items
    (every output is also checked against the oracle by the per-item launch's
    own tests)."""
    announce("forward persistent vs per-item, paged + lambda mask")
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(977)
    P = 256
    lens = [int(x) for x in rng.integers(1, 700, size=300)]
    tasks, n_vp = I.paged_varlen_tasks(lens, P)
    hq, hkv, d = 16, 4, 128
    T = sum(lens)
    masks = np.array([(int(rng.integers(0, 200)), int(rng.integers(0, 64))) for _ in range(len(tasks))], dtype=np.int32)
    n_phys = n_vp + 5
    table = I.page_table(n_vp, n_phys, 978)
    Q = I.randn_bf16((T, hq, d), 979).to(dev)
    Ks = I.page_store(I.randn_bf16((n_vp * P, hkv, d), 980), table, P, n_phys).to(dev)
    Vs = I.page_store(I.randn_bf16((n_vp * P, hkv, d), 981), table, P, n_phys).to(dev)
    outs = []
    for launch in ("persistent", "per_item"):
        O = torch.full((T, hq, d), float("nan"), dtype=torch.bfloat16, device=dev)
        LSE = torch.full((T, hq), float("nan"), device=dev)
        ca.forward(ca.make_shape(hq, hkv, d, T, n_phys * P, T, launch=launch), tasks, Q, Ks, Vs, O, LSE,
                   masks=masks, pages=ca.kv_pages(table, P))
        outs.append((O, LSE))
    torch.cuda.synchronize()
    (Op, Lp), (Oi, Li) = outs
    assert bool(torch.isfinite(Lp).all())
    assert torch.equal(Op.view(torch.int16), Oi.view(torch.int16))
    assert torch.equal(Lp, Li)
