"""Parity at full benchmark size for the sparse-mask, paged-K/V and CA-task
training paths, in the launch configurations the benchmark times:

* the 512K training batch under the lambda mask (sink 64, window 4096): the
  mask probe (K = 0, V = (-1)^position) checked on every row and head against
  its closed form, and the fp64 oracle on sampled rows;
* the 131K headline batch over shuffled 512-row pages: bit for bit equal to
  the unpaged launch over the same virtual K/V;
* the backward of the 262K CA-task batch (34B shape): per task and KV head,
  sum_j dK_j = 0 and sum_j dV_j = sum_i sum_{h in group} dO_i (rows of P sum
  to one and rows of dS to zero), on every task."""

import numpy as np
import pytest

import oracle
from long_context_core_amd import ca
from long_context_core_amd import inputs as I
from tests.gpu_util import announce, check_forward, torch_cuda, widen

pytestmark = pytest.mark.gpu

WINDOW, SINK = 4096, 64


def doc_positions(doc_lens):
    return np.concatenate([np.arange(l) for l in doc_lens]).astype(np.int64)


def sign_sum(a, b):
    """sum of (-1)^p for p in [a, b] (0 where b < a), elementwise."""
    n = np.maximum(b - a + 1, 0)
    return np.where(n % 2 == 1, np.where(a % 2 == 0, 1.0, -1.0), 0.0)


def lambda_probe_expect(pos):
    """Mean of (-1)^p over the keys a query at document position qp sees
    under the lambda mask, and their count: the window (qp - WINDOW, qp] and
    the sink [0, SINK)."""
    lo_w = np.maximum(0, pos - WINDOW + 1)
    n_win = pos - lo_w + 1
    hi_s = np.minimum(SINK, lo_w)                    # sink keys below the window: [0, hi_s)
    n = n_win + hi_s
    s = sign_sum(lo_w, pos) + sign_sum(np.zeros_like(hi_s), hi_s - 1)
    return s / n, n


def test_lambda_mask_512k_probe_all_rows():
    announce("fullsize 512k lambda mask (sink 64, window 4096) probe, all rows")
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    w = I.train_8b_prolong_512k()
    tasks = I.lambda_tasks(w.doc_lens, window=WINDOW, sink=SINK)
    T = w.q_rows
    pos = doc_positions(w.doc_lens)
    Q = I.randn_bf16((T, w.hq, w.d), 231, device=dev)
    K = torch.zeros((T, w.hkv, w.d), dtype=torch.bfloat16, device=dev)
    sign = torch.from_numpy(np.where(pos % 2 == 0, 1.0, -1.0).astype(np.float32)).to(dev)
    V = sign[:, None, None].expand(T, w.hkv, w.d).to(torch.bfloat16).contiguous()
    O = torch.empty((T, w.hq, w.d), dtype=torch.bfloat16, device=dev)
    LSE = torch.empty((T, w.hq), device=dev)
    ca.forward(ca.make_shape(w.hq, w.hkv, w.d, T, T, T), tasks, Q, K, V, O, LSE)
    torch.cuda.synchronize()
    exp_o, cnt = lambda_probe_expect(pos)
    e = torch.from_numpy(exp_o).to(dev)
    c = torch.from_numpy(cnt.astype(np.float64)).to(dev)
    err = (O.float() - e[:, None, None].float()).abs().amax(dim=(1, 2))
    bad = int((err >= (0.25 / c).float()).sum())
    dl = float((LSE.double() - torch.log(c)[:, None]).abs().max())
    print("512k lambda probe: rows=%d bad_rows=%d max|dLSE|=%.2e" % (T, bad, dl), flush=True)
    assert bad == 0 and dl < 1e-4


def test_lambda_mask_512k_sampled_rows():
    announce("fullsize 512k lambda mask sampled rows vs the oracle")
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    w = I.train_8b_prolong_512k()
    tasks = I.lambda_tasks(w.doc_lens, window=WINDOW, sink=SINK)
    T = w.q_rows
    Q = I.randn_bf16((T, w.hq, w.d), 232, device=dev)
    K = I.randn_bf16((T, w.hkv, w.d), 233, device=dev)
    V = I.randn_bf16((T, w.hkv, w.d), 234, device=dev)
    O = torch.empty((T, w.hq, w.d), dtype=torch.bfloat16, device=dev)
    LSE = torch.empty((T, w.hq), device=dev)
    ca.forward(ca.make_shape(w.hq, w.hkv, w.d, T, T, T), tasks, Q, K, V, O, LSE)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    heads = list(range(0, w.hq, 4))
    got_o, got_l, ref_o, ref_l = [], [], [], []
    for t in tasks[np.argsort(-tasks[:, 3])[:6]]:       # the six longest documents
        q_off, kv_off, o_off, q_len = (int(x) for x in t[:4])
        rows = np.unique(np.concatenate([[0, 63, 64, SINK + WINDOW - 1, SINK + WINDOW, q_len - 1],
                                         rng.integers(0, q_len, 4)]))
        rows = rows[rows < q_len]
        for r in rows:
            # The row's visible keys by the mask's definition: the sink [0, SINK)
            # and the window (r - WINDOW, r].  Softmax does not depend on key
            # order, so the oracle gets exactly these keys as one context that
            # the row sees whole.
            lo = max(0, r - WINDOW + 1)
            keep = np.unique(np.concatenate([np.arange(min(SINK, r + 1)), np.arange(lo, r + 1)]))
            kidx = torch.from_numpy(kv_off + keep).to(dev)
            ks = widen(K[kidx])
            vs = widen(V[kidx])
            qs = widen(Q[q_off + r:q_off + r + 1])
            task = np.array([0, 0, 0, 1, len(keep), len(keep) - 1, 0])
            o1, l1 = oracle.forward_rows(task, np.array([0]), qs, ks, vs, w.scale)
            ref_o.append(o1[:, heads])
            ref_l.append(l1[:, heads])
            got_o.append(widen(O[o_off + r:o_off + r + 1])[:, heads])
            got_l.append(widen(LSE[o_off + r:o_off + r + 1])[:, heads])
    check_forward(np.concatenate(got_o), np.concatenate(got_l), np.concatenate(ref_o), np.concatenate(ref_l),
                  "512k-lambda-sampled")


def test_paged_131k_bitwise_equals_unpaged():
    announce("fullsize 131k headline over shuffled 512-row pages vs unpaged")
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    P = 512
    w = I.llama8b_packed_131k_paged(P)
    n_vp = w.kv_rows // P
    Q = I.randn_bf16((w.q_rows, w.hq, w.d), 241, device=dev)
    Kv = I.randn_bf16((w.kv_rows, w.hkv, w.d), 242, device=dev)
    Vv = I.randn_bf16((w.kv_rows, w.hkv, w.d), 243, device=dev)
    table = I.page_table(n_vp, n_vp + 16, 244)
    idx = torch.from_numpy(table.astype(np.int64)).to(dev)
    Ks = torch.full(((n_vp + 16) * P, w.hkv, w.d), float("nan"), dtype=torch.bfloat16, device=dev)
    Vs = torch.full_like(Ks, float("nan"))
    Ks.view(n_vp + 16, -1)[idx] = Kv.view(n_vp, -1)
    Vs.view(n_vp + 16, -1)[idx] = Vv.view(n_vp, -1)
    outs = []
    for paged in (True, False):
        O = torch.empty((w.q_rows, w.hq, w.d), dtype=torch.bfloat16, device=dev)
        LSE = torch.empty((w.q_rows, w.hq), device=dev)
        if paged:
            ca.forward(ca.make_shape(w.hq, w.hkv, w.d, w.q_rows, Ks.shape[0], w.q_rows), w.tasks, Q, Ks, Vs, O, LSE,
                       pages=ca.kv_pages(table, P))
        else:
            ca.forward(ca.make_shape(w.hq, w.hkv, w.d, w.q_rows, w.kv_rows, w.q_rows), w.tasks, Q, Kv, Vv, O, LSE)
        outs.append((O, LSE))
    torch.cuda.synchronize()
    (Op, Lp), (Ou, Lu) = outs
    same_o = torch.equal(Op.view(torch.int16), Ou.view(torch.int16))
    same_l = torch.equal(Lp, Lu)
    print("paged 131k: O identical %s, LSE identical %s" % (same_o, same_l), flush=True)
    assert same_o and same_l
    # and the unpaged launch against the oracle on a few rows of the longest document
    t = w.tasks[int(np.argmax(w.tasks[:, 3]))]
    q_off, kv_off, o_off, q_len = (int(x) for x in t[:4])
    rows = np.array([0, 1, q_len // 2, q_len - 1])
    ridx = torch.from_numpy(o_off + rows).to(dev)
    got_o = widen(Ou[ridx])
    got_l = widen(Lu[ridx])
    ref_o, ref_l = [], []
    for r in rows:
        task = np.array([0, 0, 0, 1, r + 1, r, 0])
        o1, l1 = oracle.forward_rows(task, np.array([0]), widen(Q[q_off + r:q_off + r + 1]),
                                     widen(Kv[kv_off:kv_off + r + 1]), widen(Vv[kv_off:kv_off + r + 1]), w.scale)
        ref_o.append(o1)
        ref_l.append(l1)
    check_forward(got_o, got_l, np.concatenate(ref_o), np.concatenate(ref_l), "paged-131k-sampled")


def test_ca_tasks_34b_backward_invariants():
    announce("fullsize 262k CA-tasks (34B) backward: per-task gradient invariants")
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    w = I.ca_tasks_34b()
    G = w.hq // w.hkv
    shape = ca.make_shape(w.hq, w.hkv, w.d, w.q_rows, w.kv_rows, w.o_rows)
    Q = I.randn_bf16((w.q_rows, w.hq, w.d), 251, device=dev)
    K = I.randn_bf16((w.kv_rows, w.hkv, w.d), 252, device=dev)
    V = I.randn_bf16((w.kv_rows, w.hkv, w.d), 253, device=dev)
    dO = I.randn_bf16((w.o_rows, w.hq, w.d), 254, device=dev)
    O = torch.empty((w.o_rows, w.hq, w.d), dtype=torch.bfloat16, device=dev)
    LSE = torch.empty((w.o_rows, w.hq), device=dev)
    ca.forward(shape, w.tasks, Q, K, V, O, LSE)
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
    ca.backward(shape, w.tasks, Q, K, V, O, dO, LSE, dQ, dK, dV)
    torch.cuda.synchronize()
    worst_k = worst_v = 0.0
    for t in w.tasks:
        q_off, kv_off, o_off, q_len, kv_len = (int(x) for x in t[:5])
        dk = dK[kv_off:kv_off + kv_len].double()
        sum_dk = dk.sum(0)
        worst_k = max(worst_k, float(sum_dk.abs().max() / dk.abs().sum(0).max()))
        sum_dv = dV[kv_off:kv_off + kv_len].double().sum(0)
        sum_do = dO[o_off:o_off + q_len].double().view(q_len, w.hkv, G, w.d).sum((0, 2))
        worst_v = max(worst_v, float((sum_dv - sum_do).abs().max() / sum_do.abs().max()))
        assert bool(torch.isfinite(dk).all())
    assert bool(torch.isfinite(dQ.float()).all())
    print("34b CA-task backward: max|sum dK|/sum|dK| = %.3e, rel max|sum dV - sum dO| = %.3e"
          % (worst_k, worst_v), flush=True)
    assert worst_k < 1e-2 and worst_v < 1e-2


# ---------------------------------------------------------------------------
# causal-blockwise and shared-question masks at 512K, one launch each
# ---------------------------------------------------------------------------

def shard_starts(tasks):
    """Indices of the first task of every query shard (consecutive tasks
    with the same q_off, o_off, q_len, q_pos0 form one)."""
    t = np.asarray(tasks)
    same = np.zeros(len(t), dtype=bool)
    same[1:] = np.all(t[1:, [0, 2, 3, 5]] == t[:-1, [0, 2, 3, 5]], axis=1) & (t[1:, 3] > 0)
    return np.flatnonzero(~same)


def probe_expect_ranges(tasks, T):
    """K = 0 and V = (-1)^(buffer row): every visible key weighs the same, so a
    row's O is the mean of (-1)^row over its visible key rows and LSE the log
    of their count.  Each context contributes the key rows
    [kv_off, kv_off + n_i), n_i = clip(q_pos0 + i - kv_pos0 + 1, 0, kv_len)."""
    ssum = np.zeros(T)
    cnt = np.zeros(T)
    for q_off, kv_off, o_off, q_len, kv_len, q_pos0, kv_pos0 in np.asarray(tasks):
        i = np.arange(q_len)
        n = np.clip(q_pos0 + i - kv_pos0 + 1, 0, kv_len)
        ssum[o_off:o_off + q_len] += sign_sum(np.full(q_len, kv_off), kv_off + n - 1)
        cnt[o_off:o_off + q_len] += n
    return ssum / np.maximum(cnt, 1), cnt


def run_probe_512k(tasks, w, label):
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    T = w.q_rows
    Q = I.randn_bf16((T, w.hq, w.d), 291, device=dev)
    K = torch.zeros((T, w.hkv, w.d), dtype=torch.bfloat16, device=dev)
    sign = torch.from_numpy(np.where(np.arange(T) % 2 == 0, 1.0, -1.0).astype(np.float32)).to(dev)
    V = sign[:, None, None].expand(T, w.hkv, w.d).to(torch.bfloat16).contiguous()
    O = torch.empty((T, w.hq, w.d), dtype=torch.bfloat16, device=dev)
    LSE = torch.empty((T, w.hq), device=dev)
    ca.forward(ca.make_shape(w.hq, w.hkv, w.d, T, T, T), tasks, Q, K, V, O, LSE)
    torch.cuda.synchronize()
    exp_o, cnt = probe_expect_ranges(tasks, T)
    e = torch.from_numpy(exp_o).to(dev)
    c = torch.from_numpy(cnt).to(dev)
    err = (O.float() - e[:, None, None].float()).abs().amax(dim=(1, 2))
    bad = int((err >= (0.25 / c).float()).sum())
    dl = float((LSE.double() - torch.log(c)[:, None]).abs().max())
    print("%s probe: rows=%d bad_rows=%d max|dLSE|=%.2e" % (label, T, bad, dl), flush=True)
    assert bad == 0 and dl < 1e-4


def sampled_shards_512k(tasks, w, picks, label, seed):
    """O and LSE of sampled rows of the picked shards (start indices into the
    table) against the oracle on the shard's own key rows."""
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    T = w.q_rows
    Q = I.randn_bf16((T, w.hq, w.d), seed, device=dev)
    K = I.randn_bf16((T, w.hkv, w.d), seed + 1, device=dev)
    V = I.randn_bf16((T, w.hkv, w.d), seed + 2, device=dev)
    O = torch.empty((T, w.hq, w.d), dtype=torch.bfloat16, device=dev)
    LSE = torch.empty((T, w.hq), device=dev)
    ca.forward(ca.make_shape(w.hq, w.hkv, w.d, T, T, T), tasks, Q, K, V, O, LSE)
    torch.cuda.synchronize()
    starts = list(shard_starts(tasks)) + [len(tasks)]
    rng = np.random.default_rng(seed)
    got_o, got_l, ref_o, ref_l = [], [], [], []
    for s0 in picks:
        s1 = starts[starts.index(s0) + 1]
        segs = np.array(tasks[s0:s1], dtype=np.int64)
        q_off, q_len = int(segs[0, 0]), int(segs[0, 3])
        rows = np.unique(np.concatenate([[0, q_len - 1], rng.integers(0, q_len, 3)]))
        # the shard's key rows, gathered context after context
        local = segs.copy()
        ks, vs, at = [], [], 0
        for k, sg in enumerate(segs):
            ks.append(widen(K[int(sg[1]):int(sg[1]) + int(sg[4])]))
            vs.append(widen(V[int(sg[1]):int(sg[1]) + int(sg[4])]))
            local[k, 1] = at
            at += int(sg[4])
        local[:, 0] = 0
        local[:, 2] = 0
        qs = widen(Q[q_off:q_off + q_len])
        o1, l1 = oracle.forward_rows(local, rows, qs, np.concatenate(ks), np.concatenate(vs), w.scale)
        ref_o.append(o1)
        ref_l.append(l1)
        idx = torch.from_numpy(int(segs[0, 2]) + rows).to(dev)
        got_o.append(widen(O[idx]))
        got_l.append(widen(LSE[idx]))
    check_forward(np.concatenate(got_o), np.concatenate(got_l), np.concatenate(ref_o), np.concatenate(ref_l), label)


def test_blockwise_512k_one_launch_probe_and_sampled():
    """Causal-blockwise mask (256-token blocks, window of 2 blocks, sink block,
    final block sees everything) over the 512K training mix, one launch: the
    probe on every row and head, and the oracle on sampled rows of blocks of
    the longest document (its final block included) and of short documents."""
    announce("fullsize 512k causal-blockwise, one launch: probe + sampled rows")
    w = I.train_8b_prolong_512k()
    tasks = I.blockwise_shards(w.doc_lens, block=256, win_blocks=2)
    run_probe_512k(tasks, w, "512k blockwise")
    starts = shard_starts(tasks)
    longest = int(np.argmax(w.doc_lens))
    d0 = int(np.sum(w.doc_lens[:longest]))
    in_long = [s for s in starts if d0 <= tasks[s][0] < d0 + w.doc_lens[longest]]
    picks = [in_long[0], in_long[1], in_long[2], in_long[len(in_long) // 2], in_long[-2], in_long[-1],
             int(starts[0]), int(starts[-1])]
    sampled_shards_512k(tasks, w, picks, "512k-blockwise-sampled", 295)


def test_shared_question_512k_one_launch_probe_and_sampled():
    """Shared-question batch (49 groups of one question and 4-16 answers over
    512K tokens), one launch: the probe on every row and head, and the oracle
    on sampled rows of questions and answers."""
    announce("fullsize 512k shared question, one launch: probe + sampled rows")
    w, groups = I.shared_question_batch()
    run_probe_512k(w.tasks, w, "512k shared question")
    starts = shard_starts(w.tasks)
    picks = [int(x) for x in starts[[0, 1, 2, len(starts) // 2, len(starts) // 2 + 1, -2, -1]]]
    sampled_shards_512k(w.tasks, w, picks, "512k-shared-question-sampled", 297)
