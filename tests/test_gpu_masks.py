"""GPU parity of the sparse masks ("Dynamic Context Parallelism", Section
2.4, Figure 6) against the fp64 oracle: the lambda mask (sink + sliding
window) through ca_forward_masked, and the causal-blockwise and
shared-question masks as partial slots combined by ca_merge."""

import math

import numpy as np
import pytest

import oracle
from long_context_core_amd import ca
from long_context_core_amd import inputs as I
from tests.gpu_util import announce, check_forward, torch_cuda, widen

pytestmark = pytest.mark.gpu


def run_forward(tasks, hq, hkv, d, T, seed, o_rows=None, out_f32=False):
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    o_rows = T if o_rows is None else o_rows
    Q = I.randn_bf16((T, hq, d), seed)
    K = I.randn_bf16((T, hkv, d), seed + 1)
    V = I.randn_bf16((T, hkv, d), seed + 2)
    shape = ca.make_shape(hq, hkv, d, T, T, o_rows, out_f32=out_f32)
    O = torch.zeros((o_rows, hq, d), dtype=torch.float32 if out_f32 else torch.bfloat16, device=dev)
    LSE = torch.full((o_rows, hq), -float("inf"), device=dev)
    ca.forward(shape, tasks, Q.to(dev), K.to(dev), V.to(dev), O, LSE)
    torch.cuda.synchronize()
    return O, LSE, Q, K, V


@pytest.mark.parametrize("window,sink,hq,hkv,d", [
    (4096, 64, 8, 2, 128), (100, 0, 8, 2, 128), (37, 5, 4, 4, 64), (1, 0, 8, 2, 128),
    (64, 64, 16, 1, 128), (200, 300, 6, 2, 64), (130, 1, 8, 8, 128)])
def test_lambda_mask_forward(window, sink, hq, hkv, d):
    announce("lambda forward window=%d sink=%d hq%d hkv%d d%d" % (window, sink, hq, hkv, d))
    docs = [1500, 1, 70, 700, 333]
    T = sum(docs)
    tasks = I.lambda_tasks(docs, window=window, sink=sink)
    O, LSE, Q, K, V = run_forward(tasks, hq, hkv, d, T, 1400 + window)
    O_ref, LSE_ref = oracle.forward(tasks, widen(Q), widen(K), widen(V), 1 / math.sqrt(d))
    check_forward(O, LSE, O_ref, LSE_ref, "lambda")


def test_lambda_mask_single_rows_and_shards():
    """Windowed single-row tasks (they take the tiled kernel) and mid-document
    shards whose window starts inside the shard's context."""
    announce("lambda forward: single rows and shards")
    rows = [(0, 0, 0, 1, 900, 899, 0, 128, 16),         # last token of a 900-token document
            (1, 900, 1, 1, 50, 49, 0, 4096, 4),
            (2, 950, 2, 300, 1000, 700, 0, 257, 33),     # shard [700, 1000) of a 1000-token document
            (302, 1950, 302, 64, 2000, 1936, 0, 64, 0)]
    T = 2000 + 1950
    tasks = np.array(rows, dtype=np.int64)
    O, LSE, Q, K, V = run_forward(tasks, 8, 2, 128, T, 1450, o_rows=366)
    O_ref, LSE_ref = oracle.forward(tasks, widen(Q), widen(K), widen(V), 1 / math.sqrt(128), o_rows=366)
    check_forward(O, LSE, O_ref, LSE_ref, "lambda rows")


def merged_gpu(tasks, parts, T, hq, hkv, d, seed):
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    O, LSE, Q, K, V = run_forward(tasks, hq, hkv, d, T, seed, o_rows=parts * T, out_f32=True)
    Om = torch.empty((T, hq, d), dtype=torch.bfloat16, device=dev)
    Lm = torch.empty((T, hq), device=dev)
    ca.merge(ca.make_shape(hq, hkv, d, T, T, T), O.view(parts, T, hq, d), LSE.view(parts, T, hq), Om, Lm)
    torch.cuda.synchronize()
    Oo, Lo = oracle.forward(tasks, widen(Q), widen(K), widen(V), 1 / math.sqrt(d), o_rows=parts * T)
    Lo = np.where(np.isnan(Lo), -np.inf, Lo)
    Oo = np.where(np.isnan(Oo), 0.0, Oo)
    O_ref, LSE_ref = oracle.merge(Oo.reshape(parts, T, hq, d), Lo.reshape(parts, T, hq))
    return Om, Lm, O_ref, LSE_ref


def test_blockwise_mask_forward():
    announce("causal-blockwise forward (2 slots + merge)")
    docs = [2100, 300, 1024]
    tasks, parts = I.blockwise_tasks(docs, block=256, win_blocks=2)
    Om, Lm, O_ref, LSE_ref = merged_gpu(tasks, parts, sum(docs), 8, 2, 128, 1460)
    check_forward(Om, Lm, O_ref, LSE_ref, "blockwise")


def test_shared_question_mask_forward():
    announce("shared-question forward (2 slots + merge)")
    question, answers = 700, [300, 129, 1000, 64]
    tasks, parts = I.shared_question_tasks(question, answers)
    Om, Lm, O_ref, LSE_ref = merged_gpu(tasks, parts, question + sum(answers), 8, 2, 128, 1470)
    check_forward(Om, Lm, O_ref, LSE_ref, "shared question")


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------

from tests.gpu_util import GRAD_REL_FRO, rel_fro   # noqa: E402


def gpu_grads(fwd_tasks, bwd_tasks, parts, T, hq, hkv, d, seed):
    """Forward (into partial slots, merged when parts > 1) then the backward
    over bwd_tasks, whose output rows are the merged rows."""
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    Q = I.randn_bf16((T, hq, d), seed)
    K = I.randn_bf16((T, hkv, d), seed + 1)
    V = I.randn_bf16((T, hkv, d), seed + 2)
    dO = I.randn_bf16((T, hq, d), seed + 3)
    Qd, Kd, Vd, dOd = Q.to(dev), K.to(dev), V.to(dev), dO.to(dev)
    shape = ca.make_shape(hq, hkv, d, T, T, T)
    O = torch.empty((T, hq, d), dtype=torch.bfloat16, device=dev)
    LSE = torch.empty((T, hq), device=dev)
    if parts == 1:
        ca.forward(shape, fwd_tasks, Qd, Kd, Vd, O, LSE)
    else:
        sp = ca.make_shape(hq, hkv, d, T, T, parts * T, out_f32=True)
        Op = torch.zeros((parts * T, hq, d), device=dev)
        Lp = torch.full((parts * T, hq), -float("inf"), device=dev)
        ca.forward(sp, fwd_tasks, Qd, Kd, Vd, Op, Lp)
        ca.merge(shape, Op.view(parts, T, hq, d), Lp.view(parts, T, hq), O, LSE)
    dQ, dK, dV = torch.empty_like(Qd), torch.empty_like(Kd), torch.empty_like(Vd)
    ca.backward(shape, bwd_tasks, Qd, Kd, Vd, O, dOd, LSE, dQ, dK, dV)
    torch.cuda.synchronize()
    return (dQ, dK, dV), Q, K, V, dO


def check_grads(got, ref, label):
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        e = rel_fro(widen(g), r)
        print("%s %s relF=%.3e" % (label, name, e), flush=True)
        assert e <= GRAD_REL_FRO, label + " " + name


@pytest.mark.parametrize("window,sink,hq,hkv,d", [
    (300, 16, 8, 2, 128), (37, 0, 4, 4, 64), (1, 0, 8, 2, 128), (130, 129, 16, 1, 128), (64, 0, 6, 2, 64)])
def test_lambda_mask_backward(window, sink, hq, hkv, d):
    announce("lambda backward window=%d sink=%d hq%d hkv%d d%d" % (window, sink, hq, hkv, d))
    docs = [900, 1, 257, 400]
    T = sum(docs)
    tasks = I.lambda_tasks(docs, window=window, sink=sink)
    got, Q, K, V, dO = gpu_grads(tasks, tasks, 1, T, hq, hkv, d, 1500 + window)
    ref = oracle.backward(tasks, widen(Q), widen(K), widen(V), widen(dO), 1 / math.sqrt(d))
    check_grads(got, ref, "lambda bwd")


def merged_row_tasks(tasks):
    """The same tasks writing (and, in the backward, reading) the merged rows."""
    t = np.array(tasks, dtype=np.int64).copy()
    t[:, 2] = t[:, 0]
    return t


def test_blockwise_mask_backward():
    announce("causal-blockwise backward (merged partials)")
    docs = [700, 200, 333]
    block, w = 128, 2
    hq, hkv, d = 4, 2, 64
    T = sum(docs)
    tasks, parts = I.blockwise_tasks(docs, block=block, win_blocks=w)
    got, Q, K, V, dO = gpu_grads(tasks, merged_row_tasks(tasks), parts, T, hq, hkv, d, 1520)
    rows_keys, start = [], 0
    for L in docs:
        nb = -(-L // block)
        for p in range(L):
            b = p // block
            if b == nb - 1:
                keys = list(range(p + 1))
            else:
                keys = sorted(set(range(min(block, p + 1))) | set(range(max(0, b - w + 1) * block, p + 1)))
            rows_keys.append([start + k for k in keys])
        start += L
    ref = oracle.backward_listed(widen(Q), widen(K), widen(V), widen(dO), 1 / math.sqrt(d), rows_keys)
    check_grads(got, ref, "blockwise bwd")


def test_shared_question_mask_backward():
    announce("shared-question backward (merged partials)")
    question, answers = 300, [150, 7, 260]
    hq, hkv, d = 4, 2, 64
    T = question + sum(answers)
    tasks, parts = I.shared_question_tasks(question, answers)
    got, Q, K, V, dO = gpu_grads(tasks, merged_row_tasks(tasks), parts, T, hq, hkv, d, 1530)
    rows_keys = [list(range(p + 1)) for p in range(question)]
    off = question
    for a in answers:
        rows_keys += [list(range(question)) + [off + j for j in range(i + 1)] for i in range(a)]
        off += a
    ref = oracle.backward_listed(widen(Q), widen(K), widen(V), widen(dO), 1 / math.sqrt(d), rows_keys)
    check_grads(got, ref, "shared-question bwd")


# ---------------------------------------------------------------------------
# one launch: query shards over several contexts (no partial slots, no merge)
# ---------------------------------------------------------------------------

def fused_grads(tasks, T, hq, hkv, d, seed, masks=None):
    """Forward and backward of one shard table in single launches; returns
    device O, LSE, the gradients and the host inputs."""
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    Q = I.randn_bf16((T, hq, d), seed)
    K = I.randn_bf16((T, hkv, d), seed + 1)
    V = I.randn_bf16((T, hkv, d), seed + 2)
    dO = I.randn_bf16((T, hq, d), seed + 3)
    Qd, Kd, Vd, dOd = Q.to(dev), K.to(dev), V.to(dev), dO.to(dev)
    shape = ca.make_shape(hq, hkv, d, T, T, T)
    O = torch.full((T, hq, d), float("nan"), dtype=torch.bfloat16, device=dev)
    LSE = torch.full((T, hq), float("nan"), device=dev)
    ca.forward(shape, tasks, Qd, Kd, Vd, O, LSE, masks=masks)
    dQ, dK, dV = torch.empty_like(Qd), torch.empty_like(Kd), torch.empty_like(Vd)
    ca.backward(shape, tasks, Qd, Kd, Vd, O, dOd, LSE, dQ, dK, dV, masks=masks)
    torch.cuda.synchronize()
    return O, LSE, (dQ, dK, dV), Q, K, V, dO


@pytest.mark.parametrize("block,w,hq,hkv,d", [(256, 2, 8, 2, 128), (128, 3, 4, 4, 64), (64, 1, 16, 1, 128)])
def test_blockwise_one_launch(block, w, hq, hkv, d):
    """Causal-blockwise mask as query shards over two contexts (sink block
    and causal window): forward and backward in one launch each, against
    the oracle (and the oracle's listed-key gradient)."""
    announce("causal-blockwise in one launch: block %d window %d hq%d hkv%d d%d" % (block, w, hq, hkv, d))
    docs = [2100, 300, 1024, 77]
    T = sum(docs)
    tasks = I.blockwise_shards(docs, block=block, win_blocks=w)
    O, LSE, got, Q, K, V, dO = fused_grads(tasks, T, hq, hkv, d, 1540 + block)
    Qw, Kw, Vw, dOw = widen(Q), widen(K), widen(V), widen(dO)
    O_ref, LSE_ref = oracle.forward(tasks, Qw, Kw, Vw, 1 / math.sqrt(d))
    check_forward(O, LSE, O_ref, LSE_ref, "blockwise one launch")
    check_grads(got, oracle.backward(tasks, Qw, Kw, Vw, dOw, 1 / math.sqrt(d)), "blockwise one launch bwd")


@pytest.mark.parametrize("hq,hkv,d", [(8, 2, 128), (4, 1, 64)])
def test_shared_question_one_launch(hq, hkv, d):
    announce("shared question in one launch: hq%d hkv%d d%d" % (hq, hkv, d))
    question, answers = 700, [300, 129, 1000, 64, 1]
    T = question + sum(answers)
    tasks = I.shared_question_shards(question, answers)
    O, LSE, got, Q, K, V, dO = fused_grads(tasks, T, hq, hkv, d, 1560 + d)
    Qw, Kw, Vw, dOw = widen(Q), widen(K), widen(V), widen(dO)
    O_ref, LSE_ref = oracle.forward(tasks, Qw, Kw, Vw, 1 / math.sqrt(d))
    check_forward(O, LSE, O_ref, LSE_ref, "shared question one launch")
    check_grads(got, oracle.backward(tasks, Qw, Kw, Vw, dOw, 1 / math.sqrt(d)), "shared question one launch bwd")


def random_shard_table(rng, T):
    """Random query shards of 1-3 contexts each over one T-row buffer: query
    row ranges tile [0, T) (ragged lengths, single rows included); each
    context is a random key range with random positions, some of them
    windowed; keys of a shard's contexts may repeat (they then count twice)."""
    rows, masks, q = [], [], 0
    while q < T:
        ql = int(min(T - q, rng.choice([1, 5, 31, 64, 100, 257, 600])))
        qp = int(rng.integers(0, 3000))
        for _ in range(int(rng.integers(1, 4))):
            kl = int(rng.integers(0, min(T, 1500)))
            ko = int(rng.integers(0, T - kl + 1))
            kp = int(rng.integers(max(0, qp - kl - 50), qp + 60))
            rows.append((q, ko, q, ql, kl, qp, kp))
            win = int(rng.choice([0, 0, 0, 1, 40, 700]))
            masks.append((win, int(rng.integers(0, 80)) if win else 0))
        q += ql
    return np.array(rows, dtype=np.int64), np.array(masks, dtype=np.int64)


@pytest.mark.parametrize("seed,hq,hkv,d", [(0, 8, 2, 128), (1, 4, 4, 64), (2, 16, 1, 128), (3, 6, 2, 64)])
def test_random_multi_context_shards(seed, hq, hkv, d):
    announce("random multi-context shards seed=%d hq%d hkv%d d%d" % (seed, hq, hkv, d))
    rng = np.random.default_rng(1580 + seed)
    T = 2400
    tasks, masks = random_shard_table(rng, T)
    O, LSE, got, Q, K, V, dO = fused_grads(tasks, T, hq, hkv, d, 1590 + seed, masks=masks)
    Qw, Kw, Vw, dOw = widen(Q), widen(K), widen(V), widen(dO)
    full = np.concatenate([tasks, masks], axis=1)
    O_ref, LSE_ref = oracle.forward(full, Qw, Kw, Vw, 1 / math.sqrt(d))
    check_forward(O, LSE, O_ref, LSE_ref, "random shards")
    check_grads(got, oracle.backward(full, Qw, Kw, Vw, dOw, 1 / math.sqrt(d)), "random shards bwd")
