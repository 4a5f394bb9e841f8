"""GPU parity of ca_backward against the fp64 oracle (small cases, element by
element) and, at the full training shape, against exact invariants and the
probe's closed forms (every row, every head)."""

import math

import numpy as np
import pytest

import oracle
from long_context_core_amd import ca
from long_context_core_amd import inputs as I
from tests.gpu_util import GRAD_REL_FRO, announce, rel_fro, torch_cuda, widen

pytestmark = pytest.mark.gpu


def gpu_fwd_bwd(tasks, hq, hkv, d, q_rows, kv_rows, o_rows, Q, K, V, dO):
    """Forward (bf16 O, LSE) then backward on the GPU; returns device tensors."""
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    Qd, Kd, Vd, dOd = Q.to(dev), K.to(dev), V.to(dev), dO.to(dev)
    shape = ca.make_shape(hq, hkv, d, q_rows, kv_rows, o_rows)
    O = torch.zeros((o_rows, hq, d), dtype=torch.bfloat16, device=dev)
    LSE = torch.full((o_rows, hq), -float("inf"), device=dev)
    ca.forward(shape, tasks, Qd, Kd, Vd, O, LSE)
    dQ = torch.full_like(Qd, float("nan"))
    dK = torch.full_like(Kd, float("nan"))
    dV = torch.full_like(Vd, float("nan"))
    ca.backward(shape, tasks, Qd, Kd, Vd, O, dOd, LSE, dQ, dK, dV)
    torch.cuda.synchronize()
    return dQ, dK, dV


def check_grads(got, ref, label):
    out = []
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        gw = widen(g)
        assert np.all(np.isfinite(gw)), label + " " + name + " not finite"
        e = rel_fro(gw, r)
        out.append(e)
        print("%s %s relF=%.3e max|d|=%.3e" % (label, name, e, float(np.max(np.abs(gw - r)))), flush=True)
        assert e <= GRAD_REL_FRO, label + " " + name
    return out


def run_small(tasks, hq, hkv, d, q_rows, kv_rows, o_rows, seed, label):
    Q = I.randn_bf16((q_rows, hq, d), seed)
    K = I.randn_bf16((kv_rows, hkv, d), seed + 1)
    V = I.randn_bf16((kv_rows, hkv, d), seed + 2)
    dO = I.randn_bf16((o_rows, hq, d), seed + 3)
    got = gpu_fwd_bwd(tasks, hq, hkv, d, q_rows, kv_rows, o_rows, Q, K, V, dO)
    ref = oracle.backward(tasks, widen(Q), widen(K), widen(V), widen(dO), 1 / math.sqrt(d))
    return check_grads(got, ref, label)


@pytest.mark.parametrize("hq,hkv,d", [(8, 2, 128), (4, 4, 64), (16, 1, 128), (6, 2, 64), (8, 4, 128), (16, 2, 64)])
def test_backward_ragged_varlen(hq, hkv, d):
    announce("backward ragged varlen hq%d hkv%d d%d" % (hq, hkv, d))
    lens = [1, 31, 33, 64, 130, 200, 257]
    T = sum(lens)
    run_small(I.varlen_tasks(lens), hq, hkv, d, T, T, T, 800 + hq + d, "bwd-ragged")


def test_backward_ca_tasks_unaligned():
    announce("backward CA-tasks unaligned")
    rng = np.random.default_rng(17)
    tasks, qo, ko = [], 0, 0
    for _ in range(6):
        doc = int(rng.integers(200, 900))
        ql = int(rng.integers(1, 200))
        end = int(rng.integers(ql, doc + 1))
        tasks.append((qo, ko, qo, ql, end, end - ql, 0))
        qo += ql
        ko += end
    run_small(np.array(tasks), 16, 2, 128, qo, ko, qo, 900, "bwd-ca-tasks")


def test_backward_shared_rows_multi_pass():
    """Ring partial tasks share query shards and KV blocks: gradients must
    sum over tasks (fp32 accumulation across passes).  Output rows of the
    partials are distinct, dO is given per partial."""
    announce("backward ring partials (shared rows)")
    T, n = 384, 3
    S = T // n
    tasks = np.array([(i * S, j * S, j * T + i * S, S, S, i * S, j * S) for i in range(n) for j in range(i + 1)])
    run_small(tasks, 8, 1, 128, T, T, n * T, 950, "bwd-ring")


def test_backward_decode_rows_and_empty():
    announce("backward decode rows and empty rows")
    tasks = np.array([(0, 0, 0, 1, 700, 699, 0), (1, 700, 1, 1, 300, 100, 0),
                      (2, 1000, 2, 40, 50, 0, 30),          # first rows see nothing
                      (42, 0, 42, 5, 0, 0, 0)])            # empty context
    run_small(tasks, 16, 2, 64, 47, 1050, 47, 970, "bwd-decode-empty")


# --------------------------------------------------------------------------
# full training shape: 524,288 tokens, ProLong-like mix, 32 / 8 heads, d = 128
# --------------------------------------------------------------------------

def doc_layout(w):
    pos = np.zeros(w.q_rows, dtype=np.int64)
    end = np.zeros(w.q_rows, dtype=np.int64)    # one past the document's last row
    for t in w.tasks:
        o, l = int(t[0]), int(t[3])
        pos[o:o + l] = np.arange(l)
        end[o:o + l] = o + l
    return pos, end


def suffix_in_doc(torch, x, end):
    """For each row j: sum of x over rows j..(end of j's document) - 1."""
    c = torch.flip(torch.cumsum(torch.flip(x, [0]), 0), [0])     # c[j] = sum_{i >= j} x[i]
    pad = torch.cat([c, torch.zeros_like(c[:1])], 0)
    return c - pad[end]


def test_backward_train_512k_invariants_and_probe():
    announce("backward full 512k prolong-like: invariants + probe closed forms")
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    w = I.train_8b_prolong_512k()
    T, hq, hkv, d, G = w.q_rows, w.hq, w.hkv, w.d, w.hq // w.hkv
    shape = ca.make_shape(hq, hkv, d, T, T, T)
    pos, end = doc_layout(w)
    end_t = torch.from_numpy(end).to(dev)

    # (1) random inputs: per document and KV head, sum_j dK_j = 0 and
    #     sum_j dV_j = sum_i sum_{h in group} dO_i
    Q = I.randn_bf16((T, hq, d), 205, device=dev)
    K = I.randn_bf16((T, hkv, d), 206, device=dev)
    V = I.randn_bf16((T, hkv, d), 207, device=dev)
    dO = I.randn_bf16((T, hq, d), 208, device=dev)
    O = torch.empty_like(Q)
    LSE = torch.empty((T, hq), device=dev)
    ca.forward(shape, w.tasks, Q, K, V, O, LSE)
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
    ca.backward(shape, w.tasks, Q, K, V, O, dO, LSE, dQ, dK, dV)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(dQ.float()).all() and torch.isfinite(dK.float()).all() and torch.isfinite(dV.float()).all())
    doc_id = torch.from_numpy(np.searchsorted(np.cumsum(w.doc_lens), np.arange(T), side="right")).to(dev)
    nd = len(w.doc_lens)
    sum_dk = torch.zeros((nd, hkv, d), dtype=torch.float64, device=dev).index_add_(0, doc_id, dK.double())
    sum_dv = torch.zeros((nd, hkv, d), dtype=torch.float64, device=dev).index_add_(0, doc_id, dV.double())
    sum_do = torch.zeros((nd, hkv, d), dtype=torch.float64, device=dev).index_add_(
        0, doc_id, dO.double().view(T, hkv, G, d).sum(2))
    scale_k = float(dK.double().abs().sum(0).max())
    e_dk = float(sum_dk.abs().max()) / scale_k
    e_dv = float((sum_dv - sum_do).abs().max() / sum_do.abs().max())
    print("512k invariants: max|sum dK|/sum|dK| = %.3e, rel max|sum dV - sum dO| = %.3e" % (e_dk, e_dv), flush=True)
    assert e_dk < 1e-2 and e_dv < 1e-2
    del Q, K, V, dO, O, LSE, dQ, dK, dV, sum_dk, sum_dv, sum_do
    torch.cuda.empty_cache()

    # (2) probe: K = 0, V = (-1)^position.  dQ = 0 exactly; dV and dK by
    #     in-document suffix sums (float64, computed here with torch).
    Q = I.randn_bf16((T, hq, d), 215, device=dev)
    dO = I.randn_bf16((T, hq, d), 218, device=dev)
    K = torch.zeros((T, hkv, d), dtype=torch.bfloat16, device=dev)
    pos_t = torch.from_numpy(pos).to(dev)
    sign = torch.where(pos_t % 2 == 0, 1.0, -1.0).double()
    V = sign.float()[:, None, None].expand(T, hkv, d).to(torch.bfloat16).contiguous()
    O = torch.empty_like(Q)
    LSE = torch.empty((T, hq), device=dev)
    ca.forward(shape, w.tasks, Q, K, V, O, LSE)
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
    ca.backward(shape, w.tasks, Q, K, V, O, dO, LSE, dQ, dK, dV)
    torch.cuda.synchronize()
    assert float(dQ.float().abs().max()) == 0.0
    inv = 1.0 / (pos_t.double() + 1.0)                                  # 1/(i+1)
    o_i = torch.where(pos_t % 2 == 0, inv, torch.zeros_like(inv))       # O_i (every channel)
    dOd = dO.double()
    dv_ref = suffix_in_doc(torch, (dOd * inv[:, None, None]).view(T, hkv, G, d).sum(2), end_t)
    e_dv = float(torch.linalg.norm(dV.double() - dv_ref) / torch.linalg.norm(dv_ref))
    a = dOd.sum(2)                                                      # [T, hq]
    Qd = Q.double()
    A = suffix_in_doc(torch, (a * inv[:, None])[:, :, None].mul(Qd).view(T, hkv, G, d).sum(2), end_t)
    B = suffix_in_doc(torch, (a * inv[:, None] * o_i[:, None])[:, :, None].mul(Qd).view(T, hkv, G, d).sum(2), end_t)
    dk_ref = (1.0 / math.sqrt(d)) * (sign[:, None, None] * A - B)
    e_dk = float(torch.linalg.norm(dK.double() - dk_ref) / torch.linalg.norm(dk_ref))
    print("512k probe: dQ == 0, relF(dV)=%.3e relF(dK)=%.3e" % (e_dv, e_dk), flush=True)
    assert e_dv <= GRAD_REL_FRO and e_dk <= GRAD_REL_FRO


def test_backward_train_prolong_like_64th_scale_full_oracle():
    """The same length recipe at 1/64 scale (8,192 tokens), checked element by
    element against the oracle."""
    announce("backward prolong-like 1/64 scale vs oracle")
    w = I.train_8b_prolong_512k(div=64)
    run_small(w.tasks, w.hq, w.hkv, w.d, w.q_rows, w.kv_rows, w.o_rows, 990, "bwd-prolong-1/64")


# --------------------------------------------------------------------------
# dK/dV tiles with more query rows than one work item should sweep: split
# into items over member or row ranges whose fp32 partial slots are summed
# --------------------------------------------------------------------------

def test_backward_split_tiles_vs_oracle():
    """A 9,000-token causal document (its first key tiles are seen by more
    than 8,192 rows: split by row ranges) and a shared question read by 30
    answers of 300 rows (split by member ranges), element by element against
    the oracle."""
    announce("backward split dK/dV tiles (row and member splits) vs oracle")
    docs = I.varlen_tasks([9000, 300])
    sq = I.shared_question_shards(200, [300] * 30)
    sq[:, [0, 1, 2]] += 9300
    tasks = np.concatenate([docs, sq])
    T = 9300 + 200 + 9000
    run_small(tasks, 2, 1, 64, T, T, T, 1010, "bwd-split-tiles")


def test_backward_split_tiles_probe():
    """Probe closed forms (K = 0, V = (-1)^position: dQ = 0 exactly, dV and
    dK by in-document suffix sums) for documents whose early key tiles are
    split over many row ranges, Llama-3-8B heads."""
    announce("backward split dK/dV tiles: probe closed forms, 40K + 20K + 5K docs")
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    lens = [40000, 20000, 5000, 77]
    w = I.Workload("split-probe", 32, 8, 128, I.varlen_tasks(lens), sum(lens), sum(lens), sum(lens), doc_lens=lens)
    T, hq, hkv, d, G = w.q_rows, w.hq, w.hkv, w.d, w.hq // w.hkv
    shape = ca.make_shape(hq, hkv, d, T, T, T)
    pos, end = doc_layout(w)
    end_t = torch.from_numpy(end).to(dev)
    Q = I.randn_bf16((T, hq, d), 1015, device=dev)
    dO = I.randn_bf16((T, hq, d), 1018, device=dev)
    K = torch.zeros((T, hkv, d), dtype=torch.bfloat16, device=dev)
    pos_t = torch.from_numpy(pos).to(dev)
    sign = torch.where(pos_t % 2 == 0, 1.0, -1.0).double()
    V = sign.float()[:, None, None].expand(T, hkv, d).to(torch.bfloat16).contiguous()
    O = torch.empty_like(Q)
    LSE = torch.empty((T, hq), device=dev)
    ca.forward(shape, w.tasks, Q, K, V, O, LSE)
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
    ca.backward(shape, w.tasks, Q, K, V, O, dO, LSE, dQ, dK, dV)
    torch.cuda.synchronize()
    assert float(dQ.float().abs().max()) == 0.0
    inv = 1.0 / (pos_t.double() + 1.0)
    o_i = torch.where(pos_t % 2 == 0, inv, torch.zeros_like(inv))
    dOd = dO.double()
    dv_ref = suffix_in_doc(torch, (dOd * inv[:, None, None]).view(T, hkv, G, d).sum(2), end_t)
    e_dv = float(torch.linalg.norm(dV.double() - dv_ref) / torch.linalg.norm(dv_ref))
    a = dOd.sum(2)
    Qd = Q.double()
    A = suffix_in_doc(torch, (a * inv[:, None])[:, :, None].mul(Qd).view(T, hkv, G, d).sum(2), end_t)
    B = suffix_in_doc(torch, (a * inv[:, None] * o_i[:, None])[:, :, None].mul(Qd).view(T, hkv, G, d).sum(2), end_t)
    dk_ref = (1.0 / math.sqrt(d)) * (sign[:, None, None] * A - B)
    e_dk = float(torch.linalg.norm(dK.double() - dk_ref) / torch.linalg.norm(dk_ref))
    # the split tiles themselves: the first 256 keys of the 40K document
    e_dk0 = float(torch.linalg.norm(dK[:256].double() - dk_ref[:256]) / torch.linalg.norm(dk_ref[:256]))
    e_dv0 = float(torch.linalg.norm(dV[:256].double() - dv_ref[:256]) / torch.linalg.norm(dv_ref[:256]))
    print("split probe: relF(dV)=%.3e relF(dK)=%.3e, first 256 keys: relF(dV)=%.3e relF(dK)=%.3e"
          % (e_dv, e_dk, e_dv0, e_dk0), flush=True)
    assert max(e_dv, e_dk, e_dv0, e_dk0) <= GRAD_REL_FRO


# --------------------------------------------------------------------------
# query shards whose items would sweep very long contexts: split over key
# chunks (fp32 partials merged by Equation 4 in the forward, summed for dQ)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("hq,hkv,d", [(8, 2, 128), (4, 1, 64)])
def test_split_long_shards_forward_and_backward_vs_oracle(hq, hkv, d):
    """A 64-row shard at the end of a 70,000-token context, a 32-row shard
    over three contexts (two 40,000-key prefixes, all visible, and its own
    rows, causal) and a short document: the long shards' items are split
    over key chunks.  O, LSE and dQ, dK, dV element by element against the
    oracle."""
    announce("split long shards (forward merge, dQ sum) hq%d hkv%d d%d" % (hq, hkv, d))
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    tasks = np.array([(0, 0, 0, 64, 70000, 69936, 0),                 # shard A
                      (64, 70000, 64, 32, 40000, 100000, 0),          # shard B: prefix 1
                      (64, 110000, 64, 32, 40000, 100000, 40000),     #          prefix 2
                      (64, 150000, 64, 32, 32, 100000, 100000),       #          own rows, causal
                      (96, 150032, 96, 300, 300, 0, 0)], dtype=np.int64)
    q_rows, kv_rows = 396, 150332
    shape = ca.make_shape(hq, hkv, d, q_rows, kv_rows, q_rows)
    assert ca.forward_queue_info(shape, tasks)["split_shards"] == 2   # both long shards
    Q = I.randn_bf16((q_rows, hq, d), 1031)
    K = I.randn_bf16((kv_rows, hkv, d), 1032)
    V = I.randn_bf16((kv_rows, hkv, d), 1033)
    dO = I.randn_bf16((q_rows, hq, d), 1034)
    Qd, Kd, Vd, dOd = Q.to(dev), K.to(dev), V.to(dev), dO.to(dev)
    O = torch.full((q_rows, hq, d), float("nan"), dtype=torch.bfloat16, device=dev)
    LSE = torch.full((q_rows, hq), float("nan"), device=dev)
    ca.forward(shape, tasks, Qd, Kd, Vd, O, LSE)
    dQ, dK, dV = torch.empty_like(Qd), torch.empty_like(Kd), torch.empty_like(Vd)
    ca.backward(shape, tasks, Qd, Kd, Vd, O, dOd, LSE, dQ, dK, dV)
    torch.cuda.synchronize()
    Qw, Kw, Vw, dOw = widen(Q), widen(K), widen(V), widen(dO)
    O_ref, LSE_ref = oracle.forward(tasks, Qw, Kw, Vw, 1 / math.sqrt(d))
    from tests.gpu_util import check_forward
    check_forward(O, LSE, O_ref, LSE_ref, "split shards fwd")
    check_grads((dQ, dK, dV), oracle.backward(tasks, Qw, Kw, Vw, dOw, 1 / math.sqrt(d)), "split shards bwd")
