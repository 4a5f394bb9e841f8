"""One GPU running every rank's share of a context-parallel ring ("Context
Parallelism for Scalable Million-Token Inference"), checked against the fp64
oracle of the unsplit attention:

* full prefill with load-balanced sharding (Section 3.5.1) and the pass-KV
  ring (Section 3.5.2): the 2N per-step partials (ca_ring_kv_step_tasks ->
  ca_forward with fp32 partial output) merged by Equation 4 (ca_merge) equal
  the causal attention of every packed sequence;
* batched decode (Section 3.6): each sequence's cache spread over N ranks by
  the prefill sharding and round-robin decode placement, each rank attending
  to its own share, the N partials merged, equal one query over the whole
  cache."""

import math

import numpy as np
import pytest

import oracle
from long_context_core_amd import ca
from long_context_core_amd import inputs as I
from tests.gpu_util import announce, check_forward, torch_cuda, widen

pytestmark = pytest.mark.gpu


def fuse_slots(tables, rows):
    """The tables of one ring step as one launch: slot j's outputs go to rows
    [j * rows, (j + 1) * rows) of the stacked partial buffer."""
    out = []
    for j, t in enumerate(tables):
        t = t.copy()
        t["o_off"] += j * rows
        out.append(t)
    return np.concatenate(out)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("N,lens", [(4, [700, 1500, 333, 64, 1]), (3, [2048, 100]), (8, [5000, 77, 1029])])
def test_load_balanced_pass_kv_ring_equals_causal_attention(N, lens, fused):
    announce("ring pass-KV, load-balanced sharding: N=%d lens=%s fused=%s" % (N, lens, fused))
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    hq, hkv, d = 8, 2, 128
    T = sum(lens)
    Q = I.randn_bf16((T, hq, d), 2601)
    K = I.randn_bf16((T, hkv, d), 2602)
    V = I.randn_bf16((T, hkv, d), 2603)
    Qd, Kd, Vd = Q.to(dev), K.to(dev), V.to(dev)
    S = 2 * N
    O_p = torch.full((S, T, hq, d), float("nan"), device=dev)
    L_p = torch.full((S, T, hq), float("nan"), device=dev)
    shape = ca.make_shape(hq, hkv, d, T, T, T, out_f32=True)
    if fused:
        # both source chunks of a step in one launch
        fshape = ca.make_shape(hq, hkv, d, T, T, 2 * T, out_f32=True)
        for step in range(N):
            tasks = fuse_slots([ca.ring_kv_step_tasks(lens, N, step, slot) for slot in (0, 1)], T)
            ca.forward(fshape, tasks, Qd, Kd, Vd, O_p[2 * step:2 * step + 2], L_p[2 * step:2 * step + 2])
    else:
        for step in range(N):
            for slot in (0, 1):
                tasks = ca.ring_kv_step_tasks(lens, N, step, slot)
                ca.forward(shape, tasks, Qd, Kd, Vd, O_p[2 * step + slot], L_p[2 * step + slot])
    torch.cuda.synchronize()
    assert not bool(torch.isnan(L_p).any()), "a partial row was left unwritten"
    Om = torch.empty((T, hq, d), device=dev, dtype=torch.bfloat16)
    Lm = torch.empty((T, hq), device=dev)
    ca.merge(ca.make_shape(hq, hkv, d, T, T, T), O_p, L_p, Om, Lm)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.forward(I.varlen_tasks(lens), widen(Q), widen(K), widen(V), 1 / math.sqrt(d))
    check_forward(Om, Lm, O_ref, L_ref, "ring-pass-kv-load-balanced")


def test_round_robin_decode_shares_merge_to_the_whole_cache():
    announce("ring pass-Q decode over round-robin cache shares: N=4, 6 sequences")
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    N, hq, hkv, d = 4, 16, 1, 128
    prefill = [3000, 129, 1, 2500, 640, 77]
    n_dec = 37                      # decode iterations so far, every sequence active
    B = len(prefill)
    lens = [p + n_dec for p in prefill]
    starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    Tk = int(starts[-1])
    K = I.randn_bf16((Tk, hkv, d), 2611)
    V = I.randn_bf16((Tk, hkv, d), 2612)
    Q = I.randn_bf16((B, hq, d), 2613)       # the newest token of each sequence
    # owner of every cached position: prefill by load-balanced chunks, decode
    # token t of sequence b by the round-robin rule
    owner = np.empty(Tk, dtype=np.int64)
    for ch in ca.ring_shard(prefill, N):
        s, b, e = int(ch["seq"]), int(ch["begin"]), int(ch["end"])
        owner[starts[s] + b:starts[s] + e] = int(ch["rank"])
    for b in range(B):
        for t in range(n_dec):
            owner[starts[b] + prefill[b] + t] = ca.ring_decode_rank(N, t, b)
    counts = np.array([[int((owner[starts[b]:starts[b + 1]] == r).sum()) for b in range(B)] for r in range(N)])
    # balance: per sequence, ranks differ by at most two prefill chunks (the
    # clipped tail) plus one decode token
    for b in range(B):
        c = -(-prefill[b] // (2 * N))
        assert counts[:, b].max() - counts[:, b].min() <= 2 * c + 1
    O_p = torch.full((N, B, hq, d), float("nan"), device=dev)
    L_p = torch.full((N, B, hq), float("nan"), device=dev)
    Qd = Q.to(dev)
    for r in range(N):
        rows = np.concatenate([np.nonzero(owner[starts[b]:starts[b + 1]] == r)[0] + starts[b] for b in range(B)])
        idx = torch.from_numpy(rows.astype(np.int64))
        Kr, Vr = K[idx].contiguous().to(dev), V[idx].contiguous().to(dev)
        loc = np.concatenate([[0], np.cumsum(counts[r])])
        # each batch entry's query attends to all of this rank's rows of its own sequence
        tasks = np.array([(b, loc[b], b, 1, counts[r][b], max(0, counts[r][b] - 1), 0) for b in range(B)],
                         dtype=np.int64)
        shape = ca.make_shape(hq, hkv, d, B, max(1, int(loc[-1])), B, out_f32=True)
        ca.forward(shape, tasks, Qd, Kr, Vr, O_p[r], L_p[r])
    torch.cuda.synchronize()
    Om = torch.empty((B, hq, d), device=dev, dtype=torch.bfloat16)
    Lm = torch.empty((B, hq), device=dev)
    ca.merge(ca.make_shape(hq, hkv, d, B, B, B), O_p, L_p, Om, Lm)
    torch.cuda.synchronize()
    whole = np.array([(b, starts[b], b, 1, lens[b], lens[b] - 1, 0) for b in range(B)], dtype=np.int64)
    O_ref, L_ref = oracle.forward(whole, widen(Q), widen(K), widen(V), 1 / math.sqrt(d))
    check_forward(Om, Lm, O_ref, L_ref, "round-robin-decode-merged")


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("N,new,cached", [(4, [700, 1, 333, 64], [3000, 128, 0, 1]), (2, [1500, 90], [777, 4096])])
def test_partial_prefill_ring_equals_attention_over_cache_and_new_tokens(N, new, cached, fused):
    announce("ring partial prefill: N=%d new=%s cached=%s fused=%s" % (N, new, cached, fused))
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    hq, hkv, d = 8, 2, 128
    Tq = sum(new)
    Tk = sum(new) + sum(cached)
    Q = I.randn_bf16((Tq, hq, d), 2621)
    K = I.randn_bf16((Tk, hkv, d), 2622)
    V = I.randn_bf16((Tk, hkv, d), 2623)
    Qd, Kd, Vd = Q.to(dev), K.to(dev), V.to(dev)
    S = 4 * N
    O_p = torch.full((S, Tq, hq, d), float("nan"), device=dev)
    L_p = torch.full((S, Tq, hq), float("nan"), device=dev)
    shape = ca.make_shape(hq, hkv, d, Tq, Tk, Tq, out_f32=True)
    if fused:
        # the four chunk pairs of a step (two cached, two new) in one launch
        fshape = ca.make_shape(hq, hkv, d, Tq, Tk, 4 * Tq, out_f32=True)
        for step in range(N):
            tasks = fuse_slots([ca.ring_prefill_step_tasks(new, cached, N, step, slot) for slot in range(4)], Tq)
            ca.forward(fshape, tasks, Qd, Kd, Vd, O_p[4 * step:4 * step + 4], L_p[4 * step:4 * step + 4])
    else:
        for step in range(N):
            for slot in range(4):
                tasks = ca.ring_prefill_step_tasks(new, cached, N, step, slot)
                ca.forward(shape, tasks, Qd, Kd, Vd, O_p[4 * step + slot], L_p[4 * step + slot])
    torch.cuda.synchronize()
    assert not bool(torch.isnan(L_p).any()), "a partial row was left unwritten"
    Om = torch.empty((Tq, hq, d), device=dev, dtype=torch.bfloat16)
    Lm = torch.empty((Tq, hq), device=dev)
    ca.merge(ca.make_shape(hq, hkv, d, Tq, Tq, Tq), O_p, L_p, Om, Lm)
    torch.cuda.synchronize()
    q0 = np.concatenate([[0], np.cumsum(new)])
    k0 = np.concatenate([[0], np.cumsum(np.array(new) + np.array(cached))])
    whole = np.array([(q0[s], k0[s], q0[s], new[s], new[s] + cached[s], cached[s], 0) for s in range(len(new))],
                     dtype=np.int64)
    O_ref, L_ref = oracle.forward(whole, widen(Q), widen(K), widen(V), 1 / math.sqrt(d))
    check_forward(Om, Lm, O_ref, L_ref, "ring-partial-prefill")
