"""Scheduled CA-tasks on the GPU: the task tables the scheduler gives each
attention server, run one server after another through ca_forward /
ca_backward on the packed batch, reproduce the attention of the whole batch
(composability of CA-tasks: "Efficient Long-context Language Model Training by
Core Attention Disaggregation", Section 4.1, Property 2), checked against the
fp64 oracle."""

import math

import numpy as np
import pytest

import oracle
from oracle import scheduler as S
from long_context_core_amd import ca
from long_context_core_amd import inputs as I
from tests.gpu_util import GRAD_REL_FRO, announce, check_forward, rel_fro, torch_cuda, widen

pytestmark = pytest.mark.gpu

HQ, HKV, D = 8, 2, 128
FPP = 4 * D * HQ


def flops_grid():
    gq, gkv = [64, 512, 4096], [64, 1024, 16384]
    return gq, gkv, [[1e-5 + FPP * S.block_pairs(min(x, y), y) / 8e14 for y in gkv] for x in gq]


def scheduled(docs, k, head_tail=False):
    gq, gkv, gt = flops_grid()
    items, before, after, comm, moves = ca.schedule(docs, k, gq, gkv, gt, FPP, HQ, HKV, D,
                                                    eps=0.02, min_shard=64, head_tail=head_tail)
    assert moves > 0
    if head_tail:
        # at least one Item was split into a head and a tail on one server
        firsts = {(int(r["doc"]), int(r["q_begin"])) for r in items}
        assert any(int(r["q_begin"]) > 0 and (int(r["doc"]), 0) in firsts for r in items)
    return [ca.sched_tasks(items[items["server"] == s], docs) for s in range(k)]


@pytest.mark.parametrize("head_tail", [False, True])
def test_scheduled_forward_equals_whole_batch(head_tail):
    announce("scheduled forward: 5 documents on 4 servers, head_tail=%s" % head_tail)
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    docs = [3000, 700, 1500, 64, 900]
    T = sum(docs)
    Q = I.randn_bf16((T, HQ, D), 1301)
    K = I.randn_bf16((T, HKV, D), 1302)
    V = I.randn_bf16((T, HKV, D), 1303)
    Qd, Kd, Vd = Q.to(dev), K.to(dev), V.to(dev)
    shape = ca.make_shape(HQ, HKV, D, T, T, T)
    O = torch.full((T, HQ, D), float("nan"), dtype=torch.bfloat16, device=dev)
    LSE = torch.full((T, HQ), float("nan"), device=dev)
    for tasks in scheduled(docs, 4, head_tail):
        if len(tasks):
            ca.forward(shape, tasks, Qd, Kd, Vd, O, LSE)
    torch.cuda.synchronize()
    O_ref, LSE_ref = oracle.forward(I.varlen_tasks(docs), widen(Q), widen(K), widen(V), 1 / math.sqrt(D))
    check_forward(O, LSE, O_ref, LSE_ref, "scheduled forward")


@pytest.mark.parametrize("head_tail", [False, True])
def test_scheduled_backward_sums_to_whole_batch(head_tail):
    announce("scheduled backward: 4 documents on 3 servers, head_tail=%s" % head_tail)
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    docs = [2500, 300, 1800, 600]
    T = sum(docs)
    Q = I.randn_bf16((T, HQ, D), 1311)
    K = I.randn_bf16((T, HKV, D), 1312)
    V = I.randn_bf16((T, HKV, D), 1313)
    dO = I.randn_bf16((T, HQ, D), 1314)
    Qd, Kd, Vd, dOd = Q.to(dev), K.to(dev), V.to(dev), dO.to(dev)
    shape = ca.make_shape(HQ, HKV, D, T, T, T)
    O = torch.empty((T, HQ, D), dtype=torch.bfloat16, device=dev)
    LSE = torch.empty((T, HQ), device=dev)
    per_server = scheduled(docs, 3, head_tail)
    for tasks in per_server:
        if len(tasks):
            ca.forward(shape, tasks, Qd, Kd, Vd, O, LSE)
    dQ = torch.zeros((T, HQ, D), device=dev)
    dK = torch.zeros((T, HKV, D), device=dev)
    dV = torch.zeros((T, HKV, D), device=dev)
    for tasks in per_server:
        if not len(tasks):
            continue
        gq, gk, gv = torch.empty_like(Qd), torch.empty_like(Kd), torch.empty_like(Vd)
        ca.backward(shape, tasks, Qd, Kd, Vd, O, dOd, LSE, gq, gk, gv)
        dQ += gq.float()
        dK += gk.float()
        dV += gv.float()
    torch.cuda.synchronize()
    ref = oracle.backward(I.varlen_tasks(docs), widen(Q), widen(K), widen(V), widen(dO), 1 / math.sqrt(D))
    for name, g, r in zip(("dQ", "dK", "dV"), (dQ, dK, dV), ref):
        e = rel_fro(widen(g), r)
        print("scheduled backward %s relF=%.3e" % (name, e), flush=True)
        assert e <= GRAD_REL_FRO, name
