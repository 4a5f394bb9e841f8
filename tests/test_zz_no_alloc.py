"""ca_forward_noalloc, the forward for callers that cannot allocate, against
ca_forward_masked (its queue in a caller workspace): bit-identical outputs on
two calls in a row, the second smaller than the first (the shared scratch
keeps the first call's queue), and the same under HIP graph capture with
other calls between the replays."""

import ctypes

import numpy as np
import pytest

from long_context_core_amd import ca
from long_context_core_amd import inputs as I
from tests.gpu_util import announce, torch_cuda

pytestmark = pytest.mark.gpu

HQ, HKV, D = 16, 2, 128


def workload(docs, n_dec, ctx, window=0, sink=0):
    """Packed causal documents (optionally windowed) followed by n_dec single
    query rows, each over its own ctx-entry cache split into 4 blocks that
    write 4 partial slots (decode items, split into chunks, merged)."""
    t = [list(r) + [window, sink] for r in I.varlen_tasks(docs)]
    T = int(sum(docs))
    kv = T
    for b in range(n_dec):
        for s in range(4):
            S = ctx // 4
            t.append([T + b, kv + s * S, T + n_dec + s * n_dec + b, 1, S, ctx - 1, s * S, 0, 0])
        kv += ctx
    return np.array(t, dtype=np.int64), T + n_dec, kv, T + 5 * n_dec


def run_pair(torch, dev, tasks, q_rows, kv_rows, o_rows, seed):
    shape = ca.make_shape(HQ, HKV, D, q_rows, kv_rows, o_rows, out_f32=True)
    Q = I.randn_bf16((q_rows, HQ, D), seed, device=dev)
    K = I.randn_bf16((kv_rows, HKV, D), seed + 1, device=dev)
    V = I.randn_bf16((kv_rows, HKV, D), seed + 2, device=dev)
    outs = []
    for noalloc in (True, False):
        O = torch.full((o_rows, HQ, D), 5.0, device=dev)
        LSE = torch.full((o_rows, HQ), 5.0, device=dev)
        if noalloc:
            ca.forward_noalloc(shape, tasks, Q, K, V, O, LSE)
        else:
            ca.forward(shape, tasks, Q, K, V, O, LSE)
        outs.append((O, LSE))
    torch.cuda.synchronize()
    (O1, L1), (O2, L2) = outs
    same = torch.equal(O1, O2) and torch.equal(L1.view(torch.int32), L2.view(torch.int32))
    print("noalloc vs workspace call: q_rows=%d kv_rows=%d tasks=%d identical=%s"
          % (q_rows, kv_rows, len(tasks), same), flush=True)
    assert same
    return Q, K, V


def test_noalloc_equals_workspace_call_twice_second_smaller():
    announce("ca_forward_noalloc vs ca_forward_masked: two calls, the second smaller")
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    big = workload([3000, 517, 1, 1200], 6, 40000, window=700, sink=16)
    small = workload([300, 45], 2, 3000)
    for k, (tasks, q_rows, kv_rows, o_rows) in enumerate((big, small)):
        run_pair(torch, dev, tasks, q_rows, kv_rows, o_rows, 2900 + 10 * k)


def test_noalloc_persistent_launch_equals_per_item_workspace_call():
    """The persistent launch from the scratch (its claim counters live there
    and are reset by a kernel before each launch): two calls in a row, the
    second smaller, each bit-identical to a one-workgroup-per-item call with a
    caller workspace."""
    announce("ca_forward_noalloc, persistent launch, two calls vs per-item workspace calls")
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(2977)
    for k, n_docs in enumerate((500, 120)):
        lens = [int(x) for x in rng.integers(1, 400, size=n_docs)]
        tasks = I.varlen_tasks(lens)
        T = sum(lens)
        sp = ca.make_shape(HQ, HKV, D, T, T, T, launch="persistent")
        si = ca.make_shape(HQ, HKV, D, T, T, T, launch="per_item")
        assert ca.forward_queue_info(sp, tasks)["persistent_workgroups"] > 0
        Q = I.randn_bf16((T, HQ, D), 2980 + k, device=dev)
        K = I.randn_bf16((T, HKV, D), 2990 + k, device=dev)
        V = I.randn_bf16((T, HKV, D), 3000 + k, device=dev)
        O1 = torch.full((T, HQ, D), float("nan"), dtype=torch.bfloat16, device=dev)
        L1 = torch.full((T, HQ), float("nan"), device=dev)
        O2, L2 = torch.empty_like(O1), torch.empty_like(L1)
        ca.forward_noalloc(sp, tasks, Q, K, V, O1, L1)
        ca.forward(si, tasks, Q, K, V, O2, L2)
        torch.cuda.synchronize()
        same = torch.equal(O1.view(torch.int16), O2.view(torch.int16)) and torch.equal(L1, L2)
        print("persistent noalloc call %d (T=%d): identical to the per-item call: %s" % (k, T, same), flush=True)
        assert same


def test_noalloc_rejects_a_queue_beyond_the_scratch():
    """A table whose queue exceeds the scratch is refused before any launch
    (CA_ERR_WORKSPACE), and the outputs stay untouched."""
    announce("ca_forward_noalloc rejects a queue beyond its scratch")
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    n = 1_100_000                                  # 1.1M windowed single rows: > 64 MiB of queue
    t = np.zeros((n, 7), dtype=np.int64)
    t[:, 0] = t[:, 2] = np.arange(n)
    t[:, 3] = 1
    t[:, 4] = 1
    masks = np.tile(np.array([[4, 0]], dtype=np.int64), (n, 1))
    shape = ca.make_shape(HQ, HKV, D, n, 1, n)
    ta, ma = ca.split_tasks(t, masks)
    assert ca.forward_workspace(shape, ta, ma) > ca.NOALLOC_SCRATCH_BYTES
    Q = torch.zeros((n, HQ, D), dtype=torch.bfloat16, device=dev)
    K = torch.zeros((1, HKV, D), dtype=torch.bfloat16, device=dev)
    O = torch.full((n, HQ, D), 3.0, dtype=torch.bfloat16, device=dev)
    LSE = torch.full((n, HQ), 3.0, device=dev)
    with pytest.raises(ca.CAError) as e:
        ca.forward_noalloc(shape, ta, Q, K, K, O, LSE, masks=ma)
    assert e.value.status == ca.CA_ERR_WORKSPACE and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((O.float() == 3.0).all()) and bool((LSE == 3.0).all())


def test_noalloc_graph_replays_equal_direct_calls():
    """Captured once; before each replay, eager work changes Q and runs a
    different ca_forward_noalloc call (which overwrites the shared scratch);
    every replay (it stores its own queue again) matches ca_forward_masked."""
    announce("ca_forward_noalloc captured in a graph, replays with other calls between")
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    tasks, q_rows, kv_rows, o_rows = workload([1000, 129], 3, 9000)
    other, oq, okv, oo = workload([2000], 1, 5000)
    shape = ca.make_shape(HQ, HKV, D, q_rows, kv_rows, o_rows, out_f32=True)
    oshape = ca.make_shape(HQ, HKV, D, oq, okv, oo, out_f32=True)
    Q = I.randn_bf16((q_rows, HQ, D), 2950, device=dev)
    K = I.randn_bf16((kv_rows, HKV, D), 2951, device=dev)
    V = I.randn_bf16((kv_rows, HKV, D), 2952, device=dev)
    Qo = I.randn_bf16((oq, HQ, D), 2953, device=dev)
    Ko = I.randn_bf16((okv, HKV, D), 2954, device=dev)
    O = torch.zeros((o_rows, HQ, D), device=dev)
    LSE = torch.zeros((o_rows, HQ), device=dev)
    O2, L2 = torch.zeros_like(O), torch.zeros_like(LSE)
    Oo, Lo = torch.zeros((oo, HQ, D), device=dev), torch.zeros((oo, HQ), device=dev)
    ca.forward_noalloc(shape, tasks, Q, K, V, O, LSE)            # first call on the device: outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ca.forward_noalloc(shape, tasks, Q, K, V, O, LSE, stream=torch.cuda.current_stream())
    for rep in range(3):
        Q.copy_(I.randn_bf16((q_rows, HQ, D), 2960 + rep, device=dev))
        ca.forward_noalloc(oshape, other, Qo, Ko, Ko, Oo, Lo)
        ca.forward(shape, tasks, Q, K, V, O2, L2)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = torch.equal(O, O2) and torch.equal(LSE.view(torch.int32), L2.view(torch.int32))
        print("replay %d identical to the workspace call: %s" % (rep, same), flush=True)
        assert same
