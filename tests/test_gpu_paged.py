"""GPU parity of paged K/V (ca_forward_paged: block tables as in the
Blockwise Attention instruction of "DCP: Addressing Input Dynamism In
Long-Context Training via Dynamic Context Parallelism", Executor Design)
against the fp64 oracle, and bit-for-bit against the unpaged forward over the
virtual K/V; plus the guarantee that no kernel reads K/V rows outside a
task's context (rows there hold NaN)."""

import math

import numpy as np
import pytest

import oracle
from long_context_core_amd import ca
from long_context_core_amd import inputs as I
from tests.gpu_util import GRAD_REL_FRO, announce, check_forward, rel_fro, torch_cuda, widen

pytestmark = pytest.mark.gpu


def run_paged(tasks, masks, hq, hkv, d, q_rows, n_vp, P, seed, extra_pages=7):
    """Paged and unpaged forward of the same virtual K/V; returns both GPU
    results and the oracle's."""
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    Q = I.randn_bf16((q_rows, hq, d), seed)
    Kv = I.randn_bf16((n_vp * P, hkv, d), seed + 1)
    Vv = I.randn_bf16((n_vp * P, hkv, d), seed + 2)
    n_phys = n_vp + extra_pages
    table = I.page_table(n_vp, n_phys, seed + 3)
    Ks = I.page_store(Kv, table, P, n_phys).to(dev)
    Vs = I.page_store(Vv, table, P, n_phys).to(dev)
    Qd = Q.to(dev)
    outs = []
    for paged in (True, False):
        O = torch.full((q_rows, hq, d), float("nan"), dtype=torch.bfloat16, device=dev)
        LSE = torch.full((q_rows, hq), float("nan"), device=dev)
        if paged:
            shape = ca.make_shape(hq, hkv, d, q_rows, n_phys * P, q_rows)
            ca.forward(shape, tasks, Qd, Ks, Vs, O, LSE, masks=masks, pages=ca.kv_pages(table, P))
        else:
            shape = ca.make_shape(hq, hkv, d, q_rows, n_vp * P, q_rows)
            ca.forward(shape, tasks, Qd, Kv.to(dev), Vv.to(dev), O, LSE, masks=masks)
        outs.append((O, LSE))
    torch.cuda.synchronize()
    t9 = tasks if masks is None else np.concatenate([tasks, np.asarray(masks)], axis=1)
    Ks_np = widen(Ks)
    Vs_np = widen(Vs)
    O_ref, L_ref = oracle.forward_paged(t9, widen(Q), Ks_np, Vs_np, table, P, 1 / math.sqrt(d), o_rows=q_rows)
    return outs, O_ref, L_ref


def check_paged(outs, O_ref, L_ref, label):
    torch = torch_cuda()
    (Op, Lp), (Ou, Lu) = outs
    check_forward(Op, Lp, O_ref, L_ref, label)
    rows = torch.from_numpy(np.flatnonzero(~np.isnan(L_ref).any(1)))
    # identical work items and arithmetic: identical bits
    assert torch.equal(Op.cpu()[rows].view(torch.int16), Ou.cpu()[rows].view(torch.int16)), label
    assert torch.equal(Lp.cpu()[rows], Lu.cpu()[rows]), label


@pytest.mark.parametrize("P", [128, 256, 1024])
@pytest.mark.parametrize("hq,hkv,d", [(8, 2, 128), (4, 4, 64), (16, 1, 128)])
def test_paged_varlen(P, hq, hkv, d):
    announce("paged forward varlen P%d hq%d hkv%d d%d" % (P, hq, hkv, d))
    docs = [1, 127, 129, 300, 64, 1000, 65, 700]
    tasks, n_vp = I.paged_varlen_tasks(docs, P)
    outs, Or, Lr = run_paged(tasks, None, hq, hkv, d, sum(docs), n_vp, P, 1500 + P + d)
    check_paged(outs, Or, Lr, "paged varlen P%d" % P)


def test_paged_ca_task_shards_and_shared_prefix():
    """Query shards of long documents (CA-tasks) over paged contexts, two
    documents sharing their first pages (a common prefix)."""
    announce("paged CA-task shards with a shared prefix")
    P = 256
    hq, hkv, d = 8, 2, 128
    # virtual pages: doc A = pages 0..11, doc B = pages 12..21; B's first 4
    # pages are A's first 4 in the table below
    tasks = np.array([
        [0, 0, 0, 300, 2500, 2200, 0],          # A: queries 2200..2499 over A[0, 2500)
        [300, 0, 300, 100, 3000, 2900, 0],      # A: queries 2900..2999 over A[0, 3000)
        [400, 12 * P, 400, 257, 2001, 1744, 0],  # B: queries 1744..2000 over B[0, 2001)
        [657, 12 * P, 657, 64, 64, 0, 0],       # B: its first 64 tokens
    ], dtype=np.int64)
    q_rows, n_vp = 721, 22
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    Q = I.randn_bf16((q_rows, hq, d), 1601)
    Kv = I.randn_bf16((n_vp * P, hkv, d), 1602)
    Vv = I.randn_bf16((n_vp * P, hkv, d), 1603)
    table = I.page_table(n_vp, n_vp + 3, 1604)
    table[12:16] = table[0:4]                   # shared prefix pages
    Kv[12 * P:16 * P] = Kv[0:4 * P]             # the virtual view of B repeats them
    Vv[12 * P:16 * P] = Vv[0:4 * P]
    used = np.unique(table)
    n_phys = n_vp + 3
    Ks = torch.full((n_phys * P, hkv, d), float("nan"), dtype=torch.bfloat16)
    Vs = torch.full((n_phys * P, hkv, d), float("nan"), dtype=torch.bfloat16)
    for v, pp in enumerate(table.tolist()):
        Ks[pp * P:(pp + 1) * P] = Kv[v * P:(v + 1) * P]
        Vs[pp * P:(pp + 1) * P] = Vv[v * P:(v + 1) * P]
    assert len(used) == n_vp - 4
    O = torch.full((q_rows, hq, d), float("nan"), dtype=torch.bfloat16, device=dev)
    LSE = torch.full((q_rows, hq), float("nan"), device=dev)
    shape = ca.make_shape(hq, hkv, d, q_rows, n_phys * P, q_rows)
    ca.forward(shape, tasks, Q.to(dev), Ks.to(dev), Vs.to(dev), O, LSE, pages=ca.kv_pages(table, P))
    torch.cuda.synchronize()
    Or, Lr = oracle.forward(tasks, widen(Q), widen(Kv), widen(Vv), 1 / math.sqrt(d), o_rows=q_rows)
    check_forward(O, LSE, Or, Lr, "paged CA-tasks shared prefix")


@pytest.mark.parametrize("hq,hkv,P", [(16, 1, 256), (8, 2, 256), (16, 1, 128), (8, 2, 1024)])
def test_paged_decode(hq, hkv, P):
    """Single-token queries over paged caches (the split-KV decode kernel,
    two tiles in flight), caches of ragged length, split into several key
    chunks; chunks of 1 to 5 tiles and 128-row pages (a new page every tile)
    cover the pipeline's ends."""
    announce("paged decode hq%d hkv%d P%d" % (hq, hkv, P))
    d = 128
    ctx = [5000, 131, 2048, 777, 9000, 1, 128, 129, 256, 257, 384, 385, 512, 640]
    t = []
    vp = 0
    for b, c in enumerate(ctx):
        t.append((b, vp * P, b, 1, c, c - 1, 0))
        vp += -(-c // P)
    tasks = np.array(t, dtype=np.int64)
    outs, Or, Lr = run_paged(tasks, None, hq, hkv, d, len(ctx), vp, P, 1700 + hq + P)
    check_paged(outs, Or, Lr, "paged decode P%d" % P)


def test_paged_lambda_mask():
    announce("paged forward with sink + sliding-window masks")
    P = 128
    docs = [3000, 130, 1500]
    tasks, n_vp = I.paged_varlen_tasks(docs, P)
    masks = np.array([[512, 64], [0, 0], [100, 3]], dtype=np.int64)
    outs, Or, Lr = run_paged(tasks, masks, 8, 2, 128, sum(docs), n_vp, P, 1800)
    check_paged(outs, Or, Lr, "paged lambda")


# ---------------------------------------------------------------------------
# No kernel reads K/V rows outside a task's context
# ---------------------------------------------------------------------------

def gapped_layout(ctx_lens, gap):
    """Contexts placed back to back with `gap` rows between them (and after
    the last one): (kv_off of each context, total rows)."""
    offs, r = [], 0
    for c in ctx_lens:
        offs.append(r)
        r += c + gap
    return offs, r


def poisoned_kv(ctx_lens, offs, rows, hkv, d, seed):
    """K, V with N(0,1) rows inside the contexts and NaN everywhere else."""
    torch = torch_cuda()
    K = torch.full((rows, hkv, d), float("nan"), dtype=torch.bfloat16)
    V = torch.full((rows, hkv, d), float("nan"), dtype=torch.bfloat16)
    Kc = I.randn_bf16((rows, hkv, d), seed)
    Vc = I.randn_bf16((rows, hkv, d), seed + 1)
    for o, c in zip(offs, ctx_lens):
        K[o:o + c] = Kc[o:o + c]
        V[o:o + c] = Vc[o:o + c]
    return K, V


def test_forward_reads_nothing_past_the_context():
    announce("forward with NaN rows around every context")
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    hq, hkv, d = 8, 2, 128
    ctx = [1, 63, 65, 100, 127, 129, 1000]
    offs, rows = gapped_layout(ctx, 77)
    tasks = np.array([(sum(ctx[:i]), offs[i], sum(ctx[:i]), c, c, 0, 0) for i, c in enumerate(ctx)],
                     dtype=np.int64)
    q_rows = sum(ctx)
    Q = I.randn_bf16((q_rows, hq, d), 1900)
    K, V = poisoned_kv(ctx, offs, rows, hkv, d, 1901)
    O = torch.full((q_rows, hq, d), float("nan"), dtype=torch.bfloat16, device=dev)
    LSE = torch.full((q_rows, hq), float("nan"), device=dev)
    ca.forward(ca.make_shape(hq, hkv, d, q_rows, rows, q_rows), tasks, Q.to(dev), K.to(dev), V.to(dev), O, LSE)
    torch.cuda.synchronize()
    Kz, Vz = torch.nan_to_num(K.float()), torch.nan_to_num(V.float())
    Or, Lr = oracle.forward(tasks, widen(Q), widen(Kz), widen(Vz), 1 / math.sqrt(d))
    check_forward(O, LSE, Or, Lr, "forward NaN-fenced contexts")


def test_decode_reads_nothing_past_the_context():
    announce("decode with NaN rows around every cache")
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    hq, hkv, d = 16, 1, 128
    ctx = [5000, 1, 129, 4097, 700]
    offs, rows = gapped_layout(ctx, 200)
    tasks = np.array([(b, offs[b], b, 1, c, c - 1, 0) for b, c in enumerate(ctx)], dtype=np.int64)
    Q = I.randn_bf16((len(ctx), hq, d), 1910)
    K, V = poisoned_kv(ctx, offs, rows, hkv, d, 1911)
    O = torch.full((len(ctx), hq, d), float("nan"), dtype=torch.bfloat16, device=dev)
    LSE = torch.full((len(ctx), hq), float("nan"), device=dev)
    ca.forward(ca.make_shape(hq, hkv, d, len(ctx), rows, len(ctx)), tasks, Q.to(dev), K.to(dev), V.to(dev),
               O, LSE)
    torch.cuda.synchronize()
    Kz, Vz = torch.nan_to_num(K.float()), torch.nan_to_num(V.float())
    Or, Lr = oracle.forward(tasks, widen(Q), widen(Kz), widen(Vz), 1 / math.sqrt(d))
    check_forward(O, LSE, Or, Lr, "decode NaN-fenced caches")


def test_backward_reads_nothing_past_the_context():
    announce("backward with NaN rows around every context")
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    hq, hkv, d = 8, 2, 128
    ctx = [1, 65, 127, 300, 129]
    offs, rows = gapped_layout(ctx, 90)
    tasks = np.array([(sum(ctx[:i]), offs[i], sum(ctx[:i]), c, c, 0, 0) for i, c in enumerate(ctx)],
                     dtype=np.int64)
    q_rows = sum(ctx)
    Q = I.randn_bf16((q_rows, hq, d), 1920)
    dO = I.randn_bf16((q_rows, hq, d), 1921)
    K, V = poisoned_kv(ctx, offs, rows, hkv, d, 1922)
    shape = ca.make_shape(hq, hkv, d, q_rows, rows, q_rows)
    Qd, Kd, Vd, dOd = Q.to(dev), K.to(dev), V.to(dev), dO.to(dev)
    O = torch.empty((q_rows, hq, d), dtype=torch.bfloat16, device=dev)
    LSE = torch.empty((q_rows, hq), device=dev)
    ca.forward(shape, tasks, Qd, Kd, Vd, O, LSE)
    dQ = torch.full_like(Qd, float("nan"))
    dK = torch.full_like(Kd, float("nan"))
    dV = torch.full_like(Vd, float("nan"))
    ca.backward(shape, tasks, Qd, Kd, Vd, O, dOd, LSE, dQ, dK, dV)
    torch.cuda.synchronize()
    Kz, Vz = torch.nan_to_num(K.float()), torch.nan_to_num(V.float())
    ref = oracle.backward(tasks, widen(Q), widen(Kz), widen(Vz), widen(dO), 1 / math.sqrt(d))
    inside = np.zeros(rows, dtype=bool)
    for o, c in zip(offs, ctx):
        inside[o:o + c] = True
    for name, g, r, sel in (("dQ", dQ, ref[0], slice(None)), ("dK", dK, ref[1], inside), ("dV", dV, ref[2], inside)):
        gw = widen(g)[sel]
        assert np.isfinite(gw).all(), name
        e = rel_fro(gw, r[sel])
        print("NaN-fenced backward %s relF=%.3e" % (name, e), flush=True)
        assert e <= GRAD_REL_FRO, name


# ---------------------------------------------------------------------------
# Paged backward
# ---------------------------------------------------------------------------

def run_paged_backward(tasks, table, P, n_phys, hq, hkv, d, q_rows, seed, masks=None):
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    Q = I.randn_bf16((q_rows, hq, d), seed)
    dO = I.randn_bf16((q_rows, hq, d), seed + 1)
    Ks = I.randn_bf16((n_phys * P, hkv, d), seed + 2)
    Vs = I.randn_bf16((n_phys * P, hkv, d), seed + 3)
    pages = ca.kv_pages(table, P)
    shape = ca.make_shape(hq, hkv, d, q_rows, n_phys * P, q_rows)
    Qd, dOd, Kd, Vd = Q.to(dev), dO.to(dev), Ks.to(dev), Vs.to(dev)
    O = torch.empty((q_rows, hq, d), dtype=torch.bfloat16, device=dev)
    LSE = torch.empty((q_rows, hq), device=dev)
    ca.forward(shape, tasks, Qd, Kd, Vd, O, LSE, masks=masks, pages=pages)
    dQ = torch.full_like(Qd, float("nan"))
    dK = torch.full_like(Kd, float("nan"))
    dV = torch.full_like(Vd, float("nan"))
    ca.backward(shape, tasks, Qd, Kd, Vd, O, dOd, LSE, dQ, dK, dV, masks=masks, pages=pages)
    torch.cuda.synchronize()
    t9 = tasks if masks is None else np.concatenate([tasks, np.asarray(masks)], axis=1)
    ref = oracle.backward_paged(t9, widen(Q), widen(Ks), widen(Vs), widen(dO), table, P, 1 / math.sqrt(d))
    return (dQ, dK, dV), ref, (Qd, Kd, Vd, O, dOd, LSE)


def check_grads(got, ref, label):
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        gw = widen(g)
        assert np.isfinite(gw).all(), label + " " + name
        e = rel_fro(gw, r)
        print("%s %s relF=%.3e" % (label, name, e), flush=True)
        assert e <= GRAD_REL_FRO, label + " " + name


@pytest.mark.parametrize("P", [128, 512])
def test_paged_backward_varlen(P):
    """Distinct pages: one pass; dK/dV of the page store, gathered back to
    virtual rows, equal the unpaged backward's bit for bit."""
    announce("paged backward varlen P%d" % P)
    torch = torch_cuda()
    hq, hkv, d = 8, 2, 128
    docs = [1, 127, 129, 300, 700, 65]
    tasks, n_vp = I.paged_varlen_tasks(docs, P)
    n_phys = n_vp + 3
    table = I.page_table(n_vp, n_phys, 2000 + P)
    got, ref, (Qd, Ks, Vs, O, dOd, LSE) = run_paged_backward(tasks, table, P, n_phys, hq, hkv, d, sum(docs),
                                                              2010 + P)
    check_grads(got, ref, "paged backward P%d" % P)
    used = np.zeros(n_phys, dtype=bool)
    used[table] = True
    for g in got[1:]:
        unread = torch.from_numpy(np.flatnonzero(~used)).to(g.device)
        assert torch.count_nonzero(g.view(n_phys, -1)[unread]).item() == 0   # unread pages: 0
    # unpaged backward over the virtual K/V
    idx = torch.from_numpy(table.astype(np.int64)).to(Ks.device)
    Kv = Ks.view(n_phys, -1)[idx].view(n_vp * P, hkv, d)
    Vv = Vs.view(n_phys, -1)[idx].view(n_vp * P, hkv, d)
    shape = ca.make_shape(hq, hkv, d, sum(docs), n_vp * P, sum(docs))
    dQu, dKu, dVu = torch.empty_like(Qd), torch.empty_like(Kv), torch.empty_like(Vv)
    ca.backward(shape, tasks, Qd, Kv, Vv, O, dOd, LSE, dQu, dKu, dVu)
    torch.cuda.synchronize()
    assert torch.equal(got[0].view(torch.int16), dQu.view(torch.int16))
    assert torch.equal(got[1].view(n_phys, -1)[idx].view(torch.int16), dKu.view(n_vp, -1).view(torch.int16))
    assert torch.equal(got[2].view(n_phys, -1)[idx].view(torch.int16), dVu.view(n_vp, -1).view(torch.int16))


def test_paged_backward_shared_prefix_pages():
    """Two documents whose tables share their first pages: the shared pages
    collect both documents' gradients (accumulating passes)."""
    announce("paged backward with shared prefix pages")
    P = 128
    hq, hkv, d = 8, 2, 128
    # doc A: virtual pages 0..5 (700 tokens), doc B: virtual pages 6..9 (500 tokens);
    # B's first two pages are A's first two
    tasks = np.array([[0, 0, 0, 700, 700, 0, 0],
                      [700, 6 * P, 700, 244, 500, 256, 0]], dtype=np.int64)   # B: its last 244 queries
    table = np.array([3, 7, 0, 5, 9, 2, 3, 7, 1, 8], dtype=np.int32)
    got, ref, _ = run_paged_backward(tasks, table, P, 11, hq, hkv, d, 944, 2100)
    check_grads(got, ref, "paged backward shared prefix")


def test_paged_backward_lambda_mask():
    announce("paged backward with sink + sliding-window masks")
    P = 256
    docs = [2000, 300]
    tasks, n_vp = I.paged_varlen_tasks(docs, P)
    masks = np.array([[300, 16], [64, 0]], dtype=np.int64)
    table = I.page_table(n_vp, n_vp + 2, 2200)
    got, ref, _ = run_paged_backward(tasks, table, P, n_vp + 2, 8, 2, 128, sum(docs), 2210, masks=masks)
    check_grads(got, ref, "paged backward lambda")
