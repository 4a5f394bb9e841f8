"""Full-size parity of the training backward and of the CA-task backward
against the fp64 oracle, on sampled rows and keys (the oracle cannot do the
whole job in seconds), in the launch configuration the benchmark times.

The backward recomputes the attention probabilities from the saved per-row
statistics ("Efficient Long-context Language Model Training by Core
Attention Disaggregation", Section 3.4, Property 1), so every sampled
gradient is exact for what it covers:

* dQ of a query row depends on that row alone (its probabilities, D and dP),
  so the oracle computes it from the row (``oracle.backward_dq_rows``);
* a key at document position j is seen only by queries at positions >= j, so
  the gradient of a document's last n keys is the backward of the shard of
  its last n queries over the document prefix (``oracle.backward`` on that
  shard), and a whole document's backward gives dK / dV of all its keys.

Query heads are checked one KV group at a time, the group rotating over rows
and documents so that every head is covered; dK and dV sum over the group's
query heads, so a group is checked whole.  Tolerance: relative Frobenius
<= 3e-2 per tensor over everything sampled."""

import math

import numpy as np
import pytest

import oracle
from long_context_core_amd import ca
from long_context_core_amd import inputs as I
from tests.gpu_util import GRAD_REL_FRO, announce, check_forward, rel_fro, torch_cuda, widen

pytestmark = pytest.mark.gpu


def rows_of(torch, X, rows, cols):
    """float64 numpy of X[rows][:, cols] (rows and cols: integer arrays)."""
    idx = torch.from_numpy(np.asarray(rows, dtype=np.int64)).to(X.device)
    return widen(X.index_select(0, idx)[:, list(cols)])


def doc_table(w):
    """(start row, length) of every packed document."""
    starts = np.concatenate([[0], np.cumsum(w.doc_lens)[:-1]]).astype(np.int64)
    return starts, np.asarray(w.doc_lens, dtype=np.int64)


class Agg:
    """Concatenates sampled GPU values and their oracle values per tensor."""

    def __init__(self):
        self.got, self.ref = {}, {}

    def add(self, name, got, ref):
        self.got.setdefault(name, []).append(np.asarray(got, dtype=np.float64).ravel())
        self.ref.setdefault(name, []).append(np.asarray(ref, dtype=np.float64).ravel())

    def check(self, label):
        for name in sorted(self.got):
            g, r = np.concatenate(self.got[name]), np.concatenate(self.ref[name])
            assert np.all(np.isfinite(g)), label + " " + name
            e = rel_fro(g, r)
            print("%s %s: %d values relF=%.3e max|d|=%.3e" % (label, name, g.size, e, float(np.max(np.abs(g - r)))),
                  flush=True)
            assert e <= GRAD_REL_FRO, label + " " + name


def sparse_rows(torch, X, first, rows, cols, n):
    """[n, len(cols), d] float64 holding X[first + r][:, cols] at row r for
    the listed rows and zeros elsewhere (pages never touched stay unmapped),
    so the oracle can index the sampled rows at their own task positions."""
    out = np.zeros((n, len(cols), X.shape[2]))
    out[rows] = rows_of(torch, X, first + rows, cols)
    return out


def check_dq_rows(torch, agg, Q, K, V, dO, dQ, scale, task, rows, group, G, heads=None, chunk=16):
    """dQ of task-relative rows (sorted), query heads of KV group `group`
    (or the listed heads of that group), against the oracle over the context
    the rows see.  Rows go to the oracle in chunks of `chunk` consecutive
    sampled rows, so each chunk's score block spans only the keys up to its
    own last row."""
    q_off, kv_off, o_off, q_len, kv_len, q_pos0, kv_pos0 = (int(x) for x in task[:7])
    gheads = list(range(group * G, (group + 1) * G))
    heads = gheads if heads is None else list(heads)
    local = [gheads.index(h) for h in heads]
    rows = np.asarray(rows, dtype=np.int64)
    n = int(rows.max()) + 1
    hi = int(np.clip(q_pos0 + rows.max() - kv_pos0 + 1, 0, kv_len))
    qs = sparse_rows(torch, Q, q_off, rows, gheads, n)
    dos = sparse_rows(torch, dO, o_off, rows, gheads, n)
    ks = widen(K[kv_off:kv_off + hi, group:group + 1])
    vs = widen(V[kv_off:kv_off + hi, group:group + 1])
    t = np.array([0, 0, 0, n, hi, q_pos0, kv_pos0])
    ref = np.concatenate([oracle.backward_dq_rows(t, rows[c:c + chunk], qs, ks, vs, dos, scale, heads=local)
                          for c in range(0, len(rows), chunk)])
    agg.add("dQ", rows_of(torch, dQ, q_off + rows, heads), ref)


def check_tail_keys(torch, agg, Q, K, V, dO, dQ, dK, dV, scale, q_off, kv_off, o_off, q_pos0, n_ctx, n, group, G):
    """The shard of the last n queries (document positions q_pos0 + q_len - n
    ... , contexts from position 0) over its prefix of n_ctx keys: its dK, dV
    on the last n keys are the whole gradient of those keys, its dQ the whole
    gradient of those rows."""
    heads = list(range(group * G, (group + 1) * G))
    rows = np.arange(n)
    qs = rows_of(torch, Q, q_off + rows, heads)
    dos = rows_of(torch, dO, o_off + rows, heads)
    ks = widen(K[kv_off:kv_off + n_ctx, group:group + 1])
    vs = widen(V[kv_off:kv_off + n_ctx, group:group + 1])
    t = np.array([[0, 0, 0, n, n_ctx, q_pos0, 0]])
    rdq, rdk, rdv = oracle.backward(t, qs, ks, vs, dos, scale)
    agg.add("dQ", rows_of(torch, dQ, q_off + rows, heads), rdq)
    agg.add("dK", widen(dK[kv_off + n_ctx - n:kv_off + n_ctx, group:group + 1]), rdk[n_ctx - n:])
    agg.add("dV", widen(dV[kv_off + n_ctx - n:kv_off + n_ctx, group:group + 1]), rdv[n_ctx - n:])


def dq_random_rows(torch, w, Q, K, V, dO, dQ, n_random=4096, seed=31):
    """dQ of n_random rows drawn uniformly over the packed batch, each on one
    query head, the head rotating with the row (every head is covered)."""
    hq, G = w.hq, w.hq // w.hkv
    starts, lens = doc_table(w)
    pick = np.sort(np.random.default_rng(seed).choice(w.q_rows, n_random, replace=False))
    doc_of = np.searchsorted(starts, pick, side="right") - 1
    agg = Agg()
    for di, (s0, L) in enumerate(zip(starts, lens)):
        rows = pick[doc_of == di] - s0
        for h in range(hq):
            sel = rows[(rows + di) % hq == h]
            if len(sel):
                check_dq_rows(torch, agg, Q, K, V, dO, dQ, w.scale, (s0, s0, s0, L, L, 0, 0), sel, h // G, G,
                              heads=[h])
    return agg


def dq_long_doc_ends(torch, w, Q, K, V, dO, dQ, long_min=16384, n_end=128):
    """dQ of the first and last n_end rows of every document longer than
    long_min, each row on the query heads of one KV group, the group rotating
    with the row (every head is covered)."""
    starts, lens = doc_table(w)
    agg = Agg()
    for s0, L in zip(starts, lens):
        if L <= long_min:
            continue
        rows = np.unique(np.concatenate([np.arange(n_end), np.arange(L - n_end, L)]))
        for g in range(w.hkv):
            check_dq_rows(torch, agg, Q, K, V, dO, dQ, w.scale, (s0, s0, s0, L, L, 0, 0), rows[rows % w.hkv == g], g,
                          w.hq // w.hkv, chunk=128)
    return agg


def dkv_documents(torch, w, Q, K, V, dO, dQ, dK, dV, short_max=8192, tail=256, which="short"):
    """which = "short": dK, dV (and dQ) of every key of each document of at
    most short_max tokens; "tail": of the last `tail` keys of every longer
    document.  One KV group per document, rotating with the document."""
    hkv, G = w.hkv, w.hq // w.hkv
    starts, lens = doc_table(w)
    agg = Agg()
    for di, (s0, L) in enumerate(zip(starts, lens)):
        g = di % hkv
        if which == "short" and L <= short_max:
            check_tail_keys(torch, agg, Q, K, V, dO, dQ, dK, dV, w.scale, s0, s0, s0, 0, L, L, g, G)
        elif which == "tail" and L > short_max:
            n = min(tail, int(L))
            check_tail_keys(torch, agg, Q, K, V, dO, dQ, dK, dV, w.scale, s0 + L - n, s0, s0 + L - n, L - n, L, n,
                            g, G)
    return agg


@pytest.fixture(scope="module")
def train_512k_grads():
    """The 524,288-token ProLong-like training batch: forward, then backward,
    on the GPU, as the benchmark launches them (computed once for the tests
    below)."""
    announce("fullsize 512k training forward + backward (random inputs)")
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    w = I.train_8b_prolong_512k()
    T, hq, hkv, d = w.q_rows, w.hq, w.hkv, w.d
    shape = ca.make_shape(hq, hkv, d, T, T, T)
    Q = I.randn_bf16((T, hq, d), 261, device=dev)
    K = I.randn_bf16((T, hkv, d), 262, device=dev)
    V = I.randn_bf16((T, hkv, d), 263, device=dev)
    dO = I.randn_bf16((T, hq, d), 264, device=dev)
    O = torch.empty_like(Q)
    LSE = torch.empty((T, hq), device=dev)
    ca.forward(shape, w.tasks, Q, K, V, O, LSE)
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
    ca.backward(shape, w.tasks, Q, K, V, O, dO, LSE, dQ, dK, dV)
    torch.cuda.synchronize()
    del O, LSE
    yield torch, w, Q, K, V, dO, dQ, dK, dV
    del Q, K, V, dO, dQ, dK, dV
    torch.cuda.empty_cache()


def test_train_512k_dq_random_rows(train_512k_grads):
    """dQ of 4,096 random rows of the 512K batch vs the oracle, one head per
    row (all 32 heads covered)."""
    announce("fullsize 512k backward: dQ of 4096 random rows vs the oracle")
    torch, w, Q, K, V, dO, dQ, dK, dV = train_512k_grads
    dq_random_rows(torch, w, Q, K, V, dO, dQ).check("512k dQ random rows")


def test_train_512k_dq_long_document_ends(train_512k_grads):
    """dQ of the first and last 128 rows of every document over 16K tokens
    vs the oracle, one KV group (4 query heads) per row, rotating."""
    announce("fullsize 512k backward: dQ of the ends of the long documents vs the oracle")
    torch, w, Q, K, V, dO, dQ, dK, dV = train_512k_grads
    dq_long_doc_ends(torch, w, Q, K, V, dO, dQ).check("512k dQ long-doc ends")


def test_train_512k_dkv_short_documents(train_512k_grads):
    """dK, dV (and dQ) of every key (row) of the documents of at most 8K
    tokens vs the oracle's backward of each whole document."""
    announce("fullsize 512k backward: dK/dV of whole short documents vs the oracle")
    torch, w, Q, K, V, dO, dQ, dK, dV = train_512k_grads
    dkv_documents(torch, w, Q, K, V, dO, dQ, dK, dV, which="short").check("512k dK/dV short docs")


def test_train_512k_dkv_last_keys_of_long_documents(train_512k_grads):
    """dK, dV of the last 256 keys of every document over 8K tokens (the
    247K-token one included) vs the oracle's backward of the document's last
    256 queries."""
    announce("fullsize 512k backward: dK/dV of the last 256 keys of the long documents vs the oracle")
    torch, w, Q, K, V, dO, dQ, dK, dV = train_512k_grads
    dkv_documents(torch, w, Q, K, V, dO, dQ, dK, dV, which="tail").check("512k dK/dV long-doc tails")


def test_train_512k_forward_sampled_vs_oracle():
    """The unmasked 512K training forward (O, LSE) on sampled rows, all 32
    heads: the first and last two rows of every document and 256 random rows."""
    announce("fullsize 512k training forward, sampled rows vs the oracle")
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    w = I.train_8b_prolong_512k()
    T = w.q_rows
    Q = I.randn_bf16((T, w.hq, w.d), 271, device=dev)
    K = I.randn_bf16((T, w.hkv, w.d), 272, device=dev)
    V = I.randn_bf16((T, w.hkv, w.d), 273, device=dev)
    O = torch.empty_like(Q)
    LSE = torch.empty((T, w.hq), device=dev)
    ca.forward(ca.make_shape(w.hq, w.hkv, w.d, T, T, T), w.tasks, Q, K, V, O, LSE)
    torch.cuda.synchronize()
    starts, lens = doc_table(w)
    pick = np.random.default_rng(32).choice(T, 256, replace=False)
    doc_of = np.searchsorted(starts, pick, side="right") - 1
    G = w.hq // w.hkv
    got_o, got_l, ref_o, ref_l = [], [], [], []
    for di, (s0, L) in enumerate(zip(starts, lens)):
        rows = np.unique(np.concatenate([pick[doc_of == di] - s0, [0, min(1, L - 1), max(0, L - 2), L - 1]]))
        n = int(rows.max()) + 1
        task = np.array([0, 0, 0, n, n, 0, 0])
        for g in range(w.hkv):          # one KV group at a time: all 32 heads in 8 groups
            heads = list(range(g * G, (g + 1) * G))
            qs = sparse_rows(torch, Q, s0, rows, heads, n)
            ks = widen(K[s0:s0 + n, g:g + 1])
            vs = widen(V[s0:s0 + n, g:g + 1])
            o1, l1 = oracle.forward_rows(task, rows, qs, ks, vs, w.scale)
            ref_o.append(o1)
            ref_l.append(l1)
            got_o.append(rows_of(torch, O, s0 + rows, heads))
            got_l.append(rows_of(torch, LSE.view(T, w.hq, 1), s0 + rows, heads)[:, :, 0])
    check_forward(np.concatenate(got_o), np.concatenate(got_l), np.concatenate(ref_o), np.concatenate(ref_l),
                  "512k-fwd-sampled")


def test_ca_tasks_34b_backward_sampled_vs_oracle():
    """The 262K-query CA-task batch (34B shape, 64 tasks, each with its own
    context copy): dQ of the first, middle and last 3 query rows of every
    task, and dK / dV of the last 3 keys of every task's context (seen only
    by its last 3 queries), each task on one KV group (8 query heads), the
    group rotating over the tasks (every head is covered)."""
    announce("fullsize 262k CA-tasks (34B) backward, 3 rows and 3 keys per task vs the oracle")
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    w = I.ca_tasks_34b()
    G = w.hq // w.hkv
    shape = ca.make_shape(w.hq, w.hkv, w.d, w.q_rows, w.kv_rows, w.o_rows)
    Q = I.randn_bf16((w.q_rows, w.hq, w.d), 281, device=dev)
    K = I.randn_bf16((w.kv_rows, w.hkv, w.d), 282, device=dev)
    V = I.randn_bf16((w.kv_rows, w.hkv, w.d), 283, device=dev)
    dO = I.randn_bf16((w.o_rows, w.hq, w.d), 284, device=dev)
    O = torch.empty((w.o_rows, w.hq, w.d), dtype=torch.bfloat16, device=dev)
    LSE = torch.empty((w.o_rows, w.hq), device=dev)
    ca.forward(shape, w.tasks, Q, K, V, O, LSE)
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
    ca.backward(shape, w.tasks, Q, K, V, O, dO, LSE, dQ, dK, dV)
    torch.cuda.synchronize()
    agg = ca_tasks_backward_checks(torch, w, Q, K, V, dO, dQ, dK, dV)
    agg.check("34b-ca-tasks-bwd-sampled")


def ca_tasks_backward_checks(torch, w, Q, K, V, dO, dQ, dK, dV, n_tail=3):
    G = w.hq // w.hkv
    agg = Agg()
    for ti, t in enumerate(w.tasks):
        q_off, kv_off, o_off, q_len, kv_len, q_pos0, kv_pos0 = (int(x) for x in t)
        g = ti % w.hkv
        check_dq_rows(torch, agg, Q, K, V, dO, dQ, w.scale, t, [0, q_len // 2], g, G)
        n = min(n_tail, q_len)
        check_tail_keys(torch, agg, Q, K, V, dO, dQ, dK, dV, w.scale, q_off + q_len - n, kv_off, o_off + q_len - n,
                        q_pos0 + q_len - n, kv_len, n, g, G)
    return agg
