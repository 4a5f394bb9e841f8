"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test pins a part of the oracle to something other than itself: a 50-digit
brute force, a closed form, a value the pages print (tests/golden), an exact
invariant, or a library routine for a special case.  Plausible mistakes (a
wrong scale, a dropped diagonal, a transposed operand, a wrong GQA group, a
sign error in the backward, a merge that ignores a partial) each fail at least
one of them — see ``test_planted_mistakes_are_caught``.
"""

import json
import math
import os

import mpmath as mp
import numpy as np
import pytest
import scipy.special

import oracle
from oracle import attention as oa
from tests import mp_brute

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_values.json")))


def rnd(shape, seed):
    """bf16-representable N(0,1) values as float64 (widened from bf16 bits)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)     # truncation is fine for pins
    return oracle.bf16_bits_to_f64(bits)


def tiny_random_case(seed, max_tokens=8):
    """A few tasks over <= max_tokens query/key rows, random positions, GQA."""
    rng = np.random.default_rng(seed)
    hkv = int(rng.integers(1, 3))
    hq = hkv * int(rng.integers(1, 4))
    d = int(rng.integers(2, 6))
    tq = int(rng.integers(1, max_tokens + 1))
    tk = int(rng.integers(1, max_tokens + 1))
    tasks = []
    q = 0
    while q < tq:
        ql = int(rng.integers(1, tq - q + 1))
        kv_off = int(rng.integers(0, tk))
        kvl = int(rng.integers(0, tk - kv_off + 1))
        kv_pos0 = int(rng.integers(0, 5))
        q_pos0 = int(rng.integers(0, 8))
        tasks.append((q, kv_off, q, ql, kvl, q_pos0, kv_pos0))
        q += ql
    Q = rnd((tq, hq, d), seed + 1)
    K = rnd((tk, hkv, d), seed + 2)
    V = rnd((tk, hkv, d), seed + 3)
    return np.array(tasks, dtype=np.int64), Q, K, V, 1.0 / math.sqrt(d)


# ---------------------------------------------------------------------------
# bf16 widening
# ---------------------------------------------------------------------------

def test_bf16_widening_matches_torch():
    torch = pytest.importorskip("torch")
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    got = oracle.bf16_bits_to_f64(bits)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin].astype(np.float64))
    assert np.array_equal(np.isnan(got), np.isnan(ref))


# ---------------------------------------------------------------------------
# P1: 50-digit brute force on <= 8 tokens
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(12))
def test_forward_matches_brute_force(seed):
    tasks, Q, K, V, scale = tiny_random_case(seed)
    O, LSE = oracle.forward(tasks, Q, K, V, scale)
    ref = mp_brute.attention(tasks, Q, K, V, scale)
    for (row, h), (o, lse) in ref.items():
        if lse == -mp.inf:
            assert LSE[row, h] == -np.inf
            assert np.all(O[row, h] == 0)
            continue
        assert abs(LSE[row, h] - float(lse)) <= 1e-12 * max(1.0, abs(float(lse)))
        for c in range(len(o)):
            assert abs(O[row, h, c] - float(o[c])) <= 1e-12


def test_gqa_group_map_matches_pages():
    g = GOLDEN["gqa_head_map_405b_tp8"]
    for h, kv in g["kv_head_of_query_head"].items():
        assert oa._group_of(int(h), g["query_heads"], g["kv_heads"]) == kv


# ---------------------------------------------------------------------------
# P2: document isolation and the pages' packing ratios
# ---------------------------------------------------------------------------

def test_packed_docs_equal_separate_attentions():
    lens = GOLDEN["packing_4000_vs_4x1000"]["packed_docs"]
    T = sum(lens)
    hq, hkv, d = 2, 1, 8
    Q, K, V = rnd((T, hq, d), 11), rnd((T, hkv, d), 12), rnd((T, hkv, d), 13)
    cu = np.cumsum([0] + lens)
    tasks = np.array([(cu[i], cu[i], cu[i], l, l, 0, 0) for i, l in enumerate(lens)])
    O, LSE = oracle.forward(tasks, Q, K, V, 1 / math.sqrt(d))
    for i, l in enumerate(lens):
        s = slice(cu[i], cu[i + 1])
        o1, lse1 = oracle.forward(np.array([(0, 0, 0, l, l, 0, 0)]), Q[s], K[s], V[s], 1 / math.sqrt(d))
        assert np.array_equal(O[s], o1)
        assert np.array_equal(LSE[s], lse1)


def test_packing_cost_ratios_from_pages():
    for key in ("packing_4000_vs_4x1000", "blog_128k_vs_8x16k"):
        g = GOLDEN[key]
        one = sum(oracle.visible_pairs_task(l, l, 0, 0) for l in g["single_doc"])
        packed = sum(oracle.visible_pairs_task(l, l, 0, 0) for l in g["packed_docs"])
        assert abs(one / packed - g["attention_cost_ratio"]) / g["attention_cost_ratio"] < 2e-3
    assert oracle.visible_pairs_task(4000, 4000, 0, 0) == 8002000
    assert sum(oracle.visible_pairs_task(1000, 1000, 0, 0) for _ in range(4)) == 2002000


def test_causal_doc_cost_cases():
    for l, pairs in GOLDEN["causal_doc_cost"]["cases"]:
        assert oracle.visible_pairs_task(l, l, 0, 0) == pairs == l * (l + 1) // 2


# ---------------------------------------------------------------------------
# P3: split + merge = unsplit (Equation 4)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n_blocks", [2, 3, 7])
def test_kv_split_merge_equals_unsplit(n_blocks):
    L, hq, hkv, d = 300, 4, 2, 16
    Q, K, V = rnd((L, hq, d), 21), rnd((L, hkv, d), 22), rnd((L, hkv, d), 23)
    scale = 1 / math.sqrt(d)
    full = np.array([(0, 0, 0, L, L, 0, 0)])
    O, LSE = oracle.forward(full, Q, K, V, scale)
    cuts = np.linspace(0, L, n_blocks + 1).astype(int)
    Op = np.zeros((n_blocks, L, hq, d))
    Lp = np.full((n_blocks, L, hq), -np.inf)
    for s in range(n_blocks):
        a, b = cuts[s], cuts[s + 1]
        part = np.array([(0, a, 0, L, b - a, 0, a)])
        o, lse = oracle.forward(part, Q, K, V, scale, o_rows=L)
        Op[s], Lp[s] = np.nan_to_num(o), lse
    Om, LSEm = oracle.merge(Op, Lp)
    assert np.max(np.abs(Om - O)) < 1e-12
    assert np.max(np.abs(LSEm - LSE)) < 1e-12


def test_query_split_tasks_equal_unsplit():
    """CA-tasks cut at arbitrary token offsets (context = prefix up to the
    shard end) reproduce the unsplit document."""
    L, hq, hkv, d = 257, 2, 1, 8
    Q, K, V = rnd((L, hq, d), 31), rnd((L, hkv, d), 32), rnd((L, hkv, d), 33)
    scale = 1 / math.sqrt(d)
    O, LSE = oracle.forward(np.array([(0, 0, 0, L, L, 0, 0)]), Q, K, V, scale)
    cuts = [0, 1, 50, 129, 200, L]
    tasks = np.array([(a, 0, a, b - a, b, a, 0) for a, b in zip(cuts[:-1], cuts[1:])])
    O2, LSE2 = oracle.forward(tasks, Q, K, V, scale)
    assert np.max(np.abs(O2 - O)) < 1e-13 and np.max(np.abs(LSE2 - LSE)) < 1e-13


def test_merge_special_cases():
    rng = np.random.default_rng(5)
    O1 = rng.standard_normal((1, 3, 2, 4))
    L1 = rng.standard_normal((1, 3, 2))
    Om, Lm = oracle.merge(O1, L1)                       # one partial: identity
    assert np.allclose(Om, O1[0], atol=1e-15) and np.allclose(Lm, L1[0], atol=1e-15)
    O2 = np.concatenate([O1, rng.standard_normal((1, 3, 2, 4))])
    L2 = np.concatenate([L1, np.full((1, 3, 2), -np.inf)])
    Om, Lm = oracle.merge(O2, L2)                       # an empty partial weighs 0
    assert np.allclose(Om, O1[0], atol=1e-15) and np.allclose(Lm, L1[0], atol=1e-15)
    Om, Lm = oracle.merge(O2, np.full((2, 3, 2), -np.inf))
    assert np.all(Om == 0) and np.all(Lm == -np.inf)
    Le = np.stack([L1[0], L1[0]])                       # equal weights: mean, LSE + ln 2
    Om, Lm = oracle.merge(O2, Le)
    assert np.allclose(Om, O2.mean(axis=0), atol=1e-15)
    assert np.allclose(Lm, L1[0] + math.log(2), atol=1e-15)


# ---------------------------------------------------------------------------
# P4: rows of P sum to 1 and equal the library softmax
# ---------------------------------------------------------------------------

def test_probabilities_are_library_softmax_and_sum_to_one():
    d = 24
    L = d                                               # V = identity => O = P
    hq, hkv = 2, 1
    Q = rnd((L, hq, d), 41)
    K = rnd((L, hkv, d), 42)
    V = np.eye(L)[:, None, :].repeat(hkv, axis=1)
    scale = 0.3
    O, LSE = oracle.forward(np.array([(0, 0, 0, L, L, 0, 0)]), Q, K, V, scale)
    assert np.allclose(O.sum(axis=2), 1.0, atol=1e-14)
    for h in range(hq):
        raw = np.einsum("id,jd->ij", Q[:, h], K[:, 0]) * scale
        masked = np.where(np.tril(np.ones((L, L), bool)), raw, -np.inf)
        assert np.allclose(O[:, h, :], scipy.special.softmax(masked, axis=1), atol=1e-14)
        assert np.allclose(LSE[:, h], scipy.special.logsumexp(masked, axis=1), atol=1e-13)


# ---------------------------------------------------------------------------
# P5: closed forms
# ---------------------------------------------------------------------------

def test_first_token_sees_one_key():
    L, hq, hkv, d = 40, 4, 2, 8
    Q, K, V = rnd((L, hq, d), 51), rnd((L, hkv, d), 52), rnd((L, hkv, d), 53)
    scale = 1 / math.sqrt(d)
    O, LSE = oracle.forward(np.array([(0, 0, 0, L, L, 0, 0)]), Q, K, V, scale)
    for h in range(hq):
        g = h // (hq // hkv)
        assert np.allclose(O[0, h], V[0, g], atol=1e-15)
        assert abs(LSE[0, h] - scale * float(np.dot(Q[0, h], K[0, g]))) < 1e-14


def test_zero_keys_count_visible_keys():
    """K = 0: LSE = ln(number of visible keys), O = mean of visible V rows."""
    tasks = np.array([(0, 0, 0, 10, 10, 0, 0), (10, 10, 10, 5, 20, 15, 0),
                      (15, 5, 15, 4, 6, 2, 3), (19, 0, 19, 3, 4, 0, 5)])
    hq, hkv, d = 2, 1, 3
    Q = rnd((22, hq, d), 61)
    K = np.zeros((30, hkv, d))
    V = rnd((30, hkv, d), 62)
    O, LSE = oracle.forward(tasks, Q, K, V, 0.7)
    for t in tasks:
        q_off, kv_off, o_off, q_len, kv_len, q_pos0, kv_pos0 = t
        for i in range(q_len):
            n = int(np.clip(q_pos0 + i - kv_pos0 + 1, 0, kv_len))
            for h in range(hq):
                if n == 0:
                    assert LSE[o_off + i, h] == -np.inf and np.all(O[o_off + i, h] == 0)
                else:
                    assert abs(LSE[o_off + i, h] - math.log(n)) < 1e-14
                    assert np.allclose(O[o_off + i, h], V[kv_off:kv_off + n, 0].mean(0), atol=1e-14)


def test_key_shift_invariance():
    L, hq, hkv, d = 50, 2, 1, 8
    Q, K, V = rnd((L, hq, d), 71), rnd((L, hkv, d), 72), rnd((L, hkv, d), 73)
    c = rnd((d,), 74)
    scale = 1 / math.sqrt(d)
    task = np.array([(0, 0, 0, L, L, 0, 0)])
    O, LSE = oracle.forward(task, Q, K, V, scale)
    O2, LSE2 = oracle.forward(task, Q, K + c, V, scale)
    assert np.allclose(O, O2, atol=1e-13)
    assert np.allclose(LSE2 - LSE, scale * np.einsum("thd,d->th", Q, c), atol=1e-12)


# ---------------------------------------------------------------------------
# P6: the parity probe (K = 0, V = (-1)^position) closed forms
# ---------------------------------------------------------------------------

def probe_inputs(tasks, q_rows, kv_rows, hq, hkv, d, seed):
    Q = rnd((q_rows, hq, d), seed)
    K = np.zeros((kv_rows, hkv, d))
    V = np.zeros((kv_rows, hkv, d))
    for t in tasks:
        kv_off, kv_len, kv_pos0 = t[1], t[4], t[6]
        pos = kv_pos0 + np.arange(kv_len)
        V[kv_off:kv_off + kv_len] = np.where(pos % 2 == 0, 1.0, -1.0)[:, None, None]
    return Q, K, V


def probe_closed_form(task):
    """O and LSE of the probe for each task row: mean of (-1)^p over the
    visible key positions, and ln of their count."""
    q_off, kv_off, o_off, q_len, kv_len, q_pos0, kv_pos0 = task
    i = np.arange(q_len)
    hi = np.clip(q_pos0 + i, kv_pos0 - 1, kv_pos0 + kv_len - 1)   # last visible position
    n = hi - kv_pos0 + 1
    # sum_{p=a}^{b} (-1)^p = (1 if a even else -1) * ((b - a) % 2 == 0)
    a = kv_pos0
    s = np.where(n > 0, np.where(a % 2 == 0, 1.0, -1.0) * ((hi - a) % 2 == 0), 0.0)
    with np.errstate(divide="ignore", invalid="ignore"):
        O = np.where(n > 0, s / np.maximum(n, 1), 0.0)
        LSE = np.where(n > 0, np.log(np.maximum(n, 1)), -np.inf)
    return O, LSE


def test_probe_closed_forms_ring_and_causal():
    T, nb = 96, 4
    S = T // nb
    tasks = np.array([(i * S, j * S, j * T + i * S, S, S, i * S, j * S)
                      for i in range(nb) for j in range(i + 1)] +
                     [(0, T, nb * T, 3, 37, 100, 0)])          # full-visibility decode-like rows
    Q, K, V = probe_inputs(tasks, T, T + 37, 2, 1, 4, 81)
    O, LSE = oracle.forward(tasks, Q, K, V, 0.5)
    for t in tasks:
        o_ref, lse_ref = probe_closed_form(t)
        r = slice(t[2], t[2] + t[3])
        assert np.allclose(O[r], o_ref[:, None, None], atol=1e-15)
        assert np.allclose(LSE[r], lse_ref[:, None], atol=1e-14)
    # causal document: O = 1/(p+1) at even p, 0 at odd p
    assert O[0, 0, 0] == 1.0 and abs(O[2, 0, 0] - 1 / 3) < 1e-15 and abs(O[3, 0, 0]) < 1e-15


# ---------------------------------------------------------------------------
# P7: backward
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [0, 3, 7])
def test_backward_matches_finite_differences(seed):
    tasks, Q, K, V, scale = tiny_random_case(100 + seed, max_tokens=5)
    dO = rnd(Q.shape, 200 + seed)
    dQ, dK, dV = oracle.backward(tasks, Q, K, V, dO, scale)
    eps = mp.mpf("1e-18")

    def fd(arr, idx, which):
        plus = arr.astype(object).copy()
        minus = arr.astype(object).copy()
        plus[idx] = mp.mpf(float(arr[idx])) + eps
        minus[idx] = mp.mpf(float(arr[idx])) - eps
        args = {"Q": Q, "K": K, "V": V}
        args[which] = plus
        lp = mp_brute.loss(tasks, args["Q"], args["K"], args["V"], dO, mp.mpf(scale))
        args[which] = minus
        lm = mp_brute.loss(tasks, args["Q"], args["K"], args["V"], dO, mp.mpf(scale))
        return float((lp - lm) / (2 * eps))

    for which, arr, grad in (("Q", Q, dQ), ("K", K, dK), ("V", V, dV)):
        for idx in np.ndindex(*arr.shape):
            assert abs(grad[idx] - fd(arr, idx, which)) < 1e-11, (which, idx)


def test_backward_invariants_per_document():
    lens = [37, 1, 64, 130]
    T = sum(lens)
    hq, hkv, d = 4, 2, 8
    Q, K, V = rnd((T, hq, d), 91), rnd((T, hkv, d), 92), rnd((T, hkv, d), 93)
    dO = rnd((T, hq, d), 94)
    cu = np.cumsum([0] + lens)
    tasks = np.array([(cu[i], cu[i], cu[i], l, l, 0, 0) for i, l in enumerate(lens)])
    dQ, dK, dV = oracle.backward(tasks, Q, K, V, dO, 1 / math.sqrt(d))
    for i in range(len(lens)):
        s = slice(cu[i], cu[i + 1])
        for g in range(hkv):
            heads = slice(g * hq // hkv, (g + 1) * hq // hkv)
            assert np.allclose(dK[s, g].sum(0), 0.0, atol=1e-12)               # rows of dS sum to 0
            assert np.allclose(dV[s, g].sum(0), dO[s, heads].sum((0, 1)), atol=1e-12)  # rows of P sum to 1


def test_backward_probe_closed_forms():
    """K = 0, V = (-1)^p: dQ = 0 exactly; dV_j = sum_h sum_{i>=j} dO_i / (i+1)."""
    L, hq, hkv, d = 40, 2, 1, 4
    task = np.array([(0, 0, 0, L, L, 0, 0)])
    Q, K, V = probe_inputs(task, L, L, hq, hkv, d, 95)
    dO = rnd((L, hq, d), 96)
    dQ, dK, dV = oracle.backward(task, Q, K, V, dO, 0.5)
    assert np.allclose(dQ, 0.0, atol=1e-15)
    w = dO / (np.arange(L) + 1.0)[:, None, None]
    ref = np.cumsum(w[::-1].sum(1), axis=0)[::-1]
    assert np.allclose(dV[:, 0], ref, atol=1e-13)


# ---------------------------------------------------------------------------
# P8 / P9: pair counts and the FLOP convention
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("nq,nkv", [(1, 1), (128, 128), (100, 1000), (4096, 70000)])
def test_shard_pair_count_identity(nq, nkv):
    pairs = oracle.visible_pairs_task(nq, nkv, nkv - nq, 0)
    assert 2 * pairs == nq * (2 * nkv - nq + 1)
    # Appendix B's continuous fraction is the large-n limit of this count
    Lq = Lkv = 2 * nkv
    full = oracle.visible_pairs_task(Lq, Lkv, 0, 0)
    frac = nq * (2 * nkv - nq) / (Lq * (2 * Lkv - Lq))
    assert abs(pairs / full - frac) <= 2.0 / Lq + 1e-12


def test_flop_convention_reproduces_pages_1m_figure():
    g = GOLDEN["llama3_405b_1m_prefill_attention_flops"]
    d = g["model_dim"] // g["query_heads"]
    T = g["tokens"]
    pairs = T * (T + 1) // 2
    total = g["layers"] * oracle.forward_flops(pairs, g["query_heads"], d)
    assert abs(total - g["attention_flops"]) / g["attention_flops"] < g["printed_precision_rel"]


def test_scale_value():
    g = GOLDEN["softmax_scale"]
    assert abs(1 / math.sqrt(g["d"]) - g["scale"]) < 1e-16


# ---------------------------------------------------------------------------
# Planted mistakes: each plausible bug fails a pin above
# ---------------------------------------------------------------------------

def test_planted_mistakes_are_caught(monkeypatch):
    """Plant a plausible bug in the oracle and check that the brute-force pin
    notices it (planted on the CPU, in the oracle only)."""
    hq, hkv, d, L = 4, 2, 3, 6
    tasks = np.array([(0, 0, 0, L, L, 0, 0)])
    Q, K, V = rnd((L, hq, d), 301), rnd((L, hkv, d), 302), rnd((L, hkv, d), 303)
    scale = 1 / math.sqrt(d)
    ref = mp_brute.attention(tasks, Q, K, V, scale)

    def max_err():
        O, LSE = oracle.forward(tasks, Q, K, V, scale)
        e = 0.0
        for (row, h), (o, lse) in ref.items():
            e = max(e, abs(LSE[row, h] - float(lse)),
                    max(abs(O[row, h, c] - float(o[c])) for c in range(d)))
        return e

    assert max_err() < 1e-12
    # (a) diagonal dropped from the mask
    orig = oa.visible_mask

    def no_diag(t, r, n):
        qpos = int(t[5]) + np.asarray(r)
        kpos = int(t[6]) + np.arange(n)
        return orig(t, r, n) & (kpos[None, :] != qpos[:, None])

    monkeypatch.setattr(oa, "visible_mask", no_diag)
    assert max_err() > 1e-3
    monkeypatch.setattr(oa, "visible_mask", orig)
    # (b) interleaved instead of contiguous GQA groups
    monkeypatch.setattr(oa, "_group_of", lambda h, hq_, hkv_: h % hkv_)
    assert max_err() > 1e-3
    monkeypatch.undo()
    # (c) scale 1/d instead of 1/sqrt(d)
    O, LSE = oracle.forward(tasks, Q, K, V, 1.0 / d)
    assert max(abs(LSE[r, h] - float(l)) for (r, h), (_, l) in ref.items()) > 1e-3
    # (d) K and V swapped
    O, LSE = oracle.forward(tasks, Q, V, K, scale)
    assert max(abs(LSE[r, h] - float(l)) for (r, h), (_, l) in ref.items()) > 1e-3
    assert max_err() < 1e-12
