"""Seeded synthetic inputs: document-length mixes, CA-task tables and bf16
tensors.

This module holds no attention arithmetic.  It only draws lengths, lays out
task descriptors and draws N(0, 1) tensors, so that the HIP library and the
fp64 oracle are fed bit-identical inputs.  The public datasets the pages train
on (ProLong, the Pile, LongAlign ...) are not available; the mixes below are
synthetic stand-ins with the shapes the pages describe.

Task-table columns (int64): q_off, kv_off, o_off, q_len, kv_len, q_pos0,
kv_pos0 — key j of a task is visible to its query i iff
kv_pos0 + j <= q_pos0 + i.
"""

from dataclasses import dataclass, field
import math

import numpy as np

TASK_COLUMNS = ("q_off", "kv_off", "o_off", "q_len", "kv_len", "q_pos0", "kv_pos0")


@dataclass
class Workload:
    """One attention call: head geometry, task table and buffer row counts."""

    name: str
    hq: int
    hkv: int
    d: int
    tasks: np.ndarray            # (n, 7) int64
    q_rows: int
    kv_rows: int
    o_rows: int
    n_parts: int = 1             # > 1: o_rows = n_parts * merged rows (partials)
    doc_lens: list = field(default_factory=list)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def merged_rows(self) -> int:
        return self.o_rows // self.n_parts


# --------------------------------------------------------------------------
# task tables
# --------------------------------------------------------------------------

def varlen_tasks(doc_lens):
    """One causal task per packed document: {cu[i], cu[i], cu[i], l, l, 0, 0}."""
    t = []
    off = 0
    for l in doc_lens:
        t.append((off, off, off, l, l, 0, 0))
        off += l
    return np.array(t, dtype=np.int64).reshape(-1, 7)


def lognormal_doc_lens(rng, total, median=2048, sigma=1.5, lo=16, hi=65536):
    """ln l ~ N(ln median, sigma^2), rounded, clipped to [lo, hi], drawn until
    ``total`` tokens are filled; the last document is truncated."""
    lens = []
    left = total
    while left > 0:
        l = int(round(math.exp(rng.normal(math.log(median), sigma))))
        l = min(max(l, lo), hi, left)
        lens.append(l)
        left -= l
    return lens


# --------------------------------------------------------------------------
# the workloads
# --------------------------------------------------------------------------

def tiny_forward():
    """1,024 packed tokens, docs [512, 256, 128, 128]; 4 query heads over one
    KV head, d = 64."""
    lens = [512, 256, 128, 128]
    return Workload("tiny-1k-docs-512-256-128-128", 4, 1, 64, varlen_tasks(lens),
                    1024, 1024, 1024, doc_lens=lens)


def llama8b_packed_131k(seed=102, total=131072):
    """Llama-3-8B attention shape (32 query heads, 8 KV heads, d = 128) over
    one packed chunk of ``total`` tokens with a long-tailed lognormal length
    mix (median ~2K, at most 64K)."""
    rng = np.random.default_rng(seed)
    lens = lognormal_doc_lens(rng, total)
    return Workload("llama3-8b-packed-%dk-lognormal" % (total // 1024), 32, 8, 128,
                    varlen_tasks(lens), total, total, total, doc_lens=lens)


def ca_tasks_34b(seed=103, n_tasks=64, total_q=262144, q_min=512, q_max=8192,
                 doc_min=16384, doc_max=524288):
    """Re-batched CA-tasks, LLaMA-34B attention shape (64 query heads, 8 KV
    heads, d = 128).  Each task is a query shard cut at a random offset of its
    own document (length log-uniform in [doc_min, doc_max]); its context is
    the document prefix up to the shard end.  Shard lengths are uniform in
    [q_min, q_max], then adjusted so that they total ``total_q`` exactly.
    Every task carries its own copy of its context, as an attention server
    receives one per task."""
    rng = np.random.default_rng(seed)
    docs = [int(round(math.exp(rng.uniform(math.log(doc_min), math.log(doc_max)))))
            for _ in range(n_tasks)]
    q = rng.integers(q_min, q_max + 1, size=n_tasks).astype(np.int64)
    q = np.clip(np.floor(q * (total_q / q.sum())).astype(np.int64), q_min, q_max)
    i = 0
    while q.sum() != total_q:                     # deterministic fix-up
        step = 1 if q.sum() < total_q else -1
        if q_min <= q[i] + step <= q_max:
            q[i] += step
        i = (i + 1) % n_tasks
    ends = [int(rng.integers(int(q[k]), docs[k] + 1)) for k in range(n_tasks)]
    t = []
    qo = ko = 0
    for k in range(n_tasks):
        ql, end = int(q[k]), ends[k]
        t.append((qo, ko, qo, ql, end, end - ql, 0))
        qo += ql
        ko += end
    return Workload("llama-34b-ca-tasks-64x-262k", 64, 8, 128, np.array(t, dtype=np.int64),
                    qo, ko, qo, doc_lens=docs)


def shard_sweep_32k(shard, seed=106, total_q=32768, ctx_max=8192):
    """One fused 32K-token chunk of query shards of ``shard`` tokens each
    (Llama-3-8B attention shape: 32 query heads, 8 KV heads, d = 128).  Shard
    k is the last ``shard`` tokens of its own document, whose earlier context
    is uniform in [0, ctx_max); every shard carries its own context.  The
    shard length is the swept variable; the aggregate query tokens are fixed."""
    rng = np.random.default_rng(seed)
    n = total_q // shard
    ctx = rng.integers(0, ctx_max, size=n)
    t = []
    ko = 0
    for k in range(n):
        c = int(ctx[k])
        t.append((k * shard, ko, k * shard, shard, c + shard, c, 0))
        ko += c + shard
    return Workload("llama3-8b-shards-%d-of-32k" % shard, 32, 8, 128, np.array(t, dtype=np.int64),
                    n * shard, ko, n * shard)


# --------------------------------------------------------------------------
# sparse-mask recipes ("Dynamic Context Parallelism", Section 2.4, Figure 6)
# --------------------------------------------------------------------------

def lambda_tasks(doc_lens, window=4096, sink=64):
    """Lambda mask per packed document: every token sees the first ``sink``
    tokens of its document and its ``window`` latest tokens (itself
    included).  (n, 9) table: the varlen tasks plus window / sink columns."""
    t = varlen_tasks(doc_lens)
    w = np.zeros((len(t), 2), dtype=np.int64)
    w[:, 0] = window
    w[:, 1] = sink
    return np.concatenate([t, w], axis=1)


def blockwise_tasks(doc_lens, block=256, win_blocks=2):
    """Causal-blockwise mask per packed document, as two partial slots to be
    merged by Equation 4 (output rows o_off in slot s are s * T + row):
    documents are cut into blocks of ``block`` tokens (in-context examples);
    a token of block b sees block 0 (the sink block), blocks b - win_blocks + 1
    .. b - 1 and its own block up to itself; the last block of a document (the
    test example) sees everything before it.  Slot 0 holds the window part
    (the causal context from the window's first block), slot 1 the sink block
    when the window does not reach it."""
    T = int(sum(doc_lens))
    t = []
    off = 0
    for L in doc_lens:
        nb = -(-L // block)
        for b in range(nb):
            q0, q1 = b * block, min(L, (b + 1) * block)
            last = b == nb - 1
            k0 = 0 if last else max(0, b - win_blocks + 1) * block
            t.append((off + q0, off + k0, off + q0, q1 - q0, q1 - k0, q0, k0))
            if not last and k0 > 0:
                t.append((off + q0, off, T + off + q0, q1 - q0, block, q0, 0))
        off += L
    return np.array(t, dtype=np.int64).reshape(-1, 7), 2


def blockwise_shards(doc_lens, block=256, win_blocks=2):
    """The causal-blockwise mask of blockwise_tasks in one launch: every block
    of a document is one query shard; a non-final block whose window does not
    reach the sink block lists two contexts, the sink block [0, block) (all
    visible) and the causal window from its first window block; the others
    list one.  Consecutive tasks with the same query rows are one shard (one
    softmax over the union of their keys), so the output needs no merge."""
    t = []
    off = 0
    for L in doc_lens:
        nb = -(-L // block)
        for b in range(nb):
            q0, q1 = b * block, min(L, (b + 1) * block)
            last = b == nb - 1
            k0 = 0 if last else max(0, b - win_blocks + 1) * block
            if not last and k0 > 0:
                t.append((off + q0, off, off + q0, q1 - q0, block, q0, 0))
            t.append((off + q0, off + k0, off + q0, q1 - q0, q1 - k0, q0, k0))
        off += L
    return np.array(t, dtype=np.int64).reshape(-1, 7)


def shared_question_shards(question, answers):
    """The shared-question mask of shared_question_tasks in one launch: the
    question is causal; every answer is one query shard over two contexts,
    the whole question (all visible) and the answer itself (causal).  Both
    contexts of an answer carry the answer's position after the question, so
    the two tasks name the same query rows and form one shard."""
    t = [(0, 0, 0, question, question, 0, 0)]
    off = question
    for a in answers:
        t.append((off, 0, off, a, question, question, 0))
        t.append((off, off, off, a, a, question, question))
        off += a
    return np.array(t, dtype=np.int64).reshape(-1, 7)


def shared_question_tasks(question, answers):
    """Shared-question mask (one question, several answers packed after it):
    the question is causal; each answer sees the whole question and itself
    causally, never another answer.  Two partial slots to be merged by
    Equation 4: slot 0 holds causal self-attention of every segment, slot 1
    the answers' attention to the question."""
    T = int(question + sum(answers))
    t = [(0, 0, 0, question, question, 0, 0)]
    off = question
    for a in answers:
        t.append((off, off, off, a, a, 0, 0))
        t.append((off, 0, T + off, a, question, question, 0))
        off += a
    return np.array(t, dtype=np.int64).reshape(-1, 7), 2


def shared_question_batch(seed=107, total=524288, q_median=2048, a_median=512, answers=(4, 16)):
    """A packed batch of shared-question groups (one question followed by
    its answers, as in RL / preference data) filling ``total`` tokens,
    Llama-3-8B attention shape: question lengths lognormal (median q_median,
    sigma 1, clipped to [256, 16384]), 4-16 answers per group with lognormal
    lengths (median a_median, sigma 1, clipped to [16, 4096]); the last group
    is cut to fit.  Returns (Workload over the one-launch shard table, list
    of (question, [answers]) per group)."""
    rng = np.random.default_rng(seed)
    groups, left = [], total
    while left > 0:
        q = int(min(max(round(math.exp(rng.normal(math.log(q_median), 1.0))), 256), 16384))
        q = min(q, left)
        left -= q
        ans = []
        for _ in range(int(rng.integers(answers[0], answers[1] + 1))):
            if left <= 0:
                break
            a = int(min(max(round(math.exp(rng.normal(math.log(a_median), 1.0))), 16), 4096, left))
            ans.append(a)
            left -= a
        groups.append((q, ans))
    tables, off = [], 0
    for q, ans in groups:
        t = shared_question_shards(q, ans)
        t[:, [0, 1, 2]] += off
        tables.append(t)
        off += q + sum(ans)
    return (Workload("llama3-8b-shared-question-%dk" % (total // 1024), 32, 8, 128, np.concatenate(tables),
                     total, total, total), groups)


def ring_prefill_405b_tp8(total=131072, n=8):
    """One GPU's share of Llama3-405B under TP8 (16 query heads, 1 KV head,
    d = 128): one causal document of ``total`` tokens split into n contiguous
    query shards and n contiguous KV blocks.  Task (i, j <= i) is shard i over
    block j and writes partial slot j: output rows o_off = j * total + i * S.
    Slots j > i are never written (they are fully masked); their LSE must hold
    -inf before the merge."""
    S = total // n
    t = []
    for i in range(n):
        for j in range(i + 1):
            t.append((i * S, j * S, j * total + i * S, S, S, i * S, j * S))
    return Workload("llama3-405b-tp8-ring-prefill-%dk-%dx%d" % (total // 1024, n, n), 16, 1, 128,
                    np.array(t, dtype=np.int64), total, total, n * total, n_parts=n,
                    doc_lens=[total])


def ring_decode_405b_tp8(batch=32, context=131072, n=8):
    """Pass-Q decode share: ``batch`` single-token queries (16 heads), each over
    its own ``context``-entry KV cache (1 KV head, d = 128), the cache split
    into n stationary blocks.  Task (b, s) writes partial slot s, row b."""
    S = context // n
    t = []
    for b in range(batch):
        for s in range(n):
            t.append((b, b * context + s * S, s * batch + b, 1, S, context - 1, s * S))
    return Workload("llama3-405b-tp8-decode-b%d-%dk" % (batch, context // 1024), 16, 1, 128,
                    np.array(t, dtype=np.int64), batch, batch * context, n * batch, n_parts=n)


def prolong_like_doc_lens(rng, total, long_lo, long_hi):
    """Half of the tokens in long documents (length log-uniform in
    [long_lo, long_hi], drawn until less than long_lo of that half remains),
    the rest in lognormal short documents; order shuffled."""
    long_budget = total // 2
    left = long_budget
    longs = []
    while left >= long_lo:
        l = int(round(math.exp(rng.uniform(math.log(long_lo), math.log(long_hi)))))
        l = min(l, left)
        longs.append(l)
        left -= l
    shorts = lognormal_doc_lens(rng, total - long_budget + left)
    lens = longs + shorts
    order = rng.permutation(len(lens))
    return [lens[k] for k in order]


def train_8b_prolong_512k(seed=105, total=524288, div=1):
    """Training shape, Llama-3-8B attention (32 / 8 heads, d = 128): one packed
    chunk of ``total // div`` tokens with a ProLong-like mix (50 % of tokens
    in docs of 64K-512K, scaled by 1/div, the rest lognormal short docs)."""
    rng = np.random.default_rng(seed)
    tot = total // div
    lens = prolong_like_doc_lens(rng, tot, 65536 // div, 524288 // div)
    return Workload("llama3-8b-train-prolong-like-%dk" % (tot // 1024), 32, 8, 128,
                    varlen_tasks(lens), tot, tot, tot, doc_lens=lens)


# --------------------------------------------------------------------------
# paged K/V layouts (block tables)
# --------------------------------------------------------------------------

def page_table(n_virtual, n_physical, seed):
    """Block table: each of n_virtual virtual pages gets a distinct physical
    page, drawn at random from n_physical >= n_virtual."""
    rng = np.random.default_rng(seed)
    return rng.permutation(int(n_physical))[:int(n_virtual)].astype(np.int32)


def page_store(X, table, page_rows, n_physical, fill=float("nan")):
    """Physical page store (torch tensor) of the virtual tensor X: virtual page
    v is copied to physical page table[v]; pages no entry names hold
    ``fill``.  X has len(table) * page_rows rows."""
    import torch
    P = int(page_rows)
    store = torch.full((int(n_physical) * P,) + tuple(X.shape[1:]), fill, dtype=X.dtype, device=X.device)
    for v, pp in enumerate(np.asarray(table).tolist()):
        store[pp * P:(pp + 1) * P] = X[v * P:(v + 1) * P]
    return store


def paged_varlen_tasks(doc_lens, page_rows):
    """Packed causal documents whose K/V live in pages: queries packed as in
    varlen_tasks, document i's context starting at its own virtual page.
    Returns (tasks, number of virtual pages)."""
    P = int(page_rows)
    t = []
    q = 0
    vp = 0
    for l in doc_lens:
        l = int(l)
        t.append((q, vp * P, q, l, l, 0, 0))
        q += l
        vp += -(-l // P)
    return np.array(t, dtype=np.int64).reshape(-1, 7), vp


def llama8b_packed_131k_paged(page_rows=512, seed=102):
    """The 131K packed Llama-3-8B batch with K/V in pages of page_rows rows
    (the data-block sizes 512 ... 4096 of the DCP page, Block Generation);
    tasks address virtual rows.  kv_rows counts the virtual rows."""
    w = llama8b_packed_131k(seed=seed)
    tasks, n_vp = paged_varlen_tasks(w.doc_lens, page_rows)
    return Workload("llama3-8b-packed-128k-lognormal-paged%d" % page_rows, w.hq, w.hkv, w.d, tasks,
                    w.q_rows, n_vp * page_rows, w.o_rows, doc_lens=w.doc_lens)


# --------------------------------------------------------------------------
# tensors
# --------------------------------------------------------------------------

def randn_bf16(shape, seed, device="cpu"):
    """N(0, 1) float32 from a seeded torch generator, rounded to bfloat16
    (round to nearest even)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return torch.randn(*shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def bf16_round_bits(x):
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even, with
    numpy integer operations only (NaN kept quiet)."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    out = np.where(nan, (u >> 16) | 0x40, rounded)
    return out.astype(np.uint16)


def randn_bf16_bits(shape, seed):
    """numpy-only variant: N(0, 1) float32 from PCG64, bfloat16 bit patterns."""
    rng = np.random.default_rng(seed)
    return bf16_round_bits(rng.standard_normal(shape, dtype=np.float32))
