"""The seeded input generators: rounding, and the workload recipes."""

import numpy as np
import pytest

from long_context_core_amd import inputs as I


def test_bf16_round_bits_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
                        np.array([0.0, -0.0, np.inf, -np.inf, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8], np.float32)])
    x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(I.bf16_round_bits(x), ref)


def test_randn_bf16_is_seeded():
    a = I.randn_bf16((4, 5), 7)
    b = I.randn_bf16((4, 5), 7)
    c = I.randn_bf16((4, 5), 8)
    assert (a.float() == b.float()).all() and not (a.float() == c.float()).all()


def check_table(w):
    t = w.tasks
    assert t.dtype == np.int64 and t.shape[1] == 7
    assert (t[:, 3] >= 0).all() and (t[:, 4] >= 0).all()
    assert (t[:, 0] + t[:, 3] <= w.q_rows).all()
    assert (t[:, 1] + t[:, 4] <= w.kv_rows).all()
    assert (t[:, 2] + t[:, 3] <= w.o_rows).all()
    # output row ranges never overlap
    order = np.argsort(t[:, 2])
    ends = t[order, 2] + t[order, 3]
    assert (t[order[1:], 2] >= ends[:-1]).all()


def test_tiny():
    w = I.tiny_forward()
    check_table(w)
    assert w.doc_lens == [512, 256, 128, 128] and (w.hq, w.hkv, w.d) == (4, 1, 64)


def test_packed_131k():
    w = I.llama8b_packed_131k()
    check_table(w)
    assert sum(w.doc_lens) == 131072 and max(w.doc_lens) <= 65536 and min(w.doc_lens) >= 1
    assert (w.hq, w.hkv, w.d) == (32, 8, 128)


def test_ca_tasks():
    w = I.ca_tasks_34b()
    check_table(w)
    t = w.tasks
    assert len(t) == 64 and t[:, 3].sum() == 262144
    assert (t[:, 3] >= 512).all() and (t[:, 3] <= 8192).all()
    assert (t[:, 5] + t[:, 3] == t[:, 4]).all()            # context = prefix up to shard end
    assert (t[:, 4] <= np.array(w.doc_lens)).all()
    assert (np.array(w.doc_lens) >= 16384).all() and (np.array(w.doc_lens) <= 524288).all()


def test_ring_tables():
    w = I.ring_prefill_405b_tp8()
    check_table(w)
    assert len(w.tasks) == 36 and w.n_parts == 8
    d = I.ring_decode_405b_tp8()
    check_table(d)
    assert len(d.tasks) == 256 and (d.tasks[:, 3] == 1).all()


def test_prolong_like():
    w = I.train_8b_prolong_512k()
    check_table(w)
    lens = np.array(w.doc_lens)
    assert lens.sum() == 524288
    long_tokens = lens[lens >= 65536].sum()
    assert 196608 <= long_tokens <= 262144


@pytest.mark.parametrize("shard", [32, 128, 8192])
def test_shard_sweep(shard):
    w = I.shard_sweep_32k(shard)
    check_table(w)
    t = w.tasks
    assert w.q_rows == 32768 and (t[:, 3] == shard).all()
    # each shard ends its document: last query sees the whole context
    assert (t[:, 5] + t[:, 3] == t[:, 4]).all() and (t[:, 6] == 0).all()
    assert (t[:, 5] >= 0).all() and (t[:, 5] < 8192).all()
    assert np.array_equal(I.shard_sweep_32k(shard).tasks, t)
