"""Host-side checks of libca.so that need no GPU: it loads, exports every
symbol include/ca.h declares, rejects bad arguments before touching the
device, and counts visible pairs exactly like the oracle."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from long_context_core_amd import ca
from long_context_core_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: validation fails first


def header_functions():
    text = open(os.path.join(ROOT, "include", "ca.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ca_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = ca.lib()
    names = header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(ca.EXPORTS)


def test_status_strings():
    assert ca.status_name(0) == "CA_OK"
    assert ca.status_name(-3) == "CA_ERR_WORKSPACE"


@pytest.mark.parametrize("seed", range(6))
def test_visible_pairs_match_oracle(seed):
    rng = np.random.default_rng(seed)
    n = 40
    t = np.zeros((n, 7), np.int64)
    t[:, 3] = rng.integers(0, 3000, n)
    t[:, 4] = rng.integers(0, 3000, n)
    t[:, 5] = rng.integers(-500, 5000, n)
    t[:, 6] = rng.integers(-500, 5000, n)
    assert ca.visible_pairs(t) == oracle.visible_pairs(t)


def test_visible_pairs_of_workloads():
    for w in (I.tiny_forward(), I.llama8b_packed_131k(), I.ca_tasks_34b(), I.ring_prefill_405b_tp8(),
              I.ring_decode_405b_tp8(), I.train_8b_prolong_512k()):
        assert ca.visible_pairs(w.tasks) == oracle.visible_pairs(w.tasks)
    assert ca.visible_pairs(I.ring_prefill_405b_tp8().tasks) == 131072 * 131073 // 2


def call_forward(shape, tasks, ws_bytes=1 << 20, ptr=FAKE):
    ta = ca.task_array(tasks)
    return ca.lib().ca_forward(ctypes.byref(shape) if shape is not None else None,
                               ta.ctypes.data_as(ctypes.c_void_p), len(ta),
                               ptr, ptr, ptr, ptr, ptr, FAKE, ws_bytes, None)


def test_forward_rejects_bad_arguments_without_launching():
    good = [(0, 0, 0, 10, 10, 0, 0)]
    s = ca.make_shape(8, 2, 128, 10, 10, 10)
    assert call_forward(None, good) == ca.CA_ERR_INVALID
    assert call_forward(ca.make_shape(8, 3, 128, 10, 10, 10), good) == ca.CA_ERR_INVALID
    assert call_forward(ca.make_shape(8, 2, 96, 10, 10, 10), good) == ca.CA_ERR_UNSUPPORTED
    assert call_forward(ca.make_shape(8, 2, 128, 10, 10, 10, scale=float("nan")), good) == ca.CA_ERR_INVALID
    for bad_scale in (0.0, -0.125):   # row maxima are taken before scaling
        assert call_forward(ca.make_shape(8, 2, 128, 10, 10, 10, scale=bad_scale), good) == ca.CA_ERR_INVALID
    assert call_forward(s, [(0, 0, 0, 11, 10, 0, 0)]) == ca.CA_ERR_INVALID     # past q_rows
    assert call_forward(s, [(0, 1, 0, 10, 10, 0, 0)]) == ca.CA_ERR_INVALID     # past kv_rows
    assert call_forward(s, [(0, 0, 5, 10, 10, 0, 0)]) == ca.CA_ERR_INVALID     # past o_rows
    assert call_forward(s, [(0, 0, 0, -1, 10, 0, 0)]) == ca.CA_ERR_INVALID
    big = 2 ** 63 - 1                                                           # off + len would overflow
    for k in range(3):
        for off in (big, big - 5, big - 9):
            t = [0, 0, 0, 10, 10, 0, 0]
            t[k] = off
            assert call_forward(s, [tuple(t)]) == ca.CA_ERR_INVALID, (k, off)
    assert call_forward(ca.make_shape(8, 2, 128, big, 10, 10), good) == ca.CA_ERR_INVALID   # rows > 2^40
    # task lengths above 2^30 (int32 tile arithmetic), in a shape large enough to hold them
    huge = ca.make_shape(8, 2, 128, 2 ** 31, 2 ** 31, 2 ** 31)
    for t in [(0, 0, 0, 2 ** 30 + 1, 10, 0, 0), (0, 0, 0, 10, 2 ** 30 + 1, 0, 0), (0, 0, 0, 10, 2 ** 31 - 1, 0, 0)]:
        assert call_forward(huge, [t]) == ca.CA_ERR_INVALID, t
        assert "above 2^30" in ca.lib().ca_last_error().decode()
        ta = ca.task_array([t])
        assert ca.lib().ca_backward_workspace(ctypes.byref(huge), ta.ctypes.data_as(ctypes.c_void_p), len(ta)) == 0
    assert call_forward(ca.make_shape(8192, 2, 128, 10, 10, 10), good) == ca.CA_ERR_INVALID  # hq > 4096
    assert call_forward(s, good, ptr=None) == ca.CA_ERR_INVALID                # NULL tensors
    need = ca.forward_workspace(s, good)
    assert need > 0
    assert call_forward(s, good, ws_bytes=need - 1) == ca.CA_ERR_WORKSPACE
    assert "workspace" in ca.lib().ca_last_error().decode()
    # nothing to do: OK without touching the device
    assert call_forward(s, [(0, 0, 0, 0, 10, 0, 0)]) == ca.CA_OK
    # launch flags: one of the two, forward only
    both = ca.make_shape(8, 2, 128, 10, 10, 10)
    both.flags = ca.CA_LAUNCH_PERSISTENT | ca.CA_LAUNCH_PER_ITEM
    assert call_forward(both, good) == ca.CA_ERR_INVALID
    unknown = ca.make_shape(8, 2, 128, 10, 10, 10)
    unknown.flags = 8
    assert call_forward(unknown, good) == ca.CA_ERR_INVALID
    for launch in ("persistent", "per_item"):
        sl = ca.make_shape(8, 2, 128, 10, 10, 10, launch=launch)
        assert ca.forward_workspace(sl, good) == need
        assert call_forward(sl, good, ws_bytes=need - 1) == ca.CA_ERR_WORKSPACE
        ta = ca.task_array(good)
        assert ca.lib().ca_backward_workspace(ctypes.byref(sl), ta.ctypes.data_as(ctypes.c_void_p), len(ta)) == 0
        assert "forward flags" in ca.lib().ca_last_error().decode()


def test_merge_rejects_bad_arguments():
    L = ca.lib()
    s = ca.make_shape(4, 1, 128, 0, 0, 0)
    assert L.ca_merge(ctypes.byref(s), 0, 10, FAKE, FAKE, FAKE, FAKE, None) == ca.CA_ERR_INVALID
    assert L.ca_merge(ctypes.byref(s), 2, -1, FAKE, FAKE, FAKE, FAKE, None) == ca.CA_ERR_INVALID
    assert L.ca_merge(ctypes.byref(s), 2, 10, None, FAKE, FAKE, FAKE, None) == ca.CA_ERR_INVALID
    s2 = ca.make_shape(4, 1, 80, 0, 0, 0)
    assert L.ca_merge(ctypes.byref(s2), 2, 10, FAKE, FAKE, FAKE, FAKE, None) == ca.CA_ERR_UNSUPPORTED
    assert L.ca_merge(ctypes.byref(s), 2, 0, FAKE, FAKE, FAKE, FAKE, None) == ca.CA_OK
    s3 = ca.make_shape(4, 1, 128, 0, 0, 0, launch="persistent")
    assert L.ca_merge(ctypes.byref(s3), 2, 10, FAKE, FAKE, FAKE, FAKE, None) == ca.CA_ERR_INVALID


def test_varlen_rejects_bad_cu_seqlens():
    L = ca.lib()
    s = ca.make_shape(4, 1, 64, 100, 100, 100)
    for cu in ([1, 10], [0, 10, 5]):
        a = np.array(cu, np.int32)
        st = L.ca_forward_varlen(ctypes.byref(s), a.ctypes.data_as(ctypes.c_void_p), len(a) - 1,
                                 FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None)
        assert st == ca.CA_ERR_INVALID


def test_masked_visible_pairs_match_the_oracle():
    """ca_visible_pairs_masked (host code) counts the sink + window mask's
    pairs exactly as the oracle does."""
    import numpy as np
    import oracle
    from long_context_core_amd import ca, inputs as I
    rng = np.random.default_rng(4)
    for _ in range(30):
        docs = [int(x) for x in rng.integers(1, 3000, size=rng.integers(1, 6))]
        t = I.lambda_tasks(docs, window=int(rng.integers(1, 5000)), sink=int(rng.integers(0, 300)))
        if rng.random() < 0.5:        # shifted positions, partial contexts
            t[:, 5] += rng.integers(0, 50, size=len(t))
        assert ca.visible_pairs(t) == oracle.visible_pairs(t)
    assert ca.visible_pairs(I.varlen_tasks([5, 7])) == oracle.visible_pairs(I.varlen_tasks([5, 7]))


def test_masked_visible_pairs_closed_form_on_random_tasks():
    """The closed-form count of ca_visible_pairs_masked against the oracle's
    row-by-row count, on tasks with arbitrary position offsets (rows before,
    inside and past the context), windows shorter and longer than the
    context, and sinks inside and past it."""
    import numpy as np
    import oracle
    rng = np.random.default_rng(11)
    rows = []
    for _ in range(400):
        q_len, kv_len = int(rng.integers(0, 300)), int(rng.integers(0, 300))
        kv_pos0 = int(rng.integers(0, 200))
        q_pos0 = kv_pos0 + int(rng.integers(-350, 350))
        window = int(rng.choice([0, 1, 2, int(rng.integers(1, 400))]))
        sink = int(rng.choice([0, 1, int(rng.integers(0, 500))]))
        rows.append((0, 0, 0, q_len, kv_len, q_pos0, kv_pos0, window, sink))
    for r in rows:
        assert ca.visible_pairs([r]) == oracle.visible_pairs([r]), r
    assert ca.visible_pairs(rows) == oracle.visible_pairs(rows)
    # lengths above 2^30 are refused; 2^30 itself is counted without a row loop
    with pytest.raises(ca.CAError):
        ca.visible_pairs([(0, 0, 0, 2 ** 30 + 1, 10, 0, 0, 64, 4)])
    L = 2 ** 30
    assert ca.visible_pairs([(0, 0, 0, L, L, 0, 0, 1, 0)]) == L           # window 1: the diagonal
    assert ca.visible_pairs([(0, 0, 0, L, L, 0, 0, L, 0)]) == L * (L + 1) // 2


def call_paged(shape, tasks, table, page_rows, reserved=0, ws_bytes=1 << 20):
    ta = ca.task_array(tasks)
    pg = ca.kv_pages(table, page_rows)
    pg.reserved = reserved
    return ca.lib().ca_forward_paged(ctypes.byref(shape), ta.ctypes.data_as(ctypes.c_void_p), None, len(ta),
                                     ctypes.byref(pg), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws_bytes, None)


def test_paged_forward_rejects_bad_page_tables():
    s = ca.make_shape(8, 2, 128, 300, 4 * 256, 300)        # 4 physical pages of 256 rows
    good = [(0, 256, 0, 300, 300, 0, 0)]                    # virtual rows [256, 556)
    table = [3, 1, 0]                                       # 3 virtual pages
    for bad_rows in (0, 64, 192, 3 << 20):
        assert call_paged(ca.make_shape(8, 2, 128, 300, 4 * 1024, 300), good, table, bad_rows) == \
            ca.CA_ERR_INVALID, bad_rows
    assert call_paged(s, good, [3, 4, 0], 256) == ca.CA_ERR_INVALID            # physical page 4 of 4
    assert call_paged(s, good, [3, -1, 0], 256) == ca.CA_ERR_INVALID
    assert call_paged(s, good, table, 256, reserved=1) == ca.CA_ERR_INVALID
    assert call_paged(s, [(0, 256, 0, 300, 600, 0, 0)], table, 256) == ca.CA_ERR_INVALID   # past 768 rows
    assert call_paged(s, [(0, 64, 0, 300, 300, 0, 0)], table, 256) == ca.CA_ERR_INVALID    # kv_off % 128
    assert "multiple of 128" in ca.lib().ca_last_error().decode()
    need = ca.forward_workspace(s, good, pages=ca.kv_pages(table, 256))
    assert need > ca.forward_workspace(s, [(0, 0, 0, 300, 300, 0, 0)])          # the table travels too
    assert call_paged(s, good, table, 256, ws_bytes=need - 1) == ca.CA_ERR_WORKSPACE
    assert ca.forward_workspace(s, good, pages=ca.kv_pages([3, 9, 0], 256)) == 0
    # a context that is empty needs no alignment; nothing to do: OK
    assert call_paged(s, [(0, 5, 0, 0, 0, 0, 0)], table, 256) == ca.CA_OK


def test_paged_backward_rejects_a_task_reading_a_page_twice():
    s = ca.make_shape(8, 2, 128, 300, 4 * 128, 300)
    tasks = ca.task_array([(0, 0, 0, 300, 300, 0, 0)])            # virtual pages 0, 1, 2
    for table, want in (([1, 2, 1], ca.CA_ERR_INVALID), ([1, 2, 3], ca.CA_OK)):
        pg = ca.kv_pages(table, 128)
        need = ca.lib().ca_backward_paged_workspace(ctypes.byref(s), tasks.ctypes.data_as(ctypes.c_void_p), None,
                                                     1, ctypes.byref(pg))
        assert (need == 0) == (want != ca.CA_OK)
    pg = ca.kv_pages([1, 2, 1], 128)
    st = ca.lib().ca_backward_paged(ctypes.byref(s), tasks.ctypes.data_as(ctypes.c_void_p), None, 1,
                                    ctypes.byref(pg), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                    1 << 30, None)
    assert st == ca.CA_ERR_INVALID and "twice" in ca.lib().ca_last_error().decode()


def test_binding_rejects_host_and_mistyped_tensors_before_the_library():
    """The Python binding checks every tensor against the shape before it
    hands bare pointers to the library: host tensors and non-tensors are
    rejected here (no GPU needed); the device-side checks (dtype, size,
    contiguity on the current device) run in the GPU tests."""
    import torch
    s = ca.make_shape(8, 2, 64, 10, 10, 10)
    t = [(0, 0, 0, 10, 10, 0, 0)]
    Q = torch.zeros((10, 8, 64), dtype=torch.bfloat16)
    K = torch.zeros((10, 2, 64), dtype=torch.bfloat16)
    O = torch.zeros((10, 8, 64), dtype=torch.bfloat16)
    L = torch.zeros((10, 8))
    ws = torch.zeros(1 << 16, dtype=torch.uint8)
    with pytest.raises(ca.CAError, match="Q: not a device tensor"):
        ca.forward(s, t, Q, K, K, O, L, ws=ws)
    with pytest.raises(ca.CAError, match="expected a torch tensor"):
        ca.forward(s, t, np.zeros((10, 8, 64), np.float32), K, K, O, L, ws=ws)
    with pytest.raises(ca.CAError, match="O_parts: not a device tensor"):
        ca.merge(s, torch.zeros((2, 10, 8, 64)), torch.zeros((2, 10, 8)), O, L)
    with pytest.raises(ca.CAError, match="Q: not a device tensor"):
        ca.backward(s, t, Q, K, K, O, O, L, Q, K, K, ws=ws)
    with pytest.raises(ca.CAError, match="Q: not a device tensor"):
        ca.forward_varlen(s, [0, 10], Q, K, K, O, L, ws=ws)


def test_forward_queue_info_launch_rule_and_splits():
    """Host-only view of the forward's launch: items, the persistent rule
    (default from 4,096 items; the flags force either way), multi-context
    shards and long shards split over key chunks."""
    w = I.llama8b_packed_131k()
    s = ca.make_shape(w.hq, w.hkv, w.d, w.q_rows, w.kv_rows, w.o_rows)
    info = ca.forward_queue_info(s, w.tasks)
    assert info["items"] >= 4096 and info["persistent_workgroups"] == 256
    assert not info["multi"] and info["split_shards"] == 0     # no item outlasts a CU's share
    si = ca.make_shape(w.hq, w.hkv, w.d, w.q_rows, w.kv_rows, w.o_rows, launch="per_item")
    assert ca.forward_queue_info(si, w.tasks)["persistent_workgroups"] == 0
    t = I.tiny_forward()                                         # 8 items: one workgroup each
    st = ca.make_shape(t.hq, t.hkv, t.d, t.q_rows, t.kv_rows, t.o_rows)
    assert ca.forward_queue_info(st, t.tasks)["persistent_workgroups"] == 0
    w = I.ca_tasks_34b()
    s = ca.make_shape(w.hq, w.hkv, w.d, w.q_rows, w.kv_rows, w.o_rows)
    info = ca.forward_queue_info(s, w.tasks)
    assert info["items"] >= 4096 and info["persistent_workgroups"] == 256
    si = ca.make_shape(w.hq, w.hkv, w.d, w.q_rows, w.kv_rows, w.o_rows, launch="per_item")
    assert ca.forward_queue_info(si, w.tasks)["persistent_workgroups"] == 0
    # a few rows at the end of a long context: split; with the same context
    # short, not split; a single row goes to the decode kernel
    s = ca.make_shape(8, 2, 128, 64, 200000, 64)
    assert ca.forward_queue_info(s, [(0, 0, 0, 64, 200000, 199936, 0)])["split_shards"] == 1
    assert ca.forward_queue_info(s, [(0, 0, 0, 64, 20000, 19936, 0)])["split_shards"] == 0
    info = ca.forward_queue_info(s, [(0, 0, 0, 1, 200000, 199999, 0)])
    assert info["items"] == 0 and info["decode_items"] > 0
    with pytest.raises(ca.CAError):
        ca.forward_queue_info(s, [(0, 0, 0, 65, 10, 0, 0)])   # past q_rows
