"""Python binding of libca.so (ctypes): argument marshalling only.

Every step of the attention path runs inside libca's HIP kernels; this module
only turns torch tensors into device pointers, task tables into ``ca_task``
arrays, and status codes into exceptions.  There is no fallback: if the
library is not built, ``lib()`` raises.
"""

import ctypes
import math
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libca.so")

CA_OK = 0
CA_ERR_INVALID = -1
CA_ERR_UNSUPPORTED = -2
CA_ERR_WORKSPACE = -3
CA_ERR_HIP = -4
CA_OUT_F32 = 1
CA_LAUNCH_PERSISTENT = 2
CA_LAUNCH_PER_ITEM = 4
_LAUNCH = {None: 0, "persistent": CA_LAUNCH_PERSISTENT, "per_item": CA_LAUNCH_PER_ITEM}

EXPORTS = (
    "ca_forward_workspace",
    "ca_forward",
    "ca_forward_varlen_workspace",
    "ca_forward_varlen",
    "ca_merge",
    "ca_backward_workspace",
    "ca_backward",
    "ca_visible_pairs",
    "ca_visible_pairs_masked",
    "ca_forward_masked_workspace",
    "ca_forward_queue_info",
    "ca_forward_masked",
    "ca_forward_paged_workspace",
    "ca_forward_paged",
    "ca_forward_prepare",
    "ca_forward_prepared",
    "ca_forward_noalloc",
    "ca_backward_masked_workspace",
    "ca_backward_masked",
    "ca_backward_paged_workspace",
    "ca_backward_paged",
    "ca_cost_time",
    "ca_schedule_max_items",
    "ca_schedule",
    "ca_sched_tasks",
    "ca_ring_plan",
    "ca_ring_select",
    "ca_ring_select_measured",
    "ca_ring_shard",
    "ca_ring_kv_step_max_tasks",
    "ca_ring_kv_step_tasks",
    "ca_ring_decode_rank",
    "ca_ring_prefill_step_max_tasks",
    "ca_ring_prefill_step_tasks",
    "ca_status_string",
    "ca_last_error",
)

# numpy view of the C struct ca_task (48 bytes, natural alignment)
TASK_DTYPE = np.dtype([("q_off", "<i8"), ("kv_off", "<i8"), ("o_off", "<i8"),
                       ("q_len", "<i4"), ("kv_len", "<i4"),
                       ("q_pos0", "<i8"), ("kv_pos0", "<i8")])
assert TASK_DTYPE.itemsize == 48

# numpy view of the C struct ca_task_mask (8 bytes)
MASK_DTYPE = np.dtype([("window", "<i4"), ("sink", "<i4")])
assert MASK_DTYPE.itemsize == 8


class Shape(ctypes.Structure):
    _fields_ = [("hq", ctypes.c_int32), ("hkv", ctypes.c_int32), ("d", ctypes.c_int32),
                ("scale", ctypes.c_float), ("flags", ctypes.c_uint32),
                ("q_rows", ctypes.c_int64), ("kv_rows", ctypes.c_int64), ("o_rows", ctypes.c_int64)]


class KVPages(ctypes.Structure):
    """ca_kv_pages: block table of paged K/V (physical page of each virtual page)."""
    _fields_ = [("table_host", ctypes.c_void_p), ("n_pages", ctypes.c_int64),
                ("page_rows", ctypes.c_int32), ("reserved", ctypes.c_int32)]


def kv_pages(table, page_rows):
    """KVPages over an int32 copy of ``table``; the struct keeps that copy alive."""
    tb = np.ascontiguousarray(np.asarray(table, dtype=np.int32).reshape(-1))
    pg = KVPages(tb.ctypes.data_as(ctypes.c_void_p) if tb.size else None, len(tb), int(page_rows), 0)
    pg._table = tb
    return pg


class SchedParams(ctypes.Structure):
    _fields_ = [("k", ctypes.c_int32), ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32), ("d", ctypes.c_int32),
                ("eps", ctypes.c_double), ("e_min", ctypes.c_double), ("min_shard", ctypes.c_int64),
                ("max_moves", ctypes.c_int32), ("head_tail", ctypes.c_int32), ("flops_per_pair", ctypes.c_double)]


class ForwardPlan(ctypes.Structure):
    """ca_forward_plan: filled by forward_prepare, read by forward_prepared."""
    _fields_ = [("opaque", ctypes.c_uint64 * 40)]


class RingModel(ctypes.Structure):
    _fields_ = [("n_ranks", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("elem_bytes", ctypes.c_int32), ("d_model", ctypes.c_double), ("compute", ctypes.c_double),
                ("bandwidth", ctypes.c_double)]


class RingTimes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_double) for n in ("attn_step", "sendrecv_kv", "sendrecv_q", "all2all", "exposed_kv",
                                               "miss_threshold", "t_threshold", "ctx_threshold", "eq5_rhs")]


RING_PASS_KV, RING_PASS_Q = 0, 1

# numpy view of the C struct ca_ring_chunk (24 bytes)
RING_CHUNK_DTYPE = np.dtype([("rank", "<i4"), ("seq", "<i4"), ("begin", "<i8"), ("end", "<i8")])
assert RING_CHUNK_DTYPE.itemsize == 24

# numpy view of the C struct ca_sched_item (24 bytes)
SCHED_ITEM_DTYPE = np.dtype([("server", "<i4"), ("doc", "<i4"), ("q_begin", "<i8"), ("q_end", "<i8")])
assert SCHED_ITEM_DTYPE.itemsize == 24


class CAError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("%s: %s" % (status_name(status), message))
        self.status = status


_lib = None


def lib():
    """The loaded libca.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libca.so is not built (run long_context_core_amd.build.build()); "
                               "there is no non-HIP fallback")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        sp = ctypes.POINTER(Shape)
        L.ca_forward_workspace.argtypes = [sp, vp, i32]
        L.ca_forward_workspace.restype = sz
        L.ca_forward.argtypes = [sp, vp, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.ca_forward.restype = ctypes.c_int
        L.ca_forward_varlen_workspace.argtypes = [sp, vp, i32]
        L.ca_forward_varlen_workspace.restype = sz
        L.ca_forward_varlen.argtypes = [sp, vp, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.ca_forward_varlen.restype = ctypes.c_int
        L.ca_merge.argtypes = [sp, i32, i64, vp, vp, vp, vp, vp]
        L.ca_merge.restype = ctypes.c_int
        L.ca_backward_workspace.argtypes = [sp, vp, i32]
        L.ca_backward_workspace.restype = sz
        L.ca_backward.argtypes = [sp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.ca_backward.restype = ctypes.c_int
        L.ca_visible_pairs.argtypes = [vp, i32]
        L.ca_visible_pairs.restype = i64
        L.ca_visible_pairs_masked.argtypes = [vp, vp, i32]
        L.ca_visible_pairs_masked.restype = i64
        L.ca_forward_masked_workspace.argtypes = [sp, vp, vp, i32]
        L.ca_forward_masked_workspace.restype = sz
        L.ca_forward_queue_info.argtypes = [sp, vp, vp, i32, ctypes.POINTER(ctypes.c_int64)]
        L.ca_forward_queue_info.restype = ctypes.c_int
        L.ca_forward_masked.argtypes = [sp, vp, vp, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.ca_forward_masked.restype = ctypes.c_int
        L.ca_forward_paged_workspace.argtypes = [sp, vp, vp, i32, vp]
        L.ca_forward_paged_workspace.restype = sz
        L.ca_forward_paged.argtypes = [sp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.ca_forward_paged.restype = ctypes.c_int
        L.ca_backward_paged_workspace.argtypes = [sp, vp, vp, i32, vp]
        L.ca_backward_paged_workspace.restype = sz
        L.ca_backward_paged.argtypes = [sp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.ca_backward_paged.restype = ctypes.c_int
        L.ca_backward_masked_workspace.argtypes = [sp, vp, vp, i32]
        L.ca_backward_masked_workspace.restype = sz
        L.ca_backward_masked.argtypes = [sp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.ca_backward_masked.restype = ctypes.c_int
        dbl = ctypes.c_double
        L.ca_cost_time.argtypes = [vp, i32, vp, i32, vp, dbl, i64, i64]
        L.ca_cost_time.restype = dbl
        L.ca_schedule_max_items.argtypes = [i32, i32, i32]
        L.ca_schedule_max_items.restype = i32
        L.ca_schedule.argtypes = [ctypes.POINTER(SchedParams), vp, i32, vp, i32, vp, i32, vp, vp, i32,
                                  vp, vp, vp, vp, vp]
        L.ca_schedule.restype = ctypes.c_int
        L.ca_sched_tasks.argtypes = [vp, i32, vp, i32, vp]
        L.ca_sched_tasks.restype = ctypes.c_int
        L.ca_ring_plan.argtypes = [ctypes.POINTER(RingModel), i64, i64, ctypes.POINTER(RingTimes)]
        L.ca_ring_plan.restype = ctypes.c_int
        L.ca_ring_select.argtypes = [ctypes.POINTER(RingModel), i64, i64, i32]
        L.ca_ring_select.restype = i32
        L.ca_ring_select_measured.argtypes = [i32, dbl, dbl, dbl, dbl, vp, vp]
        L.ca_ring_select_measured.restype = i32
        L.ca_ring_shard.argtypes = [i32, vp, i32, vp]
        L.ca_ring_shard.restype = ctypes.c_int
        L.ca_ring_kv_step_max_tasks.argtypes = [i32, i32]
        L.ca_ring_kv_step_max_tasks.restype = i32
        L.ca_ring_kv_step_tasks.argtypes = [i32, i32, i32, vp, i32, vp, i32, vp]
        L.ca_ring_kv_step_tasks.restype = ctypes.c_int
        L.ca_ring_prefill_step_max_tasks.argtypes = [i32, i32]
        L.ca_ring_prefill_step_max_tasks.restype = i32
        L.ca_ring_prefill_step_tasks.argtypes = [i32, i32, i32, vp, vp, i32, vp, i32, vp]
        L.ca_ring_prefill_step_tasks.restype = ctypes.c_int
        L.ca_ring_decode_rank.argtypes = [i32, i64, i32]
        L.ca_ring_decode_rank.restype = i32
        L.ca_forward_prepare.argtypes = [sp, vp, vp, i32, vp, vp, sz, vp, ctypes.POINTER(ForwardPlan)]
        L.ca_forward_prepare.restype = ctypes.c_int
        L.ca_forward_prepared.argtypes = [ctypes.POINTER(ForwardPlan), vp, vp, vp, vp, vp, vp]
        L.ca_forward_prepared.restype = ctypes.c_int
        L.ca_forward_noalloc.argtypes = [sp, vp, vp, i32, vp, vp, vp, vp, vp, vp]
        L.ca_forward_noalloc.restype = ctypes.c_int
        L.ca_status_string.argtypes = [ctypes.c_int]
        L.ca_status_string.restype = ctypes.c_char_p
        L.ca_last_error.argtypes = []
        L.ca_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_name(status):
    return lib().ca_status_string(int(status)).decode()


def _check(status):
    if status != CA_OK:
        raise CAError(status, lib().ca_last_error().decode())


def task_array(tasks):
    """(n, 7) int table (q_off, kv_off, o_off, q_len, kv_len, q_pos0, kv_pos0)
    -> contiguous ca_task records (records pass through unchanged)."""
    if isinstance(tasks, np.ndarray) and tasks.dtype == TASK_DTYPE:
        return np.ascontiguousarray(tasks)
    t = np.asarray(tasks, dtype=np.int64).reshape(-1, 7)
    a = np.zeros(len(t), dtype=TASK_DTYPE)
    for i, name in enumerate(TASK_DTYPE.names):
        a[name] = t[:, i]
    return a


def make_shape(hq, hkv, d, q_rows, kv_rows, o_rows, scale=None, out_f32=False, launch=None):
    """launch: None (the library picks), "persistent" or "per_item": how the
    forward's tiled kernel is launched (results are bit-identical)."""
    s = Shape()
    s.hq, s.hkv, s.d = int(hq), int(hkv), int(d)
    s.scale = float(1.0 / math.sqrt(d) if scale is None else scale)
    s.flags = (CA_OUT_F32 if out_f32 else 0) | _LAUNCH[launch]
    s.q_rows, s.kv_rows, s.o_rows = int(q_rows), int(kv_rows), int(o_rows)
    return s


def _ptr(x):
    if x is None:
        return None
    return ctypes.c_void_p(x.data_ptr())


def _dtype(name):
    import torch
    return {"bf16": torch.bfloat16, "f32": torch.float32, "u8": torch.uint8}[name]


def _need(x, what, dtype, numel):
    """The library reads and writes device buffers through bare pointers, with
    sizes taken from the shape: check here that each tensor is a contiguous
    tensor of the right dtype on the current device holding at least that
    many elements, so that a wrong buffer raises instead of reaching a
    kernel."""
    import torch
    if not isinstance(x, torch.Tensor):
        raise CAError(CA_ERR_INVALID, "%s: expected a torch tensor, got %s" % (what, type(x).__name__))
    if not x.is_cuda:
        raise CAError(CA_ERR_INVALID, "%s: not a device tensor (%s)" % (what, x.device))
    if x.device.index != torch.cuda.current_device():
        raise CAError(CA_ERR_INVALID, "%s: on %s, the current device is cuda:%d"
                      % (what, x.device, torch.cuda.current_device()))
    if x.dtype != _dtype(dtype):
        raise CAError(CA_ERR_INVALID, "%s: dtype %s, expected %s" % (what, x.dtype, _dtype(dtype)))
    if not x.is_contiguous():
        raise CAError(CA_ERR_INVALID, "%s: not contiguous" % what)
    if x.numel() < numel:
        raise CAError(CA_ERR_INVALID, "%s: %d elements, the call needs %d" % (what, x.numel(), numel))


def _ws_bytes(ws):
    _need(ws, "workspace", "u8", 0)
    return ws.numel()


def _check_forward_tensors(shape, Q, K, V, O, LSE):
    hq, hkv, d = int(shape.hq), int(shape.hkv), int(shape.d)
    _need(Q, "Q", "bf16", shape.q_rows * hq * d)
    _need(K, "K", "bf16", shape.kv_rows * hkv * d)
    _need(V, "V", "bf16", shape.kv_rows * hkv * d)
    _need(O, "O", "f32" if shape.flags & CA_OUT_F32 else "bf16", shape.o_rows * hq * d)
    _need(LSE, "LSE", "f32", shape.o_rows * hq)


def _stream_ptr(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _tasks_ptr(ta):
    return ta.ctypes.data_as(ctypes.c_void_p) if len(ta) else None


def split_tasks(tasks, masks=None):
    """(ca_task records, ca_task_mask records or None) from an (n, 7) table
    plus optional masks, or an (n, 9) table whose last two columns are
    window and sink."""
    if not (isinstance(tasks, np.ndarray) and tasks.dtype == TASK_DTYPE):
        t = np.asarray(tasks, dtype=np.int64)
        t = t.reshape(-1, t.shape[-1]) if t.size else t.reshape(0, 7)
        if t.shape[1] == 9:
            if masks is None:
                masks = t[:, 7:9]
            t = t[:, :7]
        tasks = t
    ta = task_array(tasks)
    if masks is None:
        return ta, None
    if isinstance(masks, np.ndarray) and masks.dtype == MASK_DTYPE:
        ma = np.ascontiguousarray(masks)
    else:
        mm = np.asarray(masks, dtype=np.int64).reshape(-1, 2)
        ma = np.zeros(len(mm), dtype=MASK_DTYPE)
        ma["window"], ma["sink"] = mm[:, 0], mm[:, 1]
    if len(ma) != len(ta):
        raise CAError(CA_ERR_INVALID, "one mask per task required")
    return ta, ma


def _mask_ptr(ma):
    return None if ma is None else ma.ctypes.data_as(ctypes.c_void_p)


def visible_pairs(tasks, masks=None):
    ta, ma = split_tasks(tasks, masks)
    n = lib().ca_visible_pairs_masked(_tasks_ptr(ta), _mask_ptr(ma), len(ta))
    if n < 0:
        raise CAError(CA_ERR_INVALID, "invalid task table")
    return int(n)


def forward_workspace(shape, tasks, masks=None, pages=None):
    ta, ma = split_tasks(tasks, masks)
    if pages is not None:
        return int(lib().ca_forward_paged_workspace(ctypes.byref(shape), _tasks_ptr(ta), _mask_ptr(ma), len(ta),
                                                    ctypes.byref(pages)))
    return int(lib().ca_forward_masked_workspace(ctypes.byref(shape), _tasks_ptr(ta), _mask_ptr(ma), len(ta)))


def forward_queue_info(shape, tasks, masks=None):
    """How the forward would launch (host only): dict with the tiled kernel's
    work items, the split-KV decode items, the persistent workgroups (0: one
    workgroup per item), whether some shard is multi-context or split, and
    the number of split shards."""
    ta, ma = split_tasks(tasks, masks)
    info = (ctypes.c_int64 * 5)()
    _check(lib().ca_forward_queue_info(ctypes.byref(shape), _tasks_ptr(ta), _mask_ptr(ma), len(ta), info))
    return {"items": int(info[0]), "decode_items": int(info[1]), "persistent_workgroups": int(info[2]),
            "multi": bool(info[3]), "split_shards": int(info[4])}


def workspace_tensor(nbytes, device, stream=None):
    """A temporary workspace from torch's caching allocator.  Its memory is
    tied to the stream that was current when it was allocated; when the call
    runs on another stream, record_stream keeps the allocator from handing the
    block to a later allocation before that stream's kernels are done."""
    import torch
    ws = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
    if stream is not None and stream != torch.cuda.current_stream(ws.device):
        ws.record_stream(stream)
    return ws


def forward(shape, tasks, Q, K, V, O, LSE, ws=None, stream=None, masks=None, pages=None):
    """ca_forward on torch tensors: Q [q_rows, hq, d] bf16, K/V [kv_rows, hkv, d]
    bf16, O [o_rows, hq, d] bf16 (fp32 with out_f32), LSE [o_rows, hq] fp32.
    With masks (or a 9-column table) it calls ca_forward_masked; with pages
    (a KVPages from kv_pages) ca_forward_paged, K/V then being page stores."""
    ta, ma = split_tasks(tasks, masks)
    _check_forward_tensors(shape, Q, K, V, O, LSE)
    if ws is None:
        ws = workspace_tensor(forward_workspace(shape, ta, ma, pages), Q.device, stream)
    wb = _ws_bytes(ws)
    if pages is not None:
        st = lib().ca_forward_paged(ctypes.byref(shape), _tasks_ptr(ta), _mask_ptr(ma), len(ta),
                                    ctypes.byref(pages), _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(LSE),
                                    _ptr(ws), wb, _stream_ptr(stream))
    elif ma is None:
        st = lib().ca_forward(ctypes.byref(shape), _tasks_ptr(ta), len(ta), _ptr(Q), _ptr(K), _ptr(V),
                              _ptr(O), _ptr(LSE), _ptr(ws), wb, _stream_ptr(stream))
    else:
        st = lib().ca_forward_masked(ctypes.byref(shape), _tasks_ptr(ta), _mask_ptr(ma), len(ta), _ptr(Q),
                                     _ptr(K), _ptr(V), _ptr(O), _ptr(LSE), _ptr(ws), wb,
                                     _stream_ptr(stream))
    _check(st)
    return O, LSE


def forward_prepare(shape, tasks, ws, stream=None, masks=None, pages=None):
    """ca_forward_prepare: the call's host work once (queue built and uploaded
    into ws on the stream); returns the plan for forward_prepared."""
    ta, ma = split_tasks(tasks, masks)
    plan = ForwardPlan()
    _check(lib().ca_forward_prepare(ctypes.byref(shape), _tasks_ptr(ta), _mask_ptr(ma), len(ta),
                                    ctypes.byref(pages) if pages is not None else None, _ptr(ws), _ws_bytes(ws),
                                    _stream_ptr(stream), ctypes.byref(plan)))
    plan._shape = Shape.from_buffer_copy(shape)
    plan._ws = ws     # the queue lives there: keep it alive with the plan
    return plan


def forward_prepared(plan, Q, K, V, O, LSE, stream=None):
    """ca_forward_prepared: kernel launches only (capturable in a HIP graph)."""
    shape = getattr(plan, "_shape", None)
    if shape is not None:
        _check_forward_tensors(shape, Q, K, V, O, LSE)
    _check(lib().ca_forward_prepared(ctypes.byref(plan), _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(LSE),
                                     _stream_ptr(stream)))
    return O, LSE


def forward_noalloc(shape, tasks, Q, K, V, O, LSE, stream=None, masks=None):
    """ca_forward_noalloc: the forward with its queue in the library's fixed
    per-GPU scratch array (no workspace, no allocation; capturable)."""
    ta, ma = split_tasks(tasks, masks)
    _check_forward_tensors(shape, Q, K, V, O, LSE)
    _check(lib().ca_forward_noalloc(ctypes.byref(shape), _tasks_ptr(ta), _mask_ptr(ma), len(ta), _ptr(Q), _ptr(K),
                                    _ptr(V), _ptr(O), _ptr(LSE), _stream_ptr(stream)))
    return O, LSE


NOALLOC_SCRATCH_BYTES = 64 << 20


def forward_varlen(shape, cu_seqlens, Q, K, V, O, LSE, ws=None, stream=None):
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    n = len(cu) - 1
    cup = cu.ctypes.data_as(ctypes.c_void_p)
    _check_forward_tensors(shape, Q, K, V, O, LSE)
    if ws is None:
        ws = workspace_tensor(lib().ca_forward_varlen_workspace(ctypes.byref(shape), cup, n), Q.device, stream)
    st = lib().ca_forward_varlen(ctypes.byref(shape), cup, n, _ptr(Q), _ptr(K), _ptr(V), _ptr(O),
                                 _ptr(LSE), _ptr(ws), _ws_bytes(ws), _stream_ptr(stream))
    _check(st)
    return O, LSE


def merge(shape, O_parts, LSE_parts, O, LSE, stream=None):
    """ca_merge: O_parts [S, n_rows, hq, d] fp32, LSE_parts [S, n_rows, hq] fp32."""
    S, n_rows = int(O_parts.shape[0]), int(O_parts.shape[1])
    hq, d = int(shape.hq), int(shape.d)
    _need(O_parts, "O_parts", "f32", S * n_rows * hq * d)
    _need(LSE_parts, "LSE_parts", "f32", S * n_rows * hq)
    _need(O, "O", "f32" if shape.flags & CA_OUT_F32 else "bf16", n_rows * hq * d)
    _need(LSE, "LSE", "f32", n_rows * hq)
    st = lib().ca_merge(ctypes.byref(shape), S, n_rows, _ptr(O_parts), _ptr(LSE_parts), _ptr(O),
                        _ptr(LSE), _stream_ptr(stream))
    _check(st)
    return O, LSE


def backward_workspace(shape, tasks, masks=None, pages=None):
    ta, ma = split_tasks(tasks, masks)
    if pages is not None:
        return int(lib().ca_backward_paged_workspace(ctypes.byref(shape), _tasks_ptr(ta), _mask_ptr(ma), len(ta),
                                                     ctypes.byref(pages)))
    return int(lib().ca_backward_masked_workspace(ctypes.byref(shape), _tasks_ptr(ta), _mask_ptr(ma), len(ta)))


def backward(shape, tasks, Q, K, V, O, dO, LSE, dQ, dK, dV, ws=None, stream=None, masks=None, pages=None):
    """ca_backward (ca_backward_masked with masks or a 9-column table,
    ca_backward_paged with pages: K, V, dK, dV are then page stores)."""
    ta, ma = split_tasks(tasks, masks)
    hq, hkv, d = int(shape.hq), int(shape.hkv), int(shape.d)
    for x, what, rows, heads in ((Q, "Q", shape.q_rows, hq), (K, "K", shape.kv_rows, hkv),
                                 (V, "V", shape.kv_rows, hkv), (O, "O", shape.o_rows, hq),
                                 (dO, "dO", shape.o_rows, hq), (dQ, "dQ", shape.q_rows, hq),
                                 (dK, "dK", shape.kv_rows, hkv), (dV, "dV", shape.kv_rows, hkv)):
        _need(x, what, "bf16", rows * heads * d)
    _need(LSE, "LSE", "f32", shape.o_rows * hq)
    if ws is None:
        ws = workspace_tensor(backward_workspace(shape, ta, ma, pages), Q.device, stream)
    wb = _ws_bytes(ws)
    if pages is not None:
        st = lib().ca_backward_paged(ctypes.byref(shape), _tasks_ptr(ta), _mask_ptr(ma), len(ta),
                                     ctypes.byref(pages), _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(dO),
                                     _ptr(LSE), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(ws), wb,
                                     _stream_ptr(stream))
    elif ma is None:
        st = lib().ca_backward(ctypes.byref(shape), _tasks_ptr(ta), len(ta), _ptr(Q), _ptr(K), _ptr(V),
                               _ptr(O), _ptr(dO), _ptr(LSE), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(ws),
                               wb, _stream_ptr(stream))
    else:
        st = lib().ca_backward_masked(ctypes.byref(shape), _tasks_ptr(ta), _mask_ptr(ma), len(ta), _ptr(Q),
                                      _ptr(K), _ptr(V), _ptr(O), _ptr(dO), _ptr(LSE), _ptr(dQ), _ptr(dK),
                                      _ptr(dV), _ptr(ws), wb, _stream_ptr(stream))
    _check(st)
    return dQ, dK, dV


# ---------------------------------------------------------------------------
# CA-task scheduling (host)
# ---------------------------------------------------------------------------

def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def cost_time(grid_q, grid_kv, grid_time, flops_per_pair, n_q, n_kv):
    """Predicted seconds of an (n_q, n_kv) block under the measured grid."""
    gq, gkv, gt = _f64(grid_q), _f64(grid_kv), _f64(grid_time)
    return lib().ca_cost_time(gq.ctypes.data, len(gq), gkv.ctypes.data, len(gkv), gt.ctypes.data,
                              float(flops_per_pair), int(n_q), int(n_kv))


def schedule(doc_lens, k, grid_q, grid_kv, grid_time, flops_per_pair, hq, hkv, d,
             eps=0.05, e_min=0.0, min_shard=128, max_moves=10000, head_tail=False):
    """Greedy placement of the documents on k attention servers (splits move
    head-tail shards when head_tail is set).  Returns
    (items as SCHED_ITEM_DTYPE records, loads_before[k], loads_after[k],
    bytes moved, number of migrations)."""
    L = lib()
    docs = np.ascontiguousarray(np.asarray(doc_lens, dtype=np.int64))
    gq, gkv, gt = _f64(grid_q), _f64(grid_kv), _f64(grid_time)
    p = SchedParams(int(k), int(hq), int(hkv), int(d), float(eps), float(e_min), int(min_shard),
                    int(max_moves), 1 if head_tail else 0, float(flops_per_pair))
    cap = L.ca_schedule_max_items(len(docs), int(k), int(max_moves))
    if cap < 0:
        raise CAError(CA_ERR_INVALID, "bad schedule size")
    items = np.zeros(max(cap, 1), dtype=SCHED_ITEM_DTYPE)
    before = np.zeros(int(k), dtype=np.float64)
    after = np.zeros(int(k), dtype=np.float64)
    n_items = ctypes.c_int32(0)
    comm = ctypes.c_double(0.0)
    moves = ctypes.c_int32(0)
    _check(L.ca_schedule(ctypes.byref(p), docs.ctypes.data, len(docs), gq.ctypes.data, len(gq),
                         gkv.ctypes.data, len(gkv), gt.ctypes.data, items.ctypes.data, len(items),
                         ctypes.byref(n_items), before.ctypes.data, after.ctypes.data,
                         ctypes.byref(comm), ctypes.byref(moves)))
    return items[:n_items.value].copy(), before, after, comm.value, moves.value


def sched_tasks(items, doc_lens):
    """ca_task records of scheduled Items over the packed batch."""
    it = np.ascontiguousarray(items, dtype=SCHED_ITEM_DTYPE)
    docs = np.ascontiguousarray(np.asarray(doc_lens, dtype=np.int64))
    out = np.zeros(len(it), dtype=TASK_DTYPE)
    _check(lib().ca_sched_tasks(it.ctypes.data, len(it), docs.ctypes.data, len(docs), out.ctypes.data))
    return out


def ring_model(n_ranks, n_heads, n_kv_heads, elem_bytes, d_model, compute, bandwidth):
    """ca_ring_model: N ranks, N_H / N_KV heads, e bytes per element, D model
    dimension, C attention FLOP/s per rank, BW SendRecv bytes/s per rank."""
    return RingModel(int(n_ranks), int(n_heads), int(n_kv_heads), int(elem_bytes), float(d_model),
                     float(compute), float(bandwidth))


def ring_plan(model, T, P):
    """Every term of the ring time model at (T, P), as a dict."""
    out = RingTimes()
    _check(lib().ca_ring_plan(ctypes.byref(model), int(T), int(P), ctypes.byref(out)))
    return {n: getattr(out, n) for n, _ in RingTimes._fields_}


def ring_select(model, T, P, refined=True):
    """RING_PASS_KV or RING_PASS_Q (Algorithm 5 when refined, else Algorithm 1)."""
    r = lib().ca_ring_select(ctypes.byref(model), int(T), int(P), 1 if refined else 0)
    if r < 0:
        raise CAError(CA_ERR_INVALID, lib().ca_last_error().decode())
    return r


def ring_select_measured(n_ranks, sendrecv_kv, sendrecv_q, attn, all2all):
    """(choice, exposed pass-KV seconds, exposed pass-Q seconds) from measured per-step times."""
    k, q = ctypes.c_double(0.0), ctypes.c_double(0.0)
    r = lib().ca_ring_select_measured(int(n_ranks), float(sendrecv_kv), float(sendrecv_q), float(attn),
                                      float(all2all), ctypes.byref(k), ctypes.byref(q))
    if r < 0:
        raise CAError(CA_ERR_INVALID, lib().ca_last_error().decode())
    return r, k.value, q.value


def ring_shard(lens, n_ranks):
    """Load-balanced chunks (RING_CHUNK_DTYPE records, (sequence, chunk) order)."""
    ls = np.ascontiguousarray(np.asarray(lens, dtype=np.int64))
    out = np.zeros(max(1, len(ls) * 2 * int(n_ranks)), dtype=RING_CHUNK_DTYPE)
    _check(lib().ca_ring_shard(int(n_ranks), ls.ctypes.data, len(ls), out.ctypes.data))
    return out[:len(ls) * 2 * int(n_ranks)]


def ring_kv_step_tasks(lens, n_ranks, step, slot):
    """ca_task records of pass-KV step `step`, slot 0 / 1, over packed sequences."""
    ls = np.ascontiguousarray(np.asarray(lens, dtype=np.int64))
    cap = lib().ca_ring_kv_step_max_tasks(int(n_ranks), len(ls))
    if cap < 0:
        raise CAError(CA_ERR_INVALID, "bad ring size")
    out = np.zeros(max(cap, 1), dtype=TASK_DTYPE)
    n = ctypes.c_int32(0)
    _check(lib().ca_ring_kv_step_tasks(int(n_ranks), int(step), int(slot), ls.ctypes.data, len(ls),
                                       out.ctypes.data, len(out), ctypes.byref(n)))
    return out[:n.value].copy()


def ring_decode_rank(n_ranks, iteration, seq):
    r = lib().ca_ring_decode_rank(int(n_ranks), int(iteration), int(seq))
    if r < 0:
        raise CAError(CA_ERR_INVALID, lib().ca_last_error().decode())
    return r


def ring_prefill_step_tasks(new_lens, cached_lens, n_ranks, step, slot):
    """ca_task records of partial-prefill ring step `step`, slot 0..3."""
    nl = np.ascontiguousarray(np.asarray(new_lens, dtype=np.int64))
    cl = np.ascontiguousarray(np.asarray(cached_lens, dtype=np.int64))
    if len(nl) != len(cl):
        raise CAError(CA_ERR_INVALID, "new_lens and cached_lens differ in length")
    cap = lib().ca_ring_prefill_step_max_tasks(int(n_ranks), len(nl))
    if cap < 0:
        raise CAError(CA_ERR_INVALID, "bad ring size")
    out = np.zeros(max(cap, 1), dtype=TASK_DTYPE)
    n = ctypes.c_int32(0)
    _check(lib().ca_ring_prefill_step_tasks(int(n_ranks), int(step), int(slot), nl.ctypes.data, cl.ctypes.data,
                                            len(nl), out.ctypes.data, len(out), ctypes.byref(n)))
    return out[:n.value].copy()
