"""CA-task profiler: the measured grid behind the scheduler's cost model
("Efficient Long-context Language Model Training by Core Attention
Disaggregation", Section 4.2, The Profiler and Cost Model).

For every grid point (n_q, n_kv) the profiler times one fused library call
holding m copies of a task whose n_q queries are the last n_q tokens of an
n_kv-token causal context (m = max(1, tokens // n_q), all copies reading the
same context rows), and records the call time divided by m: the cost of one
such task inside a fused call, the regime that the pages' composability
property describes.  Grid points with n_q > n_kv are timed as n_kv-query
blocks.  The scheduling itself (ca_schedule) is native code in libca; this
module only drives the timing runs.
"""

import numpy as np

from . import ca
from . import inputs as I


def profile_grid(grid_q, grid_kv, hq, hkv, d, tokens=32768, backward=False, reps=3, warmup=1,
                 device="cuda:0", seed=700):
    """Seconds per task at each grid point, as a [len(grid_q)][len(grid_kv)]
    list, timed with HIP events on the current stream.  backward=True times a
    forward plus a backward call (the pages' profiled unit)."""
    import torch
    dev = torch.device(device)
    stream = torch.cuda.current_stream()
    max_q = max(min(int(q), int(kv)) for q in grid_q for kv in grid_kv)
    q_rows = max(tokens, max_q)
    kv_rows = int(max(grid_kv))
    Q = I.randn_bf16((q_rows, hq, d), seed, device=dev)
    K = I.randn_bf16((kv_rows, hkv, d), seed + 1, device=dev)
    V = I.randn_bf16((kv_rows, hkv, d), seed + 2, device=dev)
    dO = I.randn_bf16((q_rows, hq, d), seed + 3, device=dev) if backward else None
    O = torch.empty((q_rows, hq, d), dtype=torch.bfloat16, device=dev)
    LSE = torch.empty((q_rows, hq), device=dev)
    grads = (torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)) if backward else None
    out = []
    for q in grid_q:
        row = []
        for kv in grid_kv:
            n_kv = int(kv)
            n_q = min(int(q), n_kv)
            m = min(max(1, tokens // n_q), q_rows // n_q)
            t = np.zeros((m, 7), dtype=np.int64)
            t[:, 0] = np.arange(m) * n_q          # q_off
            t[:, 1] = 0                           # kv_off: shared context
            t[:, 2] = t[:, 0]                     # o_off
            t[:, 3] = n_q
            t[:, 4] = n_kv
            t[:, 5] = n_kv - n_q                  # q_pos0: last n_q tokens
            t[:, 6] = 0
            tasks = ca.task_array(t)
            shape = ca.make_shape(hq, hkv, d, q_rows, kv_rows, q_rows)
            ws = ca.workspace_tensor(ca.forward_workspace(shape, tasks), dev)
            bws = ca.workspace_tensor(ca.backward_workspace(shape, tasks), dev) if backward else None

            def call():
                ca.forward(shape, tasks, Q, K, V, O, LSE, ws=ws, stream=stream)
                if backward:
                    ca.backward(shape, tasks, Q, K, V, O, dO, LSE, *grads, ws=bws, stream=stream)

            for _ in range(warmup):
                call()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                call()
            b.record(stream)
            torch.cuda.synchronize()
            row.append(a.elapsed_time(b) / 1e3 / reps / m)
        out.append(row)
    return out
