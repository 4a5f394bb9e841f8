"""Helpers shared by the GPU parity tests: device tensors from the seeded
generators, widening for the oracle, and the tolerance checks.

Tolerances (stated for this path): on O, max |O_gpu - O_ref| <= 2e-2 and
||O_gpu - O_ref||_F / ||O_ref||_F <= 1e-2; on LSE, max |dLSE| <= 1e-3 over
rows with a finite LSE (and -inf exactly where the oracle has -inf); on dQ,
dK, dV, relative Frobenius error <= 3e-2 per tensor.
"""

import sys

import numpy as np
import pytest

import oracle

O_MAX_ABS = 2e-2
O_REL_FRO = 1e-2
LSE_MAX_ABS = 1e-3
GRAD_REL_FRO = 3e-2


def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def announce(msg):
    """Name the case before any GPU work, so a failure that ends the process
    still says which case it was."""
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


def widen(t):
    """bf16 / fp32 torch tensor (any device) -> float64 numpy (numpy passes
    through as float64)."""
    import torch
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return oracle.bf16_bits_to_f64(t.view(torch.int16).numpy())
    return t.double().numpy()


def check_forward(O_gpu, LSE_gpu, O_ref, LSE_ref, label=""):
    """Compare on rows the oracle covers (its NaN marks uncovered rows)."""
    O_gpu = widen(O_gpu)
    LSE_gpu = widen(LSE_gpu)
    covered = ~np.isnan(LSE_ref)
    assert covered.any()
    ref_inf = np.isneginf(LSE_ref) & covered
    assert np.array_equal(np.isneginf(LSE_gpu) & covered, ref_inf), label + ": -inf rows differ"
    fin = covered & ~ref_inf
    dl = np.abs(LSE_gpu[fin] - LSE_ref[fin])
    max_dlse = float(dl.max()) if dl.size else 0.0
    Og, Or = O_gpu[covered], O_ref[covered]
    assert np.all(np.isfinite(Og)), label + ": non-finite O"
    max_do = float(np.max(np.abs(Og - Or))) if Og.size else 0.0
    nrm = float(np.linalg.norm(Or))
    rel = float(np.linalg.norm(Og - Or) / nrm) if nrm > 0 else float(np.linalg.norm(Og))
    print("%s: max|dO|=%.3e relF(O)=%.3e max|dLSE|=%.3e" % (label, max_do, rel, max_dlse), flush=True)
    assert max_do <= O_MAX_ABS, label
    assert rel <= O_REL_FRO, label
    assert max_dlse <= LSE_MAX_ABS, label
    return max_do, rel, max_dlse


def rel_fro(a, b):
    nb = float(np.linalg.norm(b))
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a))
