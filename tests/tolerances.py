"""Acceptance bounds for the HIP path against the fp64 oracle.

Per-token loss: |L_gpu - L_ref| <= 1e-4 + 1e-3 |L_ref|.
Gradients (dz, dh, dW): max |g_gpu - g_ref| <= 2e-3 * max |g_ref|
(bf16 inputs, fp32 accumulation).  Row selection, gather and scatter are
compared bit for bit.
"""
import numpy as np

LOSS_ATOL = 1e-4
LOSS_RTOL = 1e-3
GRAD_REL = 2e-3


def loss_err(got, ref):
    """Largest ratio |got-ref| / (atol + rtol|ref|); <= 1 passes."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref) / (LOSS_ATOL + LOSS_RTOL * np.abs(ref))))


def grad_err(got, ref):
    """max|got-ref| / (GRAD_REL * max|ref|); <= 1 passes (0/0 counts as 0)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.size == 0:
        return 0.0
    d = float(np.max(np.abs(got - ref)))
    s = GRAD_REL * float(np.max(np.abs(ref)))
    if s == 0.0:
        return 0.0 if d == 0.0 else float("inf")
    return d / s


def assert_loss_close(got, ref, what="loss"):
    e = loss_err(got, ref)
    assert e <= 1.0, f"{what}: worst |dL| / (1e-4 + 1e-3|L|) = {e:.3g}"


def assert_grad_close(got, ref, what="grad"):
    e = grad_err(got, ref)
    assert e <= 1.0, f"{what}: max|d| / (2e-3 max|ref|) = {e:.3g}"
