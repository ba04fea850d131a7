"""Comparison metrics between a device result and the oracle (test infrastructure).

Tolerances of the rotated W4G128 path:
  * rotated activations X' (fp16): max relative error <= 2e-3, with each
    element's denominator floored at 1 % of the RMS of its (token, group) slice
    of the oracle, because elements that cancel to near zero have no meaningful
    relative error. fp32 arithmetic through 8 stages contributes at most about
    24 * 2^-24 * |x_group| ~ 1.4e-6 |x_group|, i.e. <= 1.6e-3 of the floor, and
    the final fp16 rounding contributes <= 2^-11 of the element itself.
  * linear output Y: ||Y - Y_ref||_F / ||Y_ref||_F <= 1e-2 and
    max |Y - Y_ref| <= 5e-2 * max |Y_ref|.
  * gradients of the transform (input, angles, scales; fp32 on the device):
    max |g - g_ref| / max(|g_ref|, rms(g_ref)) <= 1e-4 over each output. A
    value goes through K stages forward and K stages back, about four fp32
    roundings per stage: 4 K 2^-24 ~ 2e-6 of the row at K = 8 (8e-6 at
    K = 32). Sums over rows add at most about sqrt(M) 2^-24 of the sum of
    the terms' magnitudes, which for terms of random sign is of the order of
    the typical entry (the rms floor covers entries that cancel).
"""
from __future__ import annotations

import numpy as np

XR_TOL = 2e-3
GRAD_TOL = 1e-4
Y_FRO_TOL = 1e-2
Y_MAX_TOL = 5e-2


def rotated_error(got, ref, group):
    """Return (floored max relative error, unfloored max relative error, count > XR_TOL)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    M, d = ref.shape
    if M == 0:
        return 0.0, 0.0, 0
    rg = ref.reshape(M, d // group, group)
    rms = np.sqrt(np.mean(rg * rg, axis=2, keepdims=True))
    floor = np.broadcast_to(0.01 * rms, rg.shape).reshape(M, d)
    err = np.abs(got - ref)
    rel = err / np.maximum(np.abs(ref), floor)
    with np.errstate(divide="ignore", invalid="ignore"):
        raw = np.where(ref != 0, err / np.abs(ref), np.where(err == 0, 0.0, np.inf))
    return float(rel.max()), float(raw.max()), int((rel > XR_TOL).sum())


def linear_error(got, ref):
    """Return (relative Frobenius error, max-abs error / max |ref|)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0, 0.0
    fro = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    mx = np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-300)
    return float(fro), float(mx)


def assert_rotated_close(got, ref, group, tol=XR_TOL):
    fl, raw, n = rotated_error(got, ref, group)
    assert fl <= tol, f"rotated activations: floored max rel err {fl:.3e} > {tol} ({n} elements; unfloored {raw:.3e})"
    return fl


def assert_linear_close(got, ref, fro_tol=Y_FRO_TOL, max_tol=Y_MAX_TOL):
    fro, mx = linear_error(got, ref)
    assert fro <= fro_tol and mx <= max_tol, f"linear: rel-Frobenius {fro:.3e}, max-abs/max {mx:.3e}"
    return fro, mx


def grad_error(got, ref):
    """max |got - ref| / max(|ref|, rms(ref)) over all entries (0 for empty)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    den = np.maximum(np.abs(ref), max(rms, 1e-300))
    return float((np.abs(got - ref) / den).max())


def assert_grad_close(got, ref, name="gradient", tol=GRAD_TOL):
    e = grad_error(got, ref)
    assert e <= tol, f"{name}: floored max rel err {e:.3e} > {tol}"
    return e
