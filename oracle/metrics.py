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
  * layer-wise loss and its straight-through gradients: per-value tolerances
    from ``layer_loss_tolerance``, derived from the device arithmetic that the
    library documents for that call (fp16 X', fp16 dequantized weights, fp16
    Y_q, fp32 sums, fp16 operands of the dY E product) against the oracle's
    plain fp64 definition; see that function.
"""
from __future__ import annotations

import numpy as np

import oracle

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


# ----------------------------------------------------------------------------
# Layer-wise loss: tolerances derived from the device's rounding points
# ----------------------------------------------------------------------------

U16 = 2.0 ** -11    # unit roundoff of fp16 round-to-nearest-even
ETA16 = 2.0 ** -25  # half the spacing of fp16 subnormals (absolute rounding bound)
U32 = 2.0 ** -24    # unit roundoff of fp32


def layer_loss_tolerance(x, w, qweight, scales, zeros, group, pairs, theta, alpha, draws=32,
                         seed=0):
    """Tolerances for a device layer loss and its gradients against the oracle's
    plain fp64 ``layer_loss``.

    The device computes Y_q as fp32 sums of fp16 X' times the fp16 rounding of
    each dequantized weight and stores Y_q in fp16; it computes Y = X W^T as
    fp32 sums of exact fp16 products, dY = 2 (Y_q - Y), and dX' = dY E
    (E = W_hat - T W) from fp16 roundings of dY and E with fp32 sums. Every
    rounding is modelled as an independent error of at most U16 |v| + ETA16
    (fp16) on the value v it rounds; X' also carries the fp32 transform's
    error (24 U32 times its group's 2-norm) and each fp32 sum of d terms an
    error of standard deviation sqrt(d) U32 sum_k |a_k b_k|. With
    Delta = (Y_q - Y)_device - (Y_q - Y), to first order
      Delta = e_y + e_x W_hat^T + X' e_w^T + (sum errors),
    with e_y, e_x, e_w the roundings of Y_q, X', W_hat. Then
      * loss: L_dev - L = 2 <diff, Delta> + ||Delta||^2. The inner product is a
        sum of independent terms: its variance is at most
        sum (b_y diff)^2 + sum (b_x (diff W_hat))^2 + sum (b_w (diff^T X'))^2
        + sum diff^2 s_acc^2 with b the bounds above; the tolerance is six
        standard deviations of 2 <diff, Delta> plus four times the bound on
        E ||Delta||^2, plus 1e-5 L for the device's fp32 partial sums;
      * gradients (linear in dX'): the error of each angle and scale gradient
        is the image of 2 Delta E and of the dY E product's roundings under
        the activation side's transform gradient. Its standard deviation is
        estimated from ``draws`` seeded draws that put +-bound (the largest
        variance a bounded rounding error can have) on every rounding; the
        tolerance is six such deviations plus GRAD_TOL of max(|g|, rms(g))
        for the fp32 gradient arithmetic itself.
    Returns (loss_tol, dtheta_tol [K][d/2], dalpha_tol [d]).
    """
    x64 = np.asarray(x).astype(np.float64)
    w64 = np.asarray(w).astype(np.float64)
    M, d = x64.shape
    N = w64.shape[0]
    xr = oracle.rotate_activations(x, pairs, theta, alpha)
    what = oracle.dequantize(qweight, scales, zeros, group)
    tw = oracle.transform_weights_f64(w, pairs, theta, alpha)
    yq = xr @ what.T
    diff = yq - x64 @ w64.T
    L = float(np.sum(diff * diff))
    gnorm = np.sqrt(np.sum(xr.reshape(M, d // group, group) ** 2, axis=2, keepdims=True))
    bx = U16 * np.abs(xr) + ETA16 + 24 * U32 * np.broadcast_to(gnorm, (M, d // group, group)).reshape(M, d)
    bw = U16 * np.abs(what) + ETA16
    by = U16 * np.abs(yq) + ETA16
    sacc = np.sqrt(d) * U32 * np.sqrt((np.abs(xr) @ np.abs(what).T) ** 2 + (np.abs(x64) @ np.abs(w64).T) ** 2)
    var = (np.sum((by * diff) ** 2) + np.sum((bx * (diff @ what)) ** 2)
           + np.sum((bw * (diff.T @ xr)) ** 2) + np.sum((diff * sacc) ** 2))
    e2 = (np.sum(by ** 2) + np.sum((bx ** 2).sum(0) * (what ** 2).sum(0))
          + np.sum((bw ** 2).sum(0) * (xr ** 2).sum(0)) + np.sum(sacc ** 2))
    loss_tol = 12.0 * np.sqrt(var) + 4.0 * e2 + 1e-5 * L
    e = what - tw
    dy = 2.0 * diff
    _, gth, gal = oracle.rotation_backward(x, dy @ e, pairs, theta, alpha, "activation")
    rng = np.random.default_rng(np.random.SeedSequence([0x544F4C, seed]))
    sign = lambda shape: rng.integers(0, 2, size=shape) * 2.0 - 1.0  # noqa: E731
    acc_th = np.zeros_like(gth)
    acc_al = np.zeros_like(gal)
    bdy = U16 * np.abs(dy) + ETA16
    be = U16 * np.abs(e) + ETA16
    for _ in range(draws):
        delta = (by * sign((M, N)) + (bx * sign((M, d))) @ what.T + xr @ (bw * sign((N, d))).T
                 + sacc * rng.standard_normal((M, N)))
        ddx = (2.0 * delta + bdy * sign((M, N))) @ e + dy @ (be * sign((N, d)))
        _, nth, nal = oracle.rotation_backward(x, ddx, pairs, theta, alpha, "activation")
        acc_th += nth * nth
        acc_al += nal * nal
    sth = np.sqrt(acc_th / draws)
    sal = np.sqrt(acc_al / draws)

    def floor(g):
        return GRAD_TOL * np.maximum(np.abs(g), np.sqrt(np.mean(g * g)) if g.size else 0.0)

    return float(loss_tol), 6.0 * sth + floor(gth), 6.0 * sal + floor(gal)


def assert_within(got, ref, tol, name):
    """Every |got - ref| <= tol (elementwise); returns the largest ratio."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    tol = np.asarray(tol, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    ratio = np.abs(got - ref) / tol
    worst = float(ratio.max())
    assert worst <= 1.0, (f"{name}: |got - ref| exceeds the derived tolerance by {worst:.2f}x "
                          f"({int((ratio > 1).sum())} of {ratio.size} values)")
    return worst
