"""CPU oracle for ParoQuant's rotated W4G128 linear layer.

TEST INFRASTRUCTURE ONLY. Only the test suite, the package's smoke check and
the benchmark's CPU-baseline leg may import this module. The product path
(the HIP library and its Python binding) never calls it, and it shares no code
with that path: the only thing both sides use is the seeded input generator
(``synthetic``), which holds none of the method's arithmetic.

Sources (the pages describing the method):
  [Notes]    Paper notes "ParoQuant: Pairwise Rotation Quantization for
             Efficient Reasoning LLM Inference" (ICLR 2026, arXiv 2511.10645):
             section "关键设计" (key design): the Givens plane rotation of a
             channel pair, the independent-rotation constraint (each channel in
             at most one pair of a stage, rotations local to a quantization
             group), the cascade of K stages (default 8) with n/2 angles per
             stage, the channel scaling diag(alpha), and the final transform
             T = (prod_t R(P_t, Theta_t)) * diag(alpha) applied to W.
             Section "损失函数 / 训练策略": per-group quantization parameters
             s (scale) and z (zero). Section "主实验": the W4G128 format.
  [CSDN]     CSDN article on ParoQuant: section 2.1 (the equivalence
             Y = XW + b = (X T^-1)(T W) + b), section 2.2 (the 2x2 Givens
             matrix [[cos, -sin], [sin, cos]] acting on (v_i, v_j)), section 2.3
             (scale first, then the rotations in sequence).
  [Abstract] arXiv 2511.10645 abstract: weight-only post-training
             quantization combining independent Givens rotations with channel
             scaling.

Readings of points the pages leave open (each is also listed in the design
notes of the repository):
  * Stage 0 of the ``pairs``/``theta`` arrays is applied first (the product
    over t = 1..K is read as "apply R_1, then R_2, ...").
  * For a stored pair (i, j): v_i <- c*v_i - s*v_j and v_j <- s*v_i + c*v_j
    (the CSDN 2x2 matrix; the notes write the same update for row i).
  * Activations: x <- x / alpha, then the SAME stages in the SAME order with the
    SAME update. This is x * T^-1 for T = R_K...R_1 diag(alpha), because
    x * R^T applies R's update to the row vector x.
  * Weights ([N][d] nn.Linear layout, i.e. the transpose of the math W):
    u <- w * alpha along d, then the stages along d.
  * Quantizer (the pages give only "s, z" and W4G128): asymmetric min/max
    round-to-nearest over 15 steps, range widened to include 0, fp16 scale,
    integer zero in [0, 15], codes clamp(rint(u/s) + z, 0, 15), ties to even.
    A zero scale becomes 1.0; an infinite or NaN scale is an error.
  * Packing: eight codes per 32-bit little-endian word (channels 8w .. 8w+7),
    the even channels in its low 16 bits and the odd ones in its high 16
    bits, 4 bits each in channel order (``pack_codes``); scales fp16 [N][d/G];
    zeros uint8 [N][d/G].
  * cos/sin: c = float32(cos(float64(theta))), s = float32(sin(...)) for the
    canonical fp32 weight transform; plain fp64 cos/sin for the fp64 parts.

Precision:
  * ``rotate_activations``, ``transform_weights_f64``, ``linear``,
    ``rotation_backward``: fp64.
  * ``transform_weights_f32`` and ``quantize_groups``: the canonical fp32
    order of operations (every product and sum rounded to fp32 on its own,
    no fused multiply-add), because the int4 codes must be reproduced bit for
    bit. numpy evaluates each elementwise operation separately, so
    ``c * a - s * b`` on float32 arrays is exactly fl(fl(c*a) - fl(s*b)).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "check_rotation_params", "cos_sin_f32", "rotate_activations",
    "transform_weights_f32", "transform_weights_f64", "quantize_groups",
    "pack_codes", "unpack_codes", "dequantize", "quantize_weights", "linear",
    "rotated_w4_linear", "rotation_backward", "layer_loss", "layer_loss_gradients",
    "QuantizeError",
]


class QuantizeError(ValueError):
    """A group's scale is infinite or NaN (the input had non-finite values)."""


# ----------------------------------------------------------------------------
# Parameters
# ----------------------------------------------------------------------------

def check_rotation_params(pairs, theta, alpha, group):
    """Validate the rotation parameters the way [Notes] "关键设计" constrains them.

    Independent rotation: inside one stage each channel belongs to exactly one
    pair (a perfect pairing; partial pairings use theta = 0), and a pair never
    leaves its quantization group.
    """
    pairs = np.asarray(pairs)
    theta = np.asarray(theta)
    alpha = np.asarray(alpha)
    d = alpha.shape[0]
    K = pairs.shape[0]
    if group <= 0 or group % 2 or d % group:
        raise ValueError("group must be even and divide d")
    if pairs.shape != (K, d // 2, 2) or theta.shape != (K, d // 2):
        raise ValueError("pairs must be [K][d/2][2] and theta [K][d/2]")
    for t in range(K):
        flat = pairs[t].reshape(-1)
        if flat.min(initial=0) < 0 or flat.max(initial=0) >= d:
            raise ValueError(f"stage {t}: channel index out of range")
        if np.bincount(flat, minlength=d).max(initial=0) != 1 or flat.size != d:
            raise ValueError(f"stage {t}: not a perfect pairing")
        if np.any(pairs[t, :, 0] // group != pairs[t, :, 1] // group):
            raise ValueError(f"stage {t}: a pair crosses a group boundary")
    if not np.all(np.isfinite(theta)):
        raise ValueError("theta must be finite")
    if not (np.all(np.isfinite(alpha)) and np.all(alpha > 0)):
        raise ValueError("alpha must be finite and positive")


def cos_sin_f32(theta):
    """fp32 rounding of the fp64 cosine and sine of each angle (reading S10)."""
    t64 = np.asarray(theta, dtype=np.float32).astype(np.float64)
    return np.cos(t64).astype(np.float32), np.sin(t64).astype(np.float32)


def _apply_stages(v, pairs, c, s):
    """Apply the K independent-rotation stages to the last axis of ``v`` in place.

    [Notes] "关键设计" / [CSDN] §2.2: for each pair (i, j) of stage t,
    (v_i, v_j) <- (c v_i - s v_j, s v_i + c v_j). Pairs of one stage are
    channel-disjoint, so the whole stage is one vectorised update. The dtype of
    ``v``, ``c`` and ``s`` fixes the precision; numpy rounds each product and
    each difference separately.
    """
    for t in range(pairs.shape[0]):
        i = pairs[t, :, 0]
        j = pairs[t, :, 1]
        a = v[..., i]
        b = v[..., j]
        v[..., i] = c[t] * a - s[t] * b
        v[..., j] = s[t] * a + c[t] * b
    return v


# ----------------------------------------------------------------------------
# Online activation transform  X' = X T^-1
# ----------------------------------------------------------------------------

def rotate_activations(x, pairs, theta, alpha):
    """X' = X * T^-1 in fp64 for T = R_K ... R_1 diag(alpha).

    [CSDN] §2.1 (the equivalence rewrite) and [Notes] "关键设计" (the form
    of T). With T^-1 = diag(alpha)^-1 R_1^T ... R_K^T, a row vector x becomes
    ((x / alpha) R_1^T) R_2^T ..., and x R^T applies R's own pair update to x.
    Input fp16 (or any float) [M][d]; output fp64 [M][d], not rounded.
    """
    v = np.asarray(x).astype(np.float64) / np.asarray(alpha, dtype=np.float32).astype(np.float64)
    t64 = np.asarray(theta, dtype=np.float32).astype(np.float64)
    return _apply_stages(v, np.asarray(pairs), np.cos(t64), np.sin(t64))


# ----------------------------------------------------------------------------
# Gradients of the transform (transform learning)
# ----------------------------------------------------------------------------

def rotation_backward(x, g, pairs, theta, alpha, side="activation"):
    """Gradients of the transform with respect to its input, angles and scales (fp64).

    [Notes] "损失函数 / 训练策略": the angles and channel scales are learned by
    minimising the layer-wise output loss, which needs these gradients.

    The transform of one row r (a token of X, or a row of W in the [N][d]
    layout): v_0 = r / alpha (side "activation", X' = X T^-1) or r * alpha
    (side "weight", T W), then each stage t in order applies the pair update
    (v_i, v_j) <- (c v_i - s v_j, s v_i + c v_j). Given g = dL/d(output) for
    every row ([M][d]), returns, by the chain rule:
      dr      [M][d]    g walked back through every stage's transpose
                        (g_i, g_j) <- (c g_i + s g_j, -s g_i + c g_j), then
                        through the scaling (/ alpha or * alpha);
      dtheta  [K][d/2]  summed over rows: g'_j v'_i - g'_i v'_j, with v' the
                        stage's outputs and g' their gradient, because
                        d v'_i / d theta = -v'_j and d v'_j / d theta = v'_i;
      dalpha  [d]       summed over rows: g_0 * d v_0 / d alpha, which is
                        -v_0 / alpha for activations and r for weights.
    The forward values of every stage are kept (fp64), then the stages are
    walked back in reverse order.
    """
    if side not in ("activation", "weight"):
        raise ValueError("side is 'activation' or 'weight'")
    r = np.asarray(x).astype(np.float64)
    gy = np.asarray(g).astype(np.float64)
    a = np.asarray(alpha, dtype=np.float32).astype(np.float64)
    t64 = np.asarray(theta, dtype=np.float32).astype(np.float64)
    c, s = np.cos(t64), np.sin(t64)
    pairs = np.asarray(pairs)
    K = pairs.shape[0]
    d = a.shape[0]
    v0 = r / a if side == "activation" else r * a
    outs = []
    v = v0
    for t in range(K):
        i, j = pairs[t, :, 0], pairs[t, :, 1]
        vi, vj = v[..., i], v[..., j]
        v = v.copy()
        v[..., i] = c[t] * vi - s[t] * vj
        v[..., j] = s[t] * vi + c[t] * vj
        outs.append(v)
    gc = gy.copy()
    dtheta = np.zeros((K, d // 2))
    for t in reversed(range(K)):
        i, j = pairs[t, :, 0], pairs[t, :, 1]
        gi, gj = gc[..., i], gc[..., j]
        dtheta[t] = (gj * outs[t][..., i] - gi * outs[t][..., j]).reshape(-1, d // 2).sum(axis=0)
        gc = gc.copy()
        gc[..., i] = c[t] * gi + s[t] * gj
        gc[..., j] = -s[t] * gi + c[t] * gj
    if side == "activation":
        dr = gc / a
        dalpha = -(gc * v0 / a).reshape(-1, d).sum(axis=0)
    else:
        dr = gc * a
        dalpha = (gc * r).reshape(-1, d).sum(axis=0)
    return dr, dtheta, dalpha


# ----------------------------------------------------------------------------
# Offline weight transform  T W
# ----------------------------------------------------------------------------

def transform_weights_f64(w, pairs, theta, alpha):
    """T * W_math in fp64, returned in the [N][d] layout (no rounding).

    [Notes] "关键设计": scale the input channels by alpha, then apply the K
    stages in order. W is stored [N][d] (nn.Linear), the transpose of the
    math W, so channel k is column k.
    """
    u = np.asarray(w).astype(np.float64) * np.asarray(alpha, dtype=np.float32).astype(np.float64)
    t64 = np.asarray(theta, dtype=np.float32).astype(np.float64)
    return _apply_stages(u, np.asarray(pairs), np.cos(t64), np.sin(t64))


def transform_weights_f32(w, pairs, theta, alpha):
    """T * W_math in the canonical fp32 order of operations ([N][d] layout).

    u_k = fl(w_k * alpha_k); per pair a = u_i, b = u_j;
    u_i = fl(fl(c a) - fl(s b)); u_j = fl(fl(s a) + fl(c b)), with the fp32
    c, s of ``cos_sin_f32``. This order is the bit-exact contract that decides
    the int4 codes.
    """
    u = np.asarray(w).astype(np.float32) * np.asarray(alpha, dtype=np.float32)
    c, s = cos_sin_f32(theta)
    return _apply_stages(u, np.asarray(pairs), c, s)


# ----------------------------------------------------------------------------
# W4G128 quantization (canonical fp32)
# ----------------------------------------------------------------------------

def quantize_groups(u, group):
    """Asymmetric round-to-nearest int4 quantization per group of ``group`` inputs.

    [Notes] "损失函数 / 训练策略" (per-group scale s and zero z) and "主实验"
    (W4G128). For each row and group, in fp32:
      mn = min(0, min u), mx = max(0, max u)
      s32 = fl(fl(mx - mn) / 15); s16 = fp16 round-to-nearest-even of s32
      s16 == 0 -> 1.0; s16 infinite or NaN -> QuantizeError
      z = clamp(rint(fl(-mn / s16)), 0, 15)
      q = clamp(rint(fl(u / s16)) + z, 0, 15)        (rint: ties to even)
    Returns codes uint8 [N][d] (unpacked), scales fp16 [N][d/G],
    zeros uint8 [N][d/G].
    """
    u = np.asarray(u, dtype=np.float32)
    N, d = u.shape
    if d % group:
        raise ValueError("group must divide d")
    if not np.all(np.isfinite(u)):
        raise QuantizeError("non-finite transformed weight")
    ug = u.reshape(N, d // group, group)
    zero = np.float32(0.0)
    mn = np.minimum(ug.min(axis=2), zero)
    mx = np.maximum(ug.max(axis=2), zero)
    s32 = (mx - mn) / np.float32(15.0)
    with np.errstate(over="ignore"):
        s16 = s32.astype(np.float16)
    if not np.all(np.isfinite(s16)):
        raise QuantizeError("group scale overflows fp16")
    s16 = np.where(s16 == 0, np.float16(1.0), s16)
    sq = s16.astype(np.float32)
    z = np.clip(np.rint((-mn) / sq), 0, 15)
    q = np.clip(np.rint(ug / sq[:, :, None]) + z[:, :, None], 0, 15)
    return (q.astype(np.uint8).reshape(N, d), s16.astype(np.float16),
            z.astype(np.uint8))


def pack_codes(codes):
    """Eight codes per 32-bit little-endian word, split by parity (reading R8):
    a word covers channels 8w .. 8w + 7; its low 16 bits hold the even
    channels 8w, 8w+2, 8w+4, 8w+6 and its high 16 bits the odd channels
    8w+1, 8w+3, 8w+5, 8w+7, four bits each in increasing channel order. So
    byte 0 = c0 | c2 << 4, byte 1 = c4 | c6 << 4, byte 2 = c1 | c3 << 4,
    byte 3 = c5 | c7 << 4 (c_i the code of channel 8w + i). The row length
    must be a multiple of 8."""
    codes = np.asarray(codes, dtype=np.uint8)
    N, d = codes.shape
    if d % 8:
        raise ValueError("the row length must be a multiple of 8")
    c = codes.reshape(N, d // 8, 8)
    out = np.empty((N, d // 8, 4), dtype=np.uint8)
    out[:, :, 0] = c[:, :, 0] | (c[:, :, 2] << 4)
    out[:, :, 1] = c[:, :, 4] | (c[:, :, 6] << 4)
    out[:, :, 2] = c[:, :, 1] | (c[:, :, 3] << 4)
    out[:, :, 3] = c[:, :, 5] | (c[:, :, 7] << 4)
    return out.reshape(N, d // 2)


def unpack_codes(qweight):
    """Inverse of ``pack_codes``."""
    qweight = np.asarray(qweight, dtype=np.uint8)
    N = qweight.shape[0]
    b = qweight.reshape(N, -1, 4)
    out = np.empty((N, b.shape[1], 8), dtype=np.uint8)
    out[:, :, 0], out[:, :, 2] = b[:, :, 0] & 0x0F, b[:, :, 0] >> 4
    out[:, :, 4], out[:, :, 6] = b[:, :, 1] & 0x0F, b[:, :, 1] >> 4
    out[:, :, 1], out[:, :, 3] = b[:, :, 2] & 0x0F, b[:, :, 2] >> 4
    out[:, :, 5], out[:, :, 7] = b[:, :, 3] & 0x0F, b[:, :, 3] >> 4
    return out.reshape(N, -1)


def dequantize(qweight, scales, zeros, group):
    """W_hat[n][k] = (q - z) * s in fp64 (exact: |q - z| <= 15, s is fp16)."""
    q = unpack_codes(qweight).astype(np.float64)
    N, d = q.shape
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)
    z = np.asarray(zeros, dtype=np.uint8).astype(np.float64)
    qg = q.reshape(N, d // group, group)
    return ((qg - z[:, :, None]) * s[:, :, None]).reshape(N, d)


def quantize_weights(w, group, pairs=None, theta=None, alpha=None):
    """Q(T W) for a rotated layer, or Q(W) when no rotation is given.

    Returns (qweight uint8 [N][d/2], scales fp16 [N][d/G], zeros uint8 [N][d/G]).
    """
    if pairs is None:
        u = np.asarray(w).astype(np.float32)
    else:
        u = transform_weights_f32(w, pairs, theta, alpha)
    codes, s16, z = quantize_groups(u, group)
    return pack_codes(codes), s16, z


# ----------------------------------------------------------------------------
# The linear layer
# ----------------------------------------------------------------------------

def linear(xr, qweight, scales, zeros, group, bias=None):
    """Y = X' * W_hat^T + b in fp64 ([CSDN] §2.1, the right-hand side).

    ``xr`` is the (unrounded) rotated activation [M][d]; the product is a plain
    fp64 matrix product.
    """
    w_hat = dequantize(qweight, scales, zeros, group)
    y = np.asarray(xr, dtype=np.float64) @ w_hat.T
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float16).astype(np.float64)[None, :]
    return y


def rotated_w4_linear(x, qweight, scales, zeros, group, pairs=None, theta=None, alpha=None,
                      bias=None):
    """The whole online path: rotate X (if a rotation is given), then the W4 linear."""
    if pairs is None:
        xr = np.asarray(x).astype(np.float64)
    else:
        xr = rotate_activations(x, pairs, theta, alpha)
    return linear(xr, qweight, scales, zeros, group, bias)


# ----------------------------------------------------------------------------
# Layer-wise output loss (transform learning)
# ----------------------------------------------------------------------------

def layer_loss(x, w, qweight, scales, zeros, group, pairs, theta, alpha, grad=False):
    """Layer-wise output loss of the quantized, transformed layer, and its
    gradients with respect to the angles and scales (fp64, no rounding).

    [Notes] "损失函数 / 训练策略": L = ||Q(D)(X') - D(X)||, here the squared
    Frobenius norm L = sum (Y_q - Y)^2 with D(X) = X W^T the layer in its
    original fp16 weights and Q(D)(X') = X' W_hat^T the 4-bit layer on the
    transformed activations (X' = X T^-1 unrounded, W_hat the exactly
    dequantized Q(T W)). Every product and sum is fp64.

    Gradients (grad=True) pass through the quantizer unchanged (the
    straight-through reading of training through Q): see
    ``layer_loss_gradients``. Returns L, or (L, dtheta [K][d/2], dalpha [d]).
    """
    xr = rotate_activations(x, pairs, theta, alpha)
    what = dequantize(qweight, scales, zeros, group)
    yq = xr @ what.T
    y = np.asarray(x).astype(np.float64) @ np.asarray(w).astype(np.float64).T
    diff = yq - y
    loss = float(np.sum(diff * diff))
    if not grad:
        return loss
    dth, dal = layer_loss_gradients(x, w, xr, what, 2.0 * diff, pairs, theta, alpha)
    return loss, dth, dal


def layer_loss_gradients(x, w, xr, what, dy, pairs, theta, alpha):
    """Straight-through angle and scale gradients of the layer loss for a given
    dL/dY_q = ``dy`` [M][N] (fp64; linear in ``dy``).

    dL/dX' = dY W_hat and dL/dW_hat = dY^T X', the latter taken as dL/d(T W);
    then each transform's own gradients (``rotation_backward``: activation side
    for X', weight side for T W), summed. ``xr`` is the unrounded X' and
    ``what`` the dequantized weights [N][d]. Returns (dtheta [K][d/2], dalpha [d]).
    """
    dy = np.asarray(dy, dtype=np.float64)
    _, dth_a, dal_a = rotation_backward(x, dy @ what, pairs, theta, alpha, "activation")
    _, dth_w, dal_w = rotation_backward(w, dy.T @ xr, pairs, theta, alpha, "weight")
    return dth_a + dth_w, dal_a + dal_w
