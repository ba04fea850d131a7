"""Pins for the CPU oracle: closed forms, brute force, invariants, worked examples.

Each test pins the oracle to something other than itself: the pages' 2x2
Givens matrix, a dense-matrix construction of T taken literally from the
notes' formula, a signed Walsh-Hadamard closed form, exact-arithmetic round
trips of the quantizer, and hand-worked examples under tests/golden/.
"""
import os

import numpy as np
import pytest

import oracle
import synthetic
from oracle import metrics

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def dense_stage(d, pairs_t, theta_t):
    """Dense d x d matrix of one stage, from the 2x2 matrix [[c, -s], [s, c]]
    acting on (v_i, v_j) (CSDN article, section 2.2)."""
    R = np.eye(d)
    for (i, j), th in zip(pairs_t, theta_t.astype(np.float64)):
        c, s = np.cos(th), np.sin(th)
        R[i, i], R[i, j], R[j, i], R[j, j] = c, -s, s, c
    return R


def dense_T(pairs, theta, alpha):
    """T = R_K ... R_1 diag(alpha), stage 0 applied first (the notes' final transform)."""
    d = alpha.shape[0]
    T = np.diag(alpha.astype(np.float64))
    for t in range(pairs.shape[0]):
        T = dense_stage(d, pairs[t], theta[t]) @ T
    return T


def small_case(seed, M=5, d=32, G=8, K=3, N=6):
    rng = synthetic.rng_for(99, seed)
    x = synthetic.draw_x(rng, M, d, 2, 20.0)
    w = synthetic.draw_w(rng, N, d, 0.02)
    pairs, theta, alpha = synthetic.draw_rotation(rng, d, G, K)
    return x, w, pairs, theta, alpha


# ----------------------------------------------------------------------------
# P1-P7: the rotation
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_p4_bruteforce_dense_T(seed):
    """Structured oracle == dense T built literally from the pages' definition."""
    x, w, pairs, theta, alpha = small_case(seed)
    T = dense_T(pairs, theta, alpha)
    # weight side: T * W_math, W_math = w^T; our layout returns (T W_math)^T
    tw = oracle.transform_weights_f64(w, pairs, theta, alpha)
    np.testing.assert_allclose(tw, (T @ w.astype(np.float64).T).T, rtol=0, atol=1e-13)
    # activation side: X T^-1 by a linear solve of the dense matrix
    xr = oracle.rotate_activations(x, pairs, theta, alpha)
    ref = np.linalg.solve(T.T, x.astype(np.float64).T).T
    np.testing.assert_allclose(xr, ref, rtol=0, atol=1e-12 * np.abs(ref).max())
    # with alpha = 1, T is orthogonal
    T1 = dense_T(pairs, theta, np.ones_like(alpha))
    np.testing.assert_allclose(T1.T @ T1, np.eye(T1.shape[0]), atol=1e-13)


def test_p1_norm_preserved_per_group():
    x, w, pairs, theta, alpha = small_case(7, M=9, d=64, G=16, K=8)
    ones = np.ones_like(alpha)
    xr = oracle.rotate_activations(x, pairs, theta, ones)
    x64 = x.astype(np.float64)
    n0 = np.linalg.norm(x64.reshape(9, 4, 16), axis=2)
    n1 = np.linalg.norm(xr.reshape(9, 4, 16), axis=2)
    np.testing.assert_allclose(n1, n0, rtol=1e-14 * 8)
    # and each stage alone is orthogonal
    for t in range(8):
        R = dense_stage(64, pairs[t], theta[t])
        np.testing.assert_allclose(R.T @ R, np.eye(64), atol=1e-15)


def test_p2_inverse_returns_input():
    """Applying stages K-1..0 with -theta and then multiplying by alpha undoes X T^-1."""
    x, w, pairs, theta, alpha = small_case(3, K=8)
    xr = oracle.rotate_activations(x, pairs, theta, alpha)
    back = oracle.rotate_activations(xr, pairs[::-1].copy(), -theta[::-1].copy(),
                                     np.ones_like(alpha)) * alpha.astype(np.float64)
    np.testing.assert_allclose(back, x.astype(np.float64), rtol=0,
                               atol=1e-13 * np.abs(x.astype(np.float64)).max())


def test_p3_invariance_xw():
    """(X T^-1)(T W) = X W before quantization (CSDN article, section 2.1)."""
    x, w, pairs, theta, alpha = small_case(4, M=7, d=64, G=16, K=8, N=10)
    lhs = oracle.rotate_activations(x, pairs, theta, alpha) @ \
        oracle.transform_weights_f64(w, pairs, theta, alpha).T
    rhs = x.astype(np.float64) @ w.astype(np.float64).T
    np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-12 * np.abs(rhs).max())


def test_p5_walsh_hadamard_closed_form():
    """G = 2^k, stage t pairs (a, a + 2^t), theta = pi/4: T = signed Walsh-Hadamard / sqrt(G)."""
    k = 5
    G = 1 << k
    d = 2 * G  # two groups: the second gets the same structure shifted by G
    pairs = np.zeros((k, d // 2, 2), np.int32)
    for t in range(k):
        lo = [a for a in range(G) if not (a >> t) & 1]
        for g in range(2):
            for p, a in enumerate(lo):
                pairs[t, g * (G // 2) + p] = (g * G + a, g * G + a + (1 << t))
    theta = np.full((k, d // 2), np.float32(np.pi / 4), np.float32)
    # the fp32 angle is not exactly pi/4: use its own cos/sin in the closed form
    th = np.float64(np.float32(np.pi / 4))
    c, s = np.cos(th), np.sin(th)
    alpha = np.ones(d, np.float32)
    Tg = np.empty((G, G))
    for a in range(G):
        for b in range(G):
            v = 1.0
            for t in range(k):
                ab, bb = (a >> t) & 1, (b >> t) & 1
                v *= {(0, 0): c, (0, 1): -s, (1, 0): s, (1, 1): c}[(ab, bb)]
            Tg[a, b] = v
    # the exact pi/4 case is the popcount sign pattern
    sign = np.array([[(-1) ** bin(~a & b & (G - 1)).count("1") for b in range(G)] for a in range(G)])
    np.testing.assert_allclose(Tg, sign / np.sqrt(G), atol=1e-6)
    eye = np.eye(d, dtype=np.float16)
    # activation side with X = I: X' = T^-1 = T^T
    xr = oracle.rotate_activations(eye, pairs, theta, alpha)
    for g in range(2):
        blk = xr[g * G:(g + 1) * G, g * G:(g + 1) * G]
        np.testing.assert_allclose(blk, Tg.T, rtol=0, atol=1e-13)
    # weight side with W = I: the [N][d] result is (T W_math)^T = T^T
    tw = oracle.transform_weights_f64(eye, pairs, theta, alpha)
    np.testing.assert_allclose(tw[:G, :G], Tg.T, rtol=0, atol=1e-13)
    assert np.all(xr[:G, G:] == 0) and np.all(xr[G:, :G] == 0)


def test_hadamard_golden_g4():
    rows = [list(map(float, ln.split())) for ln in open(os.path.join(GOLDEN, "hadamard_g4.txt"))
            if ln.strip() and not ln.startswith("#")]
    T = np.array(rows) / 2.0
    pairs = np.array([[[0, 1], [2, 3]], [[0, 2], [1, 3]]], np.int32)
    theta = np.full((2, 2), np.pi / 4, np.float32)
    alpha = np.ones(4, np.float32)
    xr = oracle.rotate_activations(np.eye(4, dtype=np.float16), pairs, theta, alpha)
    np.testing.assert_allclose(xr, T.T, atol=1e-7)
    tw = oracle.transform_weights_f64(np.eye(4, dtype=np.float16), pairs, theta, alpha)
    np.testing.assert_allclose(tw, T.T, atol=1e-7)
    # canonical fp32 path agrees to fp32 precision
    tw32 = oracle.transform_weights_f32(np.eye(4, dtype=np.float16), pairs, theta, alpha)
    np.testing.assert_allclose(tw32, T.T, atol=1e-6)


def test_p6_sign_convention_quarter_turn():
    """One pair (i, j) = (1, 3), theta = pi/2: e_i -> e_j and e_j -> -e_i."""
    d = 4
    pairs = np.array([[[1, 3], [0, 2]]], np.int32)
    theta = np.array([[np.pi / 2, 0.0]], np.float32)
    alpha = np.ones(d, np.float32)
    xr = oracle.rotate_activations(np.eye(d, dtype=np.float16), pairs, theta, alpha)
    np.testing.assert_allclose(xr[1], [0, 0, 0, 1], atol=1e-7)
    np.testing.assert_allclose(xr[3], [0, -1, 0, 0], atol=1e-7)
    np.testing.assert_allclose(xr[0], [1, 0, 0, 0], atol=0)
    # swapping the stored order of a pair is the same as negating its angle
    pairs2 = pairs.copy()
    pairs2[0, 0] = [3, 1]
    theta2 = theta.copy()
    theta2[0, 0] = -theta[0, 0]
    x = synthetic.draw_x(synthetic.rng_for(99, 50), 3, d, 0)
    np.testing.assert_allclose(oracle.rotate_activations(x, pairs2, theta2, alpha),
                               oracle.rotate_activations(x, pairs, theta, alpha), atol=1e-15)


def test_p7_k0_is_channel_scaling():
    x, w, pairs, theta, alpha = small_case(5)
    p0 = pairs[:0]
    t0 = theta[:0]
    np.testing.assert_array_equal(oracle.rotate_activations(x, p0, t0, alpha),
                                  x.astype(np.float64) / alpha.astype(np.float64))
    np.testing.assert_array_equal(oracle.transform_weights_f32(w, p0, t0, alpha),
                                  w.astype(np.float32) * alpha)


def test_fp32_transform_matches_scalar_loop_and_f64():
    """Canonical fp32 transform: vectorised == scalar loop bit for bit; close to fp64."""
    x, w, pairs, theta, alpha = small_case(6, d=16, G=8, K=4, N=3)
    got = oracle.transform_weights_f32(w, pairs, theta, alpha)
    f32 = np.float32
    ref = np.empty_like(got)
    for n in range(w.shape[0]):
        u = [f32(w[n, k]) * f32(alpha[k]) for k in range(16)]
        for t in range(4):
            for (i, j), th in zip(pairs[t], theta[t]):
                c = f32(np.cos(np.float64(th)))
                s = f32(np.sin(np.float64(th)))
                a, b = u[i], u[j]
                u[i] = f32(f32(c * a) - f32(s * b))
                u[j] = f32(f32(s * a) + f32(c * b))
        ref[n] = u
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))
    f64 = oracle.transform_weights_f64(w, pairs, theta, alpha)
    np.testing.assert_allclose(got, f64, rtol=0, atol=1e-6 * np.abs(f64).max())


def test_param_validation():
    d, G = 16, 8
    pairs, theta, alpha = synthetic.draw_rotation(synthetic.rng_for(99, 9), d, G, 2)
    oracle.check_rotation_params(pairs, theta, alpha, G)
    bad = pairs.copy()
    bad[0, 0, 1] = bad[0, 1, 0]  # duplicate channel
    with pytest.raises(ValueError):
        oracle.check_rotation_params(bad, theta, alpha, G)
    cross = pairs.copy()
    # swap one member between the two groups -> crosses a group
    a = cross[1, 0, 0]
    b = cross[1, G // 2, 0]
    cross[1, 0, 0], cross[1, G // 2, 0] = b, a
    with pytest.raises(ValueError):
        oracle.check_rotation_params(cross, theta, alpha, G)
    with pytest.raises(ValueError):
        oracle.check_rotation_params(pairs, theta, -alpha, G)


# ----------------------------------------------------------------------------
# R1-R6: the quantizer
# ----------------------------------------------------------------------------

def read_quant_golden():
    path = os.path.join(os.path.dirname(__file__), "golden", "quantize_worked.txt")
    cases, packed = [], None
    for ln in open(path):
        ln = ln.strip()
        if not ln or ln.startswith("#"):
            continue
        if ln.startswith("packed"):
            packed = bytes(int(b, 16) for b in ln.split()[1:])
            continue
        u, sz, q = [p.split() for p in ln.split("|")]
        cases.append((np.array(u, np.float32), int(sz[0], 16), int(sz[1]), np.array(q, np.uint8)))
    return cases, packed


def test_quantize_worked_examples():
    cases, packed = read_quant_golden()
    assert len(cases) == 6
    for u, s_bits, z, q in cases:
        codes, s16, zeros = oracle.quantize_groups(u[None, :], 4)
        assert int(s16.view(np.uint16)[0, 0]) == s_bits
        assert int(zeros[0, 0]) == z
        np.testing.assert_array_equal(codes[0], q)
    # all six as one row of six groups, packed by hand
    row = np.concatenate([c[0] for c in cases])[None, :]
    codes, s16, zeros = oracle.quantize_groups(row, 4)
    assert oracle.pack_codes(codes)[0].tobytes() == packed


def test_r1_r2_r3_on_random_groups():
    rng = synthetic.rng_for(99, 11)
    w = synthetic.draw_w(rng, 64, 512, 0.02, n_outlier_cols=5, factor=10.0)
    pairs, theta, alpha = synthetic.draw_rotation(rng, 512, 128, 8)
    u = oracle.transform_weights_f32(w, pairs, theta, alpha)
    codes, s16, z = oracle.quantize_groups(u, 128)
    sq = s16.astype(np.float64)
    assert codes.max() <= 15 and z.max() <= 15
    ug = u.reshape(64, 4, 128).astype(np.float64)
    qg = codes.reshape(64, 4, 128).astype(np.float64)
    # R1: the minimum maps to code 0 when negative; otherwise the maximum is 15
    neg = ug.min(axis=2) < 0
    assert np.all(np.where(neg, qg.min(axis=2) == 0, qg.max(axis=2) == 15))
    # R2: reconstruction error <= (0.5 + 15 * 2^-11) * s
    rec = (qg - z[:, :, None]) * sq[:, :, None]
    bound = (0.5 + 15 * 2.0 ** -11) * sq[:, :, None] * (1 + 1e-6)
    assert np.all(np.abs(ug - rec) <= bound)
    # R3: each code is the nearest of the 16 grid points (up to the fp32 quotient's rounding)
    grid = (np.arange(16)[None, None, None, :] - z[:, :, None, None]) * sq[:, :, None, None]
    dist = np.abs(ug[..., None] - grid)
    mine = np.take_along_axis(dist, qg.astype(np.int64)[..., None], axis=3)[..., 0]
    assert np.all(mine <= dist.min(axis=3) + np.abs(ug) * 2.0 ** -22 + 1e-30)


def test_r4_grid_aligned_round_trip():
    rng = synthetic.rng_for(99, 12)
    N, d, G = 40, 256, 128
    s16 = np.abs(rng.standard_normal((N, d // G)) * 0.01).astype(np.float16)
    s16 = np.where(s16 < np.float16(1e-3), np.float16(1e-3), s16).astype(np.float16)
    z = rng.integers(0, 16, size=(N, d // G)).astype(np.uint8)
    q = rng.integers(0, 16, size=(N, d // G, G)).astype(np.uint8)
    q[:, :, 0] = 0
    q[:, :, 1] = 15
    u = ((q.astype(np.float32) - z[:, :, None].astype(np.float32)) *
         s16[:, :, None].astype(np.float32)).reshape(N, d)
    codes, s_out, z_out = oracle.quantize_groups(u, G)
    np.testing.assert_array_equal(s_out.view(np.uint16), s16.view(np.uint16))
    np.testing.assert_array_equal(z_out, z)
    np.testing.assert_array_equal(codes, q.reshape(N, d))


def test_r5_packing_and_one_hot_linear():
    rng = synthetic.rng_for(99, 13)
    codes = rng.integers(0, 16, size=(7, 32)).astype(np.uint8)
    packed = oracle.pack_codes(codes)
    np.testing.assert_array_equal(oracle.unpack_codes(packed), codes)
    # word layout: even channels in the low half, odd channels in the high half
    word = oracle.pack_codes(np.array([[1, 2, 3, 4, 5, 6, 7, 8]], np.uint8))[0].view("<u4")[0]
    assert word == 0x86427531
    # one-hot activations read out single dequantized weights plus the bias
    scales = (rng.random((7, 2)) * 0.1 + 0.01).astype(np.float16)
    zeros = rng.integers(0, 16, size=(7, 2)).astype(np.uint8)
    bias = rng.standard_normal(7).astype(np.float16)
    y = oracle.linear(np.eye(32), packed, scales, zeros, 16, bias)
    for k in range(32):
        for n in range(7):
            g = k // 16
            want = (int(codes[n, k]) - int(zeros[n, g])) * float(scales[n, g]) + float(bias[n])
            assert y[k, n] == want


def test_r6_zero_angles_equal_k0_codes():
    rng = synthetic.rng_for(99, 14)
    w = synthetic.draw_w(rng, 16, 256, 0.02)
    pairs, theta, alpha = synthetic.draw_rotation(rng, 256, 128, 8)
    zero = np.zeros_like(theta)
    a = oracle.quantize_weights(w, 128, pairs, zero, alpha)
    b = oracle.quantize_weights(w, 128, pairs[:0], theta[:0], alpha)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x.view(np.uint8), y.view(np.uint8))
    c, s = oracle.cos_sin_f32(zero)
    assert np.all(c == 1) and np.all(s == 0)


def test_quantizer_degenerate_and_overflow():
    codes, s16, z = oracle.quantize_groups(np.zeros((2, 8), np.float32), 4)
    assert np.all(codes == 0) and np.all(z == 0) and np.all(s16 == 1.0)
    with pytest.raises(oracle.QuantizeError):
        oracle.quantize_groups(np.array([[1e6, -1e6, 0, 0]], np.float32), 4)
    with pytest.raises(oracle.QuantizeError):
        oracle.quantize_groups(np.array([[np.inf, 0, 0, 0]], np.float32), 4)


# ----------------------------------------------------------------------------
# L1-L2: the linear
# ----------------------------------------------------------------------------

def test_l1_linear_against_python_loops():
    rng = synthetic.rng_for(99, 15)
    M, N, d, G = 3, 5, 32, 16
    x = rng.standard_normal((M, d))
    codes = rng.integers(0, 16, size=(N, d)).astype(np.uint8)
    qweight = oracle.pack_codes(codes)
    scales = (rng.random((N, 2)) * 0.1 + 0.01).astype(np.float16)
    zeros = rng.integers(0, 16, size=(N, 2)).astype(np.uint8)
    bias = rng.standard_normal(N).astype(np.float16)
    y = oracle.linear(x, qweight, scales, zeros, G, bias)
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(d):
                acc += x[m, k] * (int(codes[n, k]) - int(zeros[n, k // G])) * float(scales[n, k // G])
            assert abs(y[m, n] - (acc + float(bias[n]))) <= 1e-12 * (1 + abs(acc))


def test_l2_codes_equal_zero_give_bias():
    N, d, G = 4, 256, 128
    zeros = np.arange(N * 2, dtype=np.uint8).reshape(N, 2) % 16
    codes = np.repeat(zeros, G, axis=1)
    qweight = oracle.pack_codes(codes)
    scales = np.full((N, 2), 0.37, np.float16)
    bias = np.array([1.5, -2.0, 0.25, 3.0], np.float16)
    x = synthetic.draw_x(synthetic.rng_for(99, 16), 3, d, 2)
    y = oracle.linear(x.astype(np.float64), qweight, scales, zeros, G, bias)
    np.testing.assert_array_equal(y, np.broadcast_to(bias.astype(np.float64), (3, N)))


def test_tiny_end_to_end_is_close_to_unquantized():
    """Sanity: the quantized rotated layer approximates X W^T (not a pin)."""
    x, layer = synthetic.tiny()
    qw, s, z = oracle.quantize_weights(layer.w, 128, layer.pairs, layer.theta, layer.alpha)
    y = oracle.rotated_w4_linear(x, qw, s, z, 128, layer.pairs, layer.theta, layer.alpha)
    ref = x.astype(np.float64) @ layer.w.astype(np.float64).T
    fro, _ = metrics.linear_error(y, ref)
    # random (untrained) angles spread the x10 outlier columns over whole groups,
    # so int4 error is large; this only guards against gross breakage
    assert fro < 0.5


def test_metrics_floor():
    ref = np.array([[1.0, 1e-9, -2.0, 0.5]])
    got = ref + np.array([[1e-4, 1e-6, 0, 0]])
    fl, raw, n = metrics.rotated_error(got, ref, 4)
    assert raw > 1 and fl < 2e-3
    # gradients: relative to each entry, floored at the rms of the output
    ref = np.array([300.0, 1.0, -1.0, 1e-12])
    rms = np.sqrt(np.mean(ref * ref))
    assert np.isclose(metrics.grad_error(ref + [3e-3, 0, 0, 0], ref), 1e-5)
    assert np.isclose(metrics.grad_error(ref + [0, 0, 0, 1e-3 * rms], ref), 1e-3)
    assert metrics.grad_error(np.zeros(0), np.zeros(0)) == 0.0


# ----------------------------------------------------------------------------
# B1-B4: gradients of the transform (transform learning)
# ----------------------------------------------------------------------------

def grid_params(seed, d, G, K):
    """Rotation parameters on coarse binary grids (theta = k / 64, alpha =
    1 + m / 64), so that theta +- 2^-9 and alpha +- 2^-9 stay exact in fp32,
    where the forward transforms round the parameters."""
    rng = synthetic.rng_for(98, seed)
    pairs = synthetic.draw_pairs(rng, d, G, K)
    theta = (rng.integers(-200, 201, size=(K, d // 2)) / 64.0).astype(np.float32)
    alpha = (1.0 + rng.integers(-16, 33, size=d) / 64.0).astype(np.float32)
    return pairs, theta, alpha


def forward(side, x, pairs, theta, alpha):
    if side == "activation":
        return oracle.rotate_activations(x, pairs, theta, alpha)
    return oracle.transform_weights_f64(x, pairs, theta, alpha)


def richardson(f, h):
    """Central difference extrapolated from steps h and h/2 (error O(h^4))."""
    d1 = (f(h) - f(-h)) / (2 * h)
    d2 = (f(h / 2) - f(-h / 2)) / h
    return (4 * d2 - d1) / 3


@pytest.mark.parametrize("side", ["activation", "weight"])
def test_b1_gradients_match_finite_differences(side):
    """d theta and d alpha against finite differences of the forward transform
    (the scalar loss L = sum g * F), d input against the dense-matrix closed form
    (X' = X T^-1 gives dX = g T^-T; rows of T W give dW = g T)."""
    d, G, K, M = 16, 8, 3, 3
    pairs, theta, alpha = grid_params(1 if side == "activation" else 2, d, G, K)
    rng = synthetic.rng_for(97, 0)
    x = synthetic.draw_x(rng, M, d, 1, 5.0)
    g = rng.standard_normal((M, d))
    dr, dth, dal = oracle.rotation_backward(x, g, pairs, theta, alpha, side)

    def loss(th, al):
        return float(np.sum(g * forward(side, x, pairs, th, al)))

    h = 2.0 ** -8
    for t in range(K):
        for p in range(d // 2):
            def f(e, t=t, p=p):
                th = theta.copy()
                th[t, p] = np.float32(theta[t, p] + e)
                assert th[t, p] == theta[t, p] + e
                return loss(th, alpha)
            assert abs(richardson(f, h) - dth[t, p]) <= 1e-9 * (1 + abs(dth[t, p]))
    for k in range(d):
        def f(e, k=k):
            al = alpha.copy()
            al[k] = np.float32(alpha[k] + e)
            assert al[k] == alpha[k] + e
            return loss(theta, al)
        assert abs(richardson(f, h) - dal[k]) <= 1e-9 * (1 + abs(dal[k]))
    T = dense_T(pairs, theta, alpha)
    want = g @ np.linalg.inv(T).T if side == "activation" else g @ T
    assert np.allclose(dr, want, rtol=1e-12, atol=1e-12)


def test_b2_k0_is_the_scaling_gradient():
    """K = 0: dX = g / alpha and d alpha = -sum g x / alpha^2 for activations;
    dW = g alpha and d alpha = sum g w for weights."""
    rng = synthetic.rng_for(97, 1)
    d, M = 64, 4
    x = synthetic.draw_x(rng, M, d, 1, 5.0)
    g = rng.standard_normal((M, d))
    alpha = synthetic.draw_alpha(rng, d)
    pairs = np.zeros((0, d // 2, 2), np.int32)
    theta = np.zeros((0, d // 2), np.float32)
    a = alpha.astype(np.float64)
    xf = x.astype(np.float64)
    dr, dth, dal = oracle.rotation_backward(x, g, pairs, theta, alpha, "activation")
    assert dth.shape == (0, d // 2)
    assert np.allclose(dr, g / a, rtol=1e-15)
    assert np.allclose(dal, -(g * xf).sum(0) / a ** 2, rtol=1e-12)
    dr, _, dal = oracle.rotation_backward(x, g, pairs, theta, alpha, "weight")
    assert np.allclose(dr, g * a, rtol=1e-15)
    assert np.allclose(dal, (g * xf).sum(0), rtol=1e-12)


def test_b3_single_pair_closed_form():
    """One pair, one stage, alpha = 1: out = (c x1 - s x2, s x1 + c x2), so
    dL/dtheta = g1 (-s x1 - c x2) + g2 (c x1 - s x2) and dx = R^T g."""
    x = np.array([[0.75, -1.5]], np.float16)
    g = np.array([[0.3, -2.0]])
    th = np.float32(0.625)
    c, s = np.cos(np.float64(th)), np.sin(np.float64(th))
    pairs = np.array([[[0, 1]]], np.int32)
    dr, dth, dal = oracle.rotation_backward(x, g, pairs, np.array([[th]]), np.ones(2, np.float32))
    x1, x2 = 0.75, -1.5
    assert np.isclose(dth[0, 0], 0.3 * (-s * x1 - c * x2) + (-2.0) * (c * x1 - s * x2), rtol=1e-14)
    assert np.allclose(dr[0], [c * 0.3 + s * -2.0, -s * 0.3 + c * -2.0], rtol=1e-14)
    # d alpha at alpha = 1: -g_0 * x with g_0 = R^T g
    assert np.allclose(dal, -dr[0] * np.array([x1, x2]), rtol=1e-14)


def test_b4_weight_side_is_activation_side_with_inverse_scales():
    """r * alpha = r / (1 / alpha): with power-of-two scales (exact inverses),
    the weight side's dW and d theta equal the activation side's at 1 / alpha,
    and d alpha follows the chain rule d/d alpha = -(1 / alpha^2) d/d(1 / alpha)."""
    rng = synthetic.rng_for(97, 2)
    d, G, K, M = 128, 64, 4, 3
    w = synthetic.draw_w(rng, M, d, 0.5)
    g = rng.standard_normal((M, d))
    pairs, theta, _ = synthetic.draw_rotation(rng, d, G, K)
    alpha = (2.0 ** rng.integers(-2, 3, size=d)).astype(np.float32)
    inv = (1.0 / alpha).astype(np.float32)
    dw, dth_w, dal_w = oracle.rotation_backward(w, g, pairs, theta, alpha, "weight")
    dx, dth_a, dal_a = oracle.rotation_backward(w, g, pairs, theta, inv, "activation")
    assert np.allclose(dw, dx, rtol=1e-13, atol=1e-13)
    assert np.allclose(dth_w, dth_a, rtol=1e-12, atol=1e-12)
    assert np.allclose(dal_w, -dal_a / alpha.astype(np.float64) ** 2, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------
# L1-L2: the layer-wise output loss and its straight-through gradients
# ----------------------------------------------------------------------------

def test_l_loss_is_the_output_error_of_the_quantized_layer():
    """L = ||X' W_hat^T - X W^T||_F^2, and with K = 0 and alpha = 1 it is the
    plain W4 layer's squared output error."""
    rng = synthetic.rng_for(96, 0)
    d, N, M, G = 128, 16, 5, 64
    x = synthetic.draw_x(rng, M, d, 1, 5.0)
    w = synthetic.draw_w(rng, N, d, 0.05)
    pairs = np.zeros((0, d // 2, 2), np.int32)
    theta = np.zeros((0, d // 2), np.float32)
    alpha = np.ones(d, np.float32)
    q, s, z = oracle.quantize_weights(w, G)
    what = oracle.dequantize(q, s, z, G)
    want = np.sum((x.astype(np.float64) @ what.T - x.astype(np.float64) @ w.astype(np.float64).T) ** 2)
    got = oracle.layer_loss(x, w, q, s, z, G, pairs, theta, alpha)
    assert np.isclose(got, want, rtol=1e-12)


def test_l_gradients_match_finite_differences_with_frozen_quantization_error():
    """The straight-through gradients equal the exact gradients of the smooth
    surrogate L~(theta, alpha) = ||X'(theta, alpha) (T W + E0)^T - X W^T||^2,
    in which the quantization error E0 = W_hat - T W is frozen at the base
    point: checked against finite differences of L~ built from the forward
    transforms alone."""
    d, N, M, G, K = 16, 6, 4, 8, 2
    pairs, theta, alpha = grid_params(3, d, G, K)
    rng = synthetic.rng_for(96, 1)
    x = synthetic.draw_x(rng, M, d, 1, 5.0)
    w = synthetic.draw_w(rng, N, d, 0.3)
    q, s, z = oracle.quantize_weights(w, G, pairs, theta, alpha)
    e0 = oracle.dequantize(q, s, z, G) - oracle.transform_weights_f64(w, pairs, theta, alpha)
    y = x.astype(np.float64) @ w.astype(np.float64).T
    _, dth, dal = oracle.layer_loss(x, w, q, s, z, G, pairs, theta, alpha, grad=True)

    def surrogate(th, al):
        xr = oracle.rotate_activations(x, pairs, th, al)
        u = oracle.transform_weights_f64(w, pairs, th, al) + e0
        return float(np.sum((xr @ u.T - y) ** 2))

    h = 2.0 ** -8
    for t in range(K):
        for p in range(d // 2):
            def f(e, t=t, p=p):
                th = theta.copy()
                th[t, p] = np.float32(theta[t, p] + e)
                return surrogate(th, alpha)
            assert abs(richardson(f, h) - dth[t, p]) <= 1e-8 * (1 + abs(dth[t, p]))
    for k in range(d):
        def f(e, k=k):
            al = alpha.copy()
            al[k] = np.float32(alpha[k] + e)
            return surrogate(theta, al)
        assert abs(richardson(f, h) - dal[k]) <= 1e-8 * (1 + abs(dal[k]))


def test_l_gradient_is_the_activation_side_through_the_quantization_error():
    """X' (T W)^T = X W^T for every angle and scale, so the two sides' terms
    through T W cancel: the straight-through gradient equals the activation
    side's gradient for dX' = dY E, E = W_hat - T W."""
    x, layer, _ = synthetic.linear_case(seed=2, M=9, d=256, N=32, group=128, K=4, bias=False)
    q, s, z = oracle.quantize_weights(layer.w, 128, layer.pairs, layer.theta, layer.alpha)
    _, dth, dal = oracle.layer_loss(x, layer.w, q, s, z, 128, layer.pairs, layer.theta, layer.alpha,
                                    grad=True)
    xr = oracle.rotate_activations(x, layer.pairs, layer.theta, layer.alpha)
    what = oracle.dequantize(q, s, z, 128)
    dy = 2.0 * (xr @ what.T - x.astype(np.float64) @ layer.w.astype(np.float64).T)
    e = what - oracle.transform_weights_f64(layer.w, layer.pairs, layer.theta, layer.alpha)
    _, dth2, dal2 = oracle.rotation_backward(x, dy @ e, layer.pairs, layer.theta, layer.alpha)
    assert np.allclose(dth, dth2, rtol=1e-9, atol=1e-9 * np.abs(dth).max())
    assert np.allclose(dal, dal2, rtol=1e-9, atol=1e-9 * np.abs(dal).max())


def _fp16_device_layer_loss(x, w, q, s, z, G, layer):
    """The layer loss as the library documents its arithmetic, simulated in
    numpy: fp16 X' and dequantized weights, fp32 sums, fp16 Y_q, fp32 Y,
    dY = 2 (Y_q - Y), and dX' from fp16 dY and E = W_hat - T W with fp32 sums
    (T W in the canonical fp32 order). Used only to check that the derived
    tolerance covers that arithmetic."""
    f32, f16 = np.float32, np.float16
    xr16 = oracle.rotate_activations(x, layer.pairs, layer.theta, layer.alpha).astype(f16)
    what = oracle.dequantize(q, s, z, G)
    yq = (xr16.astype(f32) @ what.astype(f16).astype(f32).T).astype(f16).astype(f32)
    y = x.astype(f32) @ layer.w.astype(f32).T
    diff = yq - y
    loss = float(np.sum(diff.astype(np.float64) ** 2))
    tw32 = oracle.transform_weights_f32(layer.w, layer.pairs, layer.theta, layer.alpha)
    e16 = (what.astype(f32) - tw32).astype(f16)
    dy16 = (f32(2.0) * diff).astype(f16)
    dxr = dy16.astype(f32) @ e16.astype(f32)
    _, dth, dal = oracle.rotation_backward(x, dxr, layer.pairs, layer.theta, layer.alpha)
    return loss, dth, dal


@pytest.mark.parametrize("M,d,N,G,K,seed", [(24, 256, 64, 128, 8, 1), (9, 512, 48, 64, 4, 2),
                                            (40, 256, 32, 256, 8, 3)])
def test_l_tolerance_covers_fp16_arithmetic_and_rejects_mistakes(M, d, N, G, K, seed):
    """The derived layer-loss tolerance holds a numpy simulation of the
    device's documented roundings, and fails planted mistakes: a dropped
    rounding-free term of the loss, a flipped gradient sign, a gradient taken
    through W_hat instead of the quantization error, and a transposed pair."""
    x, layer, _ = synthetic.linear_case(seed=seed, M=M, d=d, N=N, group=G, K=K, bias=False)
    q, s, z = oracle.quantize_weights(layer.w, G, layer.pairs, layer.theta, layer.alpha)
    ref = oracle.layer_loss(x, layer.w, q, s, z, G, layer.pairs, layer.theta, layer.alpha, grad=True)
    tl, tth, tal = metrics.layer_loss_tolerance(x, layer.w, q, s, z, G, layer.pairs, layer.theta,
                                                layer.alpha)
    loss, dth, dal = _fp16_device_layer_loss(x, layer.w, q, s, z, G, layer)
    assert abs(loss - ref[0]) <= tl
    metrics.assert_within(dth, ref[1], tth, "dtheta")
    metrics.assert_within(dal, ref[2], tal, "dalpha")
    # the tolerance is far below the size of a structural mistake
    assert tl < 0.01 * ref[0]
    with pytest.raises(AssertionError):
        metrics.assert_within(-dal, ref[2], tal, "dalpha (sign)")
    what = oracle.dequantize(q, s, z, G)
    xr = oracle.rotate_activations(x, layer.pairs, layer.theta, layer.alpha)
    dy = 2.0 * (xr @ what.T - x.astype(np.float64) @ layer.w.astype(np.float64).T)
    _, wth, wal = oracle.rotation_backward(x, dy @ what, layer.pairs, layer.theta, layer.alpha)
    with pytest.raises(AssertionError):
        metrics.assert_within(wal, ref[2], tal, "dalpha (through W_hat)")
    swapped = layer.pairs[:, :, ::-1].copy()
    sth, _ = oracle.layer_loss_gradients(x, layer.w, xr, what, dy, swapped, layer.theta, layer.alpha)
    with pytest.raises(AssertionError):
        metrics.assert_within(sth, ref[1], tth, "dtheta (swapped pair)")


# ----------------------------------------------------------------------------
# S1-S6: choosing the channel pairs (oracle.pairs)
# ----------------------------------------------------------------------------

from oracle import pairs as opairs  # noqa: E402


def _golden(name):
    path = os.path.join(os.path.dirname(__file__), "golden", name)
    return [ln.split() for ln in open(path) if ln.strip() and not ln.startswith("#")]


def test_s1_splitmix64_reference_outputs():
    """The generator reproduces the published SplitMix64 outputs."""
    for row in _golden("splitmix64.txt"):
        rng = opairs.SplitMix64(int(row[0]))
        assert [rng.next() for _ in row[1:]] == [int(v) for v in row[1:]]


def test_s2_shuffle_is_uniform():
    """Fisher-Yates from SplitMix64 draws every permutation of 3 items equally
    often (chi-square over 60000 draws); the common mistake of drawing j from
    all n positions at every step gives frequencies 4/27 .. 5/27 and fails."""
    rng = opairs.SplitMix64(7)
    counts = {}
    n = 60000
    for _ in range(n):
        key = tuple(opairs.shuffle(rng, 3))
        counts[key] = counts.get(key, 0) + 1
    assert len(counts) == 6
    exp = n / 6
    chi2 = sum((c - exp) ** 2 / exp for c in counts.values())
    assert chi2 < 25.7  # 5 degrees of freedom, p = 1e-4


def _assert_valid_plan(p, d, G):
    theta = np.zeros(p.shape[:2], np.float32)
    oracle.check_rotation_params(p, theta, np.ones(d, np.float32), G)


def test_s3_random_pairs_never_repeat_and_complete_a_factorization():
    """Every stage is a perfect pairing inside the groups and no unordered pair
    occurs twice in a group; with G = 4 and K = 3 the three stages use each of
    the six pairs of the group exactly once (the one-factorization of K4)."""
    for d, G, K, seed in [(256, 128, 8, 1), (128, 64, 16, 2), (512, 256, 8, 3), (64, 8, 4, 4)]:
        p = opairs.pairs_random(d, G, K, seed)
        _assert_valid_plan(p, d, G)
        for g in range(d // G):
            sl = p[:, g * (G // 2):(g + 1) * (G // 2)].reshape(-1, 2)
            keys = {frozenset(map(int, r)) for r in sl}
            assert len(keys) == sl.shape[0]
    for seed in range(20):
        p = opairs.pairs_random(8, 4, 3, seed)
        for g in range(2):
            sl = p[:, 2 * g:2 * g + 2].reshape(-1, 2) - 4 * g
            assert sorted(tuple(sorted(map(int, r))) for r in sl) == \
                [(0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3)]


def test_s4_gap_pairs_hand_worked():
    rows = _golden("pairs_by_gap_g8.txt")
    cases = []
    for r in rows:
        if r[0] == "score":
            cases.append([np.array([float(v) for v in r[1:]], np.float32), []])
        else:
            cases[-1][1].append(np.array([int(v) for v in r[1:]]).reshape(4, 2))
    for score, stages in cases:
        p = opairs.pairs_by_gap(score, 8, len(stages))
        for t, want in enumerate(stages):
            assert np.array_equal(p[t], want), (t, p[t], want)


def _matchings(items):
    if not items:
        yield []
        return
    a = items[0]
    for k in range(1, len(items)):
        rest = items[1:k] + items[k + 1:]
        for m in _matchings(rest):
            yield [(a, items[k])] + m


def test_s5_gap_pairs_reach_the_largest_total_difference():
    """Brute force over all 105 perfect pairings of 8 channels: every stage's
    total |score_i - score_j| equals the largest any pairing reaches, and the
    stages' pairs are distinct."""
    rng = synthetic.rng_for(98, 0)
    for trial in range(5):
        s = rng.standard_normal(8).astype(np.float32)
        best = max(sum(abs(float(s[a]) - float(s[b])) for a, b in m) for m in _matchings(list(range(8))))
        p = opairs.pairs_by_gap(s, 8, 4)
        _assert_valid_plan(p, 8, 8)
        seen = set()
        for t in range(4):
            tot = sum(abs(float(s[a]) - float(s[b])) for a, b in p[t])
            assert abs(tot - best) <= 1e-6 * max(1.0, best)
            for a, b in p[t]:
                assert float(s[a]) >= float(s[b])
                key = frozenset((int(a), int(b)))
                assert key not in seen
                seen.add(key)


def test_s6_sparsify_keeps_the_largest_angles():
    """Brute force: the kept pairs are the n_keep largest |theta| (ties by
    position), with their angle unchanged; all others are 0."""
    theta = np.array([[0.5, -2.0, 0.1, 2.0], [-0.5, 3.0, 0.0, -0.1]], np.float32)
    got = opairs.sparsify_angles(theta, 4)
    assert np.array_equal(got, np.array([[0.5, -2.0, 0.0, 2.0], [0.0, 3.0, 0.0, 0.0]], np.float32))
    rng = synthetic.rng_for(98, 1)
    th = rng.uniform(-np.pi, np.pi, size=(3, 16)).astype(np.float32)
    th[1, 3] = th[0, 5]  # a tie
    for n in (0, 1, 7, 24, 48):
        got = opairs.sparsify_angles(th, n)
        flat = [(abs(float(v)), i) for i, v in enumerate(th.reshape(-1))]
        chosen = {i for _, i in sorted(flat, key=lambda e: (-e[0], e[1]))[:n]}
        for i, v in enumerate(got.reshape(-1)):
            assert v == (th.reshape(-1)[i] if i in chosen else 0.0)
