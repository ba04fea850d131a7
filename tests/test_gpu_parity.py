"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

* rotation: X' within the floored max relative error 2e-3 of the fp64 oracle;
* quantization: qweight, scales and zeros byte-for-byte equal to the oracle's
  canonical fp32 quantizer;
* linear: ||Y - Y_ref||_F / ||Y_ref||_F <= 1e-2 and max|Y - Y_ref| <= 5e-2 max|Y_ref|
  against the fp64 oracle on the same codes.

Full-size workloads are checked on sampled token rows / weight rows (every row
is independent, so the oracle computes them one by one) in the same launch
configuration the benchmark times.
"""
import ctypes

import numpy as np
import pytest

import oracle
import synthetic
from oracle import metrics

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def paro():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rotated_w4_linear_amd as p
    p.load_library()
    return p


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def log(msg):
    print(msg, flush=True)


# ----------------------------------------------------------------------------
# rotation
# ----------------------------------------------------------------------------

def check_rotation(paro, x, layer, rows=None, inplace=False):
    r = paro.Rotation(layer.pairs, layer.theta, layer.alpha, layer.group)
    xd = dev(x)
    if inplace:
        yd = paro.paro_rotate(r, xd, xd)
    else:
        yd = paro.paro_rotate(r, xd)
    got = host(yd)
    idx = np.arange(x.shape[0]) if rows is None else rows
    ref = oracle.rotate_activations(x[idx], layer.pairs, layer.theta, layer.alpha)
    err = metrics.assert_rotated_close(got[idx], ref, layer.group)
    r.close()
    return err, got


def test_rotate_tiny(paro):
    x, layer = synthetic.tiny()
    log("rotate tiny 4x256 G128 K8")
    check_rotation(paro, x, layer)


@pytest.mark.parametrize("M", [1, 4, 16])
def test_rotate_decode(paro, M):
    layer = synthetic.decode_layer()
    log(f"rotate decode M={M}")
    check_rotation(paro, synthetic.decode_x(M), layer)


@pytest.mark.parametrize("G,K,d,M", [(64, 8, 512, 37), (256, 8, 512, 37), (128, 1, 384, 9),
                                     (128, 0, 256, 5), (256, 0, 512, 3), (64, 0, 256, 2),
                                     (128, 3, 1024, 100), (256, 5, 768, 19), (128, 16, 256, 7),
                                     (64, 32, 256, 5), (256, 12, 512, 6), (128, 2, 128, 1),
                                     (256, 3, 512, 2050), (256, 2, 768, 4101)])
def test_rotate_shapes(paro, G, K, d, M):
    log(f"rotate G={G} K={K} d={d} M={M}")
    x, layer = synthetic.rotation_case(seed=G + K * 7 + d + M, M=M, d=d, group=G, K=K)
    check_rotation(paro, x, layer)


def test_rotate_general_form_and_identity_angles(paro):
    log("rotate with theta=1e-7 pairs (general 2x2 form)")
    x, layer = synthetic.rotation_case(seed=11, M=33, d=512, group=128, K=8)
    theta0 = layer.theta.copy()
    layer.theta[:, ::3] = 1e-7
    img, lay = paro.paro_rotation_plan_host(layer.pairs, layer.theta, layer.alpha, 128)
    assert not lay["fast"]
    check_rotation(paro, x, layer)
    log("rotate with theta=0 pairs (identity pairs, factored form)")
    layer.theta[:] = theta0
    layer.theta[:, ::3] = 0.0
    img, lay = paro.paro_rotation_plan_host(layer.pairs, layer.theta, layer.alpha, 128)
    assert lay["fast"]
    check_rotation(paro, x, layer)
    # all angles zero: X' = X / alpha exactly up to the fp16 rounding
    layer.theta[:] = 0.0
    _, got = check_rotation(paro, x, layer)
    want = (x.astype(np.float64) / layer.alpha.astype(np.float64)).astype(np.float16)
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


@pytest.mark.parametrize("keep,G,K,d,M", [(0.1, 128, 8, 4096, 300), (0.1, 128, 8, 4096, 1),
                                           (0.05, 128, 8, 14336, 70), (0.1, 64, 8, 512, 37),
                                           (0.1, 256, 8, 1024, 19), (0.02, 128, 16, 512, 9)])
def test_rotate_sparse_pairing(paro, keep, G, K, d, M):
    """Sparse pairings (most theta = 0): the kernel runs the compacted schedule
    of fewer stages than K."""
    log(f"rotate sparse keep={keep} G={G} K={K} d={d} M={M}")
    x, layer = synthetic.sparse_rotation_case(seed=int(keep * 1000) + d + M, M=M, d=d, group=G,
                                              K=K, keep=keep)
    _, lay = paro.paro_rotation_plan_host(layer.pairs, layer.theta, layer.alpha, G)
    assert lay["stages"] < K and lay["fast"]
    check_rotation(paro, x, layer)


@pytest.mark.parametrize("keep", [1.0, 0.1])
def test_rotate_quarter_turns(paro, keep):
    """Quarter turns (cos ~ 4e-8 for the float angle) in dense and sparse
    pairings: the factored form carries them with large coefficient ratios."""
    log(f"rotate quarter turns keep={keep}")
    x, layer = synthetic.sparse_rotation_case(seed=23, M=45, d=2048, group=128, K=8, keep=keep)
    nz = np.argwhere(layer.theta != 0.0)
    for t, p in nz[::50 if keep == 1.0 else 16]:
        layer.theta[t, p] = np.float32(np.pi / 2)
    check_rotation(paro, x, layer)


def test_rotate_inplace_and_empty(paro):
    log("rotate in place / M=0")
    x, layer = synthetic.rotation_case(seed=3, M=21, d=512, group=128, K=8)
    check_rotation(paro, x, layer, inplace=True)
    r = paro.Rotation(layer.pairs, layer.theta, layer.alpha, 128)
    empty = torch.empty((0, 512), dtype=torch.float16, device="cuda")
    out = paro.paro_rotate(r, empty)
    assert out.shape == (0, 512)
    # token counts past the 32-bit row index are rejected before any launch
    lib = paro.load_library()
    buf = torch.zeros((4, 512), dtype=torch.float16, device="cuda")
    st = lib.paro_rotate(r.handle, ctypes.c_void_p(buf.data_ptr()), ctypes.c_void_p(buf.data_ptr()),
                         ctypes.c_int64(2 ** 31), None)
    assert paro.STATUS[st] == "PARO_ERR_SHAPE"


def test_rotate_256_general_form_and_in_place(paro):
    """256-channel segments, whose packed outputs go through the store
    permutation before the stores: the general 2x2 form, and in place (each
    wavefront's next batch is loaded before it stores the current one)."""
    log("rotate G=256 general form, in place")
    x, layer = synthetic.rotation_case(seed=13, M=29, d=1024, group=256, K=8)
    layer.theta[:, ::3] = 1e-7
    _, lay = paro.paro_rotation_plan_host(layer.pairs, layer.theta, layer.alpha, 256)
    assert not lay["fast"] and lay["seg_ch"] == 256
    check_rotation(paro, x, layer)
    check_rotation(paro, x, layer, inplace=True)
    log("rotate G=256 factored form in place, 8200 rows")
    x, layer = synthetic.rotation_case(seed=14, M=8200, d=512, group=256, K=8)
    check_rotation(paro, x, layer, rows=np.r_[0:40, 4090:4110, 8160:8200], inplace=True)


def test_rotate_deterministic(paro):
    x, layer = synthetic.rotation_case(seed=4, M=333, d=1024, group=128, K=8)
    r = paro.Rotation(layer.pairs, layer.theta, layer.alpha, 128)
    xd = dev(x)
    a = host(paro.paro_rotate(r, xd))
    b = host(paro.paro_rotate(r, xd))
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


@pytest.mark.parametrize("point", list(range(27)))
def test_rotate_sweep_full_size(paro, point):
    """The 27 sweep points at M = 8192 (the benchmark's launch), 96 sampled rows checked."""
    x, layer = synthetic.sweep(point)
    d, K, G = synthetic.sweep_points()[point]
    log(f"rotate sweep point {point}: d={d} K={K} G={G}")
    rows = np.sort(synthetic.rng_for(3000, point).choice(x.shape[0], 96, replace=False))
    rows[-1] = x.shape[0] - 1
    check_rotation(paro, x, layer, rows=rows)


@pytest.mark.parametrize("which", ["mlp", "down"])
def test_rotate_prefill_configs_sampled(paro, which):
    """X' of the prefill configurations' own inputs (MLP: 8192 x 4096, N(0, 1)
    with 1 % outlier channels; down-proj: 2048 x 14336, Student-t(3)) at the
    full-size launch, 2e-3 on 128 sampled rows including the last."""
    x, layer = synthetic.prefill_mlp() if which == "mlp" else synthetic.prefill_down()
    log(f"rotate prefill {which} {x.shape[0]}x{x.shape[1]} (sampled rows)")
    rows = np.sort(synthetic.rng_for(3100, 0 if which == "mlp" else 1).choice(x.shape[0], 128, replace=False))
    rows[-1] = x.shape[0] - 1
    check_rotation(paro, x, layer, rows=rows)


# ----------------------------------------------------------------------------
# quantization
# ----------------------------------------------------------------------------

def check_quantize(paro, layer, rotated=True, rows=None, group=None):
    group = group or layer.group
    r = paro.Rotation(layer.pairs, layer.theta, layer.alpha, layer.group) if rotated else None
    qw, s, z = paro.paro_quantize_weights(r, dev(layer.w), group)
    qw, s, z = host(qw), host(s), host(z)
    idx = np.arange(layer.w.shape[0]) if rows is None else rows
    if rotated:
        rq, rs, rz = oracle.quantize_weights(layer.w[idx], group, layer.pairs, layer.theta, layer.alpha)
    else:
        rq, rs, rz = oracle.quantize_weights(layer.w[idx], group)
    for name, g, w in (("qweight", qw[idx], rq), ("scales", s[idx].view(np.uint16), rs.view(np.uint16)),
                       ("zeros", z[idx], rz)):
        bad = np.argwhere(g != w)
        assert bad.size == 0, f"{name}: {len(bad)} mismatches, first at {bad[0]}: {g[tuple(bad[0])]} vs {w[tuple(bad[0])]}"
    return qw, s, z


def test_quantize_tiny(paro):
    log("quantize tiny")
    _, layer = synthetic.tiny()
    check_quantize(paro, layer)
    check_quantize(paro, layer, rotated=False)


def test_quantize_decode_layer_full(paro):
    log("quantize decode layer 4096x4096 (all rows)")
    check_quantize(paro, synthetic.decode_layer())


@pytest.mark.parametrize("which", ["mlp", "down"])
def test_quantize_prefill_layers_sampled(paro, which):
    _, layer = synthetic.prefill_mlp() if which == "mlp" else synthetic.prefill_down()
    rows = np.sort(synthetic.rng_for(3100, 0 if which == "mlp" else 1).choice(layer.w.shape[0], 384, replace=False))
    log(f"quantize {which} {layer.w.shape} on {len(rows)} sampled rows")
    check_quantize(paro, layer, rows=rows)
    check_quantize(paro, layer, rotated=False, rows=rows[:64])


@pytest.mark.parametrize("G", [64, 256])
def test_quantize_other_groups(paro, G):
    log(f"quantize group {G}")
    rng = synthetic.rng_for(3200, G)
    w = synthetic.draw_w(rng, 40, 512, 0.02, n_outlier_cols=3)
    pairs, theta, alpha = synthetic.draw_rotation(rng, 512, G, 5)
    check_quantize(paro, synthetic.Layer(w, pairs, theta, alpha, G))


def test_quantize_zero_angles_equal_plain_scaled(paro):
    """theta = 0: codes equal the K = 0 (scale-only) codes bit for bit."""
    rng = synthetic.rng_for(3300, 0)
    w = synthetic.draw_w(rng, 32, 256, 0.02)
    pairs, theta, alpha = synthetic.draw_rotation(rng, 256, 128, 8)
    a = paro.paro_quantize_weights(paro.Rotation(pairs, np.zeros_like(theta), alpha, 128), dev(w), 128)
    b = paro.paro_quantize_weights(paro.Rotation(pairs[:0], theta[:0], alpha, 128), dev(w), 128)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_quantize_nonfinite_weight_is_an_error(paro):
    w = synthetic.draw_w(synthetic.rng_for(3400, 0), 8, 256, 0.02)
    w[3, 17] = np.float16(np.inf)
    with pytest.raises(paro.ParoError) as e:
        paro.paro_quantize_weights(None, dev(w), 128)
    assert e.value.status == -4
    big = np.full((4, 256), 60000, np.float16)
    big[:, ::2] = -60000
    with pytest.raises(paro.ParoError):
        # range 120000 / 15 = 8000 fits; scaled by alpha = 16 it overflows fp16
        pairs, theta, _ = synthetic.draw_rotation(synthetic.rng_for(3400, 1), 256, 128, 1)
        paro.paro_quantize_weights(paro.Rotation(pairs, theta, np.full(256, 16.0, np.float32), 128),
                                   dev(big), 128)


# ----------------------------------------------------------------------------
# the linear layer
# ----------------------------------------------------------------------------

def check_linear(paro, x, layer, bias=None, rotated=True, rows=None):
    G = layer.group
    r = paro.Rotation(layer.pairs, layer.theta, layer.alpha, G) if rotated else None
    qw, s, z = paro.paro_quantize_weights(r, dev(layer.w), G)
    y = host(paro.paro_w4_linear(r, dev(x), qw, s, z, dev(bias) if bias is not None else None, group=G))
    qw, s, z = host(qw), host(s), host(z)
    idx = np.arange(x.shape[0]) if rows is None else rows
    if rotated:
        ref = oracle.rotated_w4_linear(x[idx], qw, s, z, G, layer.pairs, layer.theta, layer.alpha, bias)
    else:
        ref = oracle.rotated_w4_linear(x[idx], qw, s, z, G, bias=bias)
    assert np.all(np.isfinite(y[idx].astype(np.float32)))
    return metrics.assert_linear_close(y[idx], ref)


def test_linear_tiny(paro):
    log("linear tiny (GEMV)")
    x, layer = synthetic.tiny()
    check_linear(paro, x, layer)
    check_linear(paro, x, layer, rotated=False)


@pytest.mark.parametrize("M", [1, 4, 16])
def test_linear_decode(paro, M):
    log(f"linear decode M={M}")
    layer = synthetic.decode_layer()
    check_linear(paro, synthetic.decode_x(M), layer)
    check_linear(paro, synthetic.decode_x(M), layer, rotated=False)


# 17 to 64 tokens take the small-batch kernel with two or four blocks of 16
# token columns (the last block ragged): 4096 -> 4096 (128-channel
# workgroups), 4096 -> 1024 (64-channel), 1152 -> 1040 (scales and zeros
# loaded one group at a time), groups of 64 and 256 (the latter transformed
# into the workspace first), and 4096 -> 8192 (2^25 weights: transformed
# into the workspace first from 17 tokens; the others from 33).
@pytest.mark.parametrize("M", [17, 32, 33, 48, 64])
@pytest.mark.parametrize("d,N,G", [(4096, 4096, 128), (4096, 1024, 128), (1152, 1040, 128), (1024, 272, 64),
                                   (1024, 272, 256), (4096, 8192, 128)])
def test_linear_small_batch_blocks(paro, M, d, N, G):
    log(f"linear small batch M={M} d={d} N={N} group={G}")
    x, layer, b = synthetic.linear_case(seed=700 + M + d + N + G, M=M, d=d, N=N, group=G)
    check_linear(paro, x, layer, bias=b)
    check_linear(paro, x, layer, rotated=False)


# (prefill shapes with fewer than 256 output tiles of 128 tokens x 256 channels
# run 64-token tiles, and with fewer than 256 of those, 64 x 128 tiles: the
# first four and (70, 128, 208), which has too few k-tiles to split k inside
# the workgroup; (1100, 512, 4112) runs 64 x 256 tiles; (2100, 512, 4112)
# runs 128-token tiles with k split in halves inside the workgroup,
# (4200, 256, 4208) without)
@pytest.mark.parametrize("M,d,N", [(65, 256, 64), (130, 512, 272), (300, 384, 128), (256, 1024, 512),
                                   (70, 128, 208), (1100, 512, 4112), (3, 512, 48), (9, 1152, 1040),
                                   (2100, 512, 4112), (4200, 256, 4208)])
def test_linear_shapes_with_bias(paro, M, d, N):
    log(f"linear M={M} d={d} N={N}")
    x, layer, b = synthetic.linear_case(seed=M + d + N, M=M, d=d, N=N)
    check_linear(paro, x, layer, bias=b)


# smaller-tile layers whose X' is at least 8 MiB and N < 4 M run with every XCD
# owning whole m-blocks (it reads an eighth of X'): k/v-proj shapes at 1024,
# 2048 and 4100 tokens (ragged M and N), and (1030, 4096, 272), whose few
# tiles also split k across workgroups; rows sampled (the last included)
@pytest.mark.parametrize("M,d,N", [(2048, 4096, 1024), (4100, 4096, 1040), (1024, 4096, 1024),
                                   (1030, 4096, 272)])
def test_linear_m_major_tiles(paro, M, d, N):
    log(f"linear m-major tiles M={M} d={d} N={N}")
    x, layer, b = synthetic.linear_case(seed=M + d + N + 5, M=M, d=d, N=N)
    rows = np.sort(synthetic.rng_for(3511, M).choice(M, 96, replace=False))
    rows[-1] = M - 1
    check_linear(paro, x, layer, bias=b, rows=rows)
    check_linear(paro, x, layer, rotated=False, rows=rows)


# shapes with at least 256 output tiles of 256 x 256 run the one-wavefront-per-SIMD
# kernel (d = 1024, 2048 and 4096 with the scale and zero panel in LDS): ragged in M
# and N, rows sampled (the last included), every column checked
@pytest.mark.parametrize("M,d,N", [(4200, 256, 8208), (2600, 512, 13008), (2304, 1024, 14336),
                                   (2600, 2048, 13008), (4100, 4096, 4112)])
def test_linear_wide_tiles(paro, M, d, N):
    log(f"linear wide tiles M={M} d={d} N={N}")
    x, layer, b = synthetic.linear_case(seed=M + d + N, M=M, d=d, N=N)
    rows = np.sort(synthetic.rng_for(3510, M).choice(M, 64, replace=False))
    rows[-1] = M - 1
    check_linear(paro, x, layer, bias=b, rows=rows)
    check_linear(paro, x, layer, rotated=False, rows=rows)


# layers with fewer than 256 output tiles of 256 x 256 and long k run
# stream-K when the workspace holds the partial tiles (full workspace): each
# XCD's tiles are laid end to end as one sequence of k-tiles and shared out
# among 16 to 32 workgroups of the XCD. With the minimum workspace the same
# call runs the smaller-tile kernel. Both against the oracle: the down-proj
# configuration (32 workgroups per XCD, each tile in two pieces, 56 groups of
# 128 per piece in the scale/zero panel), 3072 tokens (ranges of 1.3 tiles:
# pieces at both ends, too many groups for the panel), ragged M and N with
# unequal XCDs (13 and 9 n-blocks), groups of 256 and of 64, 24 and 16
# workgroups per XCD (tiles cut in 2 or 4 equal pieces), and layers that do
# not take stream-K (q/o-proj at 2048 tokens: the smaller-tile kernel; 448
# tiles of 256 x 256: one per workgroup).
@pytest.mark.parametrize("M,d,N,G,sk", [(2048, 14336, 4096, 128, True), (3072, 14336, 4096, 128, True),
                                        (2600, 8192, 3088, 128, True), (1500, 16384, 4096, 256, True),
                                        (1300, 8192, 4096, 64, True), (1000, 8192, 2064, 128, True),
                                        (600, 14336, 4096, 128, True), (2048, 4096, 4096, 128, False),
                                        (2048, 4096, 14336, 128, False)])
def test_linear_stream_k(paro, M, d, N, G, sk):
    log(f"linear stream-k M={M} d={d} N={N} group={G}")
    x, layer, b = synthetic.linear_case(seed=M + d + N + 7, M=M, d=d, N=N, group=G)
    assert layer.group == G
    r = paro.Rotation(layer.pairs, layer.theta, layer.alpha, G)
    qw, s, z = paro.paro_quantize_weights(r, dev(layer.w), G)
    rows = np.sort(synthetic.rng_for(3520, M).choice(M, 48, replace=False))
    rows[-1] = M - 1
    ref = oracle.rotated_w4_linear(x[rows], host(qw), host(s), host(z), G, layer.pairs, layer.theta,
                                   layer.alpha, b)
    full = paro.paro_w4_linear_workspace_size(r, M, N, d)
    minimum = 16384 + (M * d * 2 + 255) // 256 * 256
    assert full == minimum + (128 << 20 if sk else 0)
    for nbytes in ((full, minimum, full) if sk else (full,)):
        ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        y = host(paro.paro_w4_linear(r, dev(x), qw, s, z, dev(b), group=G, workspace=ws))
        assert np.all(np.isfinite(y[rows].astype(np.float32)))
        metrics.assert_linear_close(y[rows], ref)
        assert int(ws[:16384].count_nonzero()) == 0  # every call leaves the counters zero
    # plain layer: the default workspace (stream-K where planned) and, with no
    # workspace at all, one tile per workgroup or the smaller-tile kernel
    refp = oracle.rotated_w4_linear(x[rows], host(qw), host(s), host(z), G, bias=b)
    yp = host(paro.paro_w4_linear(None, dev(x), qw, s, z, dev(b), group=G))
    metrics.assert_linear_close(yp[rows], refp)
    lib = paro.load_library()
    xd, bd = dev(x), dev(b)
    y0 = torch.empty((M, N), dtype=torch.float16, device="cuda")
    vp = ctypes.c_void_p
    rc = lib.paro_w4_linear(None, vp(xd.data_ptr()), vp(qw.data_ptr()), vp(s.data_ptr()), vp(z.data_ptr()),
                            vp(bd.data_ptr()), vp(y0.data_ptr()), M, N, d, G, None, 0,
                            vp(torch.cuda.current_stream().cuda_stream))
    assert paro.STATUS[rc] == "PARO_OK"
    metrics.assert_linear_close(host(y0)[rows], refp)


# 65 to a few hundred tokens on the 64 x 128-tile kernel: with the full
# workspace k is also split across 2 or 4 workgroups per tile (fp32 partial
# tiles, the last to arrive adds them in split order); with the minimum
# workspace it is not. Both against the oracle, ragged M and N included.
@pytest.mark.parametrize("M,d,N,G", [(65, 4096, 4096, 128), (128, 4096, 4112, 128), (200, 2048, 1040, 128),
                                     (256, 4096, 4096, 64), (130, 14336, 4096, 128)])
def test_linear_narrow_split(paro, M, d, N, G):
    log(f"linear narrow split M={M} d={d} N={N} group={G}")
    x, layer, b = synthetic.linear_case(seed=M + d + N + 11, M=M, d=d, N=N, group=G)
    r = paro.Rotation(layer.pairs, layer.theta, layer.alpha, G)
    qw, s, z = paro.paro_quantize_weights(r, dev(layer.w), G)
    rows = np.sort(synthetic.rng_for(3530, M).choice(M, min(M, 40), replace=False))
    rows[-1] = M - 1
    ref = oracle.rotated_w4_linear(x[rows], host(qw), host(s), host(z), G, layer.pairs, layer.theta,
                                   layer.alpha, b)
    full = paro.paro_w4_linear_workspace_size(r, M, N, d)
    minimum = 16384 + (M * d * 2 + 255) // 256 * 256
    assert full > minimum
    for nbytes in (full, minimum, full):
        ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        y = host(paro.paro_w4_linear(r, dev(x), qw, s, z, dev(b), group=G, workspace=ws))
        metrics.assert_linear_close(y[rows], ref)
        assert int(ws[:16384].count_nonzero()) == 0
    refp = oracle.rotated_w4_linear(x[rows], host(qw), host(s), host(z), G, bias=b)
    yp = host(paro.paro_w4_linear(None, dev(x), qw, s, z, dev(b), group=G))
    metrics.assert_linear_close(yp[rows], refp)
    r.close()


def test_linear_gemv_vs_gemm_same_rows(paro):
    """Rows 0..15 through the GEMV (M = 16) and the GEMM (M = 40) agree."""
    x, layer, b = synthetic.linear_case(seed=5, M=40, d=1024, N=256)
    r = paro.Rotation(layer.pairs, layer.theta, layer.alpha, 128)
    qw, s, z = paro.paro_quantize_weights(r, dev(layer.w), 128)
    xd = dev(x)
    y_gemm = host(paro.paro_w4_linear(r, xd, qw, s, z, dev(b)))
    y_gemv = host(paro.paro_w4_linear(r, xd[:16].contiguous(), qw, s, z, dev(b)))
    fro, mx = metrics.linear_error(y_gemv, y_gemm[:16])
    assert fro < 1e-3 and mx < 5e-3


def test_linear_one_hot_reads_weights(paro):
    """X = e_k (no rotation) reads out dequantized weight columns plus the bias (GEMV and GEMM)."""
    d, N = 256, 64
    x, layer, b = synthetic.linear_case(seed=6, M=1, d=d, N=N)
    qw, s, z = paro.paro_quantize_weights(None, dev(layer.w), 128)
    w_hat = oracle.dequantize(host(qw), host(s), host(z), 128)
    for rows in (np.arange(0, 16), np.arange(0, d)):
        eye = np.zeros((len(rows), d), np.float16)
        eye[np.arange(len(rows)), rows] = 1
        y = host(paro.paro_w4_linear(None, dev(eye), qw, s, z, dev(b))).astype(np.float64)
        want = (w_hat[:, rows].T + b.astype(np.float64)[None, :]).astype(np.float16).astype(np.float64)
        # fp16 rounding of (q - z) * s in the kernel, then of the sum with the bias
        assert np.max(np.abs(y - want)) <= 2 * 2.0 ** -10 * (np.abs(want).max() + 1)


def test_linear_workspace_errors(paro):
    x, layer, b = synthetic.linear_case(seed=7, M=8, d=256, N=32)
    r = paro.Rotation(layer.pairs, layer.theta, layer.alpha, 128)
    qw, s, z = paro.paro_quantize_weights(r, dev(layer.w), 128)
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(paro.ParoError) as e:
        paro.paro_w4_linear(r, dev(x), qw, s, z, workspace=small)
    assert e.value.status == -7
    assert paro.paro_w4_linear_workspace_size(r, 8, 32, 256) >= 16384
    assert paro.paro_w4_linear_workspace_size(r, 65, 32, 256) >= 16384 + 65 * 256 * 2


# ----------------------------------------------------------------------------
# small batches (M <= 64): one kernel, transform fused in, split over k
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("M,d,N", [(1, 640, 400), (16, 640, 400), (5, 384, 48), (2, 4096, 4096),
                                   (16, 14336, 256), (11, 1152, 1040), (1, 128, 16),
                                   (3, 4096, 14336), (16, 14336, 4096), (24, 4096, 1024), (40, 1152, 1040),
                                   (64, 14336, 4096), (16, 4096, 4096), (12, 4096, 1024), (8, 14336, 256),
                                   (5, 14336, 144)])
def test_decode_fused_equals_rotate_then_plain(paro, M, d, N):
    """The fused transform yields the X' bits paro_rotate yields and the k-split
    sum order does not depend on where X' came from: equal outputs bit for bit.
    (8, 14336, 256) and (5, 14336, 144) take the grouped reduction of 28
    k-slices (few outputs per n-block), the latter with a ragged n-block."""
    log(f"decode fused vs separate M={M} d={d} N={N}")
    x, layer, b = synthetic.linear_case(seed=40 + M + d, M=M, d=d, N=N)
    r = paro.Rotation(layer.pairs, layer.theta, layer.alpha, 128)
    qw, s, z = paro.paro_quantize_weights(r, dev(layer.w), 128)
    xd = dev(x)
    y_fused = host(paro.paro_w4_linear(r, xd, qw, s, z, dev(b)))
    y_sep = host(paro.paro_w4_linear(None, paro.paro_rotate(r, xd), qw, s, z, dev(b)))
    assert np.array_equal(y_fused.view(np.uint16), y_sep.view(np.uint16))
    ref = oracle.rotated_w4_linear(x, host(qw), host(s), host(z), 128, layer.pairs, layer.theta,
                                   layer.alpha, b)
    metrics.assert_linear_close(y_fused, ref)


@pytest.mark.parametrize("M,d,N", [(1, 4096, 640), (16, 2048, 384)])
def test_decode_unaligned_group_params(paro, M, d, N):
    """Scales and zeros placed at odd addresses take the per-group load path
    instead of the vector loads; both give the same output bit for bit."""
    log(f"decode scales/zeros at odd offsets M={M} d={d} N={N}")
    x, layer, b = synthetic.linear_case(seed=80 + M, M=M, d=d, N=N)
    r = paro.Rotation(layer.pairs, layer.theta, layer.alpha, 128)
    qw, s, z = paro.paro_quantize_weights(r, dev(layer.w), 128)
    xd, bd = dev(x), dev(b)
    y_aligned = host(paro.paro_w4_linear(r, xd, qw, s, z, bd))
    s_buf = torch.zeros(s.numel() + 1, dtype=s.dtype, device="cuda")
    z_buf = torch.zeros(z.numel() + 1, dtype=z.dtype, device="cuda")
    s_odd = s_buf[1:].view(s.shape)
    z_odd = z_buf[1:].view(z.shape)
    s_odd.copy_(s)
    z_odd.copy_(z)
    assert s_odd.data_ptr() % 8 != 0 and z_odd.data_ptr() % 4 != 0
    y_odd = host(paro.paro_w4_linear(r, xd, qw, s_odd, z_odd, bd))
    assert np.array_equal(y_aligned.view(np.uint16), y_odd.view(np.uint16))
    ref = oracle.rotated_w4_linear(x, host(qw), host(s), host(z), 128, layer.pairs, layer.theta,
                                   layer.alpha, b)
    metrics.assert_linear_close(y_aligned, ref)


@pytest.mark.parametrize("K", [12, 32, 0, 3])
def test_decode_other_stage_counts(paro, K):
    """K > 8 rotates into the workspace first; K = 0 and K < 8 run fused."""
    log(f"decode plan K={K}")
    x, layer, b = synthetic.linear_case(seed=60 + K, M=7, d=1024, N=272, K=K)
    check_linear(paro, x, layer, bias=b)


@pytest.mark.parametrize("group", [64, 256])
def test_linear_rejects_other_rotation_groups(paro, group):
    x, layer, b = synthetic.linear_case(seed=65, M=3, d=512, N=32, group=group)
    r = paro.Rotation(layer.pairs, layer.theta, layer.alpha, group)
    qw, s, z = paro.paro_quantize_weights(None, dev(layer.w), 128)
    with pytest.raises(paro.ParoError) as e:
        paro.paro_w4_linear(r, dev(x), qw, s, z)
    assert e.value.status == -2


@pytest.mark.parametrize("G", [64, 256])
@pytest.mark.parametrize("M,d,N", [(1, 1024, 256), (5, 768, 144), (16, 2048, 128), (130, 1024, 272),
                                   (300, 512, 128), (1, 4096, 1024)])
def test_linear_other_groups(paro, G, M, d, N):
    """W4G64 and W4G256: rotation and quantization groups of 64 or 256 channels
    (the small-batch kernel fuses the transform for G = 64; G = 256 rotates
    into the workspace first)."""
    if d % G:
        pytest.skip("d is not a multiple of the group")
    log(f"linear group {G} M={M} d={d} N={N}")
    x, layer, b = synthetic.linear_case(seed=300 + G + M, M=M, d=d, N=N, group=G)
    check_quantize(paro, layer, group=G)
    check_linear(paro, x, layer, bias=b)
    check_linear(paro, x, layer, rotated=False)


def test_decode_general_form(paro):
    log("decode with theta=1e-7 pairs (general 2x2 form, fused)")
    x, layer, b = synthetic.linear_case(seed=71, M=6, d=768, N=144)
    layer.theta[:, ::3] = 1e-7
    _, lay = paro.paro_rotation_plan_host(layer.pairs, layer.theta, layer.alpha, 128)
    assert not lay["fast"]
    check_linear(paro, x, layer, bias=b)


@pytest.mark.parametrize("M,d,N", [(1, 4096, 4096), (16, 4096, 1024), (300, 4096, 512)])
def test_linear_sparse_pairing(paro, M, d, N):
    """A sparse pairing (10 % of the pairs rotate): compacted activation
    schedule in the fused small-batch kernel and in the prefill path, weights
    transformed with all K canonical stages."""
    log(f"linear sparse pairing M={M} d={d} N={N}")
    x, layer, b = synthetic.linear_case(seed=90 + M, M=M, d=d, N=N)
    rng = np.random.default_rng(91 + M)
    layer.theta[rng.random(layer.theta.shape) >= 0.1] = 0.0
    _, lay = paro.paro_rotation_plan_host(layer.pairs, layer.theta, layer.alpha, 128)
    assert lay["stages"] < 8 and lay["fast"]
    check_quantize(paro, layer)
    check_linear(paro, x, layer, bias=b)


def test_decode_workspace_reuse(paro):
    """The arrival counters return to zero: repeated calls, and calls of other
    sizes, on one workspace give identical results."""
    log("decode workspace reuse")
    cases = [synthetic.linear_case(seed=80 + i, M=M, d=d, N=N)
             for i, (M, d, N) in enumerate([(16, 640, 400), (1, 4096, 4096), (3, 1024, 96)])]
    need = 0
    prepared = []
    for x, layer, b in cases:
        r = paro.Rotation(layer.pairs, layer.theta, layer.alpha, 128)
        qw, s, z = paro.paro_quantize_weights(r, dev(layer.w), 128)
        prepared.append((r, dev(x), qw, s, z, dev(b)))
        need = max(need, paro.paro_w4_linear_workspace_size(r, x.shape[0], qw.shape[0], x.shape[1]))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    first = [host(paro.paro_w4_linear(*p[:5], p[5], workspace=ws)) for p in prepared]
    again = [host(paro.paro_w4_linear(*p[:5], p[5], workspace=ws)) for p in reversed(prepared)][::-1]
    for a, c in zip(first, again):
        assert np.array_equal(a.view(np.uint16), c.view(np.uint16))
    counters = host(ws[:16384].view(torch.int32))
    assert not counters.any()
    for (x, layer, b), y, p in zip(cases, first, prepared):
        ref = oracle.rotated_w4_linear(x, host(p[2]), host(p[3]), host(p[4]), 128, layer.pairs,
                                       layer.theta, layer.alpha, b)
        metrics.assert_linear_close(y, ref)


@pytest.mark.slow
def test_decode_more_n_blocks_than_counters(paro):
    """N = 4096 * 128 + 128 output channels: more n-blocks than the 4096
    arrival counters, so the launch is split; sampled channels of both parts."""
    M, d, N = 2, 640, 4096 * 128 + 128
    log(f"decode M={M} d={d} N={N} (split launch)")
    rng = synthetic.rng_for(3600, 0)
    x = synthetic.draw_x(rng, M, d, synthetic.n_outliers(d), 20.0)
    pairs, theta, alpha = synthetic.draw_rotation(rng, d, 128, 8)
    w = (rng.standard_normal((N, d), dtype=np.float32) * np.float32(0.02)).astype(np.float16)
    b = synthetic.draw_bias(rng, N)
    r = paro.Rotation(pairs, theta, alpha, 128)
    wd = dev(w)
    del w
    qw, s, z = paro.paro_quantize_weights(r, wd, 128)
    del wd
    y = host(paro.paro_w4_linear(r, dev(x), qw, s, z, dev(b)))
    cols = np.concatenate([np.arange(0, 32), np.arange(N - 160, N),
                           np.sort(rng.choice(N, 64, replace=False))])
    ci = torch.from_numpy(cols).cuda()
    ref = oracle.rotated_w4_linear(x, host(qw[ci]), host(s[ci]), host(z[ci]), 128, pairs, theta,
                                   alpha, b[cols])
    metrics.assert_linear_close(y[:, cols], ref)


def test_linear_prefill_mlp_sampled(paro):
    log("linear prefill MLP 8192x4096 -> 14336 (sampled rows)")
    x, layer = synthetic.prefill_mlp()
    rows = np.sort(synthetic.rng_for(3500, 0).choice(x.shape[0], 48, replace=False))
    rows[-1] = x.shape[0] - 1
    check_linear(paro, x, layer, rows=rows)


def test_linear_prefill_down_sampled(paro):
    log("linear prefill down 2048x14336 -> 4096 (sampled rows)")
    x, layer = synthetic.prefill_down()
    rows = np.sort(synthetic.rng_for(3500, 1).choice(x.shape[0], 48, replace=False))
    rows[-1] = x.shape[0] - 1
    check_linear(paro, x, layer, rows=rows)


@pytest.mark.parametrize("index", list(range(7)))
def test_decoder_chain_linear(paro, index):
    """One linear of the Llama-3-8B decoder-layer chain (q, k, v, o, gate, up,
    down; each with its own rotation, group 128, K = 8) at M = 1, 16 and 2048
    tokens, rotated W4 against the oracle: every row at M <= 16, 24 sampled
    rows (including the last) at M = 2048."""
    name, layer = synthetic.decoder_layer()[index]
    N, d = layer.w.shape
    r = paro.Rotation(layer.pairs, layer.theta, layer.alpha, 128)
    qw, s, z = paro.paro_quantize_weights(r, dev(layer.w), 128)
    qh, sh, zh = host(qw), host(s), host(z)
    for M in (1, 16, 2048):
        log(f"chain {name} {d}->{N} M={M}")
        x = synthetic.decoder_x(index, M)
        y = host(paro.paro_w4_linear(r, dev(x), qw, s, z))
        rows = np.arange(M)
        if M > 16:
            rows = np.sort(synthetic.rng_for(3600, index).choice(M, 24, replace=False))
            rows[-1] = M - 1
        ref = oracle.rotated_w4_linear(x[rows], qh, sh, zh, 128, layer.pairs, layer.theta, layer.alpha)
        fro, mx = metrics.assert_linear_close(y[rows], ref)
        log(f"  rel-Frobenius {fro:.2e}, max {mx:.2e}")
    r.close()


# ----------------------------------------------------------------------------
# plans from the library's pair selection (random + de-duplication, largest
# gaps, top-10% sparsification) through the same kernels
# ----------------------------------------------------------------------------

def selected_layer(paro, kind, d=4096, N=1024, G=128, K=8):
    rng = synthetic.rng_for(3700, {"random": 0, "gap": 1, "top10": 2}[kind])
    w = synthetic.draw_w(rng, N, d, 0.02, n_outlier_cols=synthetic.n_outliers(d), factor=10.0)
    theta = synthetic.draw_theta(rng, d, K)
    alpha = synthetic.draw_alpha(rng, d)
    if kind == "gap":
        pairs = paro.paro_pairs_by_gap(np.abs(w.astype(np.float32)).max(axis=0), G, K)
    else:
        pairs = paro.paro_pairs_random(d, G, K, 0x5041524F + d)
    if kind == "top10":
        theta = paro.paro_sparsify_angles(theta, int(round(0.1 * theta.size)))
    return synthetic.Layer(w, pairs, theta, alpha, G)


@pytest.mark.parametrize("kind", ["random", "gap", "top10"])
def test_selected_pairings_through_the_kernels(paro, kind):
    """Plans built by paro_pairs_random / paro_pairs_by_gap (score: the largest
    |W| of each input channel) / paro_sparsify_angles (10% of the pairs kept):
    X' at 2e-3, codes bit-exact on sampled rows, the linear at M = 16 and 300."""
    layer = selected_layer(paro, kind)
    log(f"selected pairing {kind}")
    x = synthetic.draw_x(synthetic.rng_for(3701, 0), 2048, layer.d, synthetic.n_outliers(layer.d), 20.0)
    rows = np.sort(synthetic.rng_for(3702, 0).choice(2048, 64, replace=False))
    rows[-1] = 2047
    check_rotation(paro, x, layer, rows=rows)
    check_quantize(paro, layer, rows=np.arange(0, layer.w.shape[0], 37))
    for M in (16, 300):
        fro, mx = check_linear(paro, x[:M], layer)
        log(f"  linear M={M}: rel-Frobenius {fro:.2e}, max {mx:.2e}")


# ----------------------------------------------------------------------------
# gradients of the transform
# ----------------------------------------------------------------------------

def backward_ref(x, g, layer, side, block=1024):
    """The oracle's gradients, its row sums taken over blocks of rows (each row
    is independent, so the block sums add up to the same sums)."""
    M, d = x.shape
    K = layer.pairs.shape[0]
    gx = np.zeros((M, d))
    dth = np.zeros((K, d // 2))
    dal = np.zeros(d)
    for m0 in range(0, max(M, 1), block):
        sl = slice(m0, min(M, m0 + block))
        a, b, c = oracle.rotation_backward(x[sl], g[sl], layer.pairs, layer.theta, layer.alpha, side)
        gx[sl] = a
        dth += b
        dal += c
    return gx, dth, dal


def check_backward(paro, x, g, layer, side, rows=None, want_gx=True):
    r = paro.Rotation(layer.pairs, layer.theta, layer.alpha, layer.group)
    gx, dth, dal = paro.paro_rotation_backward(r, dev(x), dev(g), side, want_gx=want_gx)
    rgx, rdth, rdal = backward_ref(x, g, layer, side)
    errs = {"dtheta": metrics.assert_grad_close(host(dth), rdth, "dtheta"),
            "dalpha": metrics.assert_grad_close(host(dal), rdal, "dalpha")}
    if want_gx:
        idx = np.arange(x.shape[0]) if rows is None else rows
        errs["gx"] = metrics.assert_grad_close(host(gx)[idx], rgx[idx], "gx")
    r.close()
    return errs


def grad_case(seed, M, d, G, K, side, keep=1.0):
    x, layer = synthetic.sparse_rotation_case(seed, M, d, G, K, keep) if keep < 1.0 else \
        synthetic.rotation_case(seed, M, d, G, K)
    if side == "weight":
        x = synthetic.draw_w(synthetic.rng_for(4000, seed), M, d, 0.02, n_outlier_cols=2)
    g = synthetic.rng_for(4100, seed).standard_normal((M, d)).astype(np.float32)
    return x, g, layer


@pytest.mark.parametrize("side", ["activation", "weight"])
@pytest.mark.parametrize("G,K,d,M", [(128, 8, 256, 5), (128, 8, 512, 37), (64, 8, 512, 9),
                                     (256, 8, 512, 21), (128, 1, 128, 3), (128, 0, 256, 4),
                                     (128, 32, 256, 11), (256, 3, 768, 1), (64, 5, 384, 300),
                                     (256, 8, 14336, 3), (128, 16, 2048, 70)])
def test_backward_shapes(paro, side, G, K, d, M):
    log(f"backward {side} G={G} K={K} d={d} M={M}")
    x, g, layer = grad_case(G + K + d + M, M, d, G, K, side)
    check_backward(paro, x, g, layer, side)


@pytest.mark.parametrize("M,d", [(1, 512), (7, 512), (8, 512), (9, 512), (17, 512), (65, 128),
                                 (1000, 4096)])
def test_backward_batch_boundaries(paro, M, d):
    """Row counts around the gradient kernel's batches (eight rows for
    128-channel segments) and chunk ends: ragged last batches repeat the last
    row with a zero gradient and must add nothing."""
    log(f"backward batch boundaries M={M} d={d}")
    x, g, layer = grad_case(5000 + M + d, M, d, 128, 8, "activation")
    check_backward(paro, x, g, layer, "activation")


def test_backward_sparse_pairing_and_no_input_gradient(paro):
    """Identities (theta = 0) still get angle gradients; gx = NULL skips the input gradient."""
    log("backward sparse pairing, gx = NULL")
    x, g, layer = grad_case(5, 40, 1024, 128, 8, "activation", keep=0.1)
    check_backward(paro, x, g, layer, "activation", want_gx=False)


def test_backward_in_place_and_empty(paro):
    log("backward in place / M = 0")
    x, g, layer = grad_case(6, 19, 512, 128, 8, "activation")
    r = paro.Rotation(layer.pairs, layer.theta, layer.alpha, 128)
    gd = dev(g)
    gx, dth, dal = paro.paro_rotation_backward(r, dev(x), gd, "activation", gx=gd)
    rgx, rdth, rdal = backward_ref(x, g, layer, "activation")
    metrics.assert_grad_close(host(gd), rgx, "gx in place")
    metrics.assert_grad_close(host(dth), rdth, "dtheta")
    e = torch.empty((0, 512), dtype=torch.float16, device="cuda")
    ge = torch.empty((0, 512), dtype=torch.float32, device="cuda")
    _, dth, dal = paro.paro_rotation_backward(r, e, ge, "activation")
    assert not host(dth).any() and not host(dal).any()


def test_backward_deterministic(paro):
    x, g, layer = grad_case(7, 300, 1024, 128, 8, "activation")
    r = paro.Rotation(layer.pairs, layer.theta, layer.alpha, 128)
    a = [host(t) for t in paro.paro_rotation_backward(r, dev(x), dev(g), "activation")]
    b = [host(t) for t in paro.paro_rotation_backward(r, dev(x), dev(g), "activation")]
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


@pytest.mark.parametrize("side", ["activation", "weight"])
def test_backward_prefill_layer(paro, side):
    """The benchmark's shape (8192 x 4096, K = 8): angle and scale gradients in
    full, input gradients on sampled rows."""
    M, d = 8192, 4096
    log(f"backward {side} {M}x{d}")
    x, g, layer = grad_case(8 if side == "activation" else 9, M, d, 128, 8, side)
    rows = np.sort(synthetic.rng_for(4200, 0).choice(M, 256, replace=False))
    check_backward(paro, x, g, layer, side, rows=rows)


# ----------------------------------------------------------------------------
# layer-wise output loss and its straight-through gradients
# ----------------------------------------------------------------------------

# The oracle's layer loss is the plain fp64 definition. The device rounds X',
# each dequantized weight and Y_q to fp16 (and the operands of dY E), so its
# loss and gradients are held to per-value tolerances derived from those
# rounding points (metrics.layer_loss_tolerance: six standard deviations of
# the rounding noise plus the fp32 gradient arithmetic's 1e-4).


def check_layer_loss(paro, M, d, N, G, K, seed, gradients=True, keep=1.0, exact=False):
    x, layer, _ = synthetic.linear_case(seed=seed, M=M, d=d, N=N, group=G, K=K, bias=False)
    if keep < 1.0:
        layer.theta[synthetic.rng_for(4300, seed).random(layer.theta.shape) >= keep] = 0.0
    if exact:
        layer.theta[:] = 0.0
        layer.alpha[:] = (2.0 ** synthetic.rng_for(4400, seed).integers(-1, 2, size=d)).astype(np.float32)
    r = paro.Rotation(layer.pairs, layer.theta, layer.alpha, G)
    qw, s, z = paro.paro_quantize_weights(r, dev(layer.w), G)
    loss, dth, dal = paro.paro_layer_loss(r, dev(x), dev(layer.w), qw, s, z, gradients=gradients)
    qh, sh, zh = host(qw), host(s), host(z)
    ref = oracle.layer_loss(x, layer.w, qh, sh, zh, G, layer.pairs, layer.theta, layer.alpha,
                            grad=gradients)
    rl = ref[0] if gradients else ref
    got = float(host(loss)[0])
    tl, tth, tal = metrics.layer_loss_tolerance(x, layer.w, qh, sh, zh, G, layer.pairs, layer.theta,
                                                layer.alpha, seed=seed)
    log(f"  loss {got:.7g} vs {rl:.7g} (tolerance {tl:.3g})")
    assert abs(got - rl) <= tl, f"loss {got} vs {rl}, tolerance {tl}"
    if gradients:
        if K:
            e = metrics.assert_within(host(dth), ref[1], tth, "dtheta")
            log(f"  dtheta error / tolerance {e:.3f}")
        e = metrics.assert_within(host(dal), ref[2], tal, "dalpha")
        log(f"  dalpha error / tolerance {e:.3f}")
    r.close()
    return got, rl


@pytest.mark.parametrize("M,d,N,G,K", [(37, 256, 64, 128, 8), (5, 512, 96, 128, 8), (300, 512, 128, 64, 4),
                                       (130, 768, 48, 128, 1), (64, 256, 32, 128, 0), (200, 1024, 256, 128, 8),
                                       (40, 512, 64, 256, 8), (12, 512, 48, 64, 8)])
def test_layer_loss_and_gradients(paro, M, d, N, G, K):
    log(f"layer loss M={M} d={d} N={N} G={G} K={K}")
    check_layer_loss(paro, M, d, N, G, K, seed=M + d + N + G + K)


@pytest.mark.parametrize("M,d,N,G", [(37, 256, 64, 128), (9, 512, 96, 128), (140, 512, 128, 64)])
def test_layer_loss_exact_case(paro, M, d, N, G):
    """Angles 0 (identity stages that still carry angle gradients) and
    power-of-two scales (X' = X / alpha exact in fp16)."""
    log(f"layer loss, exact case M={M} d={d} N={N} G={G}")
    check_layer_loss(paro, M, d, N, G, 8, seed=M + d, exact=True)


def test_layer_loss_without_gradients_and_sparse(paro):
    log("layer loss: loss only; sparse pairing")
    check_layer_loss(paro, 77, 512, 64, 128, 8, seed=3, gradients=False)
    check_layer_loss(paro, 77, 512, 64, 128, 8, seed=4, keep=0.1)


def test_layer_loss_empty(paro):
    x, layer, _ = synthetic.linear_case(seed=5, M=1, d=256, N=32, bias=False)
    r = paro.Rotation(layer.pairs, layer.theta, layer.alpha, 128)
    qw, s, z = paro.paro_quantize_weights(r, dev(layer.w), 128)
    e = torch.empty((0, 256), dtype=torch.float16, device="cuda")
    loss, dth, dal = paro.paro_layer_loss(r, e, dev(layer.w), qw, s, z)
    assert float(host(loss)[0]) == 0.0 and not host(dth).any() and not host(dal).any()


def test_layer_loss_workspace_reused_across_sizes(paro):
    """One zero-filled workspace serves a call at M = 16 and then one at M = 8
    (d = 1024: the small-batch linear splits k, so its arrival counters are
    used): both results hold and the counters are left at zero."""
    d, N, G = 1024, 256, 128
    x, layer, _ = synthetic.linear_case(seed=71, M=16, d=d, N=N, group=G, K=8, bias=False)
    r = paro.Rotation(layer.pairs, layer.theta, layer.alpha, G)
    qw, s, z = paro.paro_quantize_weights(r, dev(layer.w), G)
    qh, sh, zh = host(qw), host(s), host(z)
    need = max(paro.load_library().paro_layer_loss_workspace_size(r.handle, M, N, d, 1) for M in (16, 8))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for M in (16, 8):
        log(f"layer loss, shared workspace, M={M}")
        loss, dth, dal = paro.paro_layer_loss(r, dev(x[:M]), dev(layer.w), qw, s, z, workspace=ws)
        ref = oracle.layer_loss(x[:M], layer.w, qh, sh, zh, G, layer.pairs, layer.theta, layer.alpha,
                                grad=True)
        tl, tth, tal = metrics.layer_loss_tolerance(x[:M], layer.w, qh, sh, zh, G, layer.pairs,
                                                    layer.theta, layer.alpha, seed=M)
        assert abs(float(host(loss)[0]) - ref[0]) <= tl
        metrics.assert_within(host(dth), ref[1], tth, "dtheta")
        metrics.assert_within(host(dal), ref[2], tal, "dalpha")
        assert not host(ws[:16384]).any(), "arrival counters not left at zero"
    r.close()


# ----------------------------------------------------------------------------
# measurement kernels (the ceilings the benchmark reports next to the peaks)
# ----------------------------------------------------------------------------

def test_stream_copy_copies(paro):
    log("measurement: device copy")
    src = torch.randint(0, 256, (3 << 20,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros_like(src)
    paro.paro_stream_copy(src, dst, blocks=300)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


def test_mfma_loop_counts_every_product(paro):
    """With every operand 1.0 each of a lane's 256 accumulators gains 16 per
    round, so each output is 4096 * iters exactly."""
    log("measurement: MFMA loop")
    src = torch.ones(4096, dtype=torch.float16, device="cuda")
    out = torch.full((7 * 256,), -1.0, dtype=torch.float32, device="cuda")
    paro.paro_mfma_loop(src, out, 7, 100)
    torch.cuda.synchronize()
    assert torch.all(out == 4096.0 * 100)
    lib = paro.load_library()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = lib.paro_mfma_loop(ctypes.c_void_p(src.data_ptr()), 12, ctypes.c_void_p(out.data_ptr()), 7, 1, stream)
    assert paro.STATUS[rc] == "PARO_ERR_SHAPE"
