"""CPU tests of the C-ABI library: exports, argument validation, rotation schedule.

No kernel is launched here. The schedule test emulates, in numpy, exactly what
the rotation kernel executes from the table image that paro_rotation_create
uploads (load selector, keep/fetch exchanges through LDS slots, two-FMA or 2x2
stage updates, deferred scales, store selector) and compares the result with
the oracle.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import synthetic
from oracle import metrics

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def paro():
    import rotated_w4_linear_amd as p
    if not os.path.exists(p.LIB_PATH):
        pytest.skip("libparo.so not built")
    p.load_library()
    return p


def header_functions():
    src = open(os.path.join(ROOT, "include", "paro.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(paro_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol(paro):
    names = header_functions()
    assert "paro_rotate" in names and "paro_w4_linear" in names and "paro_quantize_weights" in names
    lib = ctypes.CDLL(paro.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/paro.h but not exported"


def test_status_strings(paro):
    lib = paro.load_library()
    for code, name in paro.STATUS.items():
        assert lib.paro_status_string(code).decode() == name
    assert lib.paro_status_string(123).decode() == "PARO_ERR_UNKNOWN"


def _create(paro, d, group, K, pairs, theta, alpha):
    lib = paro.load_library()
    h = ctypes.c_void_p()
    pairs = np.ascontiguousarray(pairs, np.int32)
    theta = np.ascontiguousarray(theta, np.float32)
    alpha = np.ascontiguousarray(alpha, np.float32)
    st = lib.paro_rotation_create(d, group, K, paro._ptr(pairs), paro._ptr(theta),
                                  paro._ptr(alpha), ctypes.byref(h))
    return st, h


def test_create_validation_errors(paro):
    d, G, K = 256, 128, 3
    pairs, theta, alpha = synthetic.draw_rotation(synthetic.rng_for(77, 1), d, G, K)
    cases = []
    dup = pairs.copy(); dup[1, 0, 1] = dup[1, 1, 0]
    cases.append(("duplicate channel", (d, G, K, dup, theta, alpha), -3))
    cross = pairs.copy(); a, b = cross[0, 0, 0], cross[0, 64, 0]
    cross[0, 0, 0], cross[0, 64, 0] = b, a
    cases.append(("pair crosses group", (d, G, K, cross, theta, alpha), -3))
    oob = pairs.copy(); oob[2, 5, 0] = d
    cases.append(("index out of range", (d, G, K, oob, theta, alpha), -3))
    same = pairs.copy(); same[0, 3, 1] = same[0, 3, 0]
    cases.append(("i == j", (d, G, K, same, theta, alpha), -3))
    bad_a = alpha.copy(); bad_a[7] = 0.0
    cases.append(("alpha zero", (d, G, K, pairs, theta, bad_a), -4))
    bad_a2 = alpha.copy(); bad_a2[9] = np.nan
    cases.append(("alpha nan", (d, G, K, pairs, theta, bad_a2), -4))
    bad_t = theta.copy(); bad_t[1, 2] = np.inf
    cases.append(("theta inf", (d, G, K, pairs, bad_t, alpha), -4))
    cases.append(("group 96", (d, 96, K, pairs, theta, alpha), -6))
    cases.append(("d not multiple of group", (d + 64, G, K, pairs, theta, alpha), -2))
    cases.append(("K too large", (d, G, 33, np.zeros((33, d // 2, 2), np.int32),
                                  np.zeros((33, d // 2), np.float32), alpha), -6))
    for name, args, want in cases:
        st, h = _create(paro, *args)
        assert st == want, f"{name}: got {st}, want {want}"
        assert not h.value
    lib = paro.load_library()
    assert lib.paro_rotation_create(d, G, K, None, None, None, None) == -1
    assert "NULL" in lib.paro_last_error().decode() or lib.paro_last_error()


def test_hot_calls_validate_before_any_launch(paro):
    lib = paro.load_library()
    # gradients of the transform: the handle comes first
    d4 = ctypes.c_void_p(16 * 1024)
    assert lib.paro_rotation_backward(None, 0, d4, d4, d4, d4, d4, 4, None, 0, None) == -1
    assert lib.paro_rotation_backward_workspace_size(None, 4) == 0
    # layer loss: the handle and the loss pointer come first
    assert lib.paro_layer_loss(None, d4, d4, d4, d4, d4, 4, 16, 256, 128, d4, None, None, None, 0,
                               None) == -1
    assert lib.paro_layer_loss_workspace_size(None, 4, 16, 256, 1) == 0
    assert lib.paro_rotate(None, None, None, 4, None) == -1
    assert lib.paro_rotate(None, None, None, 0, None) == -1  # handle still required
    dummy = ctypes.c_void_p(16 * 1024)
    bad = ctypes.c_void_p(16 * 1024 + 2)
    # null handle
    assert lib.paro_rotate(None, dummy, dummy, 4, None) == -1
    # w4_linear: groups other than 64, 128, 256 are unsupported; N % 16, d % 128,
    # d % group are shape errors
    args = [None, dummy, dummy, dummy, dummy, None, dummy]
    assert lib.paro_w4_linear(*args, 4, 64, 256, 32, None, 0, None) == -6
    assert lib.paro_w4_linear(*args, 4, 64, 256, 512, None, 0, None) == -6
    assert lib.paro_w4_linear(*args, 4, 64, 384, 256, None, 0, None) == -2
    assert lib.paro_w4_linear(*args, 4, 60, 256, 128, None, 0, None) == -2
    assert lib.paro_w4_linear(*args, 4, 64, 200, 128, None, 0, None) == -2
    assert lib.paro_w4_linear(*args, -1, 64, 256, 128, None, 0, None) == -2
    # sizes past the kernels' 32-bit tile offsets are unsupported
    assert lib.paro_w4_linear(*args, 4, 64, 1 << 23, 128, None, 0, None) == -6
    assert lib.paro_w4_linear(*args, 4, 1 << 31, 256, 128, None, 0, None) == -6
    # small batches: ceil(d / 512) * M * N * 4 bytes of partial sums must stay below 2^31
    assert lib.paro_w4_linear(*args, 16, 1 << 24, 1 << 16, 128, None, 0, None) == -6
    assert lib.paro_w4_linear(None, bad, dummy, dummy, dummy, None, dummy, 4, 64, 256, 128,
                              None, 0, None) == -5
    assert lib.paro_w4_linear(None, None, dummy, dummy, dummy, None, dummy, 4, 64, 256, 128,
                              None, 0, None) == -1
    # M == 0 is a successful no-op, even without a GPU
    assert lib.paro_w4_linear(*args, 0, 64, 256, 128, None, 0, None) == 0
    # quantize: unsupported group, shape mismatch
    assert lib.paro_quantize_weights(None, dummy, 8, 256, 96, dummy, dummy, dummy, None) == -6
    assert lib.paro_quantize_weights(None, dummy, 8, 200, 128, dummy, dummy, dummy, None) == -2
    assert lib.paro_quantize_weights(None, None, 8, 256, 128, dummy, dummy, dummy, None) == -1
    # workspace: none for plain large-batch calls; counters + fp32 partial sums
    # [ceil(d / 512)][M][N] for small batches; + X' for rotated large batches
    assert lib.paro_w4_linear_workspace_size(None, 65, 64, 256) == 0
    # (65 tokens, 64 -> 4096 channels: two 64 x 128 tiles, k split across 4
    # workgroups each: fp32 partial tiles of 32 KB)
    assert lib.paro_w4_linear_workspace_size(None, 65, 64, 4096) == 16384 + 2 * 4 * 32768
    assert lib.paro_w4_linear_workspace_size(None, 64, 64, 4096) == 16384 + 8 * 64 * 64 * 4
    assert lib.paro_w4_linear_workspace_size(None, 16, 64, 4096) == 16384 + 8 * 16 * 64 * 4
    assert lib.paro_w4_linear_workspace_size(None, 1, 64, 512) == 16384
    assert lib.paro_w4_linear_workspace_size(None, 0, 64, 512) == 0
    lib.paro_rotation_destroy(None)  # no-op


# ----------------------------------------------------------------------------
# schedule emulation
# ----------------------------------------------------------------------------

SEL_LOAD_KEEP, SEL_LOAD_SWAP = 0x03020100, 0x01000302
SEL_STORE_X, SEL_STORE_B = 0x03020100, 0x01000302


def f32(a):
    return np.asarray(a, dtype=np.float32)


def fma32(a, b, c):
    """fp32 fused multiply-add (exact product in fp64, one final rounding)."""
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(np.float32)


def field_major(img, lay, segs):
    """The schedules of the image as [segment][field][virtual lane]: the library
    stores four consecutive fields of a lane side by side,
    [segment][words / 4][lane][4], and after them the store permutation."""
    nv = lay["seg_ch"] // 2
    W = lay["words"]
    assert W % 4 == 0 and img.size == segs * W * nv + segs * nv * 2
    return img[:segs * W * nv].reshape(segs, W // 4, nv, 4).transpose(0, 1, 3, 2).reshape(segs, W, nv)


def store_permutation(img, lay, segs):
    """The store permutation after the schedules: [segment][virtual lane] LDS
    write and read slots of the packed output words."""
    nv = lay["seg_ch"] // 2
    perm = img[segs * lay["words"] * nv:].reshape(segs, nv, 2)
    assert np.all(perm % 16 == 0)
    return perm[:, :, 0] // 16, perm[:, :, 1] // 16


def emulate_rotate(img, lay, x, K, d):
    """Runs the plan image the way the activation kernel does: the kernel executes
    lay["stages"] stages, at most the K stages of the layer."""
    assert 0 <= lay["stages"] <= K
    K = lay["stages"]
    nv = lay["seg_ch"] // 2
    W = lay["words"]
    C = 2 if lay["fast"] else 4
    segs = d // lay["seg_ch"]
    tab = field_major(img, lay, segs)
    pws, prs = store_permutation(img, lay, segs)
    M = x.shape[0]
    out = np.zeros((M, d), np.float16)
    for s in range(segs):
        t = tab[s]
        seg = x[:, s * lay["seg_ch"]:(s + 1) * lay["seg_ch"]].astype(np.float32)
        ff = 3 + 2 * K + C * K
        lo, hi = seg[:, 0::2], seg[:, 1::2]          # [M][nv]
        keep = t[0] == SEL_LOAD_KEEP
        assert np.all((t[0] == SEL_LOAD_KEEP) | (t[0] == SEL_LOAD_SWAP))
        X = np.where(keep, lo, hi)
        B = np.where(keep, hi, lo)

        def exchange(tau, B):
            wr = t[1 + 2 * tau] // 16
            rd = t[2 + 2 * tau] // 16
            lds = np.zeros((M, nv), np.float32)
            lds[:, wr] = B
            return lds[:, rd]
        if K > 0:
            B = exchange(0, B)
            for st in range(K):
                cf = [f32(t[3 + 2 * K + C * st + e].view(np.float32)) for e in range(C)]
                a, b = X, B
                if C == 2:
                    X, B = fma32(cf[0], b, a), fma32(cf[1], a, b)
                else:
                    X = fma32(cf[1], b, (cf[0] * a).astype(np.float32))
                    B = fma32(cf[2], a, (cf[3] * b).astype(np.float32))
                B = exchange(st + 1, B)
        o = out[:, s * lay["seg_ch"]:(s + 1) * lay["seg_ch"]]
        lamX = t[ff].view(np.float32)
        lamB = t[ff + 1].view(np.float32)
        q = t[ff + 2] // 4
        sel = t[ff + 3]
        ox = (X * lamX).astype(np.float16)
        ob = (B * lamB).astype(np.float16)
        first = np.where(sel == SEL_STORE_X, ox, ob)
        second = np.where(sel == SEL_STORE_X, ob, ox)
        assert np.all((sel == SEL_STORE_X) | (sel == SEL_STORE_B))
        assert sorted(q.tolist()) == list(range(nv))
        if K == 0:
            # no exchange: every lane still holds the natural pair it loaded
            assert np.array_equal(q, np.arange(nv))
            o[:, 0::2] = first
            o[:, 1::2] = second
            continue
        # the activation kernel with 256-channel segments: the packed words
        # go through the store permutation and lane w stores natural pair w
        pw, pr = pws[s], prs[s]
        assert sorted(pw.tolist()) == list(range(nv)) and sorted(pr.tolist()) == list(range(nv))
        lds = np.zeros((M, nv, 2), np.float16)
        lds[:, pw, 0] = first
        lds[:, pw, 1] = second
        o[:, 0::2] = lds[:, pr, 0]
        o[:, 1::2] = lds[:, pr, 1]
        # with 128-channel segments, and in the small-batch kernel, each lane
        # places its pair at its store offset instead: the same layout
        placed = np.zeros((M, lay["seg_ch"]), np.float16)
        placed[:, 2 * q] = first
        placed[:, 2 * q + 1] = second
        assert np.array_equal(placed, o)
    return out


def check_slots_conflict_free(img, lay, K, d):
    """gfx950 16-byte LDS accesses: writes conflict-free when every 8 consecutive
    lanes hit slots distinct mod 8, reads when every 16 consecutive lanes hit
    slots distinct mod 16."""
    assert 0 <= lay["stages"] <= K
    K = lay["stages"]
    nv = lay["seg_ch"] // 2
    tab = field_major(img, lay, d // lay["seg_ch"])
    pws, prs = store_permutation(img, lay, d // lay["seg_ch"])
    for s in range(tab.shape[0]):
        # the K + 1 exchanges, then (with stages) the store permutation
        for tau in range(K + 2 if K > 0 else K + 1):
            if tau <= K:
                wr = tab[s, 1 + 2 * tau] // 16
                rd = tab[s, 2 + 2 * tau] // 16
            else:
                wr, rd = pws[s], prs[s]
            assert sorted(wr.tolist()) == list(range(nv))
            assert sorted(rd.tolist()) == list(range(nv))
            for blk in range(nv // 8):
                assert len(set((wr[8 * blk:8 * blk + 8] % 8).tolist())) == 8
            for blk in range(nv // 16):
                assert len(set((rd[16 * blk:16 * blk + 16] % 16).tolist())) == 16


@pytest.mark.parametrize("G,K,d,M", [(128, 8, 256, 5), (128, 1, 256, 3), (64, 8, 256, 4),
                                     (256, 8, 512, 3), (256, 2, 256, 2), (128, 0, 256, 3),
                                     (64, 3, 384, 2), (128, 4, 512, 2)])
def test_schedule_emulation_matches_oracle(paro, G, K, d, M):
    x, layer = synthetic.rotation_case(seed=G * 100 + K * 10 + M, M=M, d=d, group=G, K=K)
    img, lay = paro.paro_rotation_plan_host(layer.pairs, layer.theta, layer.alpha, G)
    assert lay["seg_ch"] == (256 if G == 256 else 128)
    if K:
        check_slots_conflict_free(img, lay, K, d)
    ref = oracle.rotate_activations(x, layer.pairs, layer.theta, layer.alpha)
    metrics.assert_rotated_close(emulate_rotate(img, lay, x, K, d), ref, G)


def test_schedule_general_form_with_near_identity_pairs(paro):
    """Rotations with |sin theta| below the factored form's threshold (theta =
    1e-7, not an exact identity) pin lane orientations that cannot all hold:
    the general 2x2 form is used."""
    d, G, K, M = 256, 128, 6, 4
    x, layer = synthetic.rotation_case(seed=5, M=M, d=d, group=G, K=K)
    theta = layer.theta.copy()
    theta[:, ::3] = 1e-7
    img, lay = paro.paro_rotation_plan_host(layer.pairs, theta, layer.alpha, G)
    assert not lay["fast"] and lay["stages"] == K
    check_slots_conflict_free(img, lay, K, d)
    ref = oracle.rotate_activations(x, layer.pairs, theta, layer.alpha)
    metrics.assert_rotated_close(emulate_rotate(img, lay, x, K, d), ref, G)


@pytest.mark.parametrize("keep,d,K,M", [(0.1, 4096, 8, 3), (0.1, 512, 8, 5), (0.2, 256, 8, 4),
                                         (0.05, 1024, 16, 3), (0.1, 256, 4, 2)])
def test_schedule_sparse_pairing_compacts_stages(paro, keep, d, K, M):
    """Sparse pairings (most theta = 0): the activation schedule runs fewer
    stages than K, with every rotation after the earlier ones on its channels,
    and still equals the oracle's K-stage product."""
    x, layer = synthetic.sparse_rotation_case(seed=int(keep * 100) + d + K, M=M, d=d, group=128,
                                              K=K, keep=keep)
    img, lay = paro.paro_rotation_plan_host(layer.pairs, layer.theta, layer.alpha, 128)
    # the least number of stages that keeps the order on every channel: the
    # longest chain of non-identity rotations linked by shared channels
    depth = np.zeros(d, np.int64)
    for t in range(K):
        for p in range(d // 2):
            if layer.theta[t, p] != 0.0:
                i, j = layer.pairs[t, p]
                depth[i] = depth[j] = max(depth[i], depth[j]) + 1
    want = int(depth.max())
    assert lay["stages"] == want < K
    assert lay["fast"]
    check_slots_conflict_free(img, lay, K, d)
    ref = oracle.rotate_activations(x, layer.pairs, layer.theta, layer.alpha)
    metrics.assert_rotated_close(emulate_rotate(img, lay, x, K, d), ref, 128)


@pytest.mark.parametrize("angle,step,seed,fast", [(np.pi / 2, 16, 18, True), (np.pi / 2, 64, 17, True),
                                                  (1e-13, 64, 17, True), (1e-13, 4, 17, False)])
def test_schedule_sparse_pairing_with_pinned_rotations(paro, angle, step, seed, fast):
    """Sparse pairings where some rotations are quarter turns (cos ~ 4e-8: the
    factored form carries them with a large coefficient ratio) or nearly
    identities (sin ~ 1e-13: their lanes must keep their registers, which ties
    the identity pairs around them; many such ties can contradict each other,
    and the plan then takes the general form)."""
    d, K = 1024, 8
    x, layer = synthetic.sparse_rotation_case(seed=seed, M=3, d=d, group=128, K=K, keep=0.1)
    nz = np.argwhere(layer.theta != 0.0)
    for t, p in nz[::step]:
        layer.theta[t, p] = np.float32(angle)
    img, lay = paro.paro_rotation_plan_host(layer.pairs, layer.theta, layer.alpha, 128)
    assert lay["fast"] == fast and lay["stages"] < K
    check_slots_conflict_free(img, lay, K, d)
    ref = oracle.rotate_activations(x, layer.pairs, layer.theta, layer.alpha)
    metrics.assert_rotated_close(emulate_rotate(img, lay, x, K, d), ref, 128)


def test_schedule_dense_pairing_keeps_all_stages(paro):
    """No identities, or identities that do not shorten the longest chain: K stages."""
    x, layer = synthetic.rotation_case(seed=9, M=2, d=512, group=128, K=6)
    _, lay = paro.paro_rotation_plan_host(layer.pairs, layer.theta, layer.alpha, 128)
    assert lay["stages"] == 6
    theta = layer.theta.copy()
    theta[:, ::3] = 0.0
    img, lay = paro.paro_rotation_plan_host(layer.pairs, theta, layer.alpha, 128)
    # exact identities become identity pairs that the factored form can carry
    assert lay["stages"] == 6 and lay["fast"]
    check_slots_conflict_free(img, lay, 6, 512)
    ref = oracle.rotate_activations(x, layer.pairs, theta, layer.alpha)
    metrics.assert_rotated_close(emulate_rotate(img, lay, x, 6, 512), ref, 128)


def test_schedule_full_decode_layer(paro):
    """The 4096-channel, K = 8 decode layer: factored form, exact on a few tokens."""
    layer = synthetic.decode_layer()
    x = synthetic.decode_x(4)
    img, lay = paro.paro_rotation_plan_host(layer.pairs, layer.theta, layer.alpha, 128)
    assert lay["fast"]
    check_slots_conflict_free(img, lay, 8, 4096)
    ref = oracle.rotate_activations(x, layer.pairs, layer.theta, layer.alpha)
    metrics.assert_rotated_close(emulate_rotate(img, lay, x, 8, 4096), ref, 128)


# ----------------------------------------------------------------------------
# channel-pair selection (host functions of the library) against the oracle
# ----------------------------------------------------------------------------

from oracle import pairs as opairs  # noqa: E402


@pytest.mark.parametrize("d,G,K,seed", [(256, 128, 8, 1), (4096, 128, 8, 0x5041524F), (128, 64, 16, 2),
                                        (512, 256, 8, 3), (8, 4, 3, 11), (640, 64, 0, 5),
                                        (2 ** 10, 8, 4, 2 ** 64 - 1)])
def test_pairs_random_equal_oracle(paro, d, G, K, seed):
    got = paro.paro_pairs_random(d, G, K, seed)
    want = opairs.pairs_random(d, G, K, seed)
    assert np.array_equal(got, want)


def test_pairs_random_infeasible_is_an_error(paro):
    """Seven greedy stages of a group of 8 can run out of unrepeated pairs;
    the library reports it where the oracle does."""
    try:
        opairs.pairs_random(64, 8, 7, 4)
        feasible = True
    except RuntimeError:
        feasible = False
    if feasible:
        assert np.array_equal(paro.paro_pairs_random(64, 8, 7, 4), opairs.pairs_random(64, 8, 7, 4))
    else:
        with pytest.raises(paro.ParoError) as ei:
            paro.paro_pairs_random(64, 8, 7, 4)
        assert ei.value.status == -4
    with pytest.raises(paro.ParoError):
        paro.paro_pairs_random(100, 8, 3, 1)  # group does not divide d
    with pytest.raises(paro.ParoError):
        paro.paro_pairs_random(64, 8, 8, 1)  # K > group - 1


@pytest.mark.parametrize("d,G,K", [(256, 128, 8), (4096, 128, 8), (512, 64, 32), (256, 256, 8), (8, 8, 4)])
def test_pairs_by_gap_equal_oracle(paro, d, G, K):
    rng = synthetic.rng_for(99, d + G + K)
    w = synthetic.draw_w(rng, 64, d, 0.02, n_outlier_cols=max(1, d // 64), factor=10.0)
    score = np.abs(w.astype(np.float32)).max(axis=0)  # the largest |W| of each input channel
    score[::7] = score[3]  # ties
    got = paro.paro_pairs_by_gap(score, G, K)
    assert np.array_equal(got, opairs.pairs_by_gap(score, G, K))
    with pytest.raises(paro.ParoError):
        paro.paro_pairs_by_gap(score, G, G // 2 + 1)
    bad = score.copy()
    bad[1] = np.nan
    with pytest.raises(paro.ParoError):
        paro.paro_pairs_by_gap(bad, G, K)


@pytest.mark.parametrize("K,d,frac", [(8, 4096, 0.1), (8, 256, 0.25), (1, 128, 0.0), (4, 512, 1.0)])
def test_sparsify_angles_equal_oracle(paro, K, d, frac):
    rng = synthetic.rng_for(99, 7 * K + d)
    theta = synthetic.draw_theta(rng, d, K)
    theta.reshape(-1)[::5] = theta.reshape(-1)[2]  # ties
    n = int(round(frac * theta.size))
    got = paro.paro_sparsify_angles(theta, n)
    assert np.array_equal(got.view(np.uint32), opairs.sparsify_angles(theta, n).view(np.uint32))
    assert int((got != 0).sum()) <= n
