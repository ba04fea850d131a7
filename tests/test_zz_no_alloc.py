"""paro_w4_linear_noalloc (the W4 linear on the library's static device
scratch) against paro_w4_linear with a caller's workspace, through the C ABI.

Both run the same kernels in the same order, so their outputs must be equal
bit for bit. Each case makes two calls in a row on the shared scratch, the
second with a smaller input; the arrival counters the small-batch kernel
keeps in that scratch must have been left at zero by the first call for the
second to be right. Also: a request larger than the scratch is refused before
anything is enqueued, and a captured call replays correctly.
"""
import gc

import numpy as np
import pytest

import synthetic

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def paro():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rotated_w4_linear_amd as p
    p.load_library()
    p.paro_device_init()
    return p


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def log(msg):
    print(msg, flush=True)


SCRATCH_BYTES = (64 << 20) + 16384  # the static scratch (include/paro.h)


def run_pair(paro, r, x, qw, s, z, bias, G):
    M, d = x.shape
    N = qw.shape[0]
    # the workspace entry point with the workspace the scratch stands for: the
    # full size when it fits (the k-split's partial tiles included), else the
    # minimum (for M > 64: X' only, or nothing for a plain layer)
    full = paro.paro_w4_linear_workspace_size(r, M, N, d)
    if full <= SCRATCH_BYTES:
        nbytes = full
    else:
        nbytes = 16384 + (M * d * 2 + 255) // 256 * 256 if r is not None else 0
    ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device="cuda")[:nbytes]
    ref = paro.paro_w4_linear(r, x, qw, s, z, bias, group=G, workspace=ws)
    y = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    paro.paro_w4_linear_noalloc(r, x, qw, s, z, y, bias, group=G)
    torch.cuda.synchronize()
    assert torch.equal(y, ref), f"noalloc differs from the workspace entry point at M={M}"


@pytest.mark.parametrize("rotated,G,d,N,Ms", [
    (True, 128, 4096, 4096, (16, 4)),      # small batch, transform fused, k split over 8 slices
    (True, 128, 4096, 4096, (48, 20)),     # small batch in blocks of 16 tokens (four, then two)
    (False, 128, 14336, 4096, (8, 1)),     # plain W4, 28 k-slices
    (True, 256, 1024, 512, (16, 5)),       # plan the small-batch kernel does not fuse: X' in the scratch
    (True, 128, 4096, 1024, (2048, 300)),  # matrix-core path, X' in the scratch
])
def test_noalloc_equals_workspace_entry_point(paro, rotated, G, d, N, Ms):
    x, layer, b = synthetic.linear_case(seed=d + N + G, M=max(Ms), d=d, N=N, group=G, K=8)
    r = paro.Rotation(layer.pairs, layer.theta, layer.alpha, G) if rotated else None
    qw, s, z = paro.paro_quantize_weights(r, dev(layer.w), G)
    xd, bd = dev(x), dev(b)
    for M in Ms:
        log(f"noalloc rotated={rotated} G={G} {d}->{N} M={M}")
        run_pair(paro, r, xd[:M].contiguous(), qw, s, z, bd, G)
    if r is not None:
        r.close()


def test_noalloc_rejects_requests_beyond_the_scratch(paro):
    d, N, M = 14336, 64, 4096  # X' alone is 112 MiB
    x, layer, _ = synthetic.linear_case(seed=9, M=1, d=d, N=N, bias=False)
    r = paro.Rotation(layer.pairs, layer.theta, layer.alpha, 128)
    qw, s, z = paro.paro_quantize_weights(r, dev(layer.w), 128)
    xd = torch.zeros((M, d), dtype=torch.float16, device="cuda")
    y = torch.full((M, N), 7.0, dtype=torch.float16, device="cuda")
    with pytest.raises(paro.ParoError) as ei:
        paro.paro_w4_linear_noalloc(r, xd, qw, s, z, y)
    assert ei.value.status == -7
    del ei  # (its traceback holds this frame: no cycle keeps r alive)
    torch.cuda.synchronize()
    assert bool((y == 7.0).all()), "a refused call wrote its output"
    r.close()


def test_noalloc_captured_call_replays(paro):
    M, d, N = 16, 2048, 1024
    x, layer, _ = synthetic.linear_case(seed=12, M=M, d=d, N=N, bias=False)
    r = paro.Rotation(layer.pairs, layer.theta, layer.alpha, 128)
    qw, s, z = paro.paro_quantize_weights(r, dev(layer.w), 128)
    xd = dev(x)
    ref = paro.paro_w4_linear(r, xd, qw, s, z)
    ref4 = paro.paro_w4_linear(r, xd[:4].contiguous(), qw, s, z)
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    # no garbage may be collected during the capture: a destroyed handle of
    # an earlier test would free device memory inside it
    gc.collect()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        paro.paro_w4_linear_noalloc(r, xd, qw, s, z, y)
    for i in range(3):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"replay {i}"
        other = torch.empty((4, N), dtype=torch.float16, device="cuda")
        paro.paro_w4_linear_noalloc(r, xd[:4].contiguous(), qw, s, z, other)  # eager use between replays
        torch.cuda.synchronize()
        assert torch.equal(other, ref4)
    r.close()
