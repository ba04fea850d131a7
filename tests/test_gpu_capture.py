"""Hot calls under HIP-graph capture, in a fresh process.

The small-batch linear splits k over workgroups that meet in one XCD's L2;
how workgroups are dispatched to XCDs is checked once per device by
paro_device_init (paro_rotation_create runs it), never by the hot call. These
tests start a child process (so that no earlier test has set the device up)
and make that process's FIRST small-batch paro_w4_linear call inside a stream
capture:
  * plain W4 on a device nobody initialised (the memory-side exchange path);
  * the rotated layer after paro_rotation_create (the XCD-local path).
Every graph replay is compared with the eager result, with eager work and
synchronisations between the replays; the two exchange paths add the same
partial sums in the same order, so their results are bit-identical.
"""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import gc
import sys
import numpy as np
import torch
sys.path.insert(0, ROOT)
import synthetic
import rotated_w4_linear_amd as paro

torch.cuda.set_device(0)
M, d, N = 4, 1024, 512
x, layer, _ = synthetic.linear_case(seed=31, M=M, d=d, N=N, group=128, K=8, bias=False)
xd = torch.from_numpy(x).cuda()
wd = torch.from_numpy(layer.w).cuda()
print("child: plain W4, first small-batch call inside a capture", flush=True)
qw, s, z = paro.paro_quantize_weights(None, wd, 128)  # offline; does not set the device up
ws = paro.new_workspace(None, M, N, d)
y = torch.empty((M, N), dtype=torch.float16, device="cuda")
gc.collect()
torch.cuda.synchronize()
g = torch.cuda.CUDAGraph()
with torch.cuda.graph(g):
    paro.paro_w4_linear(None, xd, qw, s, z, y=y, workspace=ws)
ref = paro.paro_w4_linear(None, xd, qw, s, z, workspace=paro.new_workspace(None, M, N, d))
torch.cuda.synchronize()
for i in range(3):
    y.zero_()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(y, ref), f"plain replay {i} differs from eager"
    _ = (xd.float() * 2).sum().item()  # eager work between replays
paro.paro_device_init()
fast = paro.paro_w4_linear(None, xd, qw, s, z, workspace=paro.new_workspace(None, M, N, d))
torch.cuda.synchronize()
assert torch.equal(fast, ref), "memory-side and XCD-local exchanges differ"

print("child: rotated layer, first rotated small-batch call inside a capture", flush=True)
r = paro.Rotation(layer.pairs, layer.theta, layer.alpha, 128)
qr, sr, zr = paro.paro_quantize_weights(r, wd, 128)
ws2 = paro.new_workspace(r, M, N, d)
y2 = torch.empty((M, N), dtype=torch.float16, device="cuda")
gc.collect()
torch.cuda.synchronize()
g2 = torch.cuda.CUDAGraph()
with torch.cuda.graph(g2):
    paro.paro_w4_linear(r, xd, qr, sr, zr, y=y2, workspace=ws2)
ref2 = paro.paro_w4_linear(r, xd, qr, sr, zr, workspace=paro.new_workspace(r, M, N, d))
torch.cuda.synchronize()
for i in range(3):
    y2.zero_()
    g2.replay()
    torch.cuda.synchronize()
    assert torch.equal(y2, ref2), f"rotated replay {i} differs from eager"
    _ = (xd.float() * 3).sum().item()
assert not ws2[:16384].any().item(), "arrival counters not left at zero"
print("child: ok", flush=True)
"""


def test_first_small_batch_call_inside_graph_capture():
    script = CHILD.replace("ROOT", repr(ROOT), 1)
    print("spawning child process for the capture test", flush=True)
    res = subprocess.run([sys.executable, "-c", script], capture_output=True, text=True,
                         timeout=150, cwd=ROOT)
    print(res.stdout, flush=True)
    assert res.returncode == 0, f"child failed ({res.returncode}):\n{res.stdout}\n{res.stderr[-4000:]}"
