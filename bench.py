"""Benchmark of the rotated W4G128 linear layer on one MI355X.

Default workload: the prefill MLP up/gate layer, 8192 tokens x 4096 -> 14336,
group 128, K = 8 rotation stages. One step is one forward pass of the layer's
hot path: one call of paro_w4_linear with the rotation handle, which launches
the online rotation X' = X T^-1 into its workspace and then the W4G128 linear
on X'. Steps are timed in blocks between two events. The plain W4 layer (same
kernel on the unrotated X and Q(W)) is timed the same way to give the
rotation's overhead.

Inputs are synthetic (seeded), resident in HBM before timing; distinct copies
of X and of the quantized weights are cycled so that caches (incl. the 256 MB
Infinity Cache) do not serve them from a previous step. Kernel durations (for
the rooflines) come from separate blocks of the same two launches made
through paro_rotate and paro_w4_linear, with HIP events recorded on the launch
stream around every launch. Timing starts only after half a second of the same
work (the GPU clock ramps up over the first tens of milliseconds of load), and
variants that are compared (rotated vs plain, W4 vs fp16) are timed in
alternating blocks.

Other workloads (``--workload``): prefill_down (2048 x 14336 -> 4096),
decode (M = 1, 4, 16 tokens, 4096 -> 4096; weight streaming), sweep (the 27
rotation-only points, 8192 x d), sparse (the transform with sparse pairings, in
which only a fraction of the pairs rotate), backward (the gradients of the
transform with respect to its input, angles and scales), calib (the layer-wise
loss with its angle and scale gradients: one transform-learning step), chain (the seven linears of a Llama-3-8B
decoder layer as rotated W4, plain W4 and dense fp16 chains), copy (a plain
device copy, for calibrating HBM byte counters).

Prints one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 MFMA
METRIC = "rotated-W4G128 linear TFLOP/s + rotation HBM GB/s; % overhead vs plain W4"



def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_sha(paths):
    """Hash of the kernel's source files (one path or a list, in order)."""
    h = hashlib.sha256()
    for path in ([paths] if isinstance(paths, str) else paths):
        with open(os.path.join(ROOT, path), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel_key):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
        ent = data[kernel_key]
        if ent.get("source_sha") != source_sha(ent["source"]):
            return None
        return ent["bytes_per_launch"]
    except Exception:
        return None


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


class Timer:
    """HIP events on the current stream around each launch."""

    def __init__(self, torch):
        self.torch = torch

    def event(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e


def setup_layer(paro, torch, x, layer, ring):
    r = paro.Rotation(layer.pairs, layer.theta, layer.alpha, layer.group)
    w = torch.from_numpy(layer.w).cuda()
    q_rot = paro.paro_quantize_weights(r, w, 128)
    q_plain = paro.paro_quantize_weights(None, w, 128)
    del w
    xs = [torch.from_numpy(x).cuda()]
    for _ in range(ring - 1):
        xs.append(xs[0].clone())
    qr = [q_rot] + [tuple(t.clone() for t in q_rot) for _ in range(ring - 1)]
    qp = [q_plain] + [tuple(t.clone() for t in q_plain) for _ in range(ring - 1)]
    torch.cuda.synchronize()
    return r, xs, qr, qp


def settle(torch, fns, min_rounds, seconds=0.5):
    """Run the callables round-robin for at least ``seconds`` of wall time and
    ``min_rounds`` rounds. The GPU clock ramps up over the first few tens of
    milliseconds of sustained work and then settles; every variant is timed
    only after that, so that none of them is measured on the ramp."""
    t0 = time.perf_counter()
    i = 0
    while i < min_rounds or time.perf_counter() - t0 < seconds:
        for f in fns:
            f(i)
        i += 1
        if i % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def graph_us(torch, step, n, out=None, seconds=0.3, replays=20):
    """GPU time per step (us) of n steps captured in one HIP graph and replayed.

    Small-batch calls take a few microseconds, less than launching them from
    Python costs, so back-to-back eager calls measure the host. The steps are
    captured once (after eager warm-up calls, which also run any first-call
    set-up) and the graph is replayed: events around the replays time the
    GPU's work alone. With ``out`` (a tensor the steps write) the replay's
    result is compared bit for bit with the eager one; the check is returned."""
    for i in range(n):
        step(i)
    torch.cuda.synchronize()
    ref = out.clone() if out is not None else None
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            step(i)
    ok = True
    for _ in range(3):
        if out is not None:
            out.zero_()
        g.replay()
        torch.cuda.synchronize()
        if ref is not None:
            ok = ok and bool(torch.equal(out.view(torch.int16), ref.view(torch.int16)))
    settle(torch, [lambda i: g.replay()], 2, seconds=seconds)
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(replays):
        g.replay()
    e.record()
    torch.cuda.synchronize()
    del g
    return s.elapsed_time(e) * 1e3 / (replays * n), ok


def time_layer(paro, torch, r, xs, qr, qp, steps, warmup, M, N, d):
    """Return per-step and per-kernel timings (ms) of the rotated and plain layer.

    The reported step is one call of the fused entry point (paro_w4_linear with
    the rotation handle: the rotation and the linear, two launches), timed over
    ``steps`` calls between two events; the plain layer is timed the same way.
    Per-kernel durations come from separate blocks that record an event around
    every launch (the events between launches cost a few percent of the step,
    so those blocks give the kernels' durations, not the step). After
    ``settle``, the four kinds of block run in alternation, twice, so that any
    remaining clock drift affects all alike; every figure averages both rounds."""
    ring = len(xs)
    xr = torch.empty((M, d), dtype=torch.float16, device="cuda")
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    wsp = paro.new_workspace(None, M, N, d)  # the plain layer's (split-k partial tiles, or none)
    T = Timer(torch)

    def rotated_step(i):
        k = i % ring
        paro.paro_rotate(r, xs[k], xr)
        e1 = T.event()
        paro.paro_w4_linear(None, xr, *qr[k], y=y, workspace=wsp)
        return e1

    def plain_step(i):
        paro.paro_w4_linear(None, xs[i % ring], *qp[i % ring], y=y, workspace=wsp)

    settle(torch, [rotated_step, plain_step], warmup)

    def rotated_block():
        ev = []
        start = T.event()
        prev = start
        for i in range(steps):
            mid = rotated_step(i)
            end = T.event()
            ev.append((prev, mid, end))
            prev = end
        torch.cuda.synchronize()
        return (start.elapsed_time(prev), [a.elapsed_time(b) for a, b, _ in ev],
                [b.elapsed_time(c) for _, b, c in ev])

    def plain_block():
        ev = []
        for i in range(steps):
            a = T.event()
            plain_step(i)
            ev.append((a, T.event()))
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev]

    # the fused entry point (rotation handle passed to paro_w4_linear) on the
    # same data, timed in the same alternation
    ws = paro.new_workspace(r, M, N, d)

    def fused_block():
        for i in range(2):
            paro.paro_w4_linear(r, xs[i % ring], *qr[i % ring], y=y, workspace=ws)
        s = T.event()
        for i in range(steps):
            paro.paro_w4_linear(r, xs[i % ring], *qr[i % ring], y=y, workspace=ws)
        e = T.event()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / steps

    def plain_total_block():
        s = T.event()
        for i in range(steps):
            plain_step(i)
        e = T.event()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / steps

    settle(torch, [lambda i: paro.paro_w4_linear(r, xs[i % ring], *qr[i % ring], y=y, workspace=ws)],
           2, seconds=0.1)
    rot, lin, plain_ms, inst, fused, plain_tot = [], [], [], [], [], []
    for _ in range(2):
        total, rot2, lin2 = rotated_block()
        inst.append(total / steps)
        rot += rot2
        lin += lin2
        plain_ms += plain_block()
        fused.append(fused_block())
        plain_tot.append(plain_total_block())

    return {
        "step_ms": float(np.mean(fused)),
        "plain_step_ms": float(np.mean(plain_tot)),
        "instrumented_step_ms": float(np.mean(inst)),
        "rot_ms": float(np.mean(rot)),
        "lin_ms": float(np.mean(lin)),
        "plain_ms": float(np.mean(plain_ms)),
        "pct": {k: [round(float(np.percentile(v, p)), 4) for p in (10, 50, 90)]
                for k, v in (("rotation_ms", rot), ("linear_ms", lin), ("plain_w4_ms", plain_ms))},
    }


def copy_rate_gbps(torch, paro, nbytes, ring=4, reps=12):
    """Read + write GB/s of the library's plain device copy (paro_stream_copy)
    of nbytes, cycling a ring of buffers (the same cold-cache condition as the
    kernels): the best over a few launch sizes, i.e. the measured ceiling of a
    read stream plus a write stream of that size. Returns (GB/s, blocks)."""
    n = (nbytes + 15) // 16 * 16
    src = [torch.ones(n, dtype=torch.uint8, device="cuda") for _ in range(ring)]
    dst = [torch.empty(n, dtype=torch.uint8, device="cuda") for _ in range(ring)]
    best = (0.0, 0)
    for blocks in (2048, 4096, 8192, 16384):
        for i in range(ring):
            paro.paro_stream_copy(src[i], dst[i], blocks)
        torch.cuda.synchronize()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        for i in range(reps):
            paro.paro_stream_copy(src[(i + 1) % ring], dst[i % ring], blocks)
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / reps
        best = max(best, (2.0 * n / (ms * 1e-3) / 1e9, blocks))
    del src, dst
    return best


def mfma_rate_tflops(torch, paro, iters=20000, reps=3):
    """fp16 matrix-core rate of the library's MFMA loop (paro_mfma_loop) on
    uniform(-1, 1) operands, one workgroup of four wavefronts per CU: the
    ceiling the matrix cores sustain under the chip's power limit (with random
    data the clock falls well below the one the datasheet peak assumes).
    Returns TFLOP/s, the best of a few runs."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    src = (torch.rand(1 << 20, device="cuda", generator=g) * 2 - 1).half()
    out = torch.empty(cus * 256, dtype=torch.float32, device="cuda")
    paro.paro_mfma_loop(src, out, cus, 500)
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(reps):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        paro.paro_mfma_loop(src, out, cus, iters)
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e)
        best = max(best, cus * 4 * 16 * iters * 32768.0 / (ms * 1e-3) / 1e12)
    del src, out
    return best


def cpu_baseline(x, layer, paro_q, N, d, target_s=12.0):
    """Time the oracle (rotation + fp64 linear) on a bounded sample of token rows."""
    import oracle
    qw, s, z = paro_q
    m = 16
    t_used = 0.0
    while True:
        t0 = time.perf_counter()
        xr = oracle.rotate_activations(x[:m], layer.pairs, layer.theta, layer.alpha)
        oracle.linear(xr, qw, s, z, 128)
        t_used = time.perf_counter() - t0
        if t_used > target_s / 4 or m >= x.shape[0]:
            break
        m = min(x.shape[0], m * 4)
    flops = 2.0 * m * N * d
    return {"value": flops / t_used / 1e12, "unit": "TFLOP/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"{m} of {x.shape[0]} token rows: fp64 rotation + dequantize + fp64 matmul "
                      f"({t_used:.1f} s)"}


def bench_layer(args, paro, torch, name, x, layer):
    M, d = x.shape
    N = layer.w.shape[0]
    # distinct copies of X and of both weight sets: > 1 GiB in total for the
    # MLP layer (10 x (64 + 2 x 30) MB), beyond the 256 MB Infinity Cache
    ring = args.ring or 10
    log(f"[bench] {name}: M={M} d={d} N={N} ring={ring}")
    r, xs, qr, qp = setup_layer(paro, torch, x, layer, ring)
    tm = time_layer(paro, torch, r, xs, qr, qp, args.steps, args.warmup, M, N, d)
    flops = 2.0 * M * N * d
    rot_bytes = 4.0 * M * d
    lin_tflops = flops / (tm["lin_ms"] * 1e-3) / 1e12
    copy_gbps, _ = copy_rate_gbps(torch, paro, M * d * 2)
    mfma_ceiling = mfma_rate_tflops(torch, paro)
    rot_gbps = rot_bytes / (tm["rot_ms"] * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(flops / (tm["step_ms"] * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(tm["step_ms"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": name, "tokens": M, "in_features": d, "out_features": N,
                   "group": 128, "stages_K": layer.K},
        "rotation_gbps": round(rot_bytes / (tm["rot_ms"] * 1e-3) / 1e9, 1),
        "rotation_ms": round(tm["rot_ms"], 4),
        "linear_ms": round(tm["lin_ms"], 4),
        "plain_w4_ms": round(tm["plain_ms"], 4),
        "plain_w4_tflops": round(flops / (tm["plain_ms"] * 1e-3) / 1e12, 3),
        "plain_w4_step_ms": round(tm["plain_step_ms"], 4),
        "instrumented_step_ms": round(tm["instrumented_step_ms"], 4),
        "overhead_vs_plain_pct": round(100.0 * (tm["step_ms"] - tm["plain_step_ms"]) / tm["plain_step_ms"], 2),
        "rotation_share_pct": round(100.0 * tm["rot_ms"] / tm["step_ms"], 2),
        "p10_p50_p90_ms": tm["pct"],
        "copy_same_bytes_gbps": round(copy_gbps, 1),
        "rotation_frac_of_copy": round(rot_gbps / copy_gbps, 4),
        "mfma_ceiling_tflops": round(mfma_ceiling, 1),
        "roofline": {"bound": "mfma", "achieved": round(lin_tflops, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(lin_tflops / MFMA_F16_PEAK_TFLOPS, 4),
                     "frac_of_mfma_ceiling": round(lin_tflops / mfma_ceiling, 4),
                     "traffic": traffic_for(f"w4_gemm:{name}")},
        "roofline_rotation": {"bound": "hbm", "achieved": round(rot_bytes / (tm["rot_ms"] * 1e-3) / 1e9, 1),
                              "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                              "frac": round(rot_bytes / (tm["rot_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                              "traffic": traffic_for(f"rotate:{name}")},
    }
    if args.cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        q = tuple(t.cpu().numpy() for t in qr[0])
        out["cpu_baseline"] = cpu_baseline(x, layer, q, N, d)
    return out


def bench_decode(args, paro, torch):
    import synthetic
    layer = synthetic.decode_layer()
    d, N = 4096, 4096
    ring = args.ring or 128   # 128 copies of the 8.8 MB packed layer: about 1.1 GB
    r = paro.Rotation(layer.pairs, layer.theta, layer.alpha, 128)
    w = torch.from_numpy(layer.w).cuda()
    q0 = paro.paro_quantize_weights(r, w, 128)
    p0 = paro.paro_quantize_weights(None, w, 128)
    qs = [q0] + [tuple(t.clone() for t in q0) for _ in range(ring - 1)]
    ps = [p0] + [tuple(t.clone() for t in p0) for _ in range(min(ring, 128) - 1)]
    T = Timer(torch)
    res = {}
    total_ms = 0.0
    total_flops = 0.0
    ms = [int(v) for v in args.decode_m.split(",")]
    for M in ms:
        x = torch.from_numpy(synthetic.decode_x(M)).cuda()
        y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        ws = paro.new_workspace(r, M, N, d)
        wsp = paro.new_workspace(None, M, N, d)
        xr = torch.empty_like(x)

        def run(kind, i):
            if kind == "rot":
                paro.paro_w4_linear(r, x, *qs[i % ring], y=y, workspace=ws)
            elif kind == "plain":
                paro.paro_w4_linear(None, x, *ps[i % len(ps)], y=y, workspace=wsp)
            else:
                paro.paro_rotate(r, x, xr)

        kinds = ("rot", "plain", "rotate_only")
        settle(torch, [lambda i, k=k: run(k, i) for k in kinds], args.warmup + 3)
        # eager back-to-back calls from Python (host-bound at these sizes; kept for reference)
        eager = {k: 0.0 for k in kinds}
        for kind in kinds:
            n = max(args.steps, 100)
            s = T.event()
            for i in range(n):
                run(kind, i)
            e = T.event()
            torch.cuda.synchronize()
            eager[kind] = s.elapsed_time(e) / n
        # GPU time: one graph per kind over the ring of weight copies, two
        # alternating rounds, the mean of both
        timing = {k: 0.0 for k in kinds}
        checks = {}
        for _ in range(2):
            for kind in kinds:
                us, ok = graph_us(torch, lambda i, k=kind: run(k, i), ring,
                                  out=xr if kind == "rotate_only" else y)
                timing[kind] += us / 1e3 / 2
                checks[kind] = checks.get(kind, True) and ok
        # packed codes + fp16 scales + u8 zeros, activations in, outputs out
        wbytes = N * d / 2 + 3 * N * d / 128 + 2 * M * d + 2 * M * N
        res[f"M{M}"] = {
            "rotated_us": round(1e3 * timing["rot"], 2), "plain_us": round(1e3 * timing["plain"], 2),
            "standalone_rotate_us": round(1e3 * timing["rotate_only"], 2),
            "rotated_gbps": round(wbytes / (timing["rot"] * 1e-3) / 1e9, 1),
            "plain_gbps": round(wbytes / (timing["plain"] * 1e-3) / 1e9, 1),
            "overhead_vs_plain_pct": round(100 * (timing["rot"] - timing["plain"]) / timing["plain"], 1),
            "eager_python_us": {k: round(1e3 * v, 2) for k, v in eager.items()},
            "graph_replay_equals_eager": checks,
        }
        total_ms += timing["rot"]
        total_flops += 2.0 * M * N * d
    g1 = res[f"M{ms[0]}"]["rotated_gbps"]
    return {
        "metric": METRIC, "value": round(total_flops / (total_ms * 1e-3) / 1e12, 4), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(total_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "decode_q_proj_4096x4096_M" + "_".join(map(str, ms)), "group": 128,
                   "stages_K": 8, "roofline_at_M": ms[0]},
        "decode": res,
        "roofline": {"bound": "hbm", "achieved": g1, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(g1 / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_for(f"w4_decode:decode_M{ms[0]}")},
    }


def bench_sweep(args, paro, torch):
    import synthetic
    T = Timer(torch)
    pts = []
    ring = args.ring or 6
    # measured ceiling: the library's plain copy of the largest point's bytes
    # (8192 x 5120 fp16 in and out), cycled over the same kind of ring
    copy_gbps, copy_blocks = copy_rate_gbps(torch, paro, 8192 * 5120 * 2, ring=ring)
    log(f"[sweep] copy ceiling {copy_gbps:.0f} GB/s ({copy_blocks} workgroups)")
    for p, (d, K, G) in enumerate(synthetic.sweep_points()):
        x, layer = synthetic.sweep(p)
        r = paro.Rotation(layer.pairs, layer.theta, layer.alpha, G)
        xs = [torch.from_numpy(x).cuda()]
        for _ in range(ring - 1):
            xs.append(xs[0].clone())
        ys = [torch.empty_like(xs[0]) for _ in range(ring)]
        settle(torch, [lambda i: paro.paro_rotate(r, xs[i % ring], ys[i % ring])], args.warmup + 2,
               seconds=0.2)
        n = max(args.steps, 30)
        s = T.event()
        for i in range(n):
            paro.paro_rotate(r, xs[i % ring], ys[i % ring])
        e = T.event()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / n
        gbps = 4.0 * x.shape[0] * d / (ms * 1e-3) / 1e9
        pts.append({"d": d, "K": K, "G": G, "us": round(ms * 1e3, 2), "gbps": round(gbps, 1),
                    "frac": round(gbps / HBM_PEAK_GBPS, 4), "frac_of_copy": round(gbps / copy_gbps, 4)})
        log(f"[sweep] d={d} K={K} G={G}: {ms*1e3:.1f} us, {gbps:.0f} GB/s")
        del xs, ys
    g = [q["gbps"] for q in pts]
    k8 = [q for q in pts if q["K"] == 8 and q["G"] == 128 and q["d"] == 4096][0]
    return {
        "metric": "rotation HBM GB/s (paro_rotate, 8192 tokens)", "value": round(float(np.mean(g)), 1),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(sum(q["us"] for q in pts) / 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "rotation_sweep_8192xd_27pts"}, "points": pts,
        "copy_ceiling_gbps": round(copy_gbps, 1), "copy_ceiling_blocks": copy_blocks,
        "roofline": {"bound": "hbm", "achieved": k8["gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": k8["frac"], "traffic": traffic_for("rotate:sweep_d4096_K8_G128")},
    }


def bench_sparse(args, paro, torch):
    """The transform with sparse pairings: each pair keeps its angle with
    probability `keep` and is an exact identity otherwise; the plan runs the
    compacted schedule (fewer stages than K)."""
    import synthetic
    T = Timer(torch)
    ring = args.ring or 6
    shapes = [(8192, 4096), (2048, 14336)]
    keeps = [1.0, 0.25, 0.1, 0.05]
    cases = []
    for M, d in shapes:
        for keep in keeps:
            x, layer = synthetic.sparse_rotation_case(seed=7, M=M, d=d, group=128, K=8, keep=keep)
            _, lay = paro.paro_rotation_plan_host(layer.pairs, layer.theta, layer.alpha, 128)
            r = paro.Rotation(layer.pairs, layer.theta, layer.alpha, 128)
            xs = [torch.from_numpy(x).cuda()]
            for _ in range(ring - 1):
                xs.append(xs[0].clone())
            ys = [torch.empty_like(xs[0]) for _ in range(ring)]
            cases.append({"M": M, "d": d, "keep": keep, "stages": lay["stages"], "fast": lay["fast"],
                          "r": r, "xs": xs, "ys": ys, "ms": []})
    fns = [lambda i, c=c: paro.paro_rotate(c["r"], c["xs"][i % ring], c["ys"][i % ring]) for c in cases]
    settle(torch, fns, args.warmup + 2)
    n = max(args.steps, 50)
    for _ in range(2):  # two rounds over all cases against clock drift
        for c, fn in zip(cases, fns):
            s = T.event()
            for i in range(n):
                fn(i)
            e = T.event()
            torch.cuda.synchronize()
            c["ms"].append(s.elapsed_time(e) / n)
    pts = []
    for c in cases:
        ms = min(c["ms"])
        gbps = 4.0 * c["M"] * c["d"] / (ms * 1e-3) / 1e9
        pts.append({"tokens": c["M"], "d": c["d"], "keep": c["keep"], "stages": c["stages"],
                    "factored": c["fast"], "us": round(ms * 1e3, 2), "gbps": round(gbps, 1),
                    "frac": round(gbps / HBM_PEAK_GBPS, 4)})
        log(f"[sparse] {c['M']}x{c['d']} keep={c['keep']}: {c['stages']} stages, "
            f"{ms*1e3:.1f} us, {gbps:.0f} GB/s")
    head = [q for q in pts if q["tokens"] == 8192 and q["keep"] == 0.1][0]
    return {
        "metric": "rotation HBM GB/s with sparse pairings (paro_rotate)", "value": head["gbps"],
        "unit": "GB/s", "n_gpus": 1, "steps": n, "warmup": args.warmup,
        "ms_per_step": round(head["us"] / 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "rotation_sparse_pairings_8192x4096_keep0.1", "group": 128, "K": 8},
        "points": pts,
        "roofline": {"bound": "hbm", "achieved": head["gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": head["frac"], "traffic": None},
    }


def bench_backward(args, paro, torch):
    """Gradients of the transform (paro_rotation_backward) at the prefill shape,
    8192 x 4096, K = 8: activation side and weight side with the input
    gradient, and the activation side with angle and scale gradients only."""
    import synthetic
    T = Timer(torch)
    M, d, K = 8192, 4096, 8
    ring = args.ring or 4
    x, layer = synthetic.rotation_case(seed=11, M=M, d=d, group=128, K=K)
    r = paro.Rotation(layer.pairs, layer.theta, layer.alpha, 128)
    g = synthetic.rng_for(4100, 11).standard_normal((M, d)).astype(np.float32)
    xs = [torch.from_numpy(x).cuda()] + [None] * (ring - 1)
    gs = [torch.from_numpy(g).cuda()] + [None] * (ring - 1)
    for k in range(1, ring):
        xs[k] = xs[0].clone()
        gs[k] = gs[0].clone()
    gx = torch.empty((M, d), dtype=torch.float32, device="cuda")
    dth = torch.empty((K, d // 2), dtype=torch.float32, device="cuda")
    dal = torch.empty((d,), dtype=torch.float32, device="cuda")
    need = paro.paro_rotation_backward_workspace_size(r, M)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    lib = paro.load_library()
    import ctypes

    def call(i, side, with_gx):
        k = i % ring
        st = lib.paro_rotation_backward(
            r.handle, paro.SIDES[side], ctypes.c_void_p(xs[k].data_ptr()),
            ctypes.c_void_p(gs[k].data_ptr()), ctypes.c_void_p(gx.data_ptr()) if with_gx else None,
            ctypes.c_void_p(dth.data_ptr()), ctypes.c_void_p(dal.data_ptr()), M,
            ctypes.c_void_p(ws.data_ptr()), need, None)
        assert st == 0, paro.STATUS.get(st, st)

    ys = [torch.empty_like(xs[0]) for _ in range(ring)]
    cases = [("activation", True), ("weight", True), ("activation", False)]
    fns = [lambda i, c=c: call(i, *c) for c in cases]
    fns.append(lambda i: paro.paro_rotate(r, xs[i % ring], ys[i % ring]))
    settle(torch, fns, args.warmup + 2)
    n = max(args.steps, 20)
    times = [[] for _ in fns]
    for _ in range(2):
        for f, tl in zip(fns, times):
            s = T.event()
            for i in range(n):
                f(i)
            e = T.event()
            torch.cuda.synchronize()
            tl.append(s.elapsed_time(e) / n)
    ms = [float(np.mean(t)) for t in times]
    part = need  # partial sums: written once, read once
    pts = []
    for (side, with_gx), t in zip(cases, ms):
        alg = (2 + 4 + (4 if with_gx else 0)) * M * d
        gbps = alg / (t * 1e-3) / 1e9
        pts.append({"side": side, "input_gradient": with_gx, "us": round(t * 1e3, 2),
                    "algorithmic_bytes": alg, "partial_sum_bytes": 2 * part, "gbps": round(gbps, 1),
                    "frac": round(gbps / HBM_PEAK_GBPS, 4)})
        log(f"[backward] {side} gx={with_gx}: {t*1e3:.1f} us, {gbps:.0f} GB/s")
    fwd_us = ms[-1] * 1e3
    log(f"[backward] forward transform for reference: {fwd_us:.1f} us")
    head = pts[0]
    return {
        "metric": "transform gradient HBM GB/s (paro_rotation_backward, 8192 x 4096, K = 8)",
        "value": head["gbps"], "unit": "GB/s", "n_gpus": 1, "steps": n, "warmup": args.warmup,
        "ms_per_step": round(head["us"] / 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "rotation_backward_8192x4096_K8", "group": 128, "K": K},
        "points": pts, "forward_transform_us": round(fwd_us, 2),
        "roofline": {"bound": "hbm", "achieved": head["gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": head["frac"],
                     "traffic": traffic_for("rotate_backward:8192x4096_K8"),
                     "note": "achieved over the whole call (gradient kernel + chunk reduction); "
                             "traffic is the gradient kernel's"},
    }


def bench_calib(args, paro, torch):
    """The layer-wise loss and its straight-through angle/scale gradients
    (paro_layer_loss) for a Llama-3-8B q_proj-shaped layer (4096 -> 4096,
    K = 8, G = 128) on a batch of 2048 calibration tokens: one step of the
    transform-learning loop, without the optimizer update."""
    import synthetic
    T = Timer(torch)
    M, d, N = 2048, 4096, 4096
    x, layer, _ = synthetic.linear_case(seed=21, M=M, d=d, N=N, bias=False)
    r = paro.Rotation(layer.pairs, layer.theta, layer.alpha, 128)
    xd = torch.from_numpy(x).cuda()
    wd = torch.from_numpy(layer.w).cuda()
    qw, sc, zr = paro.paro_quantize_weights(r, wd, 128)
    lib = paro.load_library()
    out = {}
    for grads in (True, False):
        need = int(lib.paro_layer_loss_workspace_size(r.handle, M, N, d, int(grads)))
        ws = torch.zeros(need, dtype=torch.uint8, device="cuda")

        def step(i, grads=grads, ws=ws):
            return paro.paro_layer_loss(r, xd, wd, qw, sc, zr, gradients=grads, workspace=ws)
        settle(torch, [step], args.warmup + 2, seconds=0.3)
        n = max(args.steps, 10)
        s = T.event()
        for i in range(n):
            res = step(i)
        e = T.event()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / n
        out[grads] = (ms, float(res[0].item()))
        log(f"[calib] gradients={grads}: {ms:.3f} ms per step, loss {out[grads][1]:.6g}")
    ms, loss = out[True]
    return {
        "metric": "transform-learning step: layer loss + angle/scale gradients (ms)", "value": round(ms, 4),
        "unit": "ms", "n_gpus": 1, "steps": max(args.steps, 10), "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16/f32", "data": "synthetic",
        "config": {"workload": "layer_loss_q_proj_2048x4096to4096_K8", "group": 128, "K": 8},
        "loss_only_ms": round(out[False][0], 4), "loss": loss,
        "calibration_tokens_per_s": round(M / (ms * 1e-3), 1),
        "roofline": None,
        "note": "three matrix-core products per step, all in this library (the W4 layer; X W^T "
                "with the loss and dY in its epilogue; dY E from fp16 operands, fp32 out); "
                "per-kernel durations in the committed rocprofv3 summary",
    }


def bench_chain(args, paro, torch):
    """The seven linears of one Llama-3-8B decoder layer in sequence (q, k, v, o,
    gate, up, down; attention and activations left out), as rotated W4G128,
    plain W4G128 and dense fp16 (torch.matmul, i.e. hipBLASLt) chains."""
    import synthetic
    layers = synthetic.decoder_layer()
    ring = args.ring or 2
    T = Timer(torch)
    plans, qr, qp, wf = [], [], [], []
    for name, layer in layers:
        r = paro.Rotation(layer.pairs, layer.theta, layer.alpha, 128)
        w = torch.from_numpy(layer.w).cuda()
        q1 = paro.paro_quantize_weights(r, w, 128)
        p1 = paro.paro_quantize_weights(None, w, 128)
        plans.append(r)
        qr.append([q1] + [tuple(t.clone() for t in q1) for _ in range(ring - 1)])
        qp.append([p1] + [tuple(t.clone() for t in p1) for _ in range(ring - 1)])
        wf.append([w] + [w.clone() for _ in range(ring - 1)])
    torch.cuda.synchronize()
    res = {}
    for M in [int(v) for v in args.chain_m.split(",")]:
        xs = [torch.from_numpy(synthetic.decoder_x(i, M)).cuda() for i in range(len(layers))]
        ys = [torch.empty((M, layers[i][1].w.shape[0]), dtype=torch.float16, device="cuda")
              for i in range(len(layers))]
        wsr = [paro.new_workspace(plans[i], M, ys[i].shape[1], xs[i].shape[1]) for i in range(len(layers))]
        wsp = [paro.new_workspace(None, M, ys[i].shape[1], xs[i].shape[1]) for i in range(len(layers))]

        def chain(kind, k):
            for i in range(len(layers)):
                if kind == "rot":
                    paro.paro_w4_linear(plans[i], xs[i], *qr[i][k], y=ys[i], workspace=wsr[i])
                elif kind == "plain":
                    paro.paro_w4_linear(None, xs[i], *qp[i][k], y=ys[i], workspace=wsp[i])
                else:
                    torch.matmul(xs[i], wf[i][k].t(), out=ys[i])

        kinds = ("rot", "plain", "fp16")
        settle(torch, [lambda k, c=c: chain(c, k % ring) for c in kinds], max(2, args.warmup))
        # eager chains launched from Python (host-bound for small M; for reference)
        eager = {c: 0.0 for c in kinds}
        for kind in kinds:
            n = max(args.steps, 20)
            s = T.event()
            for k in range(n):
                chain(kind, k % ring)
            e = T.event()
            torch.cuda.synchronize()
            eager[kind] = s.elapsed_time(e) / n
        # GPU time: each chain captured in a HIP graph (over the ring of weight
        # copies) and replayed; two alternating rounds, the mean of both
        timing = {c: 0.0 for c in kinds}
        checks = {}
        for _ in range(2):
            for kind in kinds:
                us, ok = graph_us(torch, lambda k, c=kind: chain(c, k % ring), max(ring, 4), out=ys[-1])
                timing[kind] += us / 1e3 / 2
                checks[kind] = checks.get(kind, True) and ok
        # per-linear GPU times, rotated W4 and fp16: each linear in a graph of
        # its own, alternating its weight copies (small layers then partly hit
        # the 256 MB Infinity Cache, for both variants alike)
        def one(kind, i, k):
            if kind == "rot":
                paro.paro_w4_linear(plans[i], xs[i], *qr[i][k], y=ys[i], workspace=wsr[i])
            else:
                torch.matmul(xs[i], wf[i][k].t(), out=ys[i])

        per = {}
        for kind in ("rot", "fp16"):
            per[kind] = [round(graph_us(torch, lambda k, c=kind, i=i: one(c, i, k % ring), 4 * ring,
                                        seconds=0.05)[0], 1) for i in range(len(layers))]
        res[f"M{M}"] = {
            "per_linear_us": {layers[i][0]: {"rotated_w4": per["rot"][i], "fp16": per["fp16"][i]}
                              for i in range(len(layers))},
            "rotated_w4_us": round(1e3 * timing["rot"], 1), "plain_w4_us": round(1e3 * timing["plain"], 1),
            "fp16_us": round(1e3 * timing["fp16"], 1),
            "speedup_vs_fp16": round(timing["fp16"] / timing["rot"], 3),
            "overhead_vs_plain_pct": round(100 * (timing["rot"] - timing["plain"]) / timing["plain"], 1),
            "eager_python_us": {k: round(1e3 * v, 1) for k, v in eager.items()},
            "graph_replay_equals_eager": checks,
        }
        log(f"[bench] chain M={M}: {res[f'M{M}']}")
    first = res[next(iter(res))]
    return {"metric": "decoder-layer linear chain speedup vs fp16 (rotated W4G128)",
            "value": first["speedup_vs_fp16"], "unit": "x", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(first["rotated_w4_us"] / 1e3, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
            "data": "synthetic",
            "config": {"workload": "llama3_8b_layer_linears_M" + args.chain_m.replace(",", "_"),
                       "group": 128, "stages_K": 8},
            "chain": res}


def bench_copy(args, paro, torch):
    """The library's plain device copy of 256 MiB (paro_stream_copy), for
    calibrating the HBM byte counters and as the measured copy ceiling."""
    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        paro.paro_stream_copy(a, b)
    torch.cuda.synchronize()
    T = Timer(torch)
    s = T.event()
    for _ in range(args.steps):
        paro.paro_stream_copy(a, b)
    e = T.event()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / args.steps
    return {"metric": "device copy GB/s (read + write)", "value": round(2 * n / (ms * 1e-3) / 1e9, 1),
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": 3, "ms_per_step": round(ms, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u8",
            "data": "synthetic", "config": {"workload": "copy_256MiB"}}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill_mlp",
                    choices=["prefill_mlp", "prefill_down", "decode", "sweep", "sparse", "backward",
                             "calib", "tiny", "copy", "chain"])
    ap.add_argument("--ring", type=int, default=0, help="distinct input copies cycled (0 = auto)")
    ap.add_argument("--decode-m", default="1,4,16", help="token counts of the decode workload")
    ap.add_argument("--chain-m", default="1,16,2048", help="token counts of the layer-chain workload")
    ap.add_argument("--no-cpu-baseline", dest="cpu_baseline", action="store_false")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the rotated W4G128 layer is built and measured on a "
              "single MI355X; sharding across GPUs is not run.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import rotated_w4_linear_amd as paro
    import synthetic
    paro.load_library()
    torch.cuda.set_device(0)

    if args.workload == "prefill_mlp":
        x, layer = synthetic.prefill_mlp()
        out = bench_layer(args, paro, torch, "prefill_mlp_8192x4096to14336", x, layer)
    elif args.workload == "prefill_down":
        x, layer = synthetic.prefill_down()
        out = bench_layer(args, paro, torch, "prefill_down_2048x14336to4096", x, layer)
    elif args.workload == "tiny":
        x, layer = synthetic.tiny()
        out = bench_layer(args, paro, torch, "tiny_4x256to256", x, layer)
    elif args.workload == "decode":
        out = bench_decode(args, paro, torch)
    elif args.workload == "sweep":
        out = bench_sweep(args, paro, torch)
    elif args.workload == "chain":
        out = bench_chain(args, paro, torch)
    elif args.workload == "sparse":
        out = bench_sparse(args, paro, torch)
    elif args.workload == "backward":
        out = bench_backward(args, paro, torch)
    elif args.workload == "calib":
        out = bench_calib(args, paro, torch)
    else:
        out = bench_copy(args, paro, torch)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
