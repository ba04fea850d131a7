"""Seeded synthetic inputs for the rotated W4G128 linear path.

This module only draws random numbers. It holds none of the method's
arithmetic (no rotation, no quantization, no product), so both the CPU
oracle's tests and the GPU path's tests can take their inputs from here.

Every draw comes from ``numpy.random.Generator(PCG64(SeedSequence([0x5041524F,
config_id, sub_id])))`` in a fixed order:

1. X: fp32 N(0,1) (or standard Student-t with 3 degrees of freedom), then
   outlier channels drawn uniformly without replacement whose whole column is
   multiplied by a factor, then round-to-nearest-even to fp16.
2. W in the [out][in] (nn.Linear) layout: fp32 N(0, 0.02); optional outlier
   input channels (columns) times a factor; then fp16.
3. Pairs: for each stage, for each group, ``perm = rng.permutation(G)`` and
   pairs (g*G + perm[2k], g*G + perm[2k+1]); layout [K][d/2][2], int32.
4. Angles: U(-pi, pi) in fp32, layout [K][d/2].
5. Channel scales alpha: exp(0.3 * N(0,1)) in fp32 (LogNormal(0, 0.3)).

The workloads stand in for the LLaMA-3-8B / Qwen3 layers and datasets that the
ParoQuant pages evaluate on (none of which are available here): the shapes
follow LLaMA-3-8B's q_proj (4096->4096), MLP up/gate (4096->14336) and
down-proj (14336->4096) layers and an 8K-token prefill; the values follow the
distributions stated for each workload below.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

SEED_TAG = 0x5041524F

TINY, DECODE, PREFILL_MLP, PREFILL_DOWN, SWEEP = 0, 1, 2, 3, 4

SWEEP_D = (2560, 4096, 5120)
SWEEP_K = (1, 4, 8)
SWEEP_G = (64, 128, 256)


def rng_for(config_id: int, sub_id: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_TAG, config_id, sub_id])))


@dataclasses.dataclass
class Layer:
    """One linear layer's parameters: weights plus the rotation's parameters."""
    w: Optional[np.ndarray]      # fp16 [N][d] or None (rotation-only workloads)
    pairs: np.ndarray            # int32 [K][d/2][2]
    theta: np.ndarray            # fp32 [K][d/2]
    alpha: np.ndarray            # fp32 [d]
    group: int

    @property
    def d(self) -> int:
        return int(self.alpha.shape[0])

    @property
    def K(self) -> int:
        return int(self.pairs.shape[0])


def draw_x(rng, M, d, n_outliers, factor=20.0, dist="normal") -> np.ndarray:
    if dist == "normal":
        x = rng.standard_normal((M, d), dtype=np.float32)
    elif dist == "t3":
        x = rng.standard_t(3, size=(M, d)).astype(np.float32)
    else:
        raise ValueError(dist)
    if n_outliers:
        cols = rng.choice(d, size=n_outliers, replace=False)
        x[:, cols] *= np.float32(factor)
    x16 = x.astype(np.float16)
    if not np.isfinite(x16).all():
        raise RuntimeError("synthetic activations overflowed fp16")
    return x16


def draw_w(rng, N, d, sigma=0.02, n_outlier_cols=0, factor=10.0) -> np.ndarray:
    w = (rng.standard_normal((N, d), dtype=np.float32) * np.float32(sigma))
    if n_outlier_cols:
        cols = rng.choice(d, size=n_outlier_cols, replace=False)
        w[:, cols] *= np.float32(factor)
    return w.astype(np.float16)


def draw_pairs(rng, d, group, K) -> np.ndarray:
    pairs = np.empty((K, d // 2, 2), dtype=np.int32)
    half = group // 2
    for t in range(K):
        for g in range(d // group):
            perm = rng.permutation(group).astype(np.int32) + g * group
            pairs[t, g * half:(g + 1) * half, 0] = perm[0::2]
            pairs[t, g * half:(g + 1) * half, 1] = perm[1::2]
    return pairs


def draw_theta(rng, d, K) -> np.ndarray:
    return rng.uniform(-np.pi, np.pi, size=(K, d // 2)).astype(np.float32)


def draw_alpha(rng, d) -> np.ndarray:
    return np.exp(np.float32(0.3) * rng.standard_normal(d, dtype=np.float32)).astype(np.float32)


def draw_rotation(rng, d, group, K):
    pairs = draw_pairs(rng, d, group, K)
    theta = draw_theta(rng, d, K)
    alpha = draw_alpha(rng, d)
    return pairs, theta, alpha


def draw_bias(rng, N) -> np.ndarray:
    return (rng.standard_normal(N, dtype=np.float32) * np.float32(0.1)).astype(np.float16)


def n_outliers(d: int) -> int:
    """The "1 % outlier channels" of the workloads: round(0.01 * d)."""
    return int(round(0.01 * d))


# ----------------------------------------------------------------------------
# The named workloads.
# ----------------------------------------------------------------------------

def tiny():
    """4 tokens x 256 channels, W 256x256, group 128, K = 8.

    X ~ N(0,1) with 4 outlier channels x20; W ~ N(0, 0.02) with 4 outlier
    input channels x10 (drawn independently of X's outliers)."""
    rng = rng_for(TINY)
    x = draw_x(rng, 4, 256, 4, 20.0)
    w = draw_w(rng, 256, 256, 0.02, n_outlier_cols=4, factor=10.0)
    pairs, theta, alpha = draw_rotation(rng, 256, 128, 8)
    return x, Layer(w, pairs, theta, alpha, 128)


def decode_layer(d=4096, N=4096, group=128, K=8) -> Layer:
    """q_proj-like 4096 -> 4096 layer shared by the decode token counts."""
    rng = rng_for(DECODE, 0)
    w = draw_w(rng, N, d, 0.02)
    pairs, theta, alpha = draw_rotation(rng, d, group, K)
    return Layer(w, pairs, theta, alpha, group)


def decode_x(M: int, d=4096) -> np.ndarray:
    """Decode activations, M in {1, 4, 16}: N(0,1) with 1 % outlier channels x20."""
    return draw_x(rng_for(DECODE, M), M, d, n_outliers(d), 20.0)


def prefill_mlp(M=8192, d=4096, N=14336, group=128, K=8):
    """MLP up/gate-like prefill: 8192 tokens, 4096 -> 14336."""
    rng = rng_for(PREFILL_MLP)
    x = draw_x(rng, M, d, n_outliers(d), 20.0)
    w = draw_w(rng, N, d, 0.02)
    pairs, theta, alpha = draw_rotation(rng, d, group, K)
    return x, Layer(w, pairs, theta, alpha, group)


def prefill_down(M=2048, d=14336, N=4096, group=128, K=8):
    """Down-proj-like prefill: 2048 tokens, 14336 -> 4096, X ~ Student-t(3)."""
    rng = rng_for(PREFILL_DOWN)
    x = draw_x(rng, M, d, 0, dist="t3")
    w = draw_w(rng, N, d, 0.02)
    pairs, theta, alpha = draw_rotation(rng, d, group, K)
    return x, Layer(w, pairs, theta, alpha, group)


def sweep_points():
    """The 27 rotation-only points (d, K, G), in a fixed order."""
    return [(d, K, G) for d in SWEEP_D for K in SWEEP_K for G in SWEEP_G]


def sweep(point: int, M=8192):
    """Rotation-only workload: X fp16 [M][d], random pairs/angles/scales."""
    d, K, G = sweep_points()[point]
    rng = rng_for(SWEEP, point)
    x = draw_x(rng, M, d, n_outliers(d), 20.0)
    pairs, theta, alpha = draw_rotation(rng, d, G, K)
    return x, Layer(None, pairs, theta, alpha, G)


def rotation_case(seed: int, M: int, d: int, group: int, K: int, x_dist="normal", outliers=True):
    """A free-form rotation case for tests (seeded by ``seed``)."""
    rng = rng_for(1000, seed)
    x = draw_x(rng, M, d, n_outliers(d) if outliers else 0, 20.0, dist=x_dist) if M > 0 \
        else np.zeros((0, d), np.float16)
    pairs, theta, alpha = draw_rotation(rng, d, group, K)
    return x, Layer(None, pairs, theta, alpha, group)


def sparse_rotation_case(seed: int, M: int, d: int, group: int, K: int, keep: float):
    """A rotation case where each pair carries its angle with probability
    ``keep`` and is otherwise an exact identity (theta = 0): a sparse pairing
    in which only a fraction of the channel pairs rotate (a random stand-in for
    keeping only the most useful pairs)."""
    x, layer = rotation_case(seed, M, d, group, K)
    rng = rng_for(1500, seed)
    drop = rng.random(layer.theta.shape) >= keep
    layer.theta[drop] = 0.0
    return x, layer


def linear_case(seed: int, M: int, d: int, N: int, group: int = 128, K: int = 8, bias=True):
    """A free-form linear-layer case for tests (seeded by ``seed``)."""
    rng = rng_for(2000, seed)
    x = draw_x(rng, M, d, n_outliers(d), 20.0) if M > 0 else np.zeros((0, d), np.float16)
    w = draw_w(rng, N, d, 0.02)
    pairs, theta, alpha = draw_rotation(rng, d, group, K)
    b = draw_bias(rng, N) if bias else None
    return x, Layer(w, pairs, theta, alpha, group), b


# Llama-3-8B decoder-layer linears (name, in_features d, out_features N).
DECODER_LINEARS = [("q_proj", 4096, 4096), ("k_proj", 4096, 1024), ("v_proj", 4096, 1024),
                   ("o_proj", 4096, 4096), ("gate_proj", 4096, 14336), ("up_proj", 4096, 14336),
                   ("down_proj", 14336, 4096)]


def decoder_layer():
    """The seven linears of one Llama-3-8B decoder layer, each with its own
    rotation (group 128, K = 8) and W ~ N(0, 0.02): [(name, Layer)]."""
    out = []
    for i, (name, d, N) in enumerate(DECODER_LINEARS):
        rng = rng_for(6, i)
        w = draw_w(rng, N, d, 0.02)
        pairs, theta, alpha = draw_rotation(rng, d, 128, 8)
        out.append((name, Layer(w, pairs, theta, alpha, 128)))
    return out


def decoder_x(i: int, M: int) -> np.ndarray:
    """Activations for linear i of decoder_layer() at M tokens (1 % outliers x20)."""
    d = DECODER_LINEARS[i][1]
    rng = rng_for(7, 1000 * i + M)
    return draw_x(rng, M, d, n_outliers(d), 20.0)

