"""CPU oracle for choosing the channel pairs of the rotation stages.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle``): only the test suite,
the package's smoke check and the benchmark's CPU-baseline leg may import it.
It shares no code with the library's host implementation.

Sources:
  [Notes] "局限与展望": the authors choose the pairs of the independent
          rotations at random, with de-duplication.
  [Notes] "核心观察": a sparse rotation keeping only the top-10% channel pairs
          matches the full rotation.
  [CSDN]  section 2.2: pairs of channels whose values differ strongly are
          preferred (saliency); every channel is in at most one pair of a
          stage; stages run group by group.

The exact rules are readings (each stated below and in the design notes).
Random draws come from SplitMix64, whose definition (the state advances by
0x9E3779B97F4A7C15; the output is the state through two xor-shift-multiply
rounds and a final xor-shift) is public, so both implementations reproduce
every draw.
"""
from __future__ import annotations

import numpy as np

MASK64 = (1 << 64) - 1


class SplitMix64:
    """SplitMix64 (Steele, Lea, Flood 2014) on Python integers."""

    def __init__(self, seed: int):
        self.state = seed & MASK64

    def next(self) -> int:
        self.state = (self.state + 0x9E3779B97F4A7C15) & MASK64
        z = self.state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
        return z ^ (z >> 31)


def shuffle(rng: SplitMix64, n: int) -> list:
    """A uniformly random permutation of 0..n-1 (Fisher-Yates from the last
    position down: position i swaps with j = r mod (i + 1))."""
    order = list(range(n))
    for i in range(n - 1, 0, -1):
        j = rng.next() % (i + 1)
        order[i], order[j] = order[j], order[i]
    return order


def pairs_random(d: int, group: int, K: int, seed: int, max_draws: int = 4096) -> np.ndarray:
    """Random pairs with de-duplication ([Notes] "局限与展望").

    Reading: for each group in order and each stage in order, draw a random
    permutation of the group's channels; walk positions 0, 2, 4, ...: the
    channel at the position takes as partner the first later channel it was
    not paired with in an earlier stage of the group, which is exchanged into
    the next position; if no such channel is left, the whole stage is drawn
    again. One SplitMix64 stream serves every draw of the call.
    Returns int32 [K][d/2][2] global channel ids (pair p of a stage in group
    p // (group / 2)), each stored as (channel, partner).
    """
    if group < 2 or group % 2 or d % group or not 0 <= K <= group - 1:
        raise ValueError("bad sizes")
    rng = SplitMix64(seed)
    half = group // 2
    out = np.zeros((K, d // 2, 2), dtype=np.int32)
    for g in range(d // group):
        seen = set()  # unordered pairs of this group used by earlier stages
        for t in range(K):
            for _ in range(max_draws):
                order = shuffle(rng, group)
                ok = True
                for i in range(0, group, 2):
                    a = order[i]
                    partner = None
                    for k in range(i + 1, group):
                        if frozenset((a, order[k])) not in seen:
                            partner = k
                            break
                    if partner is None:
                        ok = False
                        break
                    order[i + 1], order[partner] = order[partner], order[i + 1]
                if ok:
                    break
            else:
                raise RuntimeError("no pairing without repeated pairs found")
            for p in range(half):
                a, b = order[2 * p], order[2 * p + 1]
                seen.add(frozenset((a, b)))
                out[t, g * half + p] = (g * group + a, g * group + b)
    return out


def pairs_by_gap(score, group: int, K: int) -> np.ndarray:
    """Pairs of channels whose values differ strongly ([CSDN] section 2.2).

    Reading: rank each group's channels by ``score`` (largest first, ties by
    channel index); stage t pairs the i-th largest with the
    ((i + t) mod (group/2))-th smallest, stored as (larger, smaller).
    """
    score = np.asarray(score, dtype=np.float32)
    d = score.shape[0]
    half = group // 2
    if group < 2 or group % 2 or d % group or not 0 <= K <= half:
        raise ValueError("bad sizes")
    if not np.all(np.isfinite(score)):
        raise ValueError("non-finite score")
    out = np.zeros((K, d // 2, 2), dtype=np.int32)
    for g in range(d // group):
        local = [float(v) for v in score[g * group:(g + 1) * group]]
        ranked = sorted(range(group), key=lambda k: (-local[k], k))
        smallest_first = ranked[::-1]
        for t in range(K):
            for i in range(half):
                out[t, g * half + i] = (g * group + ranked[i], g * group + smallest_first[(i + t) % half])
    return out


def sparsify_angles(theta, n_keep: int) -> np.ndarray:
    """Keep the ``n_keep`` strongest rotations ([Notes] "核心观察", top-10%).

    Reading: rank every pair of the plan by |theta| (largest first; ties: the
    earlier stage and pair first); the first n_keep keep their angle, the
    others become exact identities (theta = 0).
    """
    theta = np.asarray(theta, dtype=np.float32)
    flat = theta.reshape(-1)
    if not 0 <= n_keep <= flat.size:
        raise ValueError("n_keep out of range")
    if not np.all(np.isfinite(flat)):
        raise ValueError("non-finite angle")
    order = np.lexsort((np.arange(flat.size), -np.abs(flat)))
    out = np.zeros_like(flat)
    keep = order[:n_keep]
    out[keep] = flat[keep]
    return out.reshape(theta.shape)
