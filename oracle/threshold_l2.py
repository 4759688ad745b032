"""fp64 CPU oracle for the Threshold-l2 keep-mask (the pruning step that
produces the mask the ragged path consumes).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU-baseline leg may import this module.  The HIP library never calls it and
shares no code with it.

The pages name Threshold-l2 as one of the four token-pruning algorithms the
pipeline is evaluated with (aissential.tech summary, "Summary") and say
nothing more about it.  The plain reading used here, stated in full:

  * the score of token j of image b is the Euclidean norm of its embedding
    row x[b, j, :] (C channels);
  * token 0 (CLS) is always kept and takes no part in the ranking;
  * among the P = N - 1 patch tokens, a patch is kept when its norm is at
    least the per-image keep-quantile q of the patch norms, the quantile
    taken with linear interpolation between order statistics.

In exact arithmetic the linear-interpolation quantile at position
q * (P - 1) lies strictly between the order statistics s_(lo) and s_(lo+1)
(lo = floor of the position) unless the position is whole, so "norm >=
quantile" keeps exactly the patches whose norm is at least the
r0-th smallest norm (0-based), r0 = ceil(q * (P - 1)); with ties the
interpolated value equals the tied order statistic, and the same holds.
That order-statistic form is what is computed here: patch j is kept when at
least r0 + 1 patch norms (its own included) are at most its own, which is
"its norm reaches the r0-th smallest".  It has no rounding of an
interpolated threshold in it, so its result is unique.

The squared norm decides, as a monotone stand-in for the norm.  It is the
fp64 sum of the exact fp64 squares of the input values, added in channel
order c = 0, 1, ..., C - 1 (one rounding per addition).  Fixing the order
makes the fp64 value unique, so a device computing the same sum in the same
order takes identical keep decisions.

Pins (tests/test_oracle_threshold.py): the channel-order sum against
math.fsum (exactly rounded), the mask against numpy's linear-interpolation
quantile rule on inputs without near-ties, a brute-force sort-and-threshold
loop on tiny inputs, the closed-form kept count P - r0 for distinct norms,
and the special cases q = 0 (every patch) and q = 1 (only the largest).
"""
from __future__ import annotations

import math

import numpy as np

from .ragged import decode


def sq_norms(x: np.ndarray, dtype: str) -> np.ndarray:
    """Squared L2 norm of every token row: x [B, N, C] device bits ->
    float64 [B, N], summed in channel order."""
    xf = decode(x, dtype)
    acc = np.zeros(xf.shape[:-1], dtype=np.float64)
    for c in range(xf.shape[-1]):
        col = xf[..., c]
        acc = acc + col * col  # the square is exact in fp64; one rounding per add
    return acc


def keep_rank(N: int, keep_quantile: float) -> int:
    """r0 = ceil(q * (P - 1)) with P = N - 1 patches: the 0-based order
    statistic a kept patch's norm must reach."""
    P = N - 1
    if P <= 0:
        return 0
    return int(math.ceil(keep_quantile * (P - 1)))


def threshold_l2_mask(x: np.ndarray, dtype: str, keep_quantile: float) -> np.ndarray:
    """uint8 [B, N]: 1 for CLS and for every patch whose norm reaches the
    per-image keep-quantile of the patch norms (order-statistic form)."""
    if not 0.0 <= keep_quantile <= 1.0:
        raise ValueError("keep_quantile must lie in [0, 1]")
    s = sq_norms(x, dtype)
    B, N = s.shape
    r0 = keep_rank(N, keep_quantile)
    mask = np.zeros((B, N), dtype=np.uint8)
    mask[:, 0] = 1
    for b in range(B):
        patches = s[b, 1:]
        # for each patch j: how many patch norms are at most its own (itself included)
        at_most = (patches[None, :] <= patches[:, None]).sum(axis=1)
        mask[b, 1:] = (at_most >= r0 + 1).astype(np.uint8)
    return mask
