"""Independent re-derivation of the hash draws from their published definition.

TEST INFRASTRUCTURE ONLY.  The library draws the random-binning hashes
(delta, u) on the host from a 64-bit seed; the oracle never needs them drawn
(it takes (delta, u) as inputs, like Q, K, V), but the draw itself is pinned
here bit for bit from the generator's published definition.

Hash law [P, Methodology 1] and [P, Theorem 2.1]: random binning features
for the Laplace kernel exp(-|x - y| / sigma) draw a bin width
delta ~ Gamma(shape 2, scale sigma) and an offset u ~ Uniform[0, delta).

Generator: SplitMix64 (G. L. Steele Jr., D. Lea, C. H. Flood, "Fast
splittable pseudorandom number generators", OOPSLA 2014), used in counter
mode: the value for counter c is the (c+1)-th output of SplitMix64 started
from state ``seed``, i.e. mix64(seed + (c + 1) * GAMMA) mod 2^64.

Draw of hash i of head h (h < 2^31, i < 2^30), for k in {0, 1, 2}:

    c_k = (h << 32) | (i << 2) | k
    z_k = mix64(seed + (c_k + 1) * GAMMA)
    U_k = ((z_k >> 12) + 0.5) * 2^-52            (exact; 0 < U_k < 1)
    delta = sigma_h * ((-log U_0) - log U_1)      (sum of two Exp(1) = Gamma(2,1))
    u     = delta * U_2

All arithmetic is IEEE binary64 in exactly this order; ``log`` is the C
library's natural logarithm (``math.log``).
"""

from __future__ import annotations

import math

import numpy as np

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15


def _mix64(z: int) -> int:
    z &= MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def splitmix64(seed: int, count: int) -> list[int]:
    """First ``count`` outputs of SplitMix64 started from state ``seed``."""
    return [_mix64(seed + (c + 1) * GAMMA) for c in range(count)]


def _u01(z: int) -> float:
    return ((z >> 12) + 0.5) * 2.0 ** -52


def sample_hashes(seed: int, sigmas, s: int) -> tuple[np.ndarray, np.ndarray]:
    """(delta, u), each float64 [H, s], for per-head sigma and s hashes."""
    sigmas = np.atleast_1d(np.asarray(sigmas, dtype=np.float64))
    H = sigmas.size
    delta = np.empty((H, s))
    u = np.empty((H, s))
    seed &= MASK64
    for h in range(H):
        for i in range(s):
            U = []
            for k in range(3):
                c = (h << 32) | (i << 2) | k
                U.append(_u01(_mix64(seed + (c + 1) * GAMMA)))
            t = (-math.log(U[0])) - math.log(U[1])
            dl = float(sigmas[h]) * t
            delta[h, i] = dl
            u[h, i] = dl * U[2]
    return delta, u
