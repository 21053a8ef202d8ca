"""Seeded random streams for the rotation and the QJL sketch (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages only say the rotation is random and seeded per cache (noze.it
"TurboQuant-MLX: quantizzare pesi e KV cache...", section "Il metodo
TurboQuant, in breve": the vector is rotated at random before quantization).
They do not name a generator, so both sides implement the same published,
counter-based one independently:

* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014): the state advances by the odd constant
  0x9E3779B97F4A7C15 and every output is the 64-bit finalizer of the new
  state (xor-shift 30, multiply, xor-shift 27, multiply, xor-shift 31).
* A uniform double in [0, 1) is the top 53 bits times 2**-53.
* Gaussians come from Box-Muller on consecutive pairs (u_a, u_b):
  r = sqrt(-2 ln(1 - u_a)), then r cos(2 pi u_b) followed by r sin(2 pi u_b).
  Matrices are filled row-major in draw order.
"""
from __future__ import annotations

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def splitmix64(seed: int, count: int) -> np.ndarray:
    """The first ``count`` SplitMix64 outputs for ``seed`` as uint64.

    Counter form: the k-th state (k = 1, 2, ...) is seed + k * golden (mod 2**64),
    and the output is the finalizer of that state.
    """
    k = np.arange(1, count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + k * _GOLDEN
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def uniform01(seed: int, count: int) -> np.ndarray:
    """Doubles in [0, 1): top 53 bits of each output times 2**-53 (exact)."""
    z = splitmix64(seed, count)
    return (z >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def gaussian(seed: int, count: int) -> np.ndarray:
    """``count`` standard normal doubles by Box-Muller over SplitMix64 pairs."""
    pairs = (count + 1) // 2
    u = uniform01(seed, 2 * pairs)
    ua, ub = u[0::2], u[1::2]
    r = np.sqrt(-2.0 * np.log(1.0 - ua))
    ang = 2.0 * np.pi * ub
    g = np.empty(2 * pairs, dtype=np.float64)
    g[0::2] = r * np.cos(ang)
    g[1::2] = r * np.sin(ang)
    return g[:count]
