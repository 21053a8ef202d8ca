"""Comparison rules between the oracle and another implementation.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Codes: a quantized index is decided by comparing a floating-point rotated
coordinate with the codebook thresholds, and an independent implementation
computes that coordinate with its own rounding.  A code may therefore differ
from the oracle's only where the oracle's coordinate lies within ``band``
(1e-6) of a threshold, only by one level, and such codes may be at most
``max_frac`` (1e-5) of all codes compared.  Sign bits of the QJL sketch follow
the same rule with the threshold 0 and |(S r)_j| < band, and are compared only
for vectors whose codes all matched (a differing code changes r).

Attention: relative L2 error ||out - ref|| / ||ref|| over the whole output,
bounded by 2e-3 (the outputs are computed from the same codes on both sides).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .codebook import lloyd_max
from .quantize import Spec

BAND = 1e-6
MAX_FRAC = 1e-5
ATTN_REL_L2 = 2e-3


@dataclass
class CodeReport:
    total: int
    mismatches: int
    in_band: int
    off_by_one: int
    ok: bool

    def __str__(self) -> str:
        return (f"codes={self.total} mismatches={self.mismatches} in_band={self.in_band} "
                f"off_by_one={self.off_by_one} ok={self.ok}")


def boundary_distance(y: np.ndarray, spec: Spec) -> np.ndarray:
    """min_j |y_i - t_j| per coordinate, with coordinate i's thresholds."""
    out = np.empty(y.shape)
    for sl, bits in ((slice(0, spec.split), spec.bits_lo), (slice(spec.split, spec.d), spec.bits_hi)):
        t = lloyd_max(spec.d, bits).boundaries
        yy = y[..., sl]
        pos = np.clip(np.searchsorted(t, yy), 1, len(t) - 1) if len(t) > 1 else np.zeros(yy.shape, int)
        dist = np.abs(yy - t[pos])
        if len(t) > 1:
            dist = np.minimum(dist, np.abs(yy - t[pos - 1]))
        out[..., sl] = dist
    return out


def compare_codes(idx_ref: np.ndarray, idx_other: np.ndarray, y_ref: np.ndarray, spec: Spec,
                  band: float = BAND, max_frac: float = MAX_FRAC) -> CodeReport:
    diff = idx_ref != idx_other
    n_mis = int(diff.sum())
    if n_mis == 0:
        return CodeReport(idx_ref.size, 0, 0, 0, True)
    dist = boundary_distance(y_ref, spec)
    in_band = int((diff & (dist < band)).sum())
    off1 = int((diff & (np.abs(idx_ref - idx_other) == 1)).sum())
    ok = (in_band == n_mis) and (off1 == n_mis) and (n_mis <= max_frac * idx_ref.size)
    return CodeReport(idx_ref.size, n_mis, in_band, off1, ok)


def compare_signs(bits_ref: np.ndarray, bits_other: np.ndarray, proj_ref: np.ndarray,
                  vec_ok: np.ndarray, band: float = BAND, max_frac: float = MAX_FRAC) -> CodeReport:
    """Sign bits [n, m]; only rows with vec_ok (no code mismatch) are compared."""
    br, bo, pr = bits_ref[vec_ok], bits_other[vec_ok], proj_ref[vec_ok]
    diff = br != bo
    n_mis = int(diff.sum())
    in_band = int((diff & (np.abs(pr) < band)).sum())
    ok = in_band == n_mis and n_mis <= max_frac * max(br.size, 1)
    return CodeReport(int(br.size), n_mis, in_band, n_mis, ok)


def rel_l2(out: np.ndarray, ref: np.ndarray) -> float:
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(np.asarray(out, np.float64) - ref) / np.linalg.norm(ref))
