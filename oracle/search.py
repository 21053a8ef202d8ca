"""Inner-product search over quantized vectors (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

noze.it "TurboQuant-MLX: quantizzare pesi e KV cache...", section "Il metodo
TurboQuant, in breve": similarity search, in place of product quantization,
is the method's second application, and the 1-bit sketch of the residual is
what removes the bias of the inner-product estimate.  For a query q and a
stored vector x with norm n, rotated unit vector y = Pi x / n, codes idx and
(with the sketch) residual r = y - c[idx], gamma = ||r||, z = sign(S r):

    est(q, x) = n ( <Pi q, c[idx]> + sqrt(pi/2)/m gamma <S Pi q, z> ),

the second term only when the spec carries the sketch.  Since Pi is
orthogonal, n <Pi q, y> = <q, x>, and over the draw of S the sketch term has
mean n <Pi q, r>, so the estimate is unbiased.
"""
from __future__ import annotations

import numpy as np

from .quantize import Spec, dequantize_rotated, rotation_of, sketch_of


def ip_scores_rotated(q: np.ndarray, yhat: np.ndarray, norms: np.ndarray, spec: Spec,
                      z: np.ndarray | None = None, gamma: np.ndarray | None = None) -> np.ndarray:
    """[nq, N] estimates from rotated unit reconstructions yhat [N, d] (and,
    with the sketch, signs z [N, m] in {-1, +1} and residual norms gamma [N])."""
    qr = np.asarray(q, np.float64) @ rotation_of(spec).T
    dots = qr @ np.asarray(yhat, np.float64).T
    if spec.qjl_m:
        u = qr @ sketch_of(spec).T
        dots = dots + np.sqrt(np.pi / 2) / spec.qjl_m * np.asarray(gamma, np.float64)[None, :] * (
            u @ np.asarray(z, np.float64).T)
    return np.asarray(norms, np.float64)[None, :] * dots


def ip_scores(q: np.ndarray, idx: np.ndarray, norms: np.ndarray, spec: Spec,
              bits: np.ndarray | None = None, gamma: np.ndarray | None = None) -> np.ndarray:
    """Estimates from stored codes idx [N, d] (and sketch bits [N, m] as 0/1)."""
    z = None if bits is None else np.where(np.asarray(bits) != 0, 1.0, -1.0)
    return ip_scores_rotated(q, dequantize_rotated(idx, spec), norms, spec, z, gamma)
