"""Random rotation Pi and QJL sketch matrix S (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

noze.it "TurboQuant-MLX: quantizzare pesi e KV cache...", section "Il metodo
TurboQuant, in breve": each vector is first rotated by a random rotation, which
makes its coordinates nearly independent with a known law.  Reading taken (the
page does not say how the rotation is drawn): a Haar-distributed orthogonal
matrix, obtained as the Q factor of a seeded Gaussian matrix after fixing the
signs so that R has a positive diagonal (Mezzadri, "How to generate random
matrices from the classical compact groups", Notices AMS 2007).  With that sign
convention the factorisation A = Pi R is unique, so any correct QR gives the
same Pi up to rounding.

The QJL stage (same section: a 1-bit quantized Johnson-Lindenstrauss transform
of the residual) uses an m x d matrix S of i.i.d. standard normal entries,
drawn from its own seed and not orthogonalised.
"""
from __future__ import annotations

import numpy as np

from .rng import gaussian


def gaussian_matrix(seed: int, rows: int, cols: int) -> np.ndarray:
    """rows x cols standard normal matrix filled row-major from ``seed``."""
    return gaussian(seed, rows * cols).reshape(rows, cols)


def rotation(seed: int, d: int) -> np.ndarray:
    """Haar orthogonal Pi (d x d, float64): Q of A = QR with diag(R) made positive.

    The rotated vector is y = Pi @ x; the inverse rotation is Pi.T.
    """
    a = gaussian_matrix(seed, d, d)
    q, r = np.linalg.qr(a)  # Householder QR (LAPACK geqrf/orgqr)
    s = np.sign(np.diag(r))
    s[s == 0] = 1.0
    return q * s[None, :]


def sketch(seed: int, m: int, d: int) -> np.ndarray:
    """QJL matrix S (m x d, float64), i.i.d. N(0, 1) from ``seed``."""
    return gaussian_matrix(seed, m, d)
