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

The same page, section "Cosa aggiunge turboquant-mlx", notes that one port
realises the random rotation with a Hadamard transform; ``hadamard_rotation``
is that option (its reading is in its docstring).

The QJL stage (section "Il metodo TurboQuant, in breve": a 1-bit quantized JL transform
of the residual) uses an m x d matrix S of i.i.d. standard normal entries,
drawn from its own seed and not orthogonalised.
"""
from __future__ import annotations

import numpy as np

from .rng import gaussian, splitmix64


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


def sylvester_hadamard(d: int) -> np.ndarray:
    """Sylvester's Hadamard matrix of order d (a power of two), float64:
    H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def hadamard_signs(seed: int, d: int) -> np.ndarray:
    """sigma_k = -1 when bit 63 of the k-th SplitMix64 output of ``seed`` is set, else +1."""
    top = splitmix64(seed, d) >> np.uint64(63)
    return np.where(top == 1, -1.0, 1.0)


def hadamard_rotation(seed: int, d: int) -> np.ndarray:
    """Randomized Hadamard rotation Pi = H_d diag(sigma) / sqrt(d) (float64).

    noze.it page, section "Cosa aggiunge turboquant-mlx": the port realises
    the random rotation as a Hadamard transform, the fast and cheap way.
    Reading taken (the page gives no construction): random sign flips drawn
    from the seed, applied before the transform, and the 1/sqrt(d) that makes
    the matrix orthogonal.  y = Pi @ x as for the Haar rotation.
    """
    return sylvester_hadamard(d) * hadamard_signs(seed, d)[None, :] / np.sqrt(d)


def sketch(seed: int, m: int, d: int) -> np.ndarray:
    """QJL matrix S (m x d, float64), i.i.d. N(0, 1) from ``seed``."""
    return gaussian_matrix(seed, m, d)
