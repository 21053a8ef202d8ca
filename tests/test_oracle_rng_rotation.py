"""Pins of the oracle's random streams, rotation and sketch (CPU only)."""
import math

import numpy as np
import pytest

from conftest import read_golden
from oracle import rng, rotation


def test_splitmix64_known_answers():
    want = [int(r[0], 16) for r in read_golden("splitmix64_seed0.txt")]
    got = [int(v) for v in rng.splitmix64(0, len(want))]
    assert got == want


def test_uniform_and_box_muller_first_pair():
    # First pair from the known-answer integers, through the math module.
    ints = [int(r[0], 16) for r in read_golden("splitmix64_seed0.txt")]
    ua = (ints[0] >> 11) * 2.0 ** -53
    ub = (ints[1] >> 11) * 2.0 ** -53
    r = math.sqrt(-2.0 * math.log(1.0 - ua))
    g = rng.gaussian(0, 4)
    assert g[0] == pytest.approx(r * math.cos(2 * math.pi * ub), rel=1e-15, abs=1e-15)
    assert g[1] == pytest.approx(r * math.sin(2 * math.pi * ub), rel=1e-15, abs=1e-15)
    u = rng.uniform01(0, 2)
    assert u[0] == ua and u[1] == ub


def test_gaussian_moments():
    n = 1_000_000
    g = rng.gaussian(123, n)
    se = 1.0 / math.sqrt(n)
    assert abs(g.mean()) < 5 * se
    assert abs(g.var() - 1.0) < 5 * math.sqrt(2.0) * se
    assert abs(np.mean(g ** 4) - 3.0) < 5 * math.sqrt(96.0) * se


def test_gaussian_odd_count_is_prefix():
    assert np.array_equal(rng.gaussian(7, 5), rng.gaussian(7, 6)[:5])


@pytest.mark.parametrize("d", [8, 128])
def test_rotation_orthogonal_and_norm_preserving(d):
    pi = rotation.rotation(0, d)
    assert np.max(np.abs(pi @ pi.T - np.eye(d))) <= 1e-13
    x = np.random.default_rng(1).standard_normal((16, d))
    y = x @ pi.T
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14, atol=0)


@pytest.mark.parametrize("seed", [0, 5])
def test_rotation_is_the_positive_diagonal_qr_factor(seed):
    # A = Pi R with R upper triangular and diag(R) > 0 fixes Pi uniquely.
    d = 128
    a = rotation.gaussian_matrix(seed, d, d)
    pi = rotation.rotation(seed, d)
    r = pi.T @ a
    assert np.max(np.abs(np.tril(r, -1))) < 1e-11
    assert np.all(np.diag(r) > 0)
    # Gram-Schmidt of the columns of A, written independently of LAPACK.
    q = np.zeros_like(a)
    for j in range(d):
        v = a[:, j].copy()
        for _ in range(2):
            v -= q[:, :j] @ (q[:, :j].T @ v)
        q[:, j] = v / np.linalg.norm(v)
    assert np.max(np.abs(q - pi)) < 1e-11


def test_rotation_is_haar_moments():
    # Haar on O(d): E[Pi_ij^2] = 1/d, E[tr Pi] = 0, E[(tr Pi)^2] = 1.
    d, n = 8, 3000
    tr = np.empty(n)
    sq = np.zeros((d, d))
    for s in range(n):
        p = rotation.rotation(1000 + s, d)
        tr[s] = np.trace(p)
        sq += p * p
    sq /= n
    assert np.max(np.abs(sq - 1.0 / d)) < 0.02
    assert abs(tr.mean()) < 5 * tr.std() / math.sqrt(n)
    assert abs(np.mean(tr ** 2) - 1.0) < 0.12


def test_sketch_is_rowmajor_gaussian_stream():
    s = rotation.sketch(1, 128, 128)
    assert s.shape == (128, 128)
    assert np.array_equal(s.ravel(), rng.gaussian(1, 128 * 128))


@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 32, 64, 128])
def test_sylvester_hadamard_is_scipys(d):
    from scipy.linalg import hadamard
    assert np.array_equal(rotation.sylvester_hadamard(d), hadamard(d).astype(np.float64))


def test_hadamard_signs_are_the_top_bits_of_splitmix64():
    want = [-1.0 if int(r[0], 16) >> 63 else 1.0 for r in read_golden("splitmix64_seed0.txt")]
    assert rotation.hadamard_signs(0, len(want)).tolist() == want


def test_hadamard_rotation_worked_example_d4():
    # seed 0: the first four SplitMix64 outputs have top bits 1, 0, 0, 1, so
    # sigma = (-1, +1, +1, -1); Pi = H_4 diag(sigma) / 2, written out by hand
    want = np.array([[-1, 1, 1, -1], [-1, -1, 1, 1], [-1, 1, -1, 1], [-1, -1, -1, -1]], dtype=np.float64) / 2.0
    assert np.array_equal(rotation.hadamard_rotation(0, 4), want)


@pytest.mark.parametrize("seed", [0, 9])
def test_hadamard_rotation_orthogonal_with_flat_entries(seed):
    d = 128
    pi = rotation.hadamard_rotation(seed, d)
    assert np.max(np.abs(pi @ pi.T - np.eye(d))) <= 1e-14
    assert np.max(np.abs(np.abs(pi) * math.sqrt(d) - 1.0)) <= 1e-15
    # first row is sigma / sqrt(d): the signs are the seed's
    assert np.array_equal(np.sign(pi[0]), rotation.hadamard_signs(seed, d))
