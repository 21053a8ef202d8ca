"""Pins of the oracle's inner-product search estimate (CPU only)."""
import dataclasses
import math

import numpy as np
import pytest

from oracle import quantize as qz
from oracle import search


def _xq(n=20, nq=3, seed=0, d=128):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((n, d)), rng.standard_normal((nq, d))


@pytest.mark.parametrize("rot", ["haar", "hadamard"])
def test_exact_reconstruction_gives_the_plain_inner_product(rot):
    # with y itself in place of the centroids (and no sketch) the estimate is
    # n <Pi q, Pi x / n> = <q, x>, for any orthogonal Pi
    x, q = _xq()
    spec = qz.Spec(bits_lo=4, bits_hi=4, rotation=rot)
    out = qz.quantize(x, spec)
    est = search.ip_scores_rotated(q, out.y, out.norms64, spec)
    assert np.max(np.abs(est - q @ x.T)) <= 1e-12 * np.abs(q @ x.T).max()


def test_zero_vector_scores_zero():
    x, q = _xq(n=4)
    x[2] = 0.0
    spec = qz.Spec(bits_lo=2, bits_hi=2, qjl_m=128)
    out = qz.quantize(x, spec)
    est = search.ip_scores(q, out.idx, out.norms64, spec, out.qjl_bits, out.rnorms)
    assert np.all(est[:, 2] == 0.0)


def test_sketch_makes_the_estimate_unbiased_over_seeds():
    # E over the sketch draw of the corrected estimate is <q, x> (the sketch
    # term has mean n <Pi q, r>); without the term the bias n <Pi q, r> stays
    x, q = _xq(n=1, nq=1, seed=3)
    x[0, :8] *= 6.0  # a vector with a large residual for a visible bias
    truth = float(q[0] @ x[0])
    est, plain = [], []
    for seed in range(600):
        spec = qz.Spec(bits_lo=2, bits_hi=2, qjl_m=128, qjl_seed=1000 + seed)
        out = qz.quantize(x, spec)
        est.append(search.ip_scores(q, out.idx, out.norms64, spec, out.qjl_bits, out.rnorms)[0, 0])
        plain.append(search.ip_scores(q, out.idx, out.norms64, dataclasses.replace(spec, qjl_m=0))[0, 0])
    est = np.array(est)
    se = est.std() / math.sqrt(len(est))
    assert abs(est.mean() - truth) < 4 * se, (est.mean(), truth, se)
    # the MSE-only estimate is the same for every sketch seed and biased by n <Pi q, r>
    assert np.ptp(plain) == 0.0
    spec = qz.Spec(bits_lo=2, bits_hi=2)
    out = qz.quantize(x, spec)
    bias = out.norms64[0] * ((qz.rotation_of(spec) @ q[0]) @ (out.y[0] - qz.dequantize_rotated(out.idx, spec)[0]))
    assert plain[0] == pytest.approx(truth - bias, rel=1e-12, abs=1e-12)
