"""The comparison rules themselves, exercised with mistakes planted in a copy of
the oracle's own codes (CPU only)."""
import numpy as np

from oracle import parity, quantize as qz


def _codes():
    spec = qz.Spec(bits_lo=4, bits_hi=4)
    x = np.random.default_rng(0).standard_normal((2048, 128))
    return spec, qz.quantize(x, spec)


def test_identical_codes_pass():
    spec, q = _codes()
    assert parity.compare_codes(q.idx, q.idx.copy(), q.y, spec).ok


def test_off_by_one_inside_band_passes():
    spec, q = _codes()
    dist = parity.boundary_distance(q.y, spec)
    n, i = np.unravel_index(np.argmin(dist), dist.shape)
    assert dist[n, i] < 1e-6
    other = q.idx.copy()
    other[n, i] += 1 if other[n, i] < 15 else -1
    rep = parity.compare_codes(q.idx, other, q.y, spec)
    assert rep.mismatches == 1 and rep.ok


def test_mismatch_outside_band_fails():
    spec, q = _codes()
    other = q.idx.copy()
    dist = parity.boundary_distance(q.y, spec)
    n, i = np.unravel_index(np.argmax(dist), dist.shape)
    other[n, i] = (other[n, i] + 1) % 16
    assert not parity.compare_codes(q.idx, other, q.y, spec).ok


def test_too_many_band_mismatches_fail():
    spec, q = _codes()
    # pretend every coordinate is in the band: the count cap still applies
    y = np.zeros_like(q.y)
    other = q.idx.copy()
    other[:10, 0] ^= 1
    rep = parity.compare_codes(q.idx, other, y, spec, max_frac=1e-6)
    assert not rep.ok


def test_rel_l2():
    a = np.ones(10)
    assert parity.rel_l2(a * (1 + 1e-3), a) == np.float64(1e-3).round(12) or abs(parity.rel_l2(a * (1 + 1e-3), a) - 1e-3) < 1e-12
