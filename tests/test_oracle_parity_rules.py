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


# ---- QJL sign bits ----------------------------------------------------------

def _signs():
    spec = qz.Spec(bits_lo=2, bits_hi=2, qjl_m=128, qjl_seed=1)
    x = np.random.default_rng(3).standard_normal((4096, 128))
    q = qz.quantize(x, spec)
    return q, np.ones(q.qjl_bits.shape[0], dtype=bool)


def test_identical_signs_pass():
    q, ok = _signs()
    rep = parity.compare_signs(q.qjl_bits, q.qjl_bits.copy(), q.qjl_proj, ok)
    assert rep.ok and rep.mismatches == 0 and rep.total == q.qjl_bits.size


def test_sign_flip_inside_band_passes():
    q, ok = _signs()
    a = np.abs(q.qjl_proj)
    n, j = np.unravel_index(np.argmin(a), a.shape)
    assert a[n, j] < 1e-6
    other = q.qjl_bits.copy()
    other[n, j] = ~other[n, j]
    rep = parity.compare_signs(q.qjl_bits, other, q.qjl_proj, ok)
    assert rep.mismatches == 1 and rep.in_band == 1 and rep.ok


def test_sign_flip_outside_band_fails():
    q, ok = _signs()
    a = np.abs(q.qjl_proj)
    n, j = np.unravel_index(np.argmax(a), a.shape)
    other = q.qjl_bits.copy()
    other[n, j] = ~other[n, j]
    rep = parity.compare_signs(q.qjl_bits, other, q.qjl_proj, ok)
    assert rep.mismatches == 1 and not rep.ok


def test_too_many_band_sign_flips_fail():
    q, ok = _signs()
    other = q.qjl_bits.copy()
    other[:4, 0] = ~other[:4, 0]
    proj = np.zeros_like(q.qjl_proj)          # pretend all lie in the band: the cap still applies
    assert parity.compare_signs(q.qjl_bits, other, proj, ok).ok          # 4 of 524288 <= 1e-5
    other[4:8, 0] = ~other[4:8, 0]
    assert not parity.compare_signs(q.qjl_bits, other, proj, ok).ok      # 8 > 5.2
    rep = parity.compare_signs(q.qjl_bits, other, proj, ok, max_frac=1e-6)
    assert not rep.ok


def test_signs_of_vectors_with_a_code_mismatch_are_not_compared():
    q, ok = _signs()
    other = q.qjl_bits.copy()
    other[5] = ~other[5]                       # every bit of vector 5 differs
    assert not parity.compare_signs(q.qjl_bits, other, q.qjl_proj, ok).ok
    ok[5] = False                              # vector 5 had a code mismatch: its residual differs
    rep = parity.compare_signs(q.qjl_bits, other, q.qjl_proj, ok)
    assert rep.ok and rep.total == q.qjl_bits.size - 128
