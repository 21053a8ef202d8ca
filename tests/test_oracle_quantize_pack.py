"""Pins of the oracle's quantizer, QJL estimator and bit layouts (CPU only)."""
import math

import numpy as np
import pytest

from compressed_kv_cache_tq_amd import workloads
from oracle import codebook as cbm
from oracle import pack, quantize as qz
from oracle.rotation import sketch


@pytest.mark.parametrize("d", [8, 128])
def test_nearest_centroid_brute_force(d):
    rng = np.random.default_rng(3)
    for bits in (1, 2, 3, 4):
        spec = qz.Spec(d=d, bits_lo=bits, bits_hi=bits, split=d)
        x = rng.standard_normal((64, d))
        q = qz.quantize(x, spec)
        c = cbm.lloyd_max(d, bits).centroids
        brute = np.argmin(np.abs(q.y[..., None] - c[None, None, :]), axis=-1)
        assert np.array_equal(brute, q.idx)


def test_mixed_split_uses_two_codebooks():
    spec = qz.Spec(bits_lo=4, bits_hi=3, split=64)
    x = np.random.default_rng(4).standard_normal((32, 128))
    q = qz.quantize(x, spec)
    assert q.idx[:, :64].max() <= 15 and q.idx[:, 64:].max() <= 7
    c4, c3 = cbm.lloyd_max(128, 4).centroids, cbm.lloyd_max(128, 3).centroids
    assert np.array_equal(np.argmin(np.abs(q.y[:, :64, None] - c4), -1), q.idx[:, :64])
    assert np.array_equal(np.argmin(np.abs(q.y[:, 64:, None] - c3), -1), q.idx[:, 64:])


def test_norm_rotation_and_zero_vector():
    spec = qz.Spec()
    pi = qz.rotation_of(spec)
    x = np.zeros((3, 128))
    x[1] = np.arange(128) / 100.0
    x[2, 5] = -3.0
    q = qz.quantize(x, spec)
    assert q.norms[0] == 0 and np.all(q.y[0] == 0)
    t = cbm.lloyd_max(128, 4).boundaries
    assert np.all(q.idx[0] == np.sum(t < 0))          # ties go to the lower index
    assert q.norms[1] == np.float32(np.sqrt(np.sum(x[1] ** 2)))
    assert q.norms[2] == np.float32(3.0)
    assert np.allclose(q.y[2], -pi[:, 5], atol=1e-15)


@pytest.mark.parametrize("rot", ["haar", "hadamard"])
@pytest.mark.parametrize("bits", [(4, 4, 128), (3, 3, 128), (4, 3, 64)])
def test_empirical_distortion_on_tiny_workload(bits, rot):
    # tiny_oracle inputs (4096 K + 4096 V, fp32 N(0,1), seed 0): the measured
    # d * mean squared error of the unit vectors matches the analytic value.
    # (For Gaussian inputs the randomized Hadamard transform also gives
    # coordinates with the uniform-sphere marginal.)
    inp = workloads.generate("tiny_oracle")
    x = np.concatenate([inp.k[0][0], inp.v[0][0]]).astype(np.float64)
    spec = qz.Spec(bits_lo=bits[0], bits_hi=bits[1], split=bits[2], rotation=rot)
    q = qz.quantize(x, spec)
    err = np.sum((q.y - qz.dequantize_rotated(q.idx, spec)) ** 2, axis=1)     # per vector
    Dlo = cbm.distortion(cbm.lloyd_max(128, bits[0]))
    Dhi = cbm.distortion(cbm.lloyd_max(128, bits[1]))
    want = (bits[2] * Dlo + (128 - bits[2]) * Dhi) / 128
    se = err.std() / math.sqrt(len(err))
    assert abs(err.mean() - want) < 3 * se, (err.mean(), want, se)
    if bits == (4, 3, 64):
        assert want == pytest.approx(0.0216, abs=2e-4)


def test_qjl_estimator_unbiased_over_seeds_and_variance():
    # For fixed q and residual r, average the sketch estimate over many QJL seeds.
    d, m, n = 128, 128, 2000
    rng = np.random.default_rng(11)
    qv = rng.standard_normal(d)
    r = rng.standard_normal(d) * 0.05
    est = np.empty(n)
    for s in range(n):
        S = sketch(10_000 + s, m, d)
        z = (S @ r) >= 0
        est[s] = qz.qjl_inner_estimate(qv, S, z, np.linalg.norm(r))
    truth = qv @ r
    var = ((math.pi / 2) * (qv @ qv) * (r @ r) - truth ** 2) / m
    assert abs(est.mean() - truth) < 4 * math.sqrt(var / n)
    assert est.var() == pytest.approx(var, rel=0.10)


def test_qjl_fields_from_quantize():
    spec = qz.Spec(bits_lo=2, bits_hi=2, qjl_m=128)
    x = np.random.default_rng(2).standard_normal((16, 128))
    q = qz.quantize(x, spec)
    r = q.y - qz.dequantize_rotated(q.idx, spec)
    S = sketch(spec.qjl_seed, 128, 128)
    assert np.array_equal(q.qjl_bits, (r @ S.T) >= 0)
    assert np.allclose(q.rnorms, np.linalg.norm(r, axis=1), rtol=1e-7)


# ---- bit layouts -----------------------------------------------------------

def test_record_worked_example_3bit():
    # idx 0..7 repeated at 3 bits, LSB first: 000 100 010 110 001 101 011 111
    # -> bytes 0x88 0xC6 0xFA, repeating every 8 coordinates.
    idx = np.tile(np.arange(8), 16)[None, :]
    rec = pack.pack_records(idx, np.full(128, 3))
    assert rec.shape == (1, 48)
    assert list(rec[0, :6]) == [0x88, 0xC6, 0xFA, 0x88, 0xC6, 0xFA]


def test_record_worked_example_4bit_and_mixed():
    idx = np.zeros((1, 128), dtype=np.int64)
    idx[0, 0], idx[0, 1], idx[0, 63] = 1, 2, 15          # 4-bit half: byte0 = 0x21, byte31 = 0xF0
    idx[0, 64], idx[0, 65], idx[0, 127] = 7, 1, 5        # 3-bit half from byte 32
    w = np.array([4] * 64 + [3] * 64)
    rec = pack.pack_records(idx, w)
    assert rec.shape == (1, 56)
    assert rec[0, 0] == 0x21 and rec[0, 31] == 0xF0
    assert rec[0, 32] == 0x0F                            # 111 then 100 -> bits 0..5 = 1,1,1,1,0,0
    assert rec[0, 55] == 0xA0                            # coord 127 at bits 189..191 of the half: 5 << 5
    assert np.count_nonzero(rec[0]) == 4


@pytest.mark.parametrize("w", [(2, 2), (3, 3), (4, 4), (4, 3), (3, 2)])
def test_record_round_trip(w):
    widths = np.array([w[0]] * 64 + [w[1]] * 64)
    rng = np.random.default_rng(0)
    idx = rng.integers(0, 1 << widths, size=(50, 128))
    rec = pack.pack_records(idx, widths)
    assert rec.shape[1] == widths.sum() // 8
    assert np.array_equal(pack.unpack_records(rec, widths), idx)


def test_tiled_worked_example():
    # 2-bit: token 9 (group 1, slot 1), coordinate 10 (group 1, row 2), code 3.
    # Group bytes G = 16 * 8 * 2 = 256; sub-block (1, 1) starts at 256 + 16 = 272;
    # inside it the code sits at bit (8*2 + 1) * 2 = 34 -> byte 276, bits 2..3.
    idx = np.zeros((10, 128), dtype=np.int64)
    idx[9, 10] = 3
    buf = pack.pack_tiled(idx, np.full(128, 2))
    assert buf.size == 32 * 32
    assert np.flatnonzero(buf).tolist() == [276] and buf[276] == 0x0C


def test_tiled_worked_example_3bit_codes_straddle_bytes():
    # 3-bit tiles: sub-block bytes 8 * 3 = 24, token-group bytes G = 16 * 24 = 384.
    # (a) token 2 (group 0, slot 2), coordinate 1 (group 0, row 1), code 7: bits
    #     (8*1 + 2) * 3 = 30, 31, 32 -> byte 3 bits 6-7 (0xC0), byte 4 bit 0 (0x01).
    # (b) token 21 (group 2, slot 5), coordinate 42 (group 5, row 2), code 5 = 0b101:
    #     sub-block at 2*384 + 5*24 = 888, bits (8*2 + 5) * 3 = 63, 64, 65 ->
    #     code bit 0 at byte 895 bit 7 (0x80), bit 2 at byte 896 bit 1 (0x02).
    # (c) tokens 8..15 (group 1), coordinate 127 (group 15, row 7), codes 0..7 in
    #     slot order: 24 bits at sub-block 384 + 15*24 = 744, bits 168..191 ->
    #     bytes 765, 766, 767 = 0x88 0xC6 0xFA (the record example's bytes).
    idx = np.zeros((32, 128), dtype=np.int64)
    idx[2, 1] = 7
    idx[21, 42] = 5
    idx[8:16, 127] = np.arange(8)
    buf = pack.pack_tiled(idx, np.full(128, 3))
    assert buf.size == 32 * 48
    want = {3: 0xC0, 4: 0x01, 895: 0x80, 896: 0x02, 765: 0x88, 766: 0xC6, 767: 0xFA}
    assert np.flatnonzero(buf).tolist() == sorted(want)
    assert all(buf[k] == v for k, v in want.items())
    assert np.array_equal(pack.unpack_tiled(buf, np.full(128, 3), 32), idx)


def test_tiled_worked_example_mixed_4_and_3_bits():
    # 3.5 bits (coordinates 0..63 at 4 bits, 64..127 at 3 bits): sub-blocks
    # q < 8 hold 32 bytes, q >= 8 hold 24, G = 8*32 + 8*24 = 448 per token group.
    #   token 3,  coord 7:   g 0, q 0,  r 7, s 3, code 10 -> bit (56+3)*4 = 236 -> byte 29 high nibble: 0xA0
    #   token 8,  coord 64:  g 1, q 8,  r 0, s 0, code 5  -> byte 448 + 256 = 704, bits 0..2: 0x05
    #   token 17, coord 70:  g 2, q 8,  r 6, s 1, code 6  -> 896 + 256 = 1152, bit (48+1)*3 = 147:
    #                        code bits 1, 2 at bits 148, 149 -> byte 1152 + 18 = 1170 bits 4, 5: 0x30
    #   token 21, coord 63:  g 2, q 7,  r 7, s 5, code 15 -> 896 + 7*32 = 1120, bit (56+5)*4 = 244 ->
    #                        byte 1150 high nibble: 0xF0
    #   token 31, coord 127: g 3, q 15, r 7, s 7, code 7  -> 3*448 + 256 + 7*24 = 1768, bit (56+7)*3 = 189
    #                        -> byte 1768 + 23 = 1791 bits 5..7: 0xE0 (the tile's last byte)
    w = np.array([4] * 64 + [3] * 64)
    idx = np.zeros((32, 128), dtype=np.int64)
    idx[3, 7], idx[8, 64], idx[17, 70], idx[21, 63], idx[31, 127] = 10, 5, 6, 15, 7
    buf = pack.pack_tiled(idx, w)
    assert buf.size == 32 * 56
    want = {29: 0xA0, 704: 0x05, 1170: 0x30, 1150: 0xF0, 1791: 0xE0}
    assert np.flatnonzero(buf).tolist() == sorted(want)
    assert all(buf[k] == v for k, v in want.items())
    assert np.array_equal(pack.unpack_tiled(buf, w, 32), idx)


@pytest.mark.parametrize("w", [(2, 2), (3, 3), (4, 4), (4, 3)])
def test_tiled_round_trip_and_partial_update(w):
    widths = np.array([w[0]] * 64 + [w[1]] * 64)
    rng = np.random.default_rng(1)
    idx = rng.integers(0, 1 << widths, size=(70, 128))
    buf = pack.pack_tiled(idx, widths)
    assert buf.size == pack.tiled_bytes(70, widths) == 3 * 32 * widths.sum() // 8
    assert np.array_equal(pack.unpack_tiled(buf, widths, 70), idx)
    # rewrite tokens 40..44 only: every other position keeps its code
    new = rng.integers(0, 1 << widths, size=(5, 128))
    pack.pack_tiled(new, widths, tok0=40, out=buf)
    want = idx.copy()
    want[40:45] = new
    assert np.array_equal(pack.unpack_tiled(buf, widths, 70), want)


def test_tiled_equals_record_bits_per_token():
    # Same multiset of bits per token in both layouts (layout is a permutation).
    widths = np.full(128, 3)
    idx = np.random.default_rng(5).integers(0, 8, size=(32, 128))
    rec = pack.pack_records(idx, widths)
    til = pack.pack_tiled(idx, widths)
    popc = lambda a: int(np.unpackbits(a).sum())
    assert popc(rec) == popc(til)


def test_fp16_norms_round_the_fp32_norm_to_nearest_even():
    """Stored fp16 norms, worked by hand: sqrt(3) = 1.7320508 lies between the
    binary16 values 1 + 749/1024 and 1 + 750/1024 and is nearer the second
    (bits 0x3EEE); 2049 and 2051 are exact fp32 norms halfway between
    binary16 neighbours (spacing 2 above 2048), which round to the even
    mantissa: 2048 (0x6800) and 2052 (0x6802), not truncated or rounded up."""
    spec = qz.Spec(bits_lo=4, bits_hi=4, norm_f16=True)
    x = np.zeros((3, 128))
    x[0, :3] = 1.0
    x[1, 5] = 2049.0
    x[2, 77] = -2051.0
    q = qz.quantize(x, spec)
    assert q.norms.dtype == np.float16
    assert q.norms.view(np.uint16).tolist() == [0x3EEE, 0x6800, 0x6802]
    # codes do not depend on how the norm is stored
    assert np.array_equal(q.idx, qz.quantize(x, qz.Spec(bits_lo=4, bits_hi=4)).idx)


def test_fp16_norms_saturate_at_the_largest_finite_value():
    """Worked by hand: 65472 = 2046 * 32 is a binary16 value (0x7BFE); 65519 is
    nearer 65504 (0x7BFF) than the next step 65536, which binary16 cannot
    hold; 65520 is the halfway point that nearest-even would send to
    infinity, and 70000 lies past it: both are stored as 65504, not +inf."""
    spec = qz.Spec(bits_lo=4, bits_hi=4, norm_f16=True)
    x = np.zeros((4, 128))
    x[0, 0], x[1, 9], x[2, 100], x[3, 127] = 65472.0, 65519.0, -65520.0, 70000.0
    q = qz.quantize(x, spec)
    assert q.norms.view(np.uint16).tolist() == [0x7BFE, 0x7BFF, 0x7BFF, 0x7BFF]
    assert np.all(np.isfinite(q.norms))
