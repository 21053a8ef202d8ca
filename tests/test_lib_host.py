"""libtq.so on the CPU: it loads, exports every symbol tq.h declares, its host
builders agree with the oracle, and bad arguments fail before any launch."""
import ctypes
import os
import re

import numpy as np
import pytest

from compressed_kv_cache_tq_amd import tq
from oracle import codebook as ocb
from oracle import rotation as orot

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(tq.LIB_PATH), reason="libtq.so not built")


def header_functions():
    text = open(os.path.join(ROOT, "include", "tq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z_0-9]+)\s*\(", text)))


def test_exports_match_header():
    names = header_functions()
    assert names == sorted(tq.EXPORTS)
    lib = tq.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert tq.format_version() == 2


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("d", [3, 128])
def test_codebook_matches_oracle(d, bits):
    c, t = tq.codebook_build(d, bits)
    cb = ocb.lloyd_max(d, bits)
    # With 256 levels the Lloyd map contracts by only ~3e-5 per step: the
    # oracle's iteration ends by its stall rule ~3e-10 from the fixed point
    # that the library reaches with Newton steps (further Lloyd steps move
    # the oracle's codebook toward the library's).
    tol = 1e-12 if bits < 8 else 1e-9
    assert np.max(np.abs(c - cb.centroids)) <= tol
    assert np.max(np.abs(t - cb.boundaries)) <= tol


@pytest.mark.parametrize("seed", [0, 7, 12345])
def test_rotation_matches_oracle(seed):
    pi = tq.rotation_build(128, seed)
    assert np.max(np.abs(pi - orot.rotation(seed, 128))) <= 1e-12


@pytest.mark.parametrize("d,seed", [(1, 0), (4, 0), (128, 0), (128, 7), (1024, 3)])
def test_hadamard_rotation_matches_oracle(d, seed):
    assert np.array_equal(tq.hadamard_rotation_build(d, seed), orot.hadamard_rotation(seed, d))


def test_hadamard_rotation_errors_and_spec_fields():
    L = tq.lib()
    m = np.zeros(16)
    for d in (0, 3, 6, 2048):
        assert L.tq_hadamard_rotation_build(d, 0, m.ctypes.data) == -1
    assert L.tq_hadamard_rotation_build(4, 0, None) == -1
    buf = np.zeros(tq.tables_bytes(), dtype=np.uint8)
    for rot, nf16 in ((3, 0), (-1, 0), (0, 2)):
        cs = tq.Spec(4).c()
        cs.rotation, cs.norm_f16 = rot, nf16
        assert tq.lib().tq_tables_build(ctypes.byref(cs), buf.ctypes.data, buf.size) == -1


@pytest.mark.parametrize("rot", [1, 2])
def test_hadamard_tables(rot):
    """Both Hadamard options (dense product, butterflies) carry the same
    matrix in the tables."""
    spec = tq.Spec(3, layout=tq.LAYOUT_TILED, rot_seed=5, rotation=rot)
    ref = orot.hadamard_rotation(5, 128)
    hdr, pi, pi_hi, pi_lo, *_ = _tables_view(spec, ref)
    assert np.array_equal(pi, ref.astype(np.float32))
    assert np.array_equal(pi_hi, (256 * ref).astype(np.float16))
    two = pi_hi.astype(np.float64) + pi_lo.astype(np.float64)
    assert np.max(np.abs(two - 256 * ref)) <= 256 * 2.0 ** -22


def test_sketch_matches_oracle():
    s = tq.sketch_build(128, 128, 1)
    assert np.max(np.abs(s - orot.sketch(1, 128, 128))) <= 1e-13


def _check_pi_frag(frag, pi_hi, pi_lo):
    """The fragment-ordered copy of pi_hi / pi_lo: [layout][hi, lo][w][t][ks][lane][e]
    holds row r(layout, w, t, lane), column 16 ks + 8 (lane // 32) + e."""
    lane = np.arange(64)
    l32 = lane % 32
    for lay in range(2):
        for w in range(2):
            for t in range(2):
                if lay:
                    row = 64 * w + 32 * t + l32
                else:
                    row = 64 * w + 32 * ((l32 >> 2) & 1) + 16 * t + 4 * (l32 >> 3) + (l32 & 3)
                for ks in range(8):
                    col = 16 * ks + 8 * (lane[:, None] // 32) + np.arange(8)[None, :]
                    assert np.array_equal(frag[lay, 0, w, t, ks], pi_hi[row[:, None], col])
                    assert np.array_equal(frag[lay, 1, w, t, ks], pi_lo[row[:, None], col])
    # every row appears: each (layout, w) covers 64 distinct rows per t pair
    for lay in range(2):
        rows = set()
        for w in range(2):
            for t in range(2):
                rows |= set((64 * w + 32 * t + l32).tolist() if lay else
                            (64 * w + 32 * ((l32 >> 2) & 1) + 16 * t + 4 * (l32 >> 3) + (l32 & 3)).tolist())
        assert rows == set(range(128))


def _tables_view(spec, ref=None):
    buf = tq.tables_build(spec)
    hdr = buf[:32].view(np.uint32)
    off = 512
    pi = buf[off: off + 65536].view(np.float32).reshape(128, 128)
    off += 65536
    pi_hi = buf[off: off + 32768].view(np.float16).reshape(128, 128)
    off += 32768
    pi_lo = buf[off: off + 32768].view(np.float16).reshape(128, 128)
    off += 32768
    s = buf[off: off + 65536].view(np.float32).reshape(128, 128)
    off += 65536
    s_hi = buf[off: off + 32768].view(np.float16).reshape(128, 128)
    off += 32768
    s_lo = buf[off: off + 32768].view(np.float16).reshape(128, 128)
    off += 32768
    pit = buf[off: off + 65536].view(np.float32).reshape(128, 128)
    off += 65536
    sit = buf[off: off + 65536].view(np.float32).reshape(128, 128)
    assert np.array_equal(pit, pi.T) and np.array_equal(sit, s.T)
    off += 65536
    b16 = buf[off: off + 3 * 32768].view(np.uint16).reshape(3, 128, 128)
    parts = (b16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = orot.rotation(0, 128) if ref is None else ref
    assert np.max(np.abs(parts.sum(0) - ref)) <= 2.0 ** -24 * np.abs(ref).max()
    off += 3 * 32768
    cells = buf[off: off + 2 * 132 * 8].view(np.uint32).reshape(2, 132, 2)
    off += 2 * 132 * 8
    frag = buf[off: off + 2 * 2 * 32768].view(np.float16).reshape(2, 2, 2, 2, 8, 64, 8)
    _check_pi_frag(frag, pi_hi, pi_lo)

    bnd = buf[32: 32 + 128].view(np.float32).reshape(2, 16)
    cen = buf[160: 160 + 128].view(np.float32).reshape(2, 16)
    cen16 = buf[288: 288 + 64].view(np.float16).reshape(2, 16)
    return hdr, pi, pi_hi, pi_lo, s, s_hi, s_lo, bnd, cen, cen16, cells


def _cen16_scale(spec):
    """The scale of each half's fp16 centroids (after cen16 in the header)."""
    return tq.tables_build(spec)[352: 360].view(np.float32)


def _eight_bit_view(spec):
    """bnd8, cen8, cen16_8 and the 8-bit cell table, which follow the
    fragment arrays at the end of the blob."""
    buf = tq.tables_build(spec)
    off = 512 + 4 * 65536 + 4 * 32768 + 3 * 32768 + 2 * 132 * 8 + 4 * 32768
    return (buf[off: off + 1024].view(np.float32), buf[off + 1024: off + 2048].view(np.float32),
            buf[off + 2048: off + 2560].view(np.float16),
            buf[off + 2560: off + 2560 + 1028 * 8].view(np.uint32).reshape(1028, 2))


def test_tables_content():
    spec = tq.Spec(4, 3, split=64, qjl_m=128)
    hdr, pi, pi_hi, pi_lo, s, s_hi, s_lo, bnd, cen, cen16, cells = _tables_view(spec)
    assert tq.tables_bytes() >= 512 + 6 * 65536 + 3 * 32768 + 2 * 132 * 8 + 4 * 32768
    assert tq.tables_bytes() % 256 == 0
    assert hdr[0] == 0x31515454 and hdr[1] == 2 and hdr[2] == 4 and hdr[3] == 3
    ref = orot.rotation(0, 128)
    assert np.array_equal(pi, ref.astype(np.float32))
    two = pi_hi.astype(np.float64) + pi_lo.astype(np.float64)
    assert np.max(np.abs(two - 256 * ref)) <= 256 * 2.0 ** -22
    assert np.array_equal(pi_hi, (256 * ref).astype(np.float16))
    sref = orot.sketch(1, 128, 128)
    assert np.array_equal(s, sref.astype(np.float32))
    assert np.max(np.abs(s_hi.astype(np.float64) + s_lo.astype(np.float64) - sref)) <= np.abs(sref).max() * 2.0 ** -21
    for h, b in ((0, 4), (1, 3)):
        cb = ocb.lloyd_max(128, b)
        L = 1 << b
        assert np.array_equal(bnd[h, : L - 1], cb.boundaries.astype(np.float32))
        assert np.all(np.isinf(bnd[h, L - 1:]))
        assert np.array_equal(cen[h, :L], cb.centroids.astype(np.float32))
        sc = float(_cen16_scale(spec)[h])
        assert np.array_equal(cen16[h, :L], (cb.centroids * sc).astype(np.float16))
        # cell table: cell c covers [(8c - 1/2)/512 - 1, (8c + 15/2)/512 - 1);
        # boundaries below it and the one boundary inside it (or +inf), from
        # the fp32 boundaries
        b32 = cb.boundaries.astype(np.float32).astype(np.float64)
        for c in range(129):
            lo, hi = (8 * c - 0.5) / 512 - 1, (8 * c + 7.5) / 512 - 1
            inside = b32[(b32 >= lo) & (b32 < hi)]
            assert len(inside) <= 1
            want = np.float32(inside[0]) if len(inside) else np.float32(np.inf)
            assert cells[h, c, 0] == want.view(np.uint32)
            assert cells[h, c, 1] == np.count_nonzero(b32 < lo)


def test_fp16_centroid_scale_minimises_the_rounding_error():
    """Each width's fp16 centroids are fp16(c s) with the s = 1 + k/2^16 in
    [1, 2) of smallest largest relative rounding error (checked by the same
    exhaustive search here), the same s for keys and values and both halves
    of a uniform width, 1 for 8-bit codes; the error is well below plain
    fp16's (2^-11 at worst): about 3.5x for 4 bits, 9x for 3, 400x for 2."""
    bound = {2: 2e-6, 3: 5e-5, 4: 1e-4}
    k = np.arange(1 << 16)
    grid = 1.0 + k / 65536.0
    for b in (2, 3, 4):
        c = ocb.lloyd_max(128, b).centroids
        v = np.abs(c)[None, :] * grid[:, None]
        err = (np.abs(v.astype(np.float16).astype(np.float64) - v) / v).max(axis=1)
        want = grid[int(np.argmin(err))]
        for spec in (tq.Spec(b), tq.Spec(b, layout=tq.LAYOUT_TILED)):
            sc = _cen16_scale(spec)
            assert sc[0] == sc[1] == np.float32(want), (b, sc, want)
        got = (c * want).astype(np.float16).astype(np.float64) / want
        assert np.max(np.abs(got - c) / np.abs(c)) <= bound[b], b
    sc = _cen16_scale(tq.Spec(4, 3, split=64))
    assert sc[0] == _cen16_scale(tq.Spec(4))[0] and sc[1] == _cen16_scale(tq.Spec(3))[0]
    assert np.all(_cen16_scale(tq.Spec(8)) == 1.0)


def test_cell_table_gives_the_codes():
    """Codes from the cell rule (code_low + (y > boundary), cell from the
    kernels' index) equal the count of boundaries below y for random and
    boundary-adjacent fp32 values."""
    for bits in (2, 3, 4):
        spec = tq.Spec(bits)
        *_, bnd, cen, cen16, cells = _tables_view(spec)
        L = 1 << bits
        b32 = bnd[0, : L - 1]
        rng = np.random.default_rng(bits)
        y = np.concatenate([rng.normal(0, 0.09, 20000), rng.uniform(-1, 1, 2000), [-1.0, 1.0, 0.0]]).astype(np.float32)
        near = np.concatenate([np.nextafter(b32, np.float32(np.inf)), np.nextafter(b32, np.float32(-np.inf)), b32])
        y = np.concatenate([y, near.astype(np.float32)])
        c = _cell_of(y)
        code = cells[0, c, 1].astype(np.int64) + (y > cells[0, c, 0].view(np.float32))
        want = np.searchsorted(b32, y, side="left")
        assert np.array_equal(code, want)


def _cell_of(y):
    """The kernels' cell index of fp32 y: bits 3..10 of the fp32 rounding
    (nearest, ties to even) of 512 y + 512 + 2^23, which float64 holds exactly."""
    u = (np.asarray(y, np.float32).astype(np.float64) * 512.0 + 8389120.0).astype(np.float32)
    return ((u.view(np.uint32) & 0x7F8) >> 3).astype(np.int64)


def test_cell_index_rounds_to_nearest_even():
    """The cell index is RNE(512 y + 512) >> 3: values on either side of a
    cell's edges, the ties exactly on them (to even: the lower edge belongs to
    the cell, the upper to the next one), and the ends of [-1, 1]."""
    for c in (0, 1, 63, 64, 65, 127, 128):
        lo, hi = (8 * c - 0.5) / 512 - 1, (8 * c + 7.5) / 512 - 1
        for y, want in ((lo, c), (hi, c + 1), ((lo + hi) / 2, c)):
            if y < -1 - 1 / 2048:
                continue  # outside the domain (|y| <= 1 up to rounding): 512 y + 512 + 2^23 < 2^23
            y32 = np.float32(y)
            assert float(y32) == y  # the edges are exact in fp32
            assert _cell_of(y32) == want, (c, y)
            assert _cell_of(np.nextafter(y32, np.float32(-2))) == want - (y == lo or y == hi), (c, y)
    assert _cell_of(np.float32(-1.0)) == 0 and _cell_of(np.float32(1.0)) == 128
    assert _cell_of(np.float32(-1 - 1 / 4096)) == 0 and _cell_of(np.float32(1 + 1 / 2048)) == 128
    assert _cell_of(np.float32(0.0)) == 64


def test_eight_bit_tables_and_cell_rule():
    """8-bit keys: the codebook arrays are the library codebook's in fp32 /
    fp16, and
    the 1024-cell rule over [-1/2, 1/2] (cell clamp(floor(1024 y + 512)),
    code = below + (y > the cell's boundary)) gives the count of boundaries
    below y for random, extreme and boundary-adjacent fp32 values."""
    bnd8, cen8, cen16_8, cells = _eight_bit_view(tq.Spec(8))
    c, t = tq.codebook_build(128, 8)      # (within 1e-9 of the oracle's, above)
    b32 = t.astype(np.float32)
    assert np.array_equal(bnd8[:255], b32) and np.isinf(bnd8[255])
    assert np.array_equal(cen8, c.astype(np.float32))
    assert np.array_equal(cen16_8, c.astype(np.float16))
    rng = np.random.default_rng(8)
    y = np.concatenate([rng.normal(0, 0.09, 50000), rng.uniform(-1, 1, 5000),
                        [-1.0, 1.0, 0.0, -0.5, 0.5, np.nextafter(np.float32(0.5), np.float32(0))]]).astype(np.float32)
    near = np.concatenate([np.nextafter(b32, np.float32(np.inf)), np.nextafter(b32, np.float32(-np.inf)), b32])
    y = np.concatenate([y, near.astype(np.float32)])
    f = np.clip(np.float32(1024) * y + np.float32(512), 0, 1024).astype(np.float32)
    c = f.astype(np.int64)
    code = cells[c, 1].astype(np.int64) + (y > cells[c, 0].view(np.float32))
    assert np.array_equal(code, np.searchsorted(b32, y, side="left"))


def test_eight_bit_spec_limits():
    L = tq.lib()
    buf = np.zeros(tq.tables_bytes() + 256, np.uint8)
    ptr = (buf.ctypes.data + 255) // 256 * 256

    def build(spec):
        return L.tq_tables_build(ctypes.byref(spec.c()), ptr, tq.tables_bytes())

    assert build(tq.Spec(8)) == 0
    assert build(tq.Spec(8, qjl_m=128)) == -2                    # no sketch with 8-bit codes
    assert build(tq.Spec(8, layout=tq.LAYOUT_TILED)) == -2       # keys only: record layout
    assert build(tq.Spec(8, 4, split=64)) == -2                  # uniform width only
    assert build(tq.Spec(4, 8, split=64)) == -2
    assert build(tq.Spec(5)) == -2
    assert tq.code_bytes(tq.Spec(8)) == 128


def test_code_bytes():
    assert tq.code_bytes(tq.Spec(4)) == 64
    assert tq.code_bytes(tq.Spec(3)) == 48
    assert tq.code_bytes(tq.Spec(2)) == 32
    assert tq.code_bytes(tq.Spec(4, 3, split=64)) == 56
    assert tq.cache_code_bytes(tq.Spec(3, layout=tq.LAYOUT_TILED), 33) == 64 * 48


@pytest.mark.parametrize("bad", [
    dict(bits_lo=5), dict(bits_lo=1), dict(split=32), dict(qjl_m=64),
    dict(qjl_m=128, layout=1), dict(bits_lo=2, bits_hi=4, split=64), dict(layout=7),
])
def test_bad_specs_rejected(bad):
    kw = dict(bits_lo=4, bits_hi=None, split=128, qjl_m=0, layout=0)
    kw.update(bad)
    spec = tq.Spec(**kw)
    buf = np.zeros(tq.tables_bytes(), dtype=np.uint8)
    cs = spec.c()
    st = tq.lib().tq_tables_build(ctypes.byref(cs), buf.ctypes.data, buf.size)
    assert st in (-1, -2)
    assert tq.last_error()


def test_quantize_argument_errors_without_launch():
    L = tq.lib()
    spec = tq.Spec(4).c()
    cache = tq.TqCache(0x1000, 0x2000, None, None, 64)
    fake_tab = ctypes.c_void_p(0x10000)
    # NULL x
    assert L.tq_quantize_kv(ctypes.byref(spec), fake_tab, 1, None, 1, 8, 0, 128, 0, ctypes.byref(cache), None) == -1
    # misaligned x
    assert L.tq_quantize_kv(ctypes.byref(spec), fake_tab, 1, 0x1002, 1, 8, 0, 128, 0, ctypes.byref(cache), None) == -1
    # beyond capacity
    assert L.tq_quantize_kv(ctypes.byref(spec), fake_tab, 1, 0x1000, 1, 65, 0, 128, 0, ctypes.byref(cache), None) == -1
    # bad dtype
    assert L.tq_quantize_kv(ctypes.byref(spec), fake_tab, 5, 0x1000, 1, 8, 0, 128, 0, ctypes.byref(cache), None) == -1
    # nothing to do: OK without touching the device
    assert L.tq_quantize_kv(ctypes.byref(spec), fake_tab, 1, 0x1000, 0, 8, 0, 128, 0, ctypes.byref(cache), None) == 0
    # tiled layout needs cap % 32 == 0
    ts = tq.Spec(3, layout=1).c()
    c2 = tq.TqCache(0x1000, 0x2000, None, None, 40)
    assert L.tq_quantize_kv(ctypes.byref(ts), fake_tab, 1, 0x1000, 1, 8, 0, 128, 0, ctypes.byref(c2), None) == -1


def test_quantize_ragged_argument_errors_without_launch():
    L = tq.lib()
    spec = tq.Spec(4).c()
    cache = tq.TqCache(0x1000, 0x2000, None, None, 64)
    tab = ctypes.c_void_p(0x10000)

    def call(n, t0=None, xo=None, x=0x1000, batch=None, hkv=2, dtype=1, sp=spec, c=cache):
        n = np.asarray(n, np.int64)
        t0 = np.zeros_like(n) if t0 is None else np.asarray(t0, np.int64)
        xo = np.zeros_like(n) if xo is None else np.asarray(xo, np.int64)
        b = len(n) if batch is None else batch
        return L.tq_quantize_kv_ragged(ctypes.byref(sp), tab, dtype, x, b, hkv, xo.ctypes.data, t0.ctypes.data,
                                       n.ctypes.data, 128 * 64, 128, ctypes.byref(c), None)

    assert call([8, 65]) == -1                      # beyond capacity
    assert call([8, 8], t0=[0, 60]) == -1           # tok0 + n beyond capacity
    assert call([8, -1]) == -1                      # negative length
    assert call([8, 8], xo=[0, 4]) == -1            # offset not a multiple of 16 bytes
    assert call([8, 8], xo=[0, -8]) == -1           # negative offset
    assert call([8, 8], hkv=0) == -1
    assert call([8, 8], dtype=5) == -1
    assert call([8, 8], x=None) == -1
    assert call([8, 8], x=0x1002) == -1             # misaligned x
    assert call([0, 0]) == 0                        # nothing to write: no launch
    assert call([8], batch=0) == 0
    assert L.tq_quantize_kv_ragged(ctypes.byref(spec), tab, 1, 0x1000, 2, 2, None, None, None, 128, 128,
                                   ctypes.byref(cache), None) == -1
    ts = tq.Spec(3, layout=1).c()
    assert call([8, 8], sp=ts, c=tq.TqCache(0x1000, 0x2000, None, None, 40)) == -1  # tiled cap % 32


def test_ip_scores_argument_errors_without_launch():
    L = tq.lib()
    spec = tq.Spec(2, qjl_m=128).c()
    db = tq.TqCache(0x1000, 0x2000, 0x3000, 0x4000, 64)
    tab = ctypes.c_void_p(0x10000)
    ws = tq.lib().tq_ip_workspace_bytes()
    assert ws >= 64 * 2 * 2 * 128 * 2

    def call(ns=2, nt=64, nq=4, ld=128, sp=spec, d=db, w=ws, q=0x5000):
        return L.tq_ip_scores(ctypes.byref(sp), tab, ctypes.byref(d), ns, nt, q, nq, 0x6000, ld, 0x8000, w, None)

    assert call(nq=0) == -2 and call(nq=65) == -2          # query count
    assert call(nt=65) == -1                                # beyond capacity
    assert call(ld=127) == -1                               # ld < n_streams * n_tok
    assert call(w=16) == -3                                 # workspace
    assert call(q=None) == -1
    assert call(d=tq.TqCache(0x1000, 0x2000, None, None, 64)) == -1  # sketch arrays missing
    assert call(sp=tq.Spec(3, layout=tq.LAYOUT_TILED).c()) == -2     # tiled layout
    assert call(sp=tq.Spec(8).c()) == -2                              # 8-bit codes
    assert call(ns=0) == 0 and call(nt=0, ld=0) == 0        # nothing to do: no launch
    assert call(ns=70000, nt=1, ld=70000, d=tq.TqCache(0x1000, 0x2000, 0x3000, 0x4000, 64)) == -2


def test_paged_argument_errors_without_launch():
    L = tq.lib()
    ks, vs = tq.Spec(4).c(), tq.Spec(3, layout=1).c()
    pool_k = tq.TqCache(0x1000, 0x2000, None, None, 64)
    pool_v = tq.TqCache(0x3000, 0x4000, None, None, 64)
    tab = ctypes.c_void_p(0x10000)

    def dec(a, kp=pool_k, max_pages=4, n_pages=8, table=0x9000):
        return L.tq_attend_decode_paged(ctypes.byref(ks), tab, ctypes.byref(kp), ctypes.byref(vs), tab,
                                        ctypes.byref(pool_v), ctypes.byref(a), 0x5000, None, None, 0x6000, table,
                                        max_pages, n_pages, 0x7000, 0x8000, 1 << 20, None)

    assert dec(tq.TqAttn(2, 8, 2, 0, 0.1, 0.0, 257)) == -1           # beyond max_pages pages
    assert dec(tq.TqAttn(2, 8, 2, 0, 0.1, 0.0, 64), table=None) == -1
    assert dec(tq.TqAttn(2, 8, 2, 0, 0.1, 0.0, 64), kp=tq.TqCache(0x1000, 0x2000, None, None, 128)) == -1
    assert dec(tq.TqAttn(2, 8, 2, 0, 0.1, 0.0, 64), n_pages=0) == -1
    assert dec(tq.TqAttn(0, 8, 2, 0, 0.1, 0.0, 64)) == 0

    def qz(n_tok, pos0=(0, 0), table=0x9000, n_pages=8, pool=pool_k, max_pages=4):
        n, p0, xo = np.asarray(n_tok, np.int64), np.asarray(pos0, np.int64), np.zeros(2, np.int64)
        return L.tq_quantize_kv_paged(ctypes.byref(ks), tab, 1, 0x1000, 2, 2, xo.ctypes.data, p0.ctypes.data,
                                      n.ctypes.data, 128 * 300, 128, table, max_pages, n_pages,
                                      ctypes.byref(pool), None)

    assert qz([10, 257]) == -1                                   # beyond max_pages pages
    assert qz([10, 10], pos0=(250, 0)) == -1
    assert qz([10, 10], table=None) == -1                        # the device table is required
    assert qz([10, 10], table=0x9002) == -1                      # ... 4-byte aligned
    assert qz([10, 10], n_pages=0) == -1
    assert qz([10, 10], n_pages=(1 << 30) + 1) == -1
    assert qz([10, 10], max_pages=0) == -1
    assert qz([10, 10], pool=tq.TqCache(0x1000, 0x2000, None, None, 96)) == -1
    assert qz([0, 0]) == 0                                       # nothing to write
    assert qz([0, 0], table=None) == -1


def test_attend_argument_errors_without_launch():
    L = tq.lib()
    ks, vs = tq.Spec(4).c(), tq.Spec(3, layout=1).c()
    kc = tq.TqCache(0x1000, 0x2000, None, None, 64)
    vc = tq.TqCache(0x3000, 0x4000, None, None, 64)
    tab = ctypes.c_void_p(0x10000)

    def call(a, ks_=ks, vs_=vs, ws=1 << 20, q=0x5000, kc_=kc):
        return L.tq_attend_decode(ctypes.byref(ks_), tab, ctypes.byref(kc_), ctypes.byref(vs_), tab,
                                  ctypes.byref(vc), ctypes.byref(a), q, None, None, 0x6000, 0x7000,
                                  0x8000, ws, None)

    assert call(tq.TqAttn(1, 6, 4, 0, 0.1, 0.0, 64)) == -1            # hq % hkv
    assert call(tq.TqAttn(1, 64, 2, 0, 0.1, 0.0, 64)) == -2           # G > 16
    assert call(tq.TqAttn(65536, 8, 2, 0, 0.1, 0.0, 64)) == -2        # batch limit
    assert call(tq.TqAttn(1, 8, 2, 0, 0.1, 0.0, 65)) == -1            # max_len > cap
    assert call(tq.TqAttn(1, 8, 2, 4, 0.1, 0.0, 64)) == -1            # sink without buffers
    assert call(tq.TqAttn(1, 8, 2, 0, 0.1, 0.0, 64), ws=16) == -3     # workspace
    assert call(tq.TqAttn(1, 8, 2, 0, 0.1, 0.0, 64), q=None) == -1
    assert call(tq.TqAttn(1, 8, 2, 0, 0.1, 0.0, 64), ks_=vs, vs_=ks) == -2  # layouts swapped
    assert call(tq.TqAttn(1, 8, 2, 513, 0.1, 0.0, 600)) == -2         # sink limit
    big = tq.TqCache(0x1000, 0x2000, None, None, (1 << 24) + 32)
    assert call(tq.TqAttn(1, 8, 2, 0, 0.1, 0.0, 64), kc_=big) == -2   # cap above 2^24
    assert call(tq.TqAttn(0, 8, 2, 0, 0.1, 0.0, 64)) == 0             # empty batch: nothing launched
    k8 = tq.Spec(8).c()
    for vspec in (tq.Spec(4, layout=1), tq.Spec(4, 3, split=64, layout=1), tq.Spec(3, 2, split=64, layout=1)):
        assert L.tq_attend_decode(ctypes.byref(k8), tab, ctypes.byref(kc), ctypes.byref(vspec.c()), tab,
                                  ctypes.byref(vc), ctypes.byref(tq.TqAttn(1, 8, 2, 0, 0.1, 0.0, 64)), 0x5000,
                                  None, None, 0x6000, 0x7000, 0x8000, 1 << 20, None) == -2  # K8: V2 or V3 only
    ws = tq.attend_workspace_bytes(2, 32, 8, 0, 32768)
    assert ws >= 2 * 32 * (2 * 128 + 4) * 4
    assert ws % 4 == 0


def test_paged_binding_wants_a_device_table_tensor():
    """The paged quantize reads its block table on the device: the binding
    refuses a host array (or a table of the wrong shape or type) before any
    call into the library."""
    torch = pytest.importorskip("torch")
    for bt in (np.zeros((2, 4), np.int32), torch.zeros((2, 4), dtype=torch.int64), torch.zeros((3, 4), dtype=torch.int32)):
        with pytest.raises(ValueError):
            tq.quantize_kv_paged(tq.Spec(4), None, None, None, hkv=2, n_tok=[1, 1], block_table=bt, n_pages=8)


def test_eight_bit_quantize_stride_limit():
    """8-bit codes have no general-kernel path: a row stride whose 32 rows
    reach 2^30 bytes is refused before any launch."""
    L = tq.lib()
    spec = tq.Spec(8)
    cache = tq.TqCache(0x1000, 0x2000, None, None, 64)
    rs = (1 << 30) // (32 * 2)  # bf16 elements
    assert L.tq_quantize_kv(ctypes.byref(spec.c()), ctypes.c_void_p(0x10000), 1, 0x4000, 1, 2, rs, rs, 0,
                            ctypes.byref(cache), None) == -2


def test_binding_refuses_a_cache_of_another_spec():
    """The C side gets bare pointers, so the binding checks that a cache was
    sized for the spec it is used with (widths, split, sketch, layout, norm
    width) and holds the streams the call touches; caches on the CPU are
    enough, nothing is launched."""
    torch = pytest.importorskip("torch")
    k4 = tq.Spec(4)
    k4h = tq.Spec(4, norm_f16=1)
    v3 = tq.Spec(3, layout=tq.LAYOUT_TILED)
    x = torch.zeros((2, 40, 128), dtype=torch.bfloat16)
    good = tq.alloc_cache(k4, 2, 64, device="cpu")
    for bad_spec in (k4h, tq.Spec(3), tq.Spec(4, 3, split=64), tq.Spec(2, qjl_m=128),
                     tq.Spec(4, layout=tq.LAYOUT_TILED)):
        with pytest.raises(ValueError):
            tq.quantize_kv(bad_spec, None, x, good)
    # an fp32-norm cache with an fp16-norm spec, and the reverse, whatever spec the cache claims
    half = tq.alloc_cache(k4h, 2, 64, device="cpu")
    with pytest.raises(ValueError):
        tq.quantize_kv(k4, None, x, tq.Cache(k4, 64, half.codes, half.norms))
    with pytest.raises(ValueError):
        tq.quantize_kv(k4h, None, x, tq.Cache(k4h, 64, good.codes, good.norms))
    # fewer streams than the call touches
    with pytest.raises(ValueError):
        tq.quantize_kv(k4, None, torch.zeros((3, 40, 128), dtype=torch.bfloat16), good)
    with pytest.raises(ValueError):
        tq.quantize_kv_ragged(k4, None, torch.zeros((4, 40, 128), dtype=torch.bfloat16), good, hkv=2,
                              n_tok=[10, 10])
    vgood = tq.alloc_cache(v3, 2, 64, device="cpu")
    q = torch.zeros((1, 8, 128))
    lens = torch.zeros(1, dtype=torch.int32)
    out = torch.zeros_like(q)
    with pytest.raises(ValueError):
        tq.attend_decode(k4, None, good, v3, None, tq.alloc_cache(tq.Spec(2, layout=tq.LAYOUT_TILED), 2, 64,
                                                                     device="cpu"),
                         q, lens, out, None, hkv=2)
    with pytest.raises(ValueError):
        tq.attend_decode(k4, None, good, v3, None, vgood, torch.zeros((2, 8, 128)), lens, out, None, hkv=2)
    with pytest.raises(ValueError):
        tq.ip_scores(tq.Spec(2, qjl_m=128), None, good, q[0], n_streams=2, n_tok=8, workspace=torch.zeros(4))
    # the right spec passes the binding's checks (the call itself would need a device)
    tq._check_cache(k4, good, 2, "ok")
    tq._check_cache(v3, vgood, 2, "ok")
    tq._check_cache(k4h, half, 2, "ok")


def test_noalloc_refuses_a_problem_beyond_its_scratch():
    """tq_attend_decode_noalloc checks the problem's partials against its
    static scratch first, before anything else and with no launch."""
    L = tq.lib()
    ks, vs = tq.Spec(4).c(), tq.Spec(3, layout=1).c()
    kc = tq.TqCache(0x1000, 0x2000, None, None, 64)
    vc = tq.TqCache(0x3000, 0x4000, None, None, 64)
    big = tq.TqAttn(4096, 32, 8, 0, 0.1, 0.0, 64)              # 131072 heads x 528 B > 8 MiB
    assert tq.attend_workspace_bytes(4096, 32, 8, 0, 64) > tq.NOALLOC_SCRATCH_BYTES
    st = L.tq_attend_decode_noalloc(ctypes.byref(ks), ctypes.c_void_p(0x10000), ctypes.byref(kc), ctypes.byref(vs),
                                    ctypes.c_void_p(0x10000), ctypes.byref(vc), ctypes.byref(big), 0x5000, None,
                                    None, 0x6000, 0x7000, None)
    assert st == -2 and "TQ_NOALLOC_SCRATCH_BYTES" in tq.last_error()
    assert L.tq_attend_decode_noalloc(ctypes.byref(ks), None, ctypes.byref(kc), ctypes.byref(vs), None,
                                      ctypes.byref(vc), None, 0x5000, None, None, 0x6000, 0x7000, None) == -1


def test_host_half_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    """The host half of the library (host.cpp, plan.cpp) built with g++ under
    -fsanitize=address,undefined (no device code: the launches are stubs that
    report no device) and driven through every host-side path: codebooks,
    rotations, sketch, tables for every spec, sizes, and the argument checks
    of every entry point up to the launch.  Any sanitizer report aborts."""
    import shutil
    import subprocess
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    csrc = os.path.join(ROOT, "compressed_kv_cache_tq_amd", "csrc")
    here = os.path.join(ROOT, "tests", "host_sanitize")
    exe = str(tmp_path / "host_san")
    cmd = [gxx, "-std=c++20", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"), "-I" + csrc,
           os.path.join(csrc, "host.cpp"), os.path.join(csrc, "plan.cpp"),
           os.path.join(here, "stubs.cpp"), os.path.join(here, "driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "host sanitizer driver ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
