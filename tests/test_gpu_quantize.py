"""GPU parity of the quantize kernel (through the C ABI) against the oracle."""
import numpy as np
import pytest

from compressed_kv_cache_tq_amd import tq, workloads
from gpu_helpers import check_quantized, read_codes, read_norms, read_signs, to_device, torch
from oracle import pack as opk

pytestmark = pytest.mark.gpu

WIDTHS = [(2, None, 128), (3, None, 128), (4, None, 128), (4, 3, 64), (3, 2, 64)]


def _data(n, seed, dtype, scale=1.0):
    x = np.random.default_rng(seed).standard_normal((1, n, 128), dtype=np.float32) * np.float32(scale)
    if dtype == "bf16":
        x = workloads.bf16_to_f32(workloads.bf16_bits(x))
    return x


def _quantize(spec, x, dtype, cap=None, tok0=0, fill=None):
    cap = cap or x.shape[1] + tok0
    tab = tq.device_tables(spec)
    cache = tq.alloc_cache(spec, x.shape[0], cap, fill=fill)
    tq.quantize_kv(spec, tab, to_device(x, dtype), cache, tok0=tok0)
    torch().cuda.synchronize()
    return cache


@pytest.mark.parametrize("layout", [tq.LAYOUT_RECORD, tq.LAYOUT_TILED])
@pytest.mark.parametrize("w", WIDTHS)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_widths_layouts(w, layout, dtype):
    print(f"[quantize] widths={w} layout={layout} dtype={dtype}", flush=True)
    spec = tq.Spec(w[0], w[1], split=w[2], layout=layout)
    n = 1000  # 31 full tiles and a ragged tail
    x = _data(n, seed=w[0] * 10 + layout, dtype=dtype)
    cache = _quantize(spec, x, dtype)
    idx = read_codes(spec, cache, 0, n)
    check_quantized(spec, x[0], idx, read_norms(cache, 0, n), label=f"{w}/{layout}/{dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_qjl(dtype):
    print(f"[quantize] qjl dtype={dtype}", flush=True)
    spec = tq.Spec(2, qjl_m=128)
    n = 777
    x = _data(n, seed=5, dtype=dtype)
    cache = _quantize(spec, x, dtype)
    idx = read_codes(spec, cache, 0, n)
    check_quantized(spec, x[0], idx, read_norms(cache, 0, n), signs=read_signs(cache, 0, n), label="qjl")


def test_quantize_multi_stream_offsets_and_zero_vector():
    print("[quantize] streams + tok0 + zero vectors", flush=True)
    for layout in (tq.LAYOUT_RECORD, tq.LAYOUT_TILED):
        spec = tq.Spec(4, 3, split=64, layout=layout)
        x = np.random.default_rng(9).standard_normal((3, 70, 128), dtype=np.float32)
        x[1, 5] = 0.0
        x[2, 69] = 0.0
        x = workloads.bf16_to_f32(workloads.bf16_bits(x))
        cap, tok0 = 160, 37
        cache = _quantize(spec, x, "bf16", cap=cap, tok0=tok0)
        for s in range(3):
            idx = read_codes(spec, cache, s, 70, tok0)
            check_quantized(spec, x[s], idx, read_norms(cache, s, 70, tok0), label=f"stream {s}")
        assert read_norms(cache, 1, 1, tok0 + 5)[0] == 0.0


def test_tiled_partial_tiles_keep_neighbours():
    print("[quantize] tiled partial update", flush=True)
    spec = tq.Spec(3, layout=tq.LAYOUT_TILED)
    cap = 128
    x = _data(cap, seed=1, dtype="bf16")
    tab = tq.device_tables(spec)
    cache = tq.alloc_cache(spec, 1, cap)
    tq.quantize_kv(spec, tab, to_device(x, "bf16"), cache)
    before = cache.codes.clone()
    y = _data(5, seed=2, dtype="bf16")
    tq.quantize_kv(spec, tab, to_device(y, "bf16"), cache, tok0=43)  # inside tile 1, not aligned
    torch().cuda.synchronize()
    idx = read_codes(spec, cache, 0, cap)
    ref = read_codes(spec, tq.Cache(spec, cap, before, cache.norms), 0, cap)
    assert np.array_equal(idx[:43], ref[:43]) and np.array_equal(idx[48:], ref[48:])
    check_quantized(spec, y[0], idx[43:48], read_norms(cache, 0, 5, 43), label="partial")


def test_record_does_not_write_outside_range():
    print("[quantize] guard bytes", flush=True)
    spec = tq.Spec(4)
    x = _data(50, seed=3, dtype="bf16")
    cap = 100
    tab = tq.device_tables(spec)
    cache = tq.alloc_cache(spec, 1, cap, fill=0xA5)
    cache.norms.fill_(-7.0)
    tq.quantize_kv(spec, tab, to_device(x, "bf16"), cache, tok0=20)
    torch().cuda.synchronize()
    raw = cache.codes.cpu().numpy().reshape(cap, 64)
    assert np.all(raw[:20] == 0xA5) and np.all(raw[70:] == 0xA5)
    nm = cache.norms.cpu().numpy()
    assert np.all(nm[:20] == -7.0) and np.all(nm[70:] == -7.0)


@pytest.mark.parametrize("name", ["tiny_oracle", "gqa_decode", "qjl", "long_context"])
def test_quantize_full_size_sampled(name):
    """Full-size workload quantized in one call per tensor (as the bench does);
    a sample of streams is checked vector by vector against the oracle."""
    print(f"[quantize] full size {name}", flush=True)
    wl = workloads.WORKLOADS[name]
    inp = workloads.generate(name)
    B, Hkv, T = len(inp.k), wl.hkv, wl.ctx
    for tensor, qs, layout in (("k", wl.k, tq.LAYOUT_RECORD), ("v", wl.v, tq.LAYOUT_TILED)):
        spec = tq.Spec(qs.bits_lo, qs.bits_hi, split=qs.split, qjl_m=qs.qjl_m if tensor == "k" else 0,
                       layout=layout)
        data = inp.k if tensor == "k" else inp.v
        X = np.stack(data).reshape(B * Hkv, T, 128)
        tab = tq.device_tables(spec)
        cache = tq.alloc_cache(spec, B * Hkv, T)
        xd = to_device(X, wl.dtype)
        tq.quantize_kv(spec, tab, xd, cache)
        torch().cuda.synchronize()
        del xd
        rng = np.random.default_rng(0)
        streams = sorted(set(rng.integers(0, B * Hkv, 2).tolist()))
        for s in streams:
            n = min(T, 16384)
            t0 = int(rng.integers(0, T - n + 1)) // 32 * 32
            idx = read_codes(spec, cache, s, n, t0)
            signs = read_signs(cache, s, n, t0) if spec.qjl_m else None
            check_quantized(spec, X[s, t0:t0 + n], idx, read_norms(cache, s, n, t0), signs=signs,
                            label=f"{name}/{tensor}/stream {s}")


def _ragged_case(spec, lens, tok0s, hkv, cap, seed, fill_first=True):
    """Fill every stream with one call, then append a ragged batch with one
    ragged call; returns (x, cache, before-codes snapshot, before-norms)."""
    B = len(lens)
    tab = tq.device_tables(spec)
    cache = tq.alloc_cache(spec, B * hkv, cap, fill=0x5A)
    if fill_first:
        base = _data(B * hkv * cap, seed=seed + 100, dtype="bf16").reshape(B * hkv, cap, 128)
        tq.quantize_kv(spec, tab, to_device(base, "bf16"), cache)
    torch().cuda.synchronize()
    before = tq.clone_cache(cache)
    L = max(max(lens), 1)
    x = _data(B * hkv * L, seed=seed, dtype="bf16").reshape(B * hkv, L, 128)
    tq.quantize_kv_ragged(spec, tab, to_device(x, "bf16"), cache, hkv=hkv, n_tok=lens, tok0=tok0s)
    torch().cuda.synchronize()
    return x, cache, before


def _check_ragged(spec, x, cache, before, lens, tok0s, hkv, label):
    cap = cache.cap
    for b, (n, t0) in enumerate(zip(lens, tok0s)):
        for h in range(hkv):
            s = b * hkv + h
            got = read_codes(spec, cache, s, cap)
            old = read_codes(spec, before, s, cap)
            keep = np.ones(cap, bool)
            keep[t0:t0 + n] = False
            assert np.array_equal(got[keep], old[keep]), f"{label}: stream {s} changed outside its range"
            nm, nm_old = read_norms(cache, s, cap), read_norms(before, s, cap)
            assert np.array_equal(nm[keep], nm_old[keep]), f"{label}: stream {s} norms changed outside"
            if n:
                check_quantized(spec, x[s, :n], got[t0:t0 + n], nm[t0:t0 + n], label=f"{label}/stream {s}")


@pytest.mark.parametrize("layout", [tq.LAYOUT_RECORD, tq.LAYOUT_TILED])
@pytest.mark.parametrize("w", [(2, None, 128), (3, None, 128), (4, 3, 64)])
def test_quantize_ragged_batch(w, layout):
    """One ragged call: lengths 0 .. several tiles, unaligned offsets (partial
    first and last tiles merge into the stored codes), two streams per
    sequence; positions outside each range keep their previous contents."""
    print(f"[quantize] ragged widths={w} layout={layout}", flush=True)
    spec = tq.Spec(w[0], w[1], split=w[2], layout=layout)
    lens = [0, 1, 33, 100, 257, 31, 64]
    tok0s = [0, 5, 31, 64, 3, 40, 96]
    _check_ragged(spec, *_ragged_case(spec, lens, tok0s, hkv=2, cap=288, seed=w[0] + 3 * layout),
                  lens, tok0s, 2, f"ragged {w}/{layout}")


def test_quantize_ragged_many_sequences_and_packed_rows():
    """More sequences than one launch takes (70), and a packed [tokens, hkv, d]
    input addressed through per-sequence offsets."""
    print("[quantize] ragged: 70 sequences; packed rows", flush=True)
    rng = np.random.default_rng(11)
    for layout in (tq.LAYOUT_RECORD, tq.LAYOUT_TILED):
        spec = tq.Spec(4, layout=layout)
        lens = rng.integers(0, 70, 70).tolist()
        tok0s = rng.integers(0, 20, 70).tolist()
        _check_ragged(spec, *_ragged_case(spec, lens, tok0s, hkv=1, cap=96, seed=21 + layout, fill_first=False),
                      lens, tok0s, 1, f"70 sequences/{layout}")
    # packed rows: sequence b's tokens are rows start_b .. start_b + n_b of a [tokens, hkv, d] tensor
    hkv, lens, tok0s = 3, [17, 0, 45, 32], [0, 0, 7, 32]
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    packed = _data(sum(lens) * hkv, seed=33, dtype="bf16").reshape(sum(lens), hkv, 128)
    for layout in (tq.LAYOUT_RECORD, tq.LAYOUT_TILED):
        spec = tq.Spec(3, layout=layout)
        tab = tq.device_tables(spec)
        cache = tq.alloc_cache(spec, len(lens) * hkv, 96)
        xd = to_device(packed, "bf16")
        tq.quantize_kv_ragged(spec, tab, xd, cache, hkv=hkv, n_tok=lens, tok0=tok0s,
                              x_off=starts * hkv * 128, x_stream_stride=128, x_row_stride=hkv * 128)
        torch().cuda.synchronize()
        for b, (n, t0) in enumerate(zip(lens, tok0s)):
            for h in range(hkv):
                if n:
                    s = b * hkv + h
                    xs = packed[starts[b]:starts[b] + n, h]
                    check_quantized(spec, xs, read_codes(spec, cache, s, n, t0), read_norms(cache, s, n, t0),
                                    label=f"packed/{layout}/stream {s}")


@pytest.mark.parametrize("n_seq", [3, 70])
def test_quantize_ragged_qjl(n_seq):
    """A spec with the sketch goes through the general kernel, one launch per
    32 sequences (70: three launches, the last one partial), with empty
    sequences skipped and every sequence's own offset and start position."""
    print(f"[quantize] ragged qjl: {n_seq} sequences", flush=True)
    spec = tq.Spec(2, qjl_m=128)
    if n_seq == 3:
        lens, tok0s, hkv = [40, 0, 77], [0, 3, 9], 2
    else:
        rng = np.random.default_rng(45)
        lens, tok0s, hkv = rng.integers(0, 78, n_seq).tolist(), rng.integers(0, 19, n_seq).tolist(), 2
        lens[5] = lens[40] = 0
    B = len(lens)
    x = _data(B * hkv * 77, seed=44, dtype="bf16").reshape(B * hkv, 77, 128)
    tab = tq.device_tables(spec)
    cache = tq.alloc_cache(spec, B * hkv, 96)
    tq.quantize_kv_ragged(spec, tab, to_device(x, "bf16"), cache, hkv=hkv, n_tok=lens, tok0=tok0s)
    torch().cuda.synchronize()
    for b, (n, t0) in enumerate(zip(lens, tok0s)):
        for h in range(hkv):
            s = b * hkv + h
            if n:
                check_quantized(spec, x[s, :n], read_codes(spec, cache, s, n, t0), read_norms(cache, s, n, t0),
                                signs=read_signs(cache, s, n, t0), label=f"ragged qjl/stream {s}")


def test_quantize_ragged_full_size_sampled():
    """The 64-sequence ragged workload (lengths 1024..32768, 128 sink tokens,
    8 KV heads) quantized with one ragged call per tensor, as the bench does;
    sampled streams checked vector by vector against the oracle."""
    print("[quantize] ragged full size", flush=True)
    wl = workloads.WORKLOADS["batched_ragged"]
    inp = workloads.generate("batched_ragged")
    B, Hkv, S = len(inp.k), wl.hkv, wl.sink
    comp = np.array([a.shape[1] - S for a in inp.k], np.int64)
    cap = int(-(-comp.max() // 32) * 32)
    rng = np.random.default_rng(5)
    seqs = sorted(set(rng.integers(0, B, 3).tolist()))
    for tensor, qs, layout in (("k", wl.k, tq.LAYOUT_RECORD), ("v", wl.v, tq.LAYOUT_TILED)):
        spec = tq.Spec(qs.bits_lo, qs.bits_hi, split=qs.split, layout=layout)
        data = inp.k if tensor == "k" else inp.v
        host = np.zeros((B * Hkv, cap, 128), np.uint16)
        for b in range(B):
            host[b * Hkv:(b + 1) * Hkv, :comp[b]] = workloads.bf16_bits(data[b][:, S:])
        xd = torch().from_numpy(host.view(np.int16)).cuda().view(torch().bfloat16)
        del host
        tab = tq.device_tables(spec)
        cache = tq.alloc_cache(spec, B * Hkv, cap)
        tq.quantize_kv_ragged(spec, tab, xd, cache, hkv=Hkv, n_tok=comp)
        torch().cuda.synchronize()
        del xd
        for b in seqs:
            h = int(rng.integers(0, Hkv))
            n = int(comp[b])
            xs = workloads.bf16_to_f32(workloads.bf16_bits(data[b][h, S:]))
            check_quantized(spec, xs, read_codes(spec, cache, b * Hkv + h, n), read_norms(cache, b * Hkv + h, n),
                            label=f"ragged/{tensor}/seq {b} head {h}")


def test_quantize_wide_row_stride_general_kernel():
    """Rows 2^24 elements apart (32 MiB of bf16) exceed the rotation kernel's
    32-bit buffer offsets, so the call goes to the general kernel; records and tiles (with partly written tiles merged) must
    still match the oracle, and the tiled neighbours must keep their codes."""
    print("[quantize] wide row stride: general kernel", flush=True)
    T = torch()
    xrs, n = 1 << 24, 3
    rng = np.random.default_rng(17)
    rows = workloads.bf16_to_f32(workloads.bf16_bits(rng.standard_normal((n, 128), dtype=np.float32)))
    flat = T.zeros(n * xrs + 128, dtype=T.bfloat16, device="cuda")
    for i in range(n):
        flat[i * xrs:i * xrs + 128] = to_device(rows[i:i + 1], "bf16")[0]
    x = flat.as_strided((1, n, 128), (n * xrs, xrs, 1))
    for layout in (tq.LAYOUT_RECORD, tq.LAYOUT_TILED):
        spec = tq.Spec(4, 3, split=64, layout=layout)
        tab = tq.device_tables(spec)
        cache = tq.alloc_cache(spec, 1, 64)
        base = _data(64, seed=18, dtype="bf16")
        tq.quantize_kv(spec, tab, to_device(base, "bf16"), cache)
        T.cuda.synchronize()
        before = read_codes(spec, cache, 0, 64)
        tq.quantize_kv(spec, tab, x, cache, tok0=30)  # positions 30..32: across a tile edge
        tq.quantize_kv_ragged(spec, tab, x, cache, hkv=1, n_tok=[2], tok0=[40], x_off=[0],
                              x_stream_stride=n * xrs, x_row_stride=xrs)
        T.cuda.synchronize()
        got = read_codes(spec, cache, 0, 64)
        keep = np.ones(64, bool)
        keep[30:33] = keep[40:42] = False
        assert np.array_equal(got[keep], before[keep]), f"layout {layout}: neighbours changed"
        check_quantized(spec, rows, got[30:33], read_norms(cache, 0, 3, 30), label=f"wide stride/{layout}")
        check_quantized(spec, rows[:2], got[40:42], read_norms(cache, 0, 2, 40), label=f"wide stride ragged/{layout}")


@pytest.mark.parametrize("layout", [tq.LAYOUT_RECORD, tq.LAYOUT_TILED])
@pytest.mark.parametrize("w", [(4, None, 128), (4, 3, 64), (2, None, 128)])
def test_quantize_hadamard_rotation(w, layout):
    """The randomized Hadamard rotation runs through the same kernels (its
    matrix sits in the tables): parity with the oracle's Hadamard Pi, with a
    ragged tail and an unaligned second append."""
    print(f"[quantize] hadamard widths={w} layout={layout}", flush=True)
    spec = tq.Spec(w[0], w[1], split=w[2], layout=layout, rot_seed=3, rotation=tq.ROT_HADAMARD)
    x = _data(1000, seed=40 + w[0] + layout, dtype="bf16")
    cache = _quantize(spec, x, "bf16", cap=1056)
    y = _data(37, seed=41, dtype="bf16")
    tq.quantize_kv(spec, tq.device_tables(spec), to_device(y, "bf16"), cache, tok0=1003)
    torch().cuda.synchronize()
    check_quantized(spec, x[0], read_codes(spec, cache, 0, 1000), read_norms(cache, 0, 1000), label=f"hadamard {w}")
    check_quantized(spec, y[0], read_codes(spec, cache, 0, 37, 1003), read_norms(cache, 0, 37, 1003),
                    label=f"hadamard append {w}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_eight_bit_keys(dtype):
    """8-bit keys (record layout, 1024-cell code table): 1000 vectors (a
    ragged tail), then three streams written from position 37 with zero
    vectors among them."""
    print(f"[quantize] 8-bit keys dtype={dtype}", flush=True)
    spec = tq.Spec(8)
    n = 1000
    x = _data(n, seed=88, dtype=dtype)
    cache = _quantize(spec, x, dtype)
    check_quantized(spec, x[0], read_codes(spec, cache, 0, n), read_norms(cache, 0, n), label=f"8-bit {dtype}")
    x = np.random.default_rng(89).standard_normal((3, 70, 128), dtype=np.float32)
    x[1, 5] = 0.0
    if dtype == "bf16":
        x = workloads.bf16_to_f32(workloads.bf16_bits(x))
    cache = _quantize(spec, x, dtype, cap=160, tok0=37)
    for s in range(3):
        check_quantized(spec, x[s], read_codes(spec, cache, s, 70, 37), read_norms(cache, s, 70, 37),
                        label=f"8-bit stream {s}")
    # a zero vector: norm 0, y = 0, code 127 (the 127 negative boundaries lie
    # below 0; the middle boundary is 0 itself, not below)
    assert read_norms(cache, 1, 1, 42)[0] == 0.0
    assert np.all(read_codes(spec, cache, 1, 1, 42) == 127)


def test_quantize_eight_bit_full_size_sampled():
    """The gqa_decode key tensor (8 x 32768 bf16 vectors with outlier
    channels) at 8 bits in one launch; sampled vectors against the oracle."""
    print("[quantize] 8-bit keys, full gqa_decode key tensor", flush=True)
    inp = workloads.generate("gqa_decode")
    spec = tq.Spec(8)
    xk = np.asarray(inp.k[0])                    # [8, 32768, 128]
    n = xk.shape[1]
    cache = _quantize(spec, xk, "bf16")
    codes = cache.codes.cpu().numpy().reshape(8, n, 128)
    norms = cache.norms.cpu().numpy().reshape(8, n)
    rng = np.random.default_rng(3)
    for s in range(8):
        rows = np.sort(rng.choice(n, 200, replace=False))
        idx = opk.unpack_records(codes[s, rows], spec.widths)
        check_quantized(spec, xk[s, rows], idx, norms[s, rows], label=f"8-bit full stream {s}")


@pytest.mark.parametrize("w", [(3, None, 128), (4, 3, 64)])
@pytest.mark.parametrize("layout", [tq.LAYOUT_RECORD, tq.LAYOUT_TILED])
def test_token_by_token_appends_equal_one_bulk_write(w, layout):
    """The decode-time pattern: 80 vectors appended one call per token (every
    value tile built up by merges into its stored words) give exactly the
    codes and norms of one bulk write of the same vectors."""
    print(f"[quantize] token-by-token appends widths={w} layout={layout}", flush=True)
    spec = tq.Spec(w[0], w[1], split=w[2], layout=layout)
    x = np.random.default_rng(17).standard_normal((2, 80, 128), dtype=np.float32)
    x = workloads.bf16_to_f32(workloads.bf16_bits(x))
    xd = to_device(x, "bf16")
    tab = tq.device_tables(spec)
    bulk = tq.alloc_cache(spec, 2, 96)
    tq.quantize_kv(spec, tab, xd, bulk)
    step = tq.alloc_cache(spec, 2, 96)
    for t in range(80):
        tq.quantize_kv(spec, tab, xd[:, t:t + 1], step, tok0=t)
    torch().cuda.synchronize()
    for s in range(2):
        assert np.array_equal(read_codes(spec, step, s, 80), read_codes(spec, bulk, s, 80))
        assert np.array_equal(read_norms(step, s, 80), read_norms(bulk, s, 80))
    check_quantized(spec, x[1], read_codes(spec, step, 1, 80), read_norms(step, 1, 80), label="appends")


def test_ragged_single_token_steps_equal_bulk_writes():
    """A decode step of a ragged batch: one tq_quantize_kv_ragged call per
    step appends one token to each live sequence at its own position
    (sequences start at different lengths and stop at different steps); the
    cache equals per-sequence bulk writes of the same vectors, both layouts."""
    print("[quantize] ragged single-token steps", flush=True)
    B, H = 6, 2
    rng = np.random.default_rng(23)
    start = rng.integers(0, 70, B)            # prefix lengths (written in bulk first)
    total = start + rng.integers(1, 40, B)     # final lengths
    x = rng.standard_normal((B * H, int(total.max()), 128), dtype=np.float32)
    x = workloads.bf16_to_f32(workloads.bf16_bits(x))
    xd = to_device(x, "bf16")
    for layout in (tq.LAYOUT_RECORD, tq.LAYOUT_TILED):
        spec = tq.Spec(4, 3, split=64, layout=layout)
        tab = tq.device_tables(spec)
        cap = int(-(-total.max() // 32) * 32)
        ref = tq.alloc_cache(spec, B * H, cap)
        tq.quantize_kv_ragged(spec, tab, xd, ref, hkv=H, n_tok=total)
        got = tq.alloc_cache(spec, B * H, cap)
        tq.quantize_kv_ragged(spec, tab, xd, got, hkv=H, n_tok=start)
        pos = start.copy()
        while np.any(pos < total):
            live = (pos < total).astype(np.int64)
            step_x = torch().zeros((B * H, 1, 128), dtype=xd.dtype, device="cuda")
            for b in range(B):
                if live[b]:
                    step_x[b * H:(b + 1) * H, 0] = xd[b * H:(b + 1) * H, pos[b]]
            tq.quantize_kv_ragged(spec, tab, step_x, got, hkv=H, n_tok=live, tok0=pos)
            pos = pos + live
        torch().cuda.synchronize()
        for s in range(B * H):
            n = int(total[s // H])
            assert np.array_equal(read_codes(spec, got, s, n), read_codes(spec, ref, s, n)), (layout, s)
            assert np.array_equal(read_norms(got, s, n), read_norms(ref, s, n)), (layout, s)


@pytest.mark.parametrize("bits,layout,qjl", [((4, None, 128), tq.LAYOUT_RECORD, 0), ((3, None, 128), tq.LAYOUT_TILED, 0),
                                             ((4, 3, 64), tq.LAYOUT_TILED, 0), ((2, None, 128), tq.LAYOUT_RECORD, 128),
                                             ((8, None, 128), tq.LAYOUT_RECORD, 0)])
def test_quantize_fp16_norms(bits, layout, qjl):
    """fp16 norms: the same codes (and sketch), the norm stored as the fp32
    norm rounded to binary16 (nearest even), within one fp16 ulp; written
    from position 37 of a stream to cover partial tiles."""
    print(f"[quantize] fp16 norms {bits} layout={layout} qjl={qjl}", flush=True)
    spec = tq.Spec(bits[0], bits[1], split=bits[2], layout=layout, qjl_m=qjl, norm_f16=1)
    x = _data(1000, seed=61, dtype="bf16")
    cache = _quantize(spec, x, "bf16", cap=1056, tok0=37)
    assert cache.norms.dtype == torch().float16
    signs = read_signs(cache, 0, 1000, 37) if qjl else None
    check_quantized(spec, x[0], read_codes(spec, cache, 0, 1000, 37), read_norms(cache, 0, 1000, 37), signs=signs,
                    label=f"fp16 norms {bits}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("bits,layout,qjl", [((4, None, 128), tq.LAYOUT_RECORD, 0), ((3, None, 128), tq.LAYOUT_TILED, 0),
                                             ((2, None, 128), tq.LAYOUT_RECORD, 128)])
def test_quantize_fp16_norms_saturate(bits, layout, qjl, dtype):
    """fp16 norms at the top of the binary16 range: a norm that would round to
    infinity is stored as 65504, as the oracle reads it; the codes do not
    depend on the norm's size."""
    print(f"[quantize] fp16 norm saturation {bits} layout={layout} qjl={qjl} {dtype}", flush=True)
    spec = tq.Spec(bits[0], bits[1], split=bits[2], layout=layout, qjl_m=qjl, norm_f16=1)
    x = _data(96, seed=62, dtype=dtype)
    big = [65472.0, 65519.0, 65520.0, 65536.0, 70000.0, 1.0e6, 65280.0] if dtype == "f32" else \
          [65280.0, 65536.0, 70144.0, 1.0e6]
    for i, v in enumerate(big):
        x[0, 3 * i + 1] = 0.0
        x[0, 3 * i + 1, (17 * i) % 128] = v
        x[0, 3 * i + 2] *= np.float32(v / 11.0)        # a full vector of that size too
    if dtype == "bf16":
        x = workloads.bf16_to_f32(workloads.bf16_bits(x))
    cache = _quantize(spec, x, dtype)
    norms = read_norms(cache, 0, 96)
    assert np.all(np.isfinite(norms.astype(np.float32))), "an fp16 norm overflowed to infinity"
    signs = read_signs(cache, 0, 96) if qjl else None
    check_quantized(spec, x[0], read_codes(spec, cache, 0, 96), norms, signs=signs, label=f"fp16 saturation {bits}")


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_quantize_hadamard_butterflies(bits):
    """TQ_ROT_HADAMARD_FWHT: the randomized Hadamard matrix applied by the
    butterfly kernel (bf16 keys, record layout).  Codes and norms pass the
    oracle's rules for the Hadamard rotation, over a ragged call with
    unaligned offsets, a partial last tile and zero vectors, with fp32 and
    fp16 norms; the dense-product Hadamard path gives the same codes up to
    band mismatches against the same oracle."""
    print(f"[quantize] hadamard butterflies {bits}-bit", flush=True)
    T = torch()
    lens = [45, 0, 130, 77]
    hkv, rows = 3, 140
    x = np.random.default_rng(70 + bits).standard_normal((len(lens) * hkv, rows, 128), dtype=np.float32)
    x[1, 3] = 0.0
    x[7, 50] = 0.0
    x = workloads.bf16_to_f32(workloads.bf16_bits(x))
    tok0 = [5, 0, 33, 0]
    for nf in (0, 1):
        fw = tq.Spec(bits, layout=tq.LAYOUT_RECORD, rotation=tq.ROT_HADAMARD_FWHT, norm_f16=nf)
        dense = tq.Spec(bits, layout=tq.LAYOUT_RECORD, rotation=tq.ROT_HADAMARD, norm_f16=nf)
        got = {}
        for spec in (fw, dense):
            cache = tq.alloc_cache(spec, len(lens) * hkv, 192, fill=0x5A)
            tq.quantize_kv_ragged(spec, tq.device_tables(spec), to_device(x, "bf16"), cache, hkv=hkv, n_tok=lens,
                                  tok0=tok0)
            T.cuda.synchronize()
            got[spec.rotation] = cache
        for b, n in enumerate(lens):
            for h in range(hkv):
                s = b * hkv + h
                if n == 0:
                    raw = got[tq.ROT_HADAMARD_FWHT].codes[s * 192 * 16 * bits:(s + 1) * 192 * 16 * bits]
                    assert T.all(raw == 0x5A), "an empty sequence was written"
                    continue
                for rot, cache in got.items():
                    check_quantized(fw if rot == tq.ROT_HADAMARD_FWHT else dense, x[s, :n],
                                    read_codes(fw, cache, s, n, tok0[b]), read_norms(cache, s, n, tok0[b]),
                                    label=f"rotation {rot} b{b} h{h} nf{nf}")
                # positions outside the written range keep their fill
                c = got[tq.ROT_HADAMARD_FWHT]
                rb = 16 * bits
                stream = c.codes[s * 192 * rb:(s + 1) * 192 * rb].view(192, rb)
                assert T.all(stream[:tok0[b]] == 0x5A) and T.all(stream[tok0[b] + n:] == 0x5A)


def test_quantize_hadamard_butterflies_many_sequences():
    """The butterfly kernel takes at most 64 sequences per launch: a ragged
    call of 150 short sequences (three launches, empty ones among them) must
    write every sequence's streams, held to the oracle's Hadamard rotation."""
    print("[quantize] hadamard butterflies: 150 sequences", flush=True)
    T = torch()
    rng = np.random.default_rng(75)
    n_seq, hkv, rows, cap = 150, 2, 40, 64
    lens = rng.integers(0, rows + 1, n_seq).tolist()
    lens[0] = lens[64] = lens[128] = 0
    tok0 = rng.integers(0, cap - rows + 1, n_seq).tolist()
    x = workloads.bf16_to_f32(workloads.bf16_bits(
        rng.standard_normal((n_seq * hkv, rows, 128), dtype=np.float32)))
    spec = tq.Spec(4, layout=tq.LAYOUT_RECORD, rotation=tq.ROT_HADAMARD_FWHT)
    cache = tq.alloc_cache(spec, n_seq * hkv, cap, fill=0x5A)
    tq.quantize_kv_ragged(spec, tq.device_tables(spec), to_device(x, "bf16"), cache, hkv=hkv, n_tok=lens, tok0=tok0)
    T.cuda.synchronize()
    rb = tq.code_bytes(spec)
    streams = cache.codes[: n_seq * hkv * cap * rb].view(n_seq * hkv, cap, rb)
    for b, n in enumerate(lens):
        for h in range(hkv):
            s = b * hkv + h
            assert T.all(streams[s, :tok0[b]] == 0x5A) and T.all(streams[s, tok0[b] + n:] == 0x5A), \
                f"sequence {b}: positions outside its range were written"
            if n:
                check_quantized(spec, x[s, :n], read_codes(spec, cache, s, n, tok0[b]),
                                read_norms(cache, s, n, tok0[b]), label=f"butterflies seq {b} head {h}")


def _extreme_scale_vectors(dtype):
    """Vectors whose elements span bf16's exponent range: groups of 24 N(0,1)
    vectors scaled by 2^e for e from -120 to +120 (squares below or above the
    fp32 range), then vectors that mix one element of 2^70 or 2^-70 with
    unit-scale ones, and zero vectors."""
    rng = np.random.default_rng(404)
    exps = [-120, -100, -80, -66, -40, 0, 40, 66, 90, 120]
    x = rng.standard_normal((len(exps) * 24 + 16, 128), dtype=np.float32)
    for g, e in enumerate(exps):
        x[24 * g:24 * (g + 1)] *= np.float32(2.0 ** e)
    tail = x[len(exps) * 24:]
    tail[0:4, 7] = np.float32(2.0 ** 70)
    tail[4:8, 100] = np.float32(2.0 ** -70)
    tail[4:8, :100] *= np.float32(2.0 ** -60)
    tail[8:12] = 0.0
    tail[12:16] *= np.float32(2.0 ** -124)
    if dtype == "bf16":
        x = workloads.bf16_to_f32(workloads.bf16_bits(x))
    return x[None]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("layout", [tq.LAYOUT_RECORD, tq.LAYOUT_TILED])
def test_quantize_extreme_scales(layout, dtype):
    """Norms from 2^-130 to 2^124: the stored norm is within 1 ulp of the
    correctly rounded one and the codes follow the oracle's band rule, where
    the squares of the elements fall below or above the fp32 range."""
    print(f"[quantize] extreme scales layout={layout} dtype={dtype}", flush=True)
    spec = tq.Spec(4, layout=layout)
    x = _extreme_scale_vectors(dtype)
    n = x.shape[1]
    cache = _quantize(spec, x, dtype)
    check_quantized(spec, x[0], read_codes(spec, cache, 0, n), read_norms(cache, 0, n), label=f"{layout}/{dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_extreme_scales_sketch(dtype):
    """The same vectors through the kernel of the sketch spec."""
    print(f"[quantize] extreme scales qjl dtype={dtype}", flush=True)
    spec = tq.Spec(2, qjl_m=128)
    x = _extreme_scale_vectors(dtype)
    n = x.shape[1]
    cache = _quantize(spec, x, dtype)
    check_quantized(spec, x[0], read_codes(spec, cache, 0, n), read_norms(cache, 0, n),
                    signs=read_signs(cache, 0, n), label=f"qjl/{dtype}")


def test_quantize_extreme_scales_butterflies():
    """The same vectors through the butterfly Hadamard kernel (bf16 records)."""
    print("[quantize] extreme scales hadamard butterflies", flush=True)
    spec = tq.Spec(4, layout=tq.LAYOUT_RECORD, rotation=tq.ROT_HADAMARD_FWHT)
    x = _extreme_scale_vectors("bf16")
    n = x.shape[1]
    cache = _quantize(spec, x, "bf16")
    check_quantized(spec, x[0], read_codes(spec, cache, 0, n), read_norms(cache, 0, n), label="fwht")
