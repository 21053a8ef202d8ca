"""GPU parity of the quantize kernel (through the C ABI) against the oracle."""
import numpy as np
import pytest

from compressed_kv_cache_tq_amd import tq, workloads
from gpu_helpers import check_quantized, read_codes, read_norms, read_signs, to_device, torch

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
