"""GPU parity of the inner-product search scores (through the C ABI) against
the oracle evaluated on the GPU's own codes.

Bound: 2e-3 relative L2 over the score matrix.  The kernel's arithmetic: the
centroids pass through fp16 (relative rounding <= 2^-11), the rotated query
through fp16 hi + lo (about 2^-22) with fp32 accumulation, so the score error
stays near 5e-4 of its magnitude; 2e-3 leaves a factor 4."""
import numpy as np
import pytest

from compressed_kv_cache_tq_amd import tq, workloads
from gpu_helpers import ospec, read_codes, read_norms, read_signs, to_device, torch
from oracle import parity
from oracle import search as osr

pytestmark = pytest.mark.gpu


def _db(spec, n_streams, n_tok, seed, cap=None):
    x = np.random.default_rng(seed).standard_normal((n_streams, n_tok, 128), dtype=np.float32)
    x = workloads.bf16_to_f32(workloads.bf16_bits(x))
    tab = tq.device_tables(spec)
    cache = tq.alloc_cache(spec, n_streams, cap or n_tok)
    tq.quantize_kv(spec, tab, to_device(x, "bf16"), cache)
    return tab, cache


def _oracle(spec, cache, q, n_streams, n_tok, cols=None):
    ref = []
    for s in range(n_streams):
        idx, nrm = read_codes(spec, cache, s, n_tok), read_norms(cache, s, n_tok)
        bits = gamma = None
        if spec.qjl_m:
            bits, gamma = read_signs(cache, s, n_tok)
        ref.append(osr.ip_scores(q, idx, nrm, ospec(spec), bits, gamma))
    return np.concatenate(ref, axis=1)


@pytest.mark.parametrize("w,qjl", [((2, None, 128), 128), ((4, None, 128), 0), ((3, None, 128), 128),
                                   ((4, 3, 64), 0), ((3, 2, 64), 128)])
def test_ip_scores_small(w, qjl):
    """Three streams of 1000 vectors (a ragged last tile), 37 queries (a
    partial query block), both rotations."""
    for rot in (tq.ROT_HAAR, tq.ROT_HADAMARD):
        print(f"[search] widths={w} qjl={qjl} rotation={rot}", flush=True)
        spec = tq.Spec(w[0], w[1], split=w[2], qjl_m=qjl, rotation=rot)
        tab, cache = _db(spec, 3, 1000, seed=w[0] + qjl)
        q = np.random.default_rng(7).standard_normal((37, 128)).astype(np.float32)
        got = tq.ip_scores(spec, tab, cache, torch().from_numpy(q).cuda(), n_streams=3, n_tok=1000)
        torch().cuda.synchronize()
        ref = _oracle(spec, cache, q, 3, 1000)
        err = parity.rel_l2(got.cpu().numpy(), ref)
        print(f"[search]   rel_l2={err:.3e}", flush=True)
        assert err <= parity.ATTN_REL_L2, f"{w}/{qjl}/{rot}: rel L2 {err:.3e}"


def test_ip_scores_layout_guard_and_odd_length():
    """ld beyond n_streams * n_tok keeps the padding columns, an odd n_tok
    takes the unaligned store path, and one query gives one row."""
    print("[search] ld, odd length, single query", flush=True)
    T = torch()
    spec = tq.Spec(2, qjl_m=128)
    tab, cache = _db(spec, 2, 333, seed=5, cap=352)
    for nq in (1, 16, 64):
        q = np.random.default_rng(nq).standard_normal((nq, 128)).astype(np.float32)
        ld = 2 * 333 + 9
        out = T.full((nq, ld), -7.0, dtype=T.float32, device="cuda")
        tq.ip_scores(spec, tab, cache, T.from_numpy(q).cuda(), n_streams=2, n_tok=333, scores=out, ld=ld)
        T.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.all(got[:, 666:] == -7.0)
        err = parity.rel_l2(got[:, :666], _oracle(spec, cache, q, 2, 333))
        assert err <= parity.ATTN_REL_L2, f"nq={nq}: rel L2 {err:.3e}"


def test_ip_scores_full_size_sampled():
    """The bench's search workload (8 streams x 131072 vectors, 2-bit codes
    with the sketch, 64 queries): sampled token columns against the oracle."""
    print("[search] full size", flush=True)
    T = torch()
    wl = workloads.SEARCH
    spec = tq.Spec(wl.bits, qjl_m=wl.qjl_m)
    rng = np.random.default_rng(0)
    x = workloads.search_database(wl)
    tab = tq.device_tables(spec)
    cache = tq.alloc_cache(spec, wl.streams, wl.n_tok)
    tq.quantize_kv(spec, tab, T.from_numpy(workloads.bf16_bits(x).view(np.int16)).cuda().view(T.bfloat16), cache)
    q = workloads.search_queries(wl)
    got = tq.ip_scores(spec, tab, cache, T.from_numpy(q).cuda(), n_streams=wl.streams, n_tok=wl.n_tok)
    T.cuda.synchronize()
    for s in sorted(set(rng.integers(0, wl.streams, 2).tolist())):
        t0 = int(rng.integers(0, wl.n_tok - 2048)) // 32 * 32
        idx, nrm = read_codes(spec, cache, s, 2048, t0), read_norms(cache, s, 2048, t0)
        bits, gamma = read_signs(cache, s, 2048, t0)
        ref = osr.ip_scores(q, idx, nrm, ospec(spec), bits, gamma)
        cols = got[:, s * wl.n_tok + t0: s * wl.n_tok + t0 + 2048].cpu().numpy()
        err = parity.rel_l2(cols, ref)
        print(f"[search]   stream {s} tokens {t0}..: rel_l2={err:.3e}", flush=True)
        assert err <= parity.ATTN_REL_L2


def test_search_rejects_eight_bit_codes():
    """Search takes codes of at most 4 bits: an 8-bit spec is refused before
    any launch."""
    spec = tq.Spec(8)
    tab = tq.device_tables(spec)
    cache = tq.alloc_cache(spec, 1, 64)
    q = torch().zeros((1, 128), dtype=torch().float32, device="cuda")
    scores = torch().empty((1, 64), dtype=torch().float32, device="cuda")
    with pytest.raises(tq.TqError):
        tq.ip_scores(spec, tab, cache, q, n_streams=1, n_tok=64, scores=scores, workspace=tq.alloc_ip_workspace())
