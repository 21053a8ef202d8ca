"""Paged caches: the quantize appends into pool pages through a device block
table and the decode reads through it.  The oracle is the reference: the codes,
norms and sketch read back through the block table pass the parity rules
against the oracle's quantization of the source vectors, and the paged decode
output is within the attention bar of the oracle's attention on those codes.
As extra checks, the same codes land at the mapped positions as in the
contiguous cache, bit for bit, and the paged decode equals the contiguous
decode exactly (same plan, same arithmetic)."""
import numpy as np
import pytest

from compressed_kv_cache_tq_amd import tq, workloads
from gpu_helpers import Run, check_quantized, oracle_attention, read_codes, read_norms, read_signs, to_device, torch
from oracle import parity

pytestmark = pytest.mark.gpu
P = tq.PAGE_TOKENS


def _tables(B, comp, n_pages, seed, junk=-1):
    """Random distinct pages per sequence; unused entries hold junk."""
    rng = np.random.default_rng(seed)
    need = [-(-int(c) // P) for c in comp]
    max_pages = max(1, max(need))
    perm = rng.permutation(n_pages)
    bt = np.full((B, max_pages), junk, np.int32)
    k = 0
    for b in range(B):
        bt[b, :need[b]] = perm[k:k + need[b]]
        k += need[b]
    assert k <= n_pages
    return bt


def _fill(pool, byte=0xAB):
    """Poison a pool so untouched positions are recognisable."""
    pool.codes.fill_(byte)
    pool.norms.fill_(-7.0)
    if pool.qjl_signs is not None:
        pool.qjl_signs.fill_(byte)
        pool.qjl_rnorms.fill_(-7.0)


def _paged_quantize(run, bt, n_pages, chunk, poison=False):
    """Appends each sequence's compressed tokens in chunks of `chunk` tokens."""
    wl, S, B, H = run.wl, run.wl.sink, run.B, run.wl.hkv
    kpool = tq.alloc_page_pool(run.kspec, n_pages, H)
    vpool = tq.alloc_page_pool(run.vspec, n_pages, H)
    if poison:
        _fill(kpool)
        _fill(vpool)
    btd = torch().from_numpy(bt).cuda()
    comp = [max(0, int(run.inp.seq_lens[b]) - S) for b in range(B)]
    xk = [to_device(run.inp.k[b], wl.dtype) for b in range(B)]
    xv = [to_device(run.inp.v[b], wl.dtype) for b in range(B)]
    for start in range(0, max(comp) + 1, chunk):
        n = [max(0, min(chunk, c - start)) for c in comp]
        if not any(n):
            continue
        # one [B*H, chunk, d] block of this chunk's rows (zeros past a sequence's end)
        T = torch()
        xkc = T.zeros((B * H, chunk, 128), dtype=xk[0].dtype, device="cuda")
        xvc = T.zeros_like(xkc)
        for b in range(B):
            if n[b]:
                xkc[b * H:(b + 1) * H, :n[b]] = xk[b][:, S + start:S + start + n[b]]
                xvc[b * H:(b + 1) * H, :n[b]] = xv[b][:, S + start:S + start + n[b]]
        pos0 = [start] * B
        tq.quantize_kv_paged(run.kspec, run.ktab, xkc, kpool, hkv=H, n_tok=n, pos0=pos0, block_table=btd,
                             n_pages=n_pages)
        tq.quantize_kv_paged(run.vspec, run.vtab, xvc, vpool, hkv=H, n_tok=n, pos0=pos0, block_table=btd,
                             n_pages=n_pages)
    torch().cuda.synchronize()
    return kpool, vpool, comp


def _gather(run, kpool, vpool, bt, comp):
    """Per (sequence, kv head): codes, norms (and sketch) of the compressed
    tokens read from the pools page by page through the block table, in the
    layout Run.gpu_codes returns."""
    H = run.wl.hkv
    K, Kn, V, Vn, Z, R = ([] for _ in range(6))
    for b in range(run.B):
        rows = [[] for _ in range(6)]
        for h in range(H):
            parts = [[] for _ in range(6)]
            for lp in range(-(-comp[b] // P)):
                n = min(P, comp[b] - lp * P)
                ps = int(bt[b, lp]) * H + h
                parts[0].append(read_codes(run.kspec, kpool, ps, n))
                parts[1].append(read_norms(kpool, ps, n))
                parts[2].append(read_codes(run.vspec, vpool, ps, n))
                parts[3].append(read_norms(vpool, ps, n))
                if run.kspec.qjl_m:
                    z, r = read_signs(kpool, ps, n)
                    parts[4].append(z)
                    parts[5].append(r)
            empty = [np.zeros((0, 128), np.int64), np.zeros(0, kpool.norms.cpu().numpy().dtype)]
            for i in range(4):
                rows[i].append(np.concatenate(parts[i]) if parts[i] else empty[i % 2])
            if run.kspec.qjl_m:
                rows[4].append(np.concatenate(parts[4]) if parts[4] else np.zeros((0, 128), bool))
                rows[5].append(np.concatenate(parts[5]) if parts[5] else np.zeros(0, np.float32))
        for dst, src in zip((K, Kn, V, Vn, Z, R), rows):
            dst.append(src)
    return K, Kn, V, Vn, (Z if run.kspec.qjl_m else None), (R if run.kspec.qjl_m else None)


def _check_against_oracle(run, kpool, vpool, bt, comp, out, label):
    """Pool contents through the block table against the oracle's quantization
    of the source vectors, and the paged decode output against the oracle's
    attention on those codes."""
    wl, S = run.wl, run.wl.sink
    K, Kn, V, Vn, Z, R = _gather(run, kpool, vpool, bt, comp)
    # the band rule's count cap applies to all codes of a tensor together
    keys = [(b, h) for b in range(run.B) if comp[b] for h in range(wl.hkv)]
    cat = lambda arrs: np.concatenate([arrs[b][h] for b, h in keys])
    xk = np.concatenate([run.inp.k[b][h, S:S + comp[b]] for b, h in keys])
    xv = np.concatenate([run.inp.v[b][h, S:S + comp[b]] for b, h in keys])
    signs = (cat(Z), cat(R)) if Z is not None else None
    check_quantized(run.kspec, xk, cat(K), cat(Kn), signs=signs, label=f"{label} keys")
    check_quantized(run.vspec, xv, cat(V), cat(Vn), label=f"{label} values")
    sk = sv = None
    if S:
        sk = [[run.inp.k[b][h, :S].astype(np.float64) for h in range(wl.hkv)] for b in range(run.B)]
        sv = [[run.inp.v[b][h, :S].astype(np.float64) for h in range(wl.hkv)] for b in range(run.B)]
    ref = oracle_attention(run.inp.q, run.kspec, run.vspec, run.inp.seq_lens, K, Kn, V, Vn, k_bits=Z, k_gamma=R,
                           sink_k=sk, sink_v=sv, sink=S, v_skip=wl.v_skip)
    err = parity.rel_l2(out.cpu().numpy(), ref)
    print(f"  {label}: paged decode vs oracle rel L2 {err:.2e}", flush=True)
    assert err <= parity.ATTN_REL_L2, f"{label}: paged decode vs oracle rel L2 {err:.3e}"


@pytest.mark.parametrize("name,ctx,batch,chunk", [
    ("tiny_oracle", None, None, 45),
    ("gqa_decode", 1500, None, 37),
    ("qjl", 1000, 2, 64),
    ("batched_ragged", 900, 5, 100),
    ("long_context", 700, None, 300),
])
def test_paged_codes_and_decode_match_contiguous(name, ctx, batch, chunk):
    print(f"[paged] {name} ctx={ctx} batch={batch} chunk={chunk}", flush=True)
    T = torch()
    run = Run(workloads.generate(name, ctx=ctx, batch=batch))
    run.quantize()
    run.attend()
    T.cuda.synchronize()
    ref_out = run.out.clone()
    wl, H, B = run.wl, run.wl.hkv, run.B
    comp = [max(0, int(run.inp.seq_lens[b]) - wl.sink) for b in range(B)]
    n_pages = sum(-(-c // P) for c in comp) + 3
    bt = _tables(B, comp, n_pages, seed=11, junk=-1 if name != "qjl" else 10 ** 6)
    kpool, vpool, comp = _paged_quantize(run, bt, n_pages, chunk)
    # the codes at every mapped position equal the contiguous cache's
    for b in range(B):
        for h in range(H):
            s = b * H + h
            for lp in range(-(-comp[b] // P)):
                n = min(P, comp[b] - lp * P)
                ps = int(bt[b, lp]) * H + h
                for spec, pool, cache in ((run.kspec, kpool, run.kc), (run.vspec, vpool, run.vc)):
                    assert np.array_equal(read_codes(spec, pool, ps, n), read_codes(spec, cache, s, n, lp * P))
                    assert np.array_equal(read_norms(pool, ps, n), read_norms(cache, s, n, lp * P))
                if run.kspec.qjl_m:
                    zp, rp = read_signs(kpool, ps, n)
                    zc, rc = read_signs(run.kc, s, n, lp * P)
                    assert np.array_equal(zp, zc) and np.array_equal(rp, rc)
    btd = T.from_numpy(bt).cuda()
    out = T.empty_like(run.q)
    tq.attend_decode_paged(run.kspec, run.ktab, kpool, run.vspec, run.vtab, vpool, run.q, run.seq_lens, out, run.ws,
                           hkv=H, block_table=btd, n_pages=n_pages, sink=wl.sink, sink_k=run.sink_k,
                           sink_v=run.sink_v, v_skip=wl.v_skip, max_len=run.max_len)
    T.cuda.synchronize()
    _check_against_oracle(run, kpool, vpool, bt, comp, out, f"paged {name}")
    assert T.equal(out, ref_out), f"{name}: paged decode differs from the contiguous decode"


def test_paged_single_split_streams_and_bad_page_ids():
    """256 streams (one split each, merged in place) and a table whose entries
    past each sequence's pages are out of the pool: they are never read."""
    print("[paged] 256 streams", flush=True)
    T = torch()
    wl = workloads.Workload("paged256", 32, 32, 8, "bf16", workloads.QSpec(4, 4), workloads.QSpec(2, 2),
                            lens_range=(129, 400), sink=128, v_skip=1e-6)
    run = Run(workloads.generate(wl))
    run.quantize()
    run.attend()
    T.cuda.synchronize()
    comp = [max(0, int(v) - 128) for v in run.inp.seq_lens]
    n_pages = sum(-(-c // P) for c in comp)
    bt = _tables(run.B, comp, n_pages, seed=3, junk=n_pages + 5)
    kpool, vpool, _ = _paged_quantize(run, bt, n_pages, 64)
    out = T.empty_like(run.q)
    tq.attend_decode_paged(run.kspec, run.ktab, kpool, run.vspec, run.vtab, vpool, run.q, run.seq_lens, out, run.ws,
                           hkv=8, block_table=T.from_numpy(bt).cuda(), n_pages=n_pages, sink=128,
                           sink_k=run.sink_k, sink_v=run.sink_v, v_skip=1e-6, max_len=run.max_len)
    T.cuda.synchronize()
    assert T.equal(out, run.out)


@pytest.mark.parametrize("name,chunk", [("gqa_decode", 37), ("qjl", 50)])
def test_paged_quantize_skips_pages_outside_the_pool(name, chunk):
    """Logical pages mapped to -1 or past the pool: their tokens are written
    nowhere (every pool page not in the table keeps its poison), the other
    pages hold the contiguous cache's codes exactly."""
    print(f"[paged] out-of-pool pages {name} chunk={chunk}", flush=True)
    run = Run(workloads.generate(name, ctx=900, batch=2))
    run.quantize()
    torch().cuda.synchronize()
    H, B = run.wl.hkv, run.B
    comp = [max(0, int(run.inp.seq_lens[b]) - run.wl.sink) for b in range(B)]
    n_pages = sum(-(-c // P) for c in comp) + 4
    bt = _tables(B, comp, n_pages, seed=5)
    bt[0, 1] = -1
    bt[1, 0] = n_pages + 3
    bt[1, 2] = 1 << 30
    used = set(int(v) for v in bt.ravel() if 0 <= v < n_pages)
    kpool, vpool, comp = _paged_quantize(run, bt, n_pages, chunk, poison=True)
    for spec, pool, cache in ((run.kspec, kpool, run.kc), (run.vspec, vpool, run.vc)):
        nb = tq.cache_code_bytes(spec, P)
        codes = pool.codes.cpu().numpy().reshape(n_pages, H, nb)
        norms = pool.norms.cpu().numpy().reshape(n_pages, H, P)
        for pg in range(n_pages):
            if pg not in used:
                assert np.all(codes[pg] == 0xAB) and np.all(norms[pg] == -7.0), f"page {pg} was written"
        for b in range(B):
            for lp in range(-(-comp[b] // P)):
                pg = int(bt[b, lp])
                if not 0 <= pg < n_pages:
                    continue
                n = min(P, comp[b] - lp * P)
                for h in range(H):
                    ps, s = pg * H + h, b * H + h
                    assert np.array_equal(read_codes(spec, pool, ps, n), read_codes(spec, cache, s, n, lp * P))
                    assert np.array_equal(read_norms(pool, ps, n), read_norms(cache, s, n, lp * P))
                    if spec.qjl_m:
                        zp, rp = read_signs(pool, ps, n)
                        zc, rc = read_signs(cache, s, n, lp * P)
                        assert np.array_equal(zp, zc) and np.array_equal(rp, rc)


@pytest.mark.parametrize("qjl", [0, 128])
def test_paged_prefill_then_token_by_token_appends(qjl):
    """The serving pattern: a paged prefill of each sequence's prefix, then
    decode steps that each append one token per live sequence at its own
    position (70 sequences: two launches of the 64-sequence table), ending
    at different steps.  Codes and decode equal the contiguous path's."""
    print(f"[paged] prefill + single-token appends, qjl={qjl}", flush=True)
    T = torch()
    wl = workloads.Workload(f"serve{qjl}", 70, 8, 2, "bf16", workloads.QSpec(2, 2, qjl_m=qjl) if qjl else workloads.QSpec(4, 4),
                            workloads.QSpec(3, 3), lens_range=(40, 300))
    run = Run(workloads.generate(wl))
    run.quantize()
    run.attend()
    T.cuda.synchronize()
    B, H = run.B, wl.hkv
    comp = [int(v) for v in run.inp.seq_lens]
    tail = np.random.default_rng(2).integers(1, 9, B)       # tokens appended one by one
    pre = [c - int(t) for c, t in zip(comp, tail)]
    n_pages = sum(-(-c // P) for c in comp) + 2
    bt = _tables(B, comp, n_pages, seed=9)
    btd = T.from_numpy(bt).cuda()
    kpool = tq.alloc_page_pool(run.kspec, n_pages, H)
    vpool = tq.alloc_page_pool(run.vspec, n_pages, H)
    xk = [to_device(run.inp.k[b], wl.dtype) for b in range(B)]
    xv = [to_device(run.inp.v[b], wl.dtype) for b in range(B)]

    def append(start, count):
        rows = max(1, max(count))
        xkc = T.zeros((B * H, rows, 128), dtype=xk[0].dtype, device="cuda")
        xvc = T.zeros_like(xkc)
        for b in range(B):
            if count[b]:
                xkc[b * H:(b + 1) * H, :count[b]] = xk[b][:, start[b]:start[b] + count[b]]
                xvc[b * H:(b + 1) * H, :count[b]] = xv[b][:, start[b]:start[b] + count[b]]
        for spec, tab, x, pool in ((run.kspec, run.ktab, xkc, kpool), (run.vspec, run.vtab, xvc, vpool)):
            tq.quantize_kv_paged(spec, tab, x, pool, hkv=H, n_tok=count, pos0=start, block_table=btd,
                                 n_pages=n_pages)

    append([0] * B, pre)
    pos = list(pre)
    for _ in range(int(tail.max())):
        count = [1 if pos[b] < comp[b] else 0 for b in range(B)]
        append(pos, count)
        pos = [p + c for p, c in zip(pos, count)]
    T.cuda.synchronize()
    assert pos == comp
    for b in range(B):
        for h in range(H):
            for lp in range(-(-comp[b] // P)):
                n = min(P, comp[b] - lp * P)
                ps, s = int(bt[b, lp]) * H + h, b * H + h
                for spec, pool, cache in ((run.kspec, kpool, run.kc), (run.vspec, vpool, run.vc)):
                    assert np.array_equal(read_codes(spec, pool, ps, n), read_codes(spec, cache, s, n, lp * P))
                    assert np.array_equal(read_norms(pool, ps, n), read_norms(cache, s, n, lp * P))
                if qjl:
                    zp, rp = read_signs(kpool, ps, n)
                    zc, rc = read_signs(run.kc, s, n, lp * P)
                    assert np.array_equal(zp, zc) and np.array_equal(rp, rc)
    out = T.empty_like(run.q)
    tq.attend_decode_paged(run.kspec, run.ktab, kpool, run.vspec, run.vtab, vpool, run.q, run.seq_lens, out, run.ws,
                           hkv=H, block_table=btd, n_pages=n_pages, max_len=run.max_len)
    T.cuda.synchronize()
    _check_against_oracle(run, kpool, vpool, bt, comp, out, f"paged serve qjl={qjl}")
    assert T.equal(out, run.out)


def test_paged_eight_bit_keys():
    """K8/V3 through the paged quantize (record tiles split at page and
    chunk edges) and the paged decode: equal to the contiguous path."""
    print("[paged] K8/V3", flush=True)
    T = torch()
    wl = workloads.Workload("pagedk8", 3, 16, 4, "bf16", workloads.QSpec(8, 8), workloads.QSpec(3, 3),
                            lens_range=(100, 700))
    run = Run(workloads.generate(wl))
    run.quantize()
    run.attend()
    T.cuda.synchronize()
    comp = [int(v) for v in run.inp.seq_lens]
    n_pages = sum(-(-c // P) for c in comp) + 1
    bt = _tables(run.B, comp, n_pages, seed=4)
    kpool, vpool, _ = _paged_quantize(run, bt, n_pages, 45)
    for b in range(run.B):
        for h in range(4):
            for lp in range(-(-comp[b] // P)):
                n = min(P, comp[b] - lp * P)
                ps, s = int(bt[b, lp]) * 4 + h, b * 4 + h
                assert np.array_equal(read_codes(run.kspec, kpool, ps, n), read_codes(run.kspec, run.kc, s, n, lp * P))
                assert np.array_equal(read_norms(kpool, ps, n), read_norms(run.kc, s, n, lp * P))
    out = T.empty_like(run.q)
    tq.attend_decode_paged(run.kspec, run.ktab, kpool, run.vspec, run.vtab, vpool, run.q, run.seq_lens, out, run.ws,
                           hkv=4, block_table=T.from_numpy(bt).cuda(), n_pages=n_pages, max_len=run.max_len)
    T.cuda.synchronize()
    _check_against_oracle(run, kpool, vpool, bt, comp, out, "paged K8/V3")
    assert T.equal(out, run.out)


def test_paged_fp16_norms():
    """fp16 norms through the paged quantize and the paged decode: equal to
    the contiguous path with fp16 norms."""
    print("[paged] fp16 norms", flush=True)
    T = torch()
    run = Run(workloads.generate("batched_ragged", ctx=700, batch=3), norm_f16=1)
    run.quantize()
    run.attend()
    T.cuda.synchronize()
    wl, H, B = run.wl, run.wl.hkv, run.B
    comp = [max(0, int(run.inp.seq_lens[b]) - wl.sink) for b in range(B)]
    n_pages = sum(-(-c // P) for c in comp) + 2
    bt = _tables(B, comp, n_pages, seed=8)
    kpool, vpool, comp = _paged_quantize(run, bt, n_pages, 50)
    assert kpool.norms.dtype == T.float16
    for b in range(B):
        for h in range(H):
            for lp in range(-(-comp[b] // P)):
                n = min(P, comp[b] - lp * P)
                ps, s = int(bt[b, lp]) * H + h, b * H + h
                for spec, pool, cache in ((run.kspec, kpool, run.kc), (run.vspec, vpool, run.vc)):
                    assert np.array_equal(read_codes(spec, pool, ps, n), read_codes(spec, cache, s, n, lp * P))
                    assert np.array_equal(read_norms(pool, ps, n), read_norms(cache, s, n, lp * P))
    out = T.empty_like(run.q)
    tq.attend_decode_paged(run.kspec, run.ktab, kpool, run.vspec, run.vtab, vpool, run.q, run.seq_lens, out, run.ws,
                           hkv=H, block_table=T.from_numpy(bt).cuda(), n_pages=n_pages, sink=wl.sink,
                           sink_k=run.sink_k, sink_v=run.sink_v, v_skip=wl.v_skip, max_len=run.max_len)
    T.cuda.synchronize()
    _check_against_oracle(run, kpool, vpool, bt, comp, out, "paged fp16 norms")
    assert T.equal(out, run.out)
