"""GPU parity of decode attention over the packed cache (through the C ABI).

The oracle reads the GPU's own codes, norms and sketch bits and evaluates the
attention in float64; the bound is 2e-3 relative L2 over the whole output."""
import dataclasses

import numpy as np
import pytest

from compressed_kv_cache_tq_amd import tq, workloads
from gpu_helpers import Run, oracle_attention, torch
from oracle import parity

pytestmark = pytest.mark.gpu


def _check(run: Run, heads=None, tol=parity.ATTN_REL_L2, label=""):
    run.quantize()
    run.attend()
    torch().cuda.synchronize()
    out = run.out.cpu().numpy().astype(np.float64)
    K, Kn, V, Vn, Z, R = run.gpu_codes(heads)
    inp, wl = run.inp, run.wl
    sk = sv = None
    if wl.sink:
        sk = [[inp.k[b][h][: wl.sink] for h in range(wl.hkv)] for b in range(run.B)]
        sv = [[inp.v[b][h][: wl.sink] for h in range(wl.hkv)] for b in range(run.B)]
    ref = oracle_attention(inp.q, run.kspec, run.vspec, inp.seq_lens, K, Kn, V, Vn, k_bits=Z, k_gamma=R,
                           sink_k=sk, sink_v=sv, sink=wl.sink, v_skip=wl.v_skip, heads=heads)
    mask = ~np.isnan(ref[..., 0])
    assert np.all(np.isfinite(out)), f"{label}: non-finite output"
    err = parity.rel_l2(out[mask], ref[mask])
    per = [parity.rel_l2(out[b, h], ref[b, h]) for b, h in zip(*np.nonzero(mask)) if np.any(ref[b, h])] or [0.0]
    print(f"[attend] {label}: rel_l2={err:.3e} worst head={max(per):.3e}", flush=True)
    assert err <= tol, f"{label}: rel L2 {err:.3e} > {tol}"
    return err


@pytest.mark.parametrize("name,ctx,batch", [
    ("tiny_oracle", None, None),
    ("gqa_decode", 2000, None),
    ("qjl", 1500, 2),
    ("long_context", 3000, None),
    ("batched_ragged", 1500, 5),
])
def test_attend_small(name, ctx, batch):
    print(f"[attend] small {name} ctx={ctx} batch={batch}", flush=True)
    _check(Run(workloads.generate(name, ctx=ctx, batch=batch)), label=f"{name} small")


@pytest.mark.parametrize("rot", [tq.ROT_HADAMARD, tq.ROT_HADAMARD_FWHT])
@pytest.mark.parametrize("name,ctx,batch", [("gqa_decode", 1500, None), ("qjl", 1000, 2), ("batched_ragged", 900, 3)])
def test_attend_hadamard_rotation(name, ctx, batch, rot):
    """Keys and values rotated by the randomized Hadamard matrix (QJL keys
    included), as a dense product or (TQ_ROT_HADAMARD_FWHT, the sketch-free
    bf16 keys) by butterflies: the oracle with the Hadamard Pi."""
    print(f"[attend] hadamard {name} rotation {rot}", flush=True)
    run = Run(workloads.generate(name, ctx=ctx, batch=batch))
    run.kspec = dataclasses.replace(run.kspec, rotation=rot)
    run.vspec = dataclasses.replace(run.vspec, rotation=rot)
    run.ktab, run.vtab = tq.device_tables(run.kspec), tq.device_tables(run.vspec)
    _check(run, label=f"{name} hadamard")


def test_attend_sink_and_peaked_v_skip():
    """Peaked scores (q x 8) so the V-skip rule drops tokens; ragged lengths
    including one equal to the sink and one shorter than it."""
    print("[attend] v-skip / sink edge cases", flush=True)
    inp = workloads.generate("batched_ragged", ctx=700, batch=4)
    inp.seq_lens[0] = 128      # only sink tokens
    inp.seq_lens[1] = 50       # shorter than the sink
    inp.q = inp.q * np.float32(8.0)
    _check(Run(inp), label="v-skip edge")


@pytest.mark.parametrize("name,ctx,batch,qs", [
    ("long_context", 3000, None, 16.0),
    ("long_context", 3000, None, 32.0),
    ("gqa_decode", 2000, None, 32.0),
    ("batched_ragged", 1500, 4, 32.0),
])
def test_attend_peaked_scores(name, ctx, batch, qs):
    """Queries scaled so the logits spread 16 or 32 times wider: softmaxes
    close to one-hot, where a score error moves weight between the top
    tokens.  The lookup tables' fp16 centroids carry a per-width scale that
    cuts their rounding error (3.5x at 4 bits, 9x at 3), which keeps these
    within the bar (with plain fp16 centroids long_context reached 3.7e-3 at
    x32)."""
    print(f"[attend] peaked scores {name} q x{qs:g}", flush=True)
    inp = workloads.generate(name, ctx=ctx, batch=batch)
    inp.q = inp.q * np.float32(qs)
    _check(Run(inp), label=f"peaked {name} q x{qs:g}")


def test_attend_gqa_g1_and_g16():
    for hq, hkv in ((8, 8), (16, 1)):
        print(f"[attend] hq={hq} hkv={hkv}", flush=True)
        wl = workloads.Workload(f"g{hq // hkv}", 2, hq, hkv, "bf16", workloads.QSpec(4, 4), workloads.QSpec(3, 3),
                                ctx=1234)
        _check(Run(workloads.generate(wl)), label=f"G={hq // hkv}")


@pytest.mark.parametrize("hq,hkv,sink", [(128, 128, 0), (256, 16, 32), (32, 8, 128)])
def test_attend_single_split_streams_merge_in_place(hq, hkv, sink):
    """256 or more (sequence, KV head) streams give one split per stream, so
    the split kernel merges its own partials (no combine launch): G = 1, 16
    and 4, ragged lengths including 0 and lengths below the sink."""
    print(f"[attend] one split per stream: hq={hq} hkv={hkv} sink={sink}", flush=True)
    B = max(1, 256 // hkv)
    wl = workloads.Workload(f"one{hq}_{hkv}_{sink}", B, hq, hkv, "bf16", workloads.QSpec(4, 4),
                            workloads.QSpec(2, 2), lens_range=(sink + 1, 200), sink=sink, v_skip=1e-6 if sink else 0.0)
    inp = workloads.generate(wl)
    inp.seq_lens[0] = 0
    if sink:
        inp.seq_lens[-1] = sink // 2
    _check(Run(inp), label=f"one split hq={hq} hkv={hkv} sink={sink}")


@pytest.mark.parametrize("kb,vb,qjl", [((3, 2), (3, 2), 0), ((4, 3), (3, 2), 128), ((3, 2), (4, 3), 0)])
def test_attend_mixed_width_combinations(kb, vb, qjl):
    """Split-width keys and values (64 coordinates at each width) in the other
    supported combinations, with and without the sketch."""
    print(f"[attend] mixed K{kb} V{vb} qjl={qjl}", flush=True)
    wl = workloads.Workload(f"mix{kb}{vb}{qjl}", 2, 8, 2, "bf16", workloads.QSpec(kb[0], kb[1], 64, qjl_m=qjl),
                            workloads.QSpec(vb[0], vb[1], 64), ctx=1111)
    _check(Run(workloads.generate(wl)), label=f"K{kb} V{vb} qjl={qjl}")


def test_attend_zero_length_sequence():
    print("[attend] zero-length sequence", flush=True)
    inp = workloads.generate("gqa_decode", ctx=300)
    run = Run(inp)
    run.quantize()
    run.seq_lens.zero_()
    run.attend()
    torch().cuda.synchronize()
    assert torch().count_nonzero(run.out).item() == 0


def test_attend_workspace_reuse():
    """Repeated calls on one workspace, and a call of another shape in
    between, give identical results: the workspace holds no state."""
    print("[attend] workspace reuse", flush=True)
    T = torch()
    run = Run(workloads.generate("gqa_decode", ctx=1000))
    run.quantize()
    big = tq.alloc_attend_workspace(4, 32, 8, 0, 4096)
    big.fill_(float("nan"))  # stale contents must not matter
    run.ws = big
    outs = []
    for _ in range(3):
        run.attend()
        T.cuda.synchronize()
        outs.append(run.out.clone())
    other = Run(workloads.generate("gqa_decode", ctx=3000))
    other.quantize()
    other.ws = big
    other.attend()
    run.attend()
    T.cuda.synchronize()
    outs.append(run.out.clone())
    for o in outs[1:]:
        assert T.equal(o, outs[0])
    _check(run, label="workspace reuse")


@pytest.mark.parametrize("name", ["tiny_oracle", "gqa_decode", "qjl", "long_context", "batched_ragged"])
def test_attend_full_size_sampled(name):
    """Full-size workload in the bench's launch configuration; the oracle
    evaluates a sample of query heads on the GPU's codes."""
    print(f"[attend] full size {name}", flush=True)
    inp = workloads.generate(name)
    run = Run(inp)
    wl = run.wl
    rng = np.random.default_rng(1)
    if name in ("tiny_oracle", "gqa_decode"):
        heads = None
    else:
        bs = sorted(set(rng.integers(0, run.B, 3).tolist()))
        heads = [(b, h) for b in bs for h in rng.choice(wl.hq, 8, replace=False).tolist()]
    _check(run, heads=heads, label=f"{name} full")


@pytest.mark.parametrize("vbits,batch,sink,ctx", [(3, 2, 0, 1111), (2, 5, 128, 0), (3, 1, 0, 3000)])
def test_attend_eight_bit_keys(vbits, batch, sink, ctx):
    """8-bit keys (K8) with 3- or 2-bit values: uniform and ragged batches,
    sink and V-skip; the oracle reads the GPU's 8-bit codes."""
    print(f"[attend] K8 V{vbits} batch={batch} sink={sink} ctx={ctx}", flush=True)
    wl = workloads.Workload(f"k8v{vbits}", batch, 32, 8, "bf16", workloads.QSpec(8, 8), workloads.QSpec(vbits, vbits),
                            ctx=ctx, lens_range=() if ctx else (sink + 1, 1500), sink=sink,
                            v_skip=1e-6 if sink else 0.0, structure="outlier_channels" if not sink else "plain")
    _check(Run(workloads.generate(wl)), label=f"K8 V{vbits}")


def test_attend_eight_bit_keys_full_gqa_shape():
    """The gqa_decode shape (8 KV heads x 32768 tokens, 32 query heads) with
    K8/V3, full output against the oracle."""
    print("[attend] K8/V3 at the gqa_decode shape", flush=True)
    inp = workloads.generate("gqa_decode")
    inp.wl = dataclasses.replace(inp.wl, k=workloads.QSpec(8, 8))
    _check(Run(inp), label="K8/V3 gqa shape")


def test_attend_per_layer_policies_share_one_workspace():
    """Per-layer K/V policies are chosen by the caller, one spec per call:
    three layers (K4/V2, K4/V4 as for a protected boundary layer, K8/V3)
    decode in turn on one workspace, each within the bound of its oracle."""
    print("[attend] per-layer policies on one workspace", flush=True)
    T = torch()
    ws = None
    runs = []
    for li, (kq, vq) in enumerate([(workloads.QSpec(4, 4), workloads.QSpec(2, 2)),
                                   (workloads.QSpec(4, 4), workloads.QSpec(4, 4)),
                                   (workloads.QSpec(8, 8), workloads.QSpec(3, 3))]):
        wl = workloads.Workload(f"layer{li}", 2, 16, 4, "bf16", kq, vq, ctx=900, seed=li)
        run = Run(workloads.generate(wl))
        ws = run.ws if ws is None else ws
        run.ws = ws
        runs.append(run)
    for run in runs:
        _check(run, label=f"layer {run.wl.name}")
    T.cuda.synchronize()


@pytest.mark.parametrize("qjl,sink", [(0, 512), (128, 0), (128, 300)])
def test_attend_sixteen_heads_per_group_edges(qjl, sink):
    """The largest group (16 query heads per KV head) with the largest sink
    (512 raw tokens, lengths below and above it), and with the sketch (the
    query fragments of 16 heads read from LDS every tile)."""
    print(f"[attend] G=16 qjl={qjl} sink={sink}", flush=True)
    kq = workloads.QSpec(2, 2, qjl_m=qjl) if qjl else workloads.QSpec(4, 4)
    wl = workloads.Workload(f"g16_{qjl}_{sink}", 3, 32, 2, "bf16", kq, workloads.QSpec(3, 3),
                            lens_range=(max(sink, 1), sink + 1500), sink=sink, v_skip=1e-6 if sink else 0.0)
    inp = workloads.generate(wl)
    if sink:
        inp.seq_lens[0] = sink // 3            # only sink tokens, fewer than the sink
    _check(Run(inp), label=f"G=16 qjl={qjl} sink={sink}")


def test_max_capacity_stream_of_identical_tokens():
    """One stream at the largest cache capacity (2^24 positions, 512 splits
    merged by the combine): every key and value is the same vector, so every
    stored code equals position 0's (sampled across the stream, including
    its last tile), and every softmax weight is equal, so each head's output
    is that one token's dequantized value, whatever the length."""
    from gpu_helpers import check_quantized, ospec, to_device
    from oracle import pack as opk
    from oracle import quantize as oqz
    print("[attend] 2^24-token stream of identical tokens", flush=True)
    T = torch()
    N = 1 << 24
    rng = np.random.default_rng(31)
    k0, v0 = (workloads.bf16_to_f32(workloads.bf16_bits(rng.standard_normal(128).astype(np.float32)))
              for _ in range(2))
    q = rng.standard_normal((1, 4, 128)).astype(np.float32)
    kspec, vspec = tq.Spec(4, layout=tq.LAYOUT_RECORD), tq.Spec(3, layout=tq.LAYOUT_TILED)
    ktab, vtab = tq.device_tables(kspec), tq.device_tables(vspec)
    kc, vc = tq.alloc_cache(kspec, 1, N), tq.alloc_cache(vspec, 1, N)
    for spec, tab, vec, cache in ((kspec, ktab, k0, kc), (vspec, vtab, v0, vc)):
        x = to_device(vec[None, None, :], "bf16").expand(1, N, 128).contiguous()
        tq.quantize_kv(spec, tab, x, cache)
        T.cuda.synchronize()
        del x

    def codes_at(spec, cache, p):
        if spec.layout == tq.LAYOUT_RECORD:
            rb = tq.code_bytes(spec)
            return opk.unpack_records(cache.codes[p * rb:(p + 1) * rb].cpu().numpy()[None], spec.widths)[0]
        tb = 32 * tq.code_bytes(spec)
        raw = cache.codes[(p // 32) * tb:(p // 32 + 1) * tb].cpu().numpy()
        return opk.unpack_tiled(raw, spec.widths, 1, p % 32)[0]

    first = {}
    for spec, cache, vec in ((kspec, kc, k0), (vspec, vc, v0)):
        c0, n0 = codes_at(spec, cache, 0), cache.norms[0:1].cpu().numpy()
        check_quantized(spec, vec[None], c0[None], n0, label="identical tokens")
        for p in (1, 31, 32, 12345, N // 2 + 7, N - 33, N - 1):
            assert np.array_equal(codes_at(spec, cache, p), c0), (spec.layout, p)
            assert cache.norms[p].item() == n0[0], (spec.layout, p)
        first[spec.layout] = (c0, float(n0[0]))
    ws = tq.alloc_attend_workspace(1, 4, 1, 0, N)
    out = T.empty((1, 4, 128), dtype=T.float32, device="cuda")
    tq.attend_decode(kspec, ktab, kc, vspec, vtab, vc, T.from_numpy(q).cuda(),
                     T.tensor([N], dtype=T.int32, device="cuda"), out, ws, hkv=1, max_len=N)
    T.cuda.synchronize()
    cv, nv = first[tq.LAYOUT_TILED]
    os_ = ospec(vspec)
    want = nv * (oqz.rotation_of(os_).T @ oqz.dequantize_rotated(cv[None], os_)[0])
    got = out.cpu().numpy().astype(np.float64)
    for h in range(4):
        assert parity.rel_l2(got[0, h], want) <= parity.ATTN_REL_L2, h


@pytest.mark.parametrize("name,ctx,batch", [("gqa_decode", 1500, None), ("qjl", 1000, 2), ("batched_ragged", 900, 3)])
def test_attend_fp16_norms(name, ctx, batch):
    """Key and value norms stored as fp16: the decode reads them through the
    fp16 variant; the oracle evaluates the attention on the GPU's codes and
    fp16 norms."""
    print(f"[attend] fp16 norms {name}", flush=True)
    _check(Run(workloads.generate(name, ctx=ctx, batch=batch), norm_f16=1), label=f"{name} fp16 norms")


def test_attend_eight_bit_keys_with_fp16_norms():
    """K8/V3 with fp16 norms (the 8-bit key instance of the fp16-norm
    decode): ragged batch, against the oracle on the GPU's codes and norms."""
    print("[attend] K8/V3 + fp16 norms", flush=True)
    wl = workloads.Workload("k8v3f16", 3, 16, 4, "bf16", workloads.QSpec(8, 8), workloads.QSpec(3, 3),
                            lens_range=(200, 1500))
    _check(Run(workloads.generate(wl), norm_f16=1), label="K8/V3 fp16 norms")
