"""Guard bands: no kernel writes outside the buffers it is given.

Each output buffer (the decode output, the attention workspace, the arrays of
a paged pool) is a view into a larger allocation whose margins hold a known
pattern; after the calls the margins must be unchanged.  The decode output
and the codes are also held to the oracle."""
import numpy as np
import pytest

from compressed_kv_cache_tq_amd import tq, workloads
from gpu_helpers import Run, to_device, torch
from oracle import parity
from test_gpu_attend import _check

pytestmark = pytest.mark.gpu
PAD = 4096  # bytes of margin on each side (keeps 16-byte alignment)
P = tq.PAGE_TOKENS


class Guarded:
    """A tensor of n elements inside margins filled with `fill`."""

    def __init__(self, n, dtype, fill):
        T = torch()
        esz = T.empty(0, dtype=dtype).element_size()
        self.pad = PAD // esz
        self.fill = fill
        self.buf = T.full((n + 2 * self.pad,), fill, dtype=dtype, device="cuda")
        self.view = self.buf[self.pad:self.pad + n]

    def intact(self) -> bool:
        T = torch()
        lo, hi = self.buf[:self.pad], self.buf[self.pad + self.view.numel():]
        want = T.full_like(lo, self.fill)
        return bool(T.equal(lo, want) and T.equal(hi, want))


def _guard_cache(spec, n_streams, cap):
    T = torch()
    nb = tq.cache_code_bytes(spec, cap)
    g = [Guarded(n_streams * nb, T.uint8, 0xA5),
         Guarded(n_streams * cap, T.float16 if spec.norm_f16 else T.float32, -7.25)]
    if spec.qjl_m:
        g += [Guarded(n_streams * cap * spec.qjl_m // 8, T.uint8, 0x5A), Guarded(n_streams * cap, T.float32, -7.25)]
    cache = tq.Cache(spec, cap, g[0].view, g[1].view, g[2].view if spec.qjl_m else None,
                     g[3].view if spec.qjl_m else None)
    return cache, g


@pytest.mark.parametrize("name,ctx,batch", [("gqa_decode", 1500, None), ("batched_ragged", 700, 4), ("qjl", 600, 2)])
def test_decode_writes_only_its_output_and_workspace(name, ctx, batch):
    print(f"[guards] decode {name}", flush=True)
    T = torch()
    run = Run(workloads.generate(name, ctx=ctx, batch=batch))
    wl = run.wl
    out = Guarded(run.q.numel(), T.float32, float("nan"))
    nws = run.ws.numel()
    ws = Guarded(nws, T.float32, -7.25)
    run.out = out.view.view(run.q.shape)
    run.ws = ws.view
    _check(run, label=f"{name} guarded")
    T.cuda.synchronize()
    # NaN margins: compare bit patterns
    assert T.equal(out.buf[:out.pad].isnan(), T.ones(out.pad, dtype=T.bool, device="cuda"))
    assert T.equal(out.buf[out.pad + out.view.numel():].isnan(), T.ones(out.pad, dtype=T.bool, device="cuda"))
    assert ws.intact(), f"{name}: the decode wrote outside its workspace"


def test_paged_calls_write_only_inside_the_pool():
    """A paged append into a pool whose arrays sit inside margins, pages in a
    scattered order including the pool's first and last page, then the paged
    decode: the margins of the pool arrays, the output and the workspace stay
    intact, and the output is the contiguous path's."""
    print("[guards] paged pool", flush=True)
    T = torch()
    for qjl in (0, 128):
        wl = workloads.Workload(f"guard{qjl}", 3, 8, 2, "bf16",
                                workloads.QSpec(2, 2, qjl_m=qjl) if qjl else workloads.QSpec(4, 4),
                                workloads.QSpec(3, 3), lens_range=(60, 250))
        run = Run(workloads.generate(wl))
        run.quantize()
        run.attend()
        T.cuda.synchronize()
        B, H = run.B, wl.hkv
        comp = [int(v) for v in run.inp.seq_lens]
        n_pages = sum(-(-c // P) for c in comp)
        perm = np.random.default_rng(3).permutation(n_pages).astype(np.int32)
        max_pages = max(-(-c // P) for c in comp)
        bt = np.full((B, max_pages), -1, np.int32)
        k = 0
        for b in range(B):
            m = -(-comp[b] // P)
            bt[b, :m] = perm[k:k + m]
            k += m
        btd = T.from_numpy(bt).cuda()
        kpool, kg = _guard_cache(run.kspec, n_pages * H, P)
        vpool, vg = _guard_cache(run.vspec, n_pages * H, P)
        xk = T.zeros((B * H, max(comp), 128), dtype=T.bfloat16, device="cuda")
        xv = T.zeros_like(xk)
        for b in range(B):
            xk[b * H:(b + 1) * H, :comp[b]] = to_device(run.inp.k[b], "bf16")
            xv[b * H:(b + 1) * H, :comp[b]] = to_device(run.inp.v[b], "bf16")
        tq.quantize_kv_paged(run.kspec, run.ktab, xk, kpool, hkv=H, n_tok=comp, block_table=btd, n_pages=n_pages)
        tq.quantize_kv_paged(run.vspec, run.vtab, xv, vpool, hkv=H, n_tok=comp, block_table=btd, n_pages=n_pages)
        out = Guarded(run.q.numel(), T.float32, -7.25)
        ws = Guarded(run.ws.numel(), T.float32, -7.25)
        tq.attend_decode_paged(run.kspec, run.ktab, kpool, run.vspec, run.vtab, vpool, run.q, run.seq_lens,
                               out.view.view(run.q.shape), ws.view, hkv=H, block_table=btd, n_pages=n_pages,
                               max_len=run.max_len)
        T.cuda.synchronize()
        for g in kg + vg:
            assert g.intact(), f"qjl={qjl}: a paged call wrote outside the pool"
        assert out.intact() and ws.intact()
        assert T.equal(out.view.view(run.q.shape), run.out)


def test_lengths_beyond_max_len_are_clamped():
    """seq_lens entries above max_len (or negative) break the call's contract;
    the split kernel clamps them into [0, max_len], so the reads stay inside
    the validated cache and such a sequence decodes as one of max_len tokens
    (a negative one as an empty sequence)."""
    print("[guards] seq_lens clamp", flush=True)
    T = torch()
    wl = workloads.Workload("clamp", 3, 8, 2, "bf16", workloads.QSpec(4, 4), workloads.QSpec(3, 3),
                            lens_range=(200, 200))
    run = Run(workloads.generate(wl))
    run.quantize()
    run.attend()
    T.cuda.synchronize()
    ref = run.out.clone()
    bad = T.tensor([200, 5000, -3], dtype=T.int32, device="cuda")
    out = T.empty_like(run.q)
    tq.attend_decode(run.kspec, run.ktab, run.kc, run.vspec, run.vtab, run.vc, run.q, bad, out, run.ws, hkv=2,
                     max_len=run.max_len)
    T.cuda.synchronize()
    assert T.equal(out[:2], ref[:2])
    assert T.equal(out[2], T.zeros_like(out[2]))
