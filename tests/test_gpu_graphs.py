"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph on the
capture stream) and replayed: every replay must give what the eager call
gives, bit for bit.  The library issues only kernel launches (no memsets,
copies or allocations), so its calls are capturable; the replays are
separated by eager work that overwrites the outputs first, so a replay that
did not run, or ran on stale arguments, shows."""
import numpy as np
import pytest

from compressed_kv_cache_tq_amd import tq, workloads
from gpu_helpers import Run, torch

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _capture(fn):
    """A graph holding fn(), after one warm-up call on a side stream."""
    T = torch()
    side = T.cuda.Stream()
    side.wait_stream(T.cuda.current_stream())
    with T.cuda.stream(side):
        fn()
    T.cuda.current_stream().wait_stream(side)
    T.cuda.synchronize()
    g = T.cuda.CUDAGraph()
    with T.cuda.graph(g):
        fn()
    T.cuda.synchronize()
    return g


@pytest.mark.parametrize("name,ctx,batch", [("gqa_decode", 3000, None), ("batched_ragged", 700, 5)])
def test_decode_replays_in_a_graph(name, ctx, batch):
    """One decode step (several splits and the combine for gqa_decode; one
    split per stream, merged in place, with sink tokens and V-skip for the
    ragged batch), through both the workspace and the allocation-free entry
    points."""
    T = torch()
    print(f"[graph] decode {name} ctx={ctx} batch={batch}", flush=True)
    run = Run(workloads.generate(name, ctx=ctx, batch=batch))
    run.quantize()
    run.attend()
    T.cuda.synchronize()
    ref = run.out.clone()
    wl = run.wl
    out2 = T.empty_like(run.q)

    def noalloc():
        tq.attend_decode_noalloc(run.kspec, run.ktab, run.kc, run.vspec, run.vtab, run.vc, run.q, run.seq_lens, out2,
                                 hkv=wl.hkv, sink=wl.sink, sink_k=run.sink_k, sink_v=run.sink_v, v_skip=wl.v_skip,
                                 max_len=run.max_len)

    for label, fn, out in (("workspace", run.attend, run.out), ("noalloc", noalloc, out2)):
        g = _capture(fn)
        for r in range(REPLAYS):
            out.fill_(float("nan"))
            run.ws.fill_(float("nan"))  # the call keeps no state in its workspace
            T.cuda.synchronize()
            g.replay()
            T.cuda.synchronize()
            assert T.equal(out, ref), f"{name}/{label}: replay {r} differs from the eager call"
        print(f"[graph] {name}/{label}: {REPLAYS} replays equal the eager call", flush=True)


def test_quantize_replays_in_a_graph():
    """A ragged quantize of keys (records) and values (tiles, including the
    launch that merges partly written tiles) captured once and replayed into
    a cache overwritten with junk before each replay."""
    T = torch()
    print("[graph] ragged quantize", flush=True)
    rng = np.random.default_rng(61)
    hkv, lens, tok0s = 2, [70, 0, 33, 100], [0, 5, 40, 3]
    B, rows = len(lens), max(lens)
    x = workloads.bf16_to_f32(workloads.bf16_bits(rng.standard_normal((B * hkv, rows, 128), dtype=np.float32)))
    xd = T.from_numpy(workloads.bf16_bits(x).view(np.int16)).cuda().view(T.bfloat16)
    for spec in (tq.Spec(4), tq.Spec(3, layout=tq.LAYOUT_TILED), tq.Spec(2, qjl_m=128)):
        what = f"{spec.bits_lo}-bit layout={spec.layout} qjl={spec.qjl_m}"
        tab = tq.device_tables(spec)
        ref = tq.alloc_cache(spec, B * hkv, 160, fill=0x5A)
        tq.quantize_kv_ragged(spec, tab, xd, ref, hkv=hkv, n_tok=lens, tok0=tok0s)
        T.cuda.synchronize()
        cache = tq.alloc_cache(spec, B * hkv, 160, fill=0x5A)
        g = _capture(lambda: tq.quantize_kv_ragged(spec, tab, xd, cache, hkv=hkv, n_tok=lens, tok0=tok0s))
        for r in range(REPLAYS):
            # back to the pre-call contents: the tiled layout keeps the codes
            # of positions the call does not write
            cache.codes.fill_(0x5A)
            cache.norms.zero_()
            if cache.qjl_signs is not None:
                cache.qjl_signs.zero_()
                cache.qjl_rnorms.zero_()
            T.cuda.synchronize()
            g.replay()
            T.cuda.synchronize()
            assert T.equal(cache.codes, ref.codes), f"{what}: replay {r}: codes differ"
            assert T.equal(cache.norms, ref.norms), f"{what}: replay {r}: norms differ"
            if cache.qjl_signs is not None:
                assert T.equal(cache.qjl_signs, ref.qjl_signs), f"{what}: replay {r}: signs differ"
                assert T.equal(cache.qjl_rnorms, ref.qjl_rnorms), f"{what}: replay {r}: residual norms differ"
        print(f"[graph] quantize {what}: {REPLAYS} replays equal the eager call", flush=True)
