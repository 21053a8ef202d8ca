"""tq_attend_decode_noalloc (the decode step with its partials in the
library's static device scratch) against tq_attend_decode with a workspace:
the same plan and kernels, so the outputs must be identical bit for bit; and
the output held to the oracle.  Two calls in a row, the second smaller, so the
second reuses scratch contents the first left behind."""
import numpy as np
import pytest

from compressed_kv_cache_tq_amd import tq, workloads
from gpu_helpers import Run, oracle_attention, torch
from oracle import parity

pytestmark = pytest.mark.gpu


def _oracle_err(run, out):
    K, Kn, V, Vn, Z, R = run.gpu_codes()
    inp, wl = run.inp, run.wl
    sk = sv = None
    if wl.sink:
        sk = [[inp.k[b][h][: wl.sink] for h in range(wl.hkv)] for b in range(run.B)]
        sv = [[inp.v[b][h][: wl.sink] for h in range(wl.hkv)] for b in range(run.B)]
    ref = oracle_attention(inp.q, run.kspec, run.vspec, inp.seq_lens, K, Kn, V, Vn, k_bits=Z, k_gamma=R,
                           sink_k=sk, sink_v=sv, sink=wl.sink, v_skip=wl.v_skip)
    return parity.rel_l2(out.cpu().numpy(), ref)


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_equals_the_workspace_entry_point(order):
    T = torch()
    cases = [("gqa_decode", 3000, None), ("batched_ragged", 700, 3)]   # several splits + combine, then one split
    for name, ctx, batch in cases:
        print(f"[noalloc] {name} ctx={ctx} batch={batch}", flush=True)
        run = Run(workloads.generate(name, ctx=ctx, batch=batch))
        run.quantize()
        run.attend()
        T.cuda.synchronize()
        ref = run.out.clone()
        wl = run.wl
        need = tq.attend_workspace_bytes(run.B, wl.hq, wl.hkv, wl.sink, run.max_len)
        assert need <= tq.NOALLOC_SCRATCH_BYTES
        out = T.full_like(run.q, float("nan"))
        tq.attend_decode_noalloc(run.kspec, run.ktab, run.kc, run.vspec, run.vtab, run.vc, run.q, run.seq_lens, out,
                                 hkv=wl.hkv, sink=wl.sink, sink_k=run.sink_k, sink_v=run.sink_v, v_skip=wl.v_skip,
                                 max_len=run.max_len)
        T.cuda.synchronize()
        assert T.equal(out, ref), f"{name}: the no-alloc decode differs from tq_attend_decode"
        err = _oracle_err(run, out)
        print(f"[noalloc] {name}: equal to tq_attend_decode, oracle rel L2 {err:.2e}", flush=True)
        assert err <= parity.ATTN_REL_L2
