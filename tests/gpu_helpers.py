"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and bring its outputs back, and evaluate the oracle on the same codes."""
from __future__ import annotations

import numpy as np

from compressed_kv_cache_tq_amd import tq, workloads
from oracle import attend as oat
from oracle import pack as opk
from oracle import parity
from oracle import quantize as oqz


def torch():
    import torch as t
    return t


def to_device(x_f32: np.ndarray, dtype: str):
    t = torch()
    if dtype == "bf16":
        bits = workloads.bf16_bits(x_f32)
        return t.from_numpy(bits.view(np.int16)).cuda().view(t.bfloat16)
    return t.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32)).cuda()


def ospec(s: tq.Spec) -> oqz.Spec:
    return oqz.Spec(bits_lo=s.bits_lo, bits_hi=s.bits_lo if s.bits_hi is None else s.bits_hi,
                    split=s.split, qjl_m=s.qjl_m, rot_seed=s.rot_seed, qjl_seed=s.qjl_seed,
                    rotation="haar" if s.rotation == tq.ROT_HAAR else "hadamard", norm_f16=bool(s.norm_f16))


def read_codes(spec: tq.Spec, cache: tq.Cache, stream: int, n_tok: int, tok0: int = 0) -> np.ndarray:
    """Unpack the GPU codes of one stream (positions tok0 .. tok0+n_tok) with the oracle's layout reader."""
    nb = tq.cache_code_bytes(spec, cache.cap)
    raw = cache.codes[stream * nb:(stream + 1) * nb].cpu().numpy()
    if spec.layout == tq.LAYOUT_TILED:
        return opk.unpack_tiled(raw, spec.widths, n_tok, tok0)
    rb = tq.code_bytes(spec)
    rec = raw.reshape(cache.cap, rb)[tok0:tok0 + n_tok]
    return opk.unpack_records(rec, spec.widths)


def read_norms(cache: tq.Cache, stream: int, n_tok: int, tok0: int = 0) -> np.ndarray:
    return cache.norms[stream * cache.cap + tok0: stream * cache.cap + tok0 + n_tok].cpu().numpy()


def read_signs(cache: tq.Cache, stream: int, n_tok: int, tok0: int = 0):
    m8 = cache.spec.qjl_m // 8
    raw = cache.qjl_signs[(stream * cache.cap + tok0) * m8:(stream * cache.cap + tok0 + n_tok) * m8].cpu().numpy()
    bits = opk.unpack_sign_bits(raw.reshape(n_tok, m8))
    rn = cache.qjl_rnorms[stream * cache.cap + tok0: stream * cache.cap + tok0 + n_tok].cpu().numpy()
    return bits, rn


def check_quantized(spec: tq.Spec, x: np.ndarray, idx_gpu: np.ndarray, norms_gpu: np.ndarray,
                    signs=None, label: str = ""):
    """Oracle quantization of the same stored values and the parity rules."""
    os_ = ospec(spec)
    q = oqz.quantize(x.astype(np.float64), os_)
    rep = parity.compare_codes(q.idx, idx_gpu, q.y, os_)
    assert rep.ok, f"{label}: {rep}"
    # norms: fp64 accumulation on the GPU -> equal to the correctly rounded
    # norm up to 1 ulp of the stored type (fp32, or fp16 rounded from fp32)
    dt = q.norms.dtype
    assert norms_gpu.dtype == dt, f"{label}: norms stored as {norms_gpu.dtype}, expected {dt}"
    ulp = np.spacing(np.maximum(q.norms, dt.type(np.finfo(dt).tiny))).astype(np.float64)
    err = np.abs(norms_gpu.astype(np.float64) - q.norms.astype(np.float64))
    assert np.all(err <= ulp), f"{label}: norms differ"
    if signs is not None:
        bits_gpu, rn_gpu = signs
        vec_ok = np.all(q.idx == idx_gpu, axis=1)
        srep = parity.compare_signs(q.qjl_bits, bits_gpu, q.qjl_proj, vec_ok)
        assert srep.ok, f"{label} signs: {srep}"
        assert np.allclose(rn_gpu[vec_ok], q.rnorms[vec_ok], rtol=2e-6, atol=1e-7), f"{label}: residual norms"
    return rep


def oracle_attention(q: np.ndarray, kspec: tq.Spec, vspec: tq.Spec, seq_lens, k_idx, k_norm, v_idx, v_norm, *,
                     k_bits=None, k_gamma=None, sink_k=None, sink_v=None, sink=0, v_skip=0.0, heads=None):
    """The oracle's batched decode attention (oracle.attend.attend) on the given
    codes, with the sketch term when the key spec has one.

    k_idx[b][kh] etc. hold the compressed tokens (already cut to L_b - sink).
    heads: optional list of (b, h) to evaluate (others left as NaN).
    """
    return oat.attend(q, ospec(kspec), ospec(vspec), seq_lens, k_idx, k_norm, v_idx, v_norm, k_bits=k_bits,
                      k_gamma=k_gamma, sink_k=sink_k, sink_v=sink_v, sink=sink, v_skip=v_skip, heads=heads)


class Run:
    """One workload pushed through the HIP path: quantize K and V, then decode attention."""

    def __init__(self, inp: workloads.Inputs, device="cuda", norm_f16: int = 0):
        t = torch()
        wl = inp.wl
        self.inp = inp
        self.wl = wl
        self.kspec = tq.Spec(wl.k.bits_lo, wl.k.bits_hi, split=wl.k.split, qjl_m=wl.k.qjl_m,
                             layout=tq.LAYOUT_RECORD, rot_seed=wl.k.rot_seed, qjl_seed=wl.k.qjl_seed,
                             norm_f16=norm_f16)
        self.vspec = tq.Spec(wl.v.bits_lo, wl.v.bits_hi, split=wl.v.split, qjl_m=0,
                             layout=tq.LAYOUT_TILED, rot_seed=wl.v.rot_seed, norm_f16=norm_f16)
        B, Hkv, S = len(inp.k), wl.hkv, wl.sink
        self.B = B
        lens = inp.seq_lens
        self.max_len = int(lens.max())
        self.cap = max(32, -(-(self.max_len - S) // 32) * 32)
        self.ktab = tq.device_tables(self.kspec)
        self.vtab = tq.device_tables(self.vspec)
        self.kc = tq.alloc_cache(self.kspec, B * Hkv, self.cap)
        self.vc = tq.alloc_cache(self.vspec, B * Hkv, self.cap)
        self.sink_k = self.sink_v = None
        if S:
            sk = np.stack([inp.k[b][:, :S] for b in range(B)])
            sv = np.stack([inp.v[b][:, :S] for b in range(B)])
            self.sink_k = t.from_numpy(workloads.bf16_bits(sk).view(np.int16)).cuda()
            self.sink_v = t.from_numpy(workloads.bf16_bits(sv).view(np.int16)).cuda()
        self.q = t.from_numpy(np.ascontiguousarray(inp.q, dtype=np.float32)).cuda()
        self.seq_lens = t.from_numpy(lens.astype(np.int32)).cuda()
        self.out = t.empty_like(self.q)
        self.ws = tq.alloc_attend_workspace(B, wl.hq, Hkv, S, self.max_len)

    def quantize(self):
        wl, S = self.wl, self.wl.sink
        for b in range(self.B):
            L = int(self.inp.seq_lens[b])
            if L <= S:
                continue
            xk = to_device(self.inp.k[b], wl.dtype)
            xv = to_device(self.inp.v[b], wl.dtype)
            kc = self.kc.streams(b * wl.hkv, wl.hkv)
            vc = self.vc.streams(b * wl.hkv, wl.hkv)
            tq.quantize_kv(self.kspec, self.ktab, xk[:, S:L], kc)
            tq.quantize_kv(self.vspec, self.vtab, xv[:, S:L], vc)

    def attend(self):
        tq.attend_decode(self.kspec, self.ktab, self.kc, self.vspec, self.vtab, self.vc, self.q, self.seq_lens,
                         self.out, self.ws, hkv=self.wl.hkv, sink=self.wl.sink, sink_k=self.sink_k,
                         sink_v=self.sink_v, v_skip=self.wl.v_skip, max_len=self.max_len)

    def gpu_codes(self, heads=None):
        """Per (b, kh): codes, norms (+ signs, rnorms) of the compressed tokens.

        heads: optional (b, query head) pairs; only their KV streams are read."""
        wl, S = self.wl, self.wl.sink
        G = wl.hq // wl.hkv
        need = None if heads is None else {(b, h // G) for b, h in heads}
        K, Kn, V, Vn, Z, R = [], [], [], [], [], []
        for b in range(self.B):
            n = max(0, int(self.inp.seq_lens[b]) - S)
            kb, knb, vb, vnb, zb, rb = [], [], [], [], [], []
            for h in range(wl.hkv):
                if need is not None and (b, h) not in need:
                    for lst in (kb, knb, vb, vnb, zb, rb):
                        lst.append(None)
                    continue
                s = b * wl.hkv + h
                kb.append(read_codes(self.kspec, self.kc, s, n))
                knb.append(read_norms(self.kc, s, n))
                vb.append(read_codes(self.vspec, self.vc, s, n))
                vnb.append(read_norms(self.vc, s, n))
                if self.kspec.qjl_m:
                    z, r = read_signs(self.kc, s, n)
                    zb.append(z)
                    rb.append(r)
            K.append(kb); Kn.append(knb); V.append(vb); Vn.append(vnb); Z.append(zb); R.append(rb)
        return K, Kn, V, Vn, (Z if self.kspec.qjl_m else None), (R if self.kspec.qjl_m else None)
