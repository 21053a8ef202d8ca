"""Seeded synthetic workloads for the packed-KV quantize + decode-attention path.

This module only draws random inputs and rounds them to bf16; it holds none of
the method's arithmetic, so both the HIP path (tests, bench) and the CPU oracle
can be fed from it.

The workloads stand in for the long-context evaluations the pages quote
(LongBench / Needle-in-a-Haystack / RULER at 3.5 bits and a 128k-context
session in NVIDIA forum "Why TurboQuant saves DGX twice"); no dataset is used.
Draws use ``numpy.random.default_rng(seed)`` in the order listed per workload;
bf16 values are float32 draws rounded to nearest even.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

D = 128


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + r) >> 16).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass(frozen=True)
class QSpec:
    """Quantizer parameters of one tensor (K or V)."""
    bits_lo: int
    bits_hi: int
    split: int = D
    qjl_m: int = 0
    rot_seed: int = 0
    qjl_seed: int = 1


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    hq: int
    hkv: int
    dtype: str                 # "f32" or "bf16": storage type of K and V
    k: QSpec
    v: QSpec
    ctx: int = 0               # uniform context length (0 -> ragged, see lens_range)
    lens_range: tuple = ()     # (lo, hi) inclusive for ragged batches
    sink: int = 0
    v_skip: float = 0.0
    structure: str = "plain"   # "plain", "outlier_channels", "channel_scales"
    seed: int = 0
    notes: str = ""


WORKLOADS: dict[str, Workload] = {
    "tiny_oracle": Workload(
        "tiny_oracle", 1, 1, 1, "f32", QSpec(4, 4), QSpec(4, 4), ctx=4096,
        notes="1 head, 4096 K and 4096 V vectors fp32 N(0,1), seed 0, K4/V4, one query"),
    "gqa_decode": Workload(
        "gqa_decode", 1, 32, 8, "bf16", QSpec(4, 4), QSpec(3, 3), ctx=32768,
        structure="outlier_channels",
        notes="batch 1, 32 q heads / 8 kv heads, ctx 32768, bf16 N(0,1), 4 key channels "
              "per head x10, K4/V3"),
    "qjl": Workload(
        "qjl", 8, 32, 8, "bf16", QSpec(2, 2, qjl_m=128), QSpec(3, 3), ctx=16384,
        notes="batch 8, 8 kv heads (32 q heads), ctx 16384, bf16 N(0,1), K 2-bit + QJL m=128, V3"),
    "long_context": Workload(
        "long_context", 1, 32, 8, "bf16", QSpec(4, 3, 64), QSpec(4, 3, 64), ctx=131072,
        structure="channel_scales",
        notes="batch 1, 8 kv heads, 32 q heads, ctx 131072, bf16 N(0,1) with per-channel "
              "scales log-uniform in [0.5, 8], 3.5 bits (coords 0-63 at 4, 64-127 at 3)"),
    "batched_ragged": Workload(
        "batched_ragged", 64, 32, 8, "bf16", QSpec(4, 4), QSpec(2, 2), lens_range=(1024, 32768),
        sink=128, v_skip=1e-6,
        notes="64 sequences, lengths U[1024, 32768], 8 kv heads (32 q heads), bf16 N(0,1), "
              "K4/V2, first 128 tokens raw bf16 sink, V skipped below weight 1e-6"),
}


@dataclass
class Inputs:
    """Drawn inputs.  K/V per sequence b: arrays [Hkv, L_b, D] (float32 values,
    exactly the stored values: bf16-rounded for bf16 workloads) plus the bf16
    bit patterns when dtype is bf16.  q: [B, Hq, D] float32."""
    wl: Workload
    seq_lens: np.ndarray
    k: list = field(default_factory=list)
    v: list = field(default_factory=list)
    k_bf16: list = field(default_factory=list)
    v_bf16: list = field(default_factory=list)
    q: np.ndarray | None = None


def _finish(x: np.ndarray, dtype: str):
    if dtype == "bf16":
        b = bf16_bits(x)
        return bf16_to_f32(b), b
    return np.ascontiguousarray(x, dtype=np.float32), None


def generate(wl: Workload | str, seed: int | None = None, ctx: int | None = None,
             batch: int | None = None) -> Inputs:
    """Draw one workload.  ``ctx``/``batch`` shrink it (same recipe, smaller sizes)."""
    wl = WORKLOADS[wl] if isinstance(wl, str) else wl
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    B = wl.batch if batch is None else batch
    f32 = np.float32
    if wl.lens_range:
        lo, hi = wl.lens_range
        if ctx is not None:
            lo, hi = min(lo, ctx), ctx
        lens = rng.integers(lo, hi, B, endpoint=True).astype(np.int64)
        ks, vs = [], []
        for b in range(B):
            ks.append(rng.standard_normal((wl.hkv, int(lens[b]), D), dtype=f32))
            vs.append(rng.standard_normal((wl.hkv, int(lens[b]), D), dtype=f32))
        q = rng.standard_normal((B, wl.hq, D), dtype=f32)
    else:
        T = wl.ctx if ctx is None else ctx
        lens = np.full(B, T, dtype=np.int64)
        K = rng.standard_normal((B, wl.hkv, T, D), dtype=f32)
        V = rng.standard_normal((B, wl.hkv, T, D), dtype=f32)
        q = rng.standard_normal((B, wl.hq, D), dtype=f32)
        if wl.structure == "outlier_channels":
            for h in range(wl.hkv):
                ch = rng.choice(D, 4, replace=False)
                K[:, h, :, ch] *= f32(10.0)
        elif wl.structure == "channel_scales":
            sk = np.exp(rng.uniform(np.log(0.5), np.log(8.0), (wl.hkv, D))).astype(f32)
            sv = np.exp(rng.uniform(np.log(0.5), np.log(8.0), (wl.hkv, D))).astype(f32)
            K *= sk[None, :, None, :]
            V *= sv[None, :, None, :]
        ks = [K[b] for b in range(B)]
        vs = [V[b] for b in range(B)]
    inp = Inputs(wl=wl, seq_lens=lens, q=q)
    for kb, vb in zip(ks, vs):
        kv, kbits = _finish(kb, wl.dtype)
        vv, vbits = _finish(vb, wl.dtype)
        inp.k.append(kv)
        inp.v.append(vv)
        inp.k_bf16.append(kbits)
        inp.v_bf16.append(vbits)
    return inp


# ---- inner-product search (the method's second application)

@dataclass(frozen=True)
class SearchWorkload:
    name: str
    streams: int        # database streams (one cache stream each)
    n_tok: int          # vectors per stream
    nq: int             # queries per call
    bits: int           # code width of the database vectors
    qjl_m: int          # sketch rows (0: none)
    seed: int = 0
    notes: str = ""


SEARCH = SearchWorkload(
    "ip_search", 8, 131072, 64, 2, 128,
    notes="1 M database vectors bf16 N(0,1) in 8 streams of 131072, 2-bit codes + 128-bit sketch "
          "(3 bits per coordinate, the inner-product setting of the method), 64 fp32 N(0,1) queries")


def _search_rng(wl: SearchWorkload):
    return np.random.default_rng(wl.seed)


def search_queries(wl: SearchWorkload = SEARCH) -> np.ndarray:
    """[nq, d] float32 N(0,1) queries (the first draws of the seed)."""
    return _search_rng(wl).standard_normal((wl.nq, D), dtype=np.float32)


def search_database(wl: SearchWorkload = SEARCH) -> np.ndarray:
    """[streams, n_tok, d] float32 N(0,1) database vectors (drawn after the queries)."""
    rng = _search_rng(wl)
    rng.standard_normal((wl.nq, D), dtype=np.float32)
    return rng.standard_normal((wl.streams, wl.n_tok, D), dtype=np.float32)
