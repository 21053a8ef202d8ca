"""Thin ctypes binding of libtq.so (include/tq.h).

Argument marshalling only: every step of quantization and decode attention
runs in the library's HIP kernels; PyTorch provides device memory and the
current stream.  The functions keep the C names without the ``tq_`` prefix.
Loading fails loudly when libtq.so has not been built.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtq.so")

D = 128
TILE = 32
QJL_M = 128
F32, BF16 = 0, 1
LAYOUT_RECORD, LAYOUT_TILED = 0, 1
ROT_HAAR, ROT_HADAMARD, ROT_HADAMARD_FWHT = 0, 1, 2
STATUS = {0: "TQ_OK", -1: "TQ_E_ARG", -2: "TQ_E_UNSUPPORTED", -3: "TQ_E_WORKSPACE", -4: "TQ_E_HIP"}

EXPORTS = [
    "tq_format_version", "tq_last_error", "tq_codebook_build", "tq_rotation_build",
    "tq_hadamard_rotation_build", "tq_sketch_build",
    "tq_tables_bytes", "tq_tables_build", "tq_code_bytes", "tq_cache_code_bytes", "tq_quantize_kv",
    "tq_quantize_kv_ragged",
    "tq_attend_workspace_bytes", "tq_attend_decode", "tq_ip_workspace_bytes", "tq_ip_scores",
    "tq_quantize_kv_paged", "tq_attend_decode_paged", "tq_attend_decode_noalloc",
]
NOALLOC_SCRATCH_BYTES = 8 << 20
IP_MAX_QUERIES = 64
PAGE_TOKENS = 64


class TqSpec(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("bits_lo", ctypes.c_int32), ("bits_hi", ctypes.c_int32),
                ("split", ctypes.c_int32), ("qjl_m", ctypes.c_int32), ("layout", ctypes.c_int32),
                ("rot_seed", ctypes.c_uint64), ("qjl_seed", ctypes.c_uint64), ("rotation", ctypes.c_int32),
                ("norm_f16", ctypes.c_int32)]


class TqCache(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("norms", ctypes.c_void_p), ("qjl_signs", ctypes.c_void_p),
                ("qjl_rnorms", ctypes.c_void_p), ("cap", ctypes.c_int64)]


class TqAttn(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32),
                ("sink", ctypes.c_int32), ("scale", ctypes.c_float), ("v_skip", ctypes.c_float),
                ("max_len", ctypes.c_int64)]


class TqError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: {STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libtq.so (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m compressed_kv_cache_tq_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, U64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_size_t
    sig = {
        "tq_format_version": (I32, []),
        "tq_last_error": (ctypes.c_char_p, []),
        "tq_codebook_build": (I32, [I32, I32, P, P]),
        "tq_rotation_build": (I32, [I32, U64, P]),
        "tq_hadamard_rotation_build": (I32, [I32, U64, P]),
        "tq_sketch_build": (I32, [I32, I32, U64, P]),
        "tq_tables_bytes": (SZ, []),
        "tq_tables_build": (I32, [ctypes.POINTER(TqSpec), P, SZ]),
        "tq_code_bytes": (SZ, [ctypes.POINTER(TqSpec)]),
        "tq_cache_code_bytes": (SZ, [ctypes.POINTER(TqSpec), I64]),
        "tq_quantize_kv": (I32, [ctypes.POINTER(TqSpec), P, I32, P, I64, I64, I64, I64, I64,
                                 ctypes.POINTER(TqCache), P]),
        "tq_quantize_kv_ragged": (I32, [ctypes.POINTER(TqSpec), P, I32, P, I32, I32, P, P, P, I64, I64,
                                        ctypes.POINTER(TqCache), P]),
        "tq_attend_workspace_bytes": (SZ, [ctypes.POINTER(TqAttn)]),
        "tq_quantize_kv_paged": (I32, [ctypes.POINTER(TqSpec), P, I32, P, I32, I32, P, P, P, I64, I64, P, I32, I64,
                                       ctypes.POINTER(TqCache), P]),
        "tq_attend_decode_paged": (I32, [ctypes.POINTER(TqSpec), P, ctypes.POINTER(TqCache), ctypes.POINTER(TqSpec), P,
                                         ctypes.POINTER(TqCache), ctypes.POINTER(TqAttn), P, P, P, P, P, I32, I64, P,
                                         P, SZ, P]),
        "tq_ip_workspace_bytes": (SZ, []),
        "tq_ip_scores": (I32, [ctypes.POINTER(TqSpec), P, ctypes.POINTER(TqCache), I64, I64, P, I32, P, I64, P, SZ,
                               P]),
        "tq_attend_decode": (I32, [ctypes.POINTER(TqSpec), P, ctypes.POINTER(TqCache), ctypes.POINTER(TqSpec), P,
                                   ctypes.POINTER(TqCache), ctypes.POINTER(TqAttn), P, P, P, P, P, P, SZ, P]),
        "tq_attend_decode_noalloc": (I32, [ctypes.POINTER(TqSpec), P, ctypes.POINTER(TqCache),
                                           ctypes.POINTER(TqSpec), P, ctypes.POINTER(TqCache),
                                           ctypes.POINTER(TqAttn), P, P, P, P, P, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype, f.argtypes = res, args
    _lib = L
    return L


def _check(st: int, where: str) -> None:
    if st != 0:
        raise TqError(st, where, lib().tq_last_error().decode())


def last_error() -> str:
    return lib().tq_last_error().decode()


def format_version() -> int:
    return lib().tq_format_version()


@dataclass(frozen=True)
class Spec:
    """Quantizer of one tensor (mirrors tq_spec)."""
    bits_lo: int
    bits_hi: int | None = None
    split: int = D
    qjl_m: int = 0
    layout: int = LAYOUT_RECORD
    rot_seed: int = 0
    qjl_seed: int = 1
    rotation: int = 0      # ROT_HAAR or ROT_HADAMARD
    norm_f16: int = 0      # 1: norms stored as fp16

    def c(self) -> TqSpec:
        return TqSpec(D, self.bits_lo, self.bits_lo if self.bits_hi is None else self.bits_hi, self.split,
                      self.qjl_m, self.layout, self.rot_seed, self.qjl_seed, self.rotation, self.norm_f16)

    @property
    def widths(self) -> np.ndarray:
        w = np.full(D, self.bits_lo if self.split == D or self.bits_hi is None else self.bits_hi, dtype=np.int64)
        w[: self.split] = self.bits_lo
        return w


# ---- host-only builders ------------------------------------------------------

def codebook_build(d: int, bits: int):
    c = np.zeros(1 << bits)
    t = np.zeros((1 << bits) - 1)
    _check(lib().tq_codebook_build(d, bits, c.ctypes.data, t.ctypes.data), "tq_codebook_build")
    return c, t


def rotation_build(d: int, seed: int) -> np.ndarray:
    m = np.zeros((d, d))
    _check(lib().tq_rotation_build(d, seed, m.ctypes.data), "tq_rotation_build")
    return m


def hadamard_rotation_build(d: int, seed: int) -> np.ndarray:
    m = np.zeros((d, d))
    _check(lib().tq_hadamard_rotation_build(d, seed, m.ctypes.data), "tq_hadamard_rotation_build")
    return m


def sketch_build(m: int, d: int, seed: int) -> np.ndarray:
    s = np.zeros((m, d))
    _check(lib().tq_sketch_build(m, d, seed, s.ctypes.data), "tq_sketch_build")
    return s


def tables_bytes() -> int:
    return int(lib().tq_tables_bytes())


def tables_build(spec: Spec) -> np.ndarray:
    """Host tables (uint8) for ``spec``."""
    n = tables_bytes()
    raw = np.zeros(n + 256, dtype=np.uint8)
    off = (-raw.ctypes.data) % 256
    buf = raw[off: off + n]
    cs = spec.c()
    _check(lib().tq_tables_build(ctypes.byref(cs), buf.ctypes.data, n), "tq_tables_build")
    return buf.copy()


def code_bytes(spec: Spec) -> int:
    cs = spec.c()
    return int(lib().tq_code_bytes(ctypes.byref(cs)))


def cache_code_bytes(spec: Spec, cap: int) -> int:
    cs = spec.c()
    return int(lib().tq_cache_code_bytes(ctypes.byref(cs), cap))


def attend_workspace_bytes(batch: int, hq: int, hkv: int, sink: int, max_len: int) -> int:
    a = TqAttn(batch, hq, hkv, sink, 0.0, 0.0, max_len)
    return int(lib().tq_attend_workspace_bytes(ctypes.byref(a)))


# ---- device-side wrappers (torch for memory and stream) ----------------------

def _torch():
    import torch
    return torch


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device=None) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def device_tables(spec: Spec, device="cuda"):
    """Device copy of the tables (256-byte aligned torch uint8 tensor)."""
    torch = _torch()
    host = torch.from_numpy(tables_build(spec))
    dev = torch.empty(host.numel() + 256, dtype=torch.uint8, device=device)
    off = (-dev.data_ptr()) % 256
    view = dev[off: off + host.numel()]
    view.copy_(host)
    return view


@dataclass
class Cache:
    """Packed cache of one tensor for n_streams streams of cap positions (torch tensors)."""
    spec: Spec
    cap: int
    codes: object
    norms: object
    qjl_signs: object = None
    qjl_rnorms: object = None

    def c(self) -> TqCache:
        return TqCache(_ptr(self.codes), _ptr(self.norms), _ptr(self.qjl_signs), _ptr(self.qjl_rnorms), self.cap)

    def streams(self, start: int, count: int) -> "Cache":
        """View of streams [start, start + count)."""
        nb = cache_code_bytes(self.spec, self.cap)
        cut = lambda t, per: None if t is None else t[start * per: (start + count) * per]
        m8 = self.spec.qjl_m // 8
        return Cache(self.spec, self.cap, cut(self.codes, nb), cut(self.norms, self.cap),
                     cut(self.qjl_signs, self.cap * m8), cut(self.qjl_rnorms, self.cap))


def alloc_cache(spec: Spec, n_streams: int, cap: int, device="cuda", fill: int | None = None) -> Cache:
    torch = _torch()
    if spec.layout == LAYOUT_TILED:
        cap = -(-cap // TILE) * TILE
    nb = cache_code_bytes(spec, cap)
    codes = torch.empty(max(n_streams * nb, 16), dtype=torch.uint8, device=device)
    if fill is not None:
        codes.fill_(fill)
    norms = torch.zeros(max(n_streams * cap, 8), dtype=torch.float16 if spec.norm_f16 else torch.float32,
                        device=device)
    signs = rn = None
    if spec.qjl_m:
        signs = torch.zeros(max(n_streams * cap * spec.qjl_m // 8, 16), dtype=torch.uint8, device=device)
        rn = torch.zeros(max(n_streams * cap, 4), dtype=torch.float32, device=device)
    return Cache(spec, cap, codes, norms, signs, rn)


def _layout_key(s: Spec):
    """The fields of a spec that fix the sizes and layout of a cache's arrays."""
    hi = s.bits_lo if s.bits_hi is None or s.split == D else s.bits_hi
    return (s.bits_lo, hi, D if hi == s.bits_lo else s.split, s.qjl_m, s.layout, int(bool(s.norm_f16)))


def _check_cache(spec: Spec, cache: Cache, n_streams: int, what: str) -> None:
    """Refuse a cache whose arrays were sized for another spec, or that holds
    fewer than n_streams streams: the C side receives bare pointers and would
    read or write past them."""
    torch = _torch()
    if _layout_key(spec) != _layout_key(cache.spec):
        raise ValueError(f"{what}: spec {spec} does not match the cache's spec {cache.spec}")
    want = torch.float16 if spec.norm_f16 else torch.float32
    if cache.norms.dtype != want:
        raise ValueError(f"{what}: norm_f16={spec.norm_f16} needs {want} norms, the cache holds {cache.norms.dtype}")
    n = max(int(n_streams), 0)
    need = [("codes", cache.codes, n * cache_code_bytes(spec, cache.cap)), ("norms", cache.norms, n * cache.cap)]
    if spec.qjl_m:
        if cache.qjl_signs is None or cache.qjl_rnorms is None:
            raise ValueError(f"{what}: the spec has a sketch, the cache has no sketch arrays")
        need += [("qjl_signs", cache.qjl_signs, n * cache.cap * spec.qjl_m // 8),
                 ("qjl_rnorms", cache.qjl_rnorms, n * cache.cap)]
    for name, t, elems in need:
        if not t.is_contiguous() or t.numel() < elems:
            raise ValueError(f"{what}: cache.{name} holds {t.numel()} elements, {n} streams need {elems}")


def quantize_kv(spec: Spec, tables, x, cache: Cache, tok0: int = 0, n_streams: int | None = None,
                n_tok: int | None = None, stream: int | None = None) -> None:
    """Quantize x ([n_streams, n_tok, d] view, float32 or bfloat16, rows 16-byte aligned)."""
    torch = _torch()
    if x.dtype == torch.float32:
        dt = F32
    elif x.dtype == torch.bfloat16:
        dt = BF16
    else:
        raise TypeError("x must be float32 or bfloat16")
    if x.dim() == 2:
        x = x.unsqueeze(0)
    if x.dim() != 3 or x.shape[-1] != D or x.stride(-1) != 1:
        raise ValueError("x must be [n_streams, n_tok, 128] with contiguous rows")
    ns = x.shape[0] if n_streams is None else n_streams
    nt = x.shape[1] if n_tok is None else n_tok
    _check_cache(spec, cache, ns, "quantize_kv")
    cs, cc = spec.c(), cache.c()
    st = _stream(x.device) if stream is None else stream
    _check(lib().tq_quantize_kv(ctypes.byref(cs), tables.data_ptr(), dt, x.data_ptr(), ns, nt, x.stride(0),
                                x.stride(1), tok0, ctypes.byref(cc), st), "tq_quantize_kv")


def quantize_kv_ragged(spec: Spec, tables, x, cache: Cache, *, hkv: int, n_tok, tok0=None, x_off=None,
                       x_stream_stride: int | None = None, x_row_stride: int | None = None,
                       stream: int | None = None) -> None:
    """Quantize a ragged batch in one call: sequence b appends n_tok[b] vectors
    to cache streams b*hkv .. b*hkv+hkv-1 at positions tok0[b] (default 0) on.

    Without x_off, x is a padded [batch*hkv, rows, d] tensor (stream b*hkv + h
    of sequence b, strides taken from it).  With x_off (elements, one per
    sequence) the strides must be given and x only supplies the base pointer,
    e.g. a packed [tokens, hkv, d] tensor with x_off[b] = start_b * hkv * d."""
    torch = _torch()
    if x.dtype == torch.float32:
        dt = F32
    elif x.dtype == torch.bfloat16:
        dt = BF16
    else:
        raise TypeError("x must be float32 or bfloat16")
    n = np.ascontiguousarray(n_tok, dtype=np.int64)
    B = n.shape[0]
    t0 = np.zeros(B, np.int64) if tok0 is None else np.ascontiguousarray(tok0, dtype=np.int64)
    if x_off is None:
        if x.dim() != 3 or x.shape[-1] != D or x.stride(-1) != 1 or x.shape[0] < B * hkv:
            raise ValueError("x must be [batch*hkv, rows, 128] with contiguous rows")
        xo = np.arange(B, dtype=np.int64) * hkv * x.stride(0)
        xss, xrs = x.stride(0), x.stride(1)
    else:
        if x_stream_stride is None or x_row_stride is None:
            raise ValueError("x_off needs x_stream_stride and x_row_stride")
        xo = np.ascontiguousarray(x_off, dtype=np.int64)
        xss, xrs = x_stream_stride, x_row_stride
    if t0.shape != (B,) or xo.shape != (B,):
        raise ValueError("n_tok, tok0 and x_off must have one entry per sequence")
    _check_cache(spec, cache, B * hkv, "quantize_kv_ragged")
    cs, cc = spec.c(), cache.c()
    st = _stream(x.device) if stream is None else stream
    _check(lib().tq_quantize_kv_ragged(ctypes.byref(cs), tables.data_ptr(), dt, x.data_ptr(), B, hkv,
                                       xo.ctypes.data, t0.ctypes.data, n.ctypes.data, xss, xrs,
                                       ctypes.byref(cc), st), "tq_quantize_kv_ragged")


def clone_cache(c: "Cache") -> "Cache":
    """Device copy of a cache (same spec and capacity)."""
    return Cache(c.spec, c.cap, c.codes.clone(), c.norms.clone(),
                 None if c.qjl_signs is None else c.qjl_signs.clone(),
                 None if c.qjl_rnorms is None else c.qjl_rnorms.clone())


def alloc_attend_workspace(batch: int, hq: int, hkv: int, sink: int, max_len: int, device="cuda"):
    """Attention workspace for tq_attend_decode (zero-filled; the call keeps no
    state in it)."""
    torch = _torch()
    n = attend_workspace_bytes(batch, hq, hkv, sink, max_len)
    return torch.zeros((n + 15) // 16 * 4, dtype=torch.float32, device=device)


def attend_decode(kspec: Spec, ktables, kcache: Cache, vspec: Spec, vtables, vcache: Cache, q, seq_lens, out,
                  workspace, *, hkv: int, sink: int = 0, sink_k=None, sink_v=None, scale: float | None = None,
                  v_skip: float = 0.0, max_len: int | None = None, stream: int | None = None) -> None:
    """One decode step: q [B, Hq, d] fp32, seq_lens int32 [B] (device), out [B, Hq, d] fp32."""
    B, Hq, _ = q.shape
    if max_len is None:
        max_len = sink + min(kcache.cap, vcache.cap)
    a = TqAttn(B, Hq, hkv, sink, (1.0 / np.sqrt(D)) if scale is None else scale, v_skip, max_len)
    _check_cache(kspec, kcache, B * hkv, "attend_decode keys")
    _check_cache(vspec, vcache, B * hkv, "attend_decode values")
    ks, vs, kc, vc = kspec.c(), vspec.c(), kcache.c(), vcache.c()
    st = _stream(q.device) if stream is None else stream
    _check(lib().tq_attend_decode(ctypes.byref(ks), ktables.data_ptr(), ctypes.byref(kc), ctypes.byref(vs),
                                  vtables.data_ptr(), ctypes.byref(vc), ctypes.byref(a), q.data_ptr(),
                                  _ptr(sink_k), _ptr(sink_v), seq_lens.data_ptr(), out.data_ptr(),
                                  workspace.data_ptr(), workspace.numel() * workspace.element_size(), st),
           "tq_attend_decode")


def attend_decode_noalloc(kspec: Spec, ktables, kcache: Cache, vspec: Spec, vtables, vcache: Cache, q, seq_lens,
                          out, *, hkv: int, sink: int = 0, sink_k=None, sink_v=None, scale: float | None = None,
                          v_skip: float = 0.0, max_len: int | None = None, stream: int | None = None) -> None:
    """attend_decode without a workspace: the partials go to the library's
    static device scratch (calls that overlap on one GPU race)."""
    B, Hq, _ = q.shape
    if max_len is None:
        max_len = sink + min(kcache.cap, vcache.cap)
    a = TqAttn(B, Hq, hkv, sink, (1.0 / np.sqrt(D)) if scale is None else scale, v_skip, max_len)
    _check_cache(kspec, kcache, B * hkv, "attend_decode_noalloc keys")
    _check_cache(vspec, vcache, B * hkv, "attend_decode_noalloc values")
    ks, vs, kc, vc = kspec.c(), vspec.c(), kcache.c(), vcache.c()
    st = _stream(q.device) if stream is None else stream
    _check(lib().tq_attend_decode_noalloc(ctypes.byref(ks), ktables.data_ptr(), ctypes.byref(kc), ctypes.byref(vs),
                                          vtables.data_ptr(), ctypes.byref(vc), ctypes.byref(a), q.data_ptr(),
                                          _ptr(sink_k), _ptr(sink_v), seq_lens.data_ptr(), out.data_ptr(), st),
           "tq_attend_decode_noalloc")


def alloc_ip_workspace(device="cuda"):
    """Workspace of ip_scores (query rows; no state is kept in it)."""
    torch = _torch()
    n = int(lib().tq_ip_workspace_bytes())
    return torch.empty((n + 15) // 16 * 4, dtype=torch.float32, device=device)


def ip_scores(spec: Spec, tables, db: Cache, q, *, n_streams: int, n_tok: int, scores=None, ld: int | None = None,
              workspace=None, stream: int | None = None):
    """Inner-product estimates of q [nq, d] (fp32, nq <= 64) against positions
    [0, n_tok) of db's first n_streams streams: scores [nq, ld], column
    s * n_tok + t for stream s, position t."""
    torch = _torch()
    nq = q.shape[0]
    ld = n_streams * n_tok if ld is None else ld
    if scores is None:
        scores = torch.empty((nq, ld), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = alloc_ip_workspace(q.device)
    _check_cache(spec, db, n_streams, "ip_scores")
    cs, cc = spec.c(), db.c()
    st = _stream(q.device) if stream is None else stream
    _check(lib().tq_ip_scores(ctypes.byref(cs), tables.data_ptr(), ctypes.byref(cc), n_streams, n_tok, q.data_ptr(),
                              nq, scores.data_ptr(), ld, workspace.data_ptr(),
                              workspace.numel() * workspace.element_size(), st), "tq_ip_scores")
    return scores


def alloc_page_pool(spec: Spec, n_pages: int, hkv: int, device="cuda") -> Cache:
    """A pool of n_pages pages of PAGE_TOKENS positions for hkv kv heads
    (stream page * hkv + h)."""
    return alloc_cache(spec, n_pages * hkv, PAGE_TOKENS, device=device)


def _dtype_code(x):
    torch = _torch()
    if x.dtype == torch.float32:
        return F32
    if x.dtype == torch.bfloat16:
        return BF16
    raise TypeError("x must be float32 or bfloat16")


def quantize_kv_paged(spec: Spec, tables, x, pool: Cache, *, hkv: int, n_tok, block_table, n_pages: int, pos0=None,
                      x_off=None, x_stream_stride: int | None = None, x_row_stride: int | None = None,
                      stream: int | None = None) -> None:
    """Append sequence b's n_tok[b] vectors at compressed positions pos0[b]..
    of a paged pool; block_table is a device int32 tensor [batch, max_pages]
    (tokens whose page lies outside [0, n_pages) are not written).  x as for
    quantize_kv_ragged."""
    n = np.ascontiguousarray(n_tok, dtype=np.int64)
    B = n.shape[0]
    p0 = np.zeros(B, np.int64) if pos0 is None else np.ascontiguousarray(pos0, dtype=np.int64)
    torch = _torch()
    if (not isinstance(block_table, torch.Tensor) or block_table.dtype != torch.int32 or block_table.dim() != 2
            or block_table.shape[0] != B or not block_table.is_contiguous()):
        raise ValueError("block_table must be a contiguous int32 tensor [batch, max_pages]")
    if x_off is None:
        if x.dim() != 3 or x.shape[-1] != D or x.stride(-1) != 1 or x.shape[0] < B * hkv:
            raise ValueError("x must be [batch*hkv, rows, 128] with contiguous rows")
        xo = np.arange(B, dtype=np.int64) * hkv * x.stride(0)
        xss, xrs = x.stride(0), x.stride(1)
    else:
        xo = np.ascontiguousarray(x_off, dtype=np.int64)
        xss, xrs = x_stream_stride, x_row_stride
    _check_cache(spec, pool, n_pages * hkv, "quantize_kv_paged")
    cs, cc = spec.c(), pool.c()
    st = _stream(x.device) if stream is None else stream
    _check(lib().tq_quantize_kv_paged(ctypes.byref(cs), tables.data_ptr(), _dtype_code(x), x.data_ptr(), B, hkv,
                                      xo.ctypes.data, p0.ctypes.data, n.ctypes.data, xss, xrs,
                                      block_table.data_ptr(), block_table.shape[1], n_pages, ctypes.byref(cc), st),
           "tq_quantize_kv_paged")


def attend_decode_paged(kspec: Spec, ktables, kpool: Cache, vspec: Spec, vtables, vpool: Cache, q, seq_lens, out,
                        workspace, *, hkv: int, block_table, n_pages: int, sink: int = 0, sink_k=None, sink_v=None,
                        scale: float | None = None, v_skip: float = 0.0, max_len: int, stream: int | None = None):
    """attend_decode over paged pools; block_table: device int32 [B, max_pages]."""
    B, Hq, _ = q.shape
    a = TqAttn(B, Hq, hkv, sink, (1.0 / np.sqrt(D)) if scale is None else scale, v_skip, max_len)
    _check_cache(kspec, kpool, n_pages * hkv, "attend_decode_paged keys")
    _check_cache(vspec, vpool, n_pages * hkv, "attend_decode_paged values")
    ks, vs, kc, vc = kspec.c(), vspec.c(), kpool.c(), vpool.c()
    st = _stream(q.device) if stream is None else stream
    _check(lib().tq_attend_decode_paged(ctypes.byref(ks), ktables.data_ptr(), ctypes.byref(kc), ctypes.byref(vs),
                                        vtables.data_ptr(), ctypes.byref(vc), ctypes.byref(a), q.data_ptr(),
                                        _ptr(sink_k), _ptr(sink_v), seq_lens.data_ptr(), block_table.data_ptr(),
                                        block_table.shape[1], n_pages, out.data_ptr(), workspace.data_ptr(),
                                        workspace.numel() * workspace.element_size(), st), "tq_attend_decode_paged")
