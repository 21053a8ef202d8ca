"""Per-vector quantization: norm, rotation, scalar codes, QJL sketch (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

noze.it "TurboQuant-MLX: quantizzare pesi e KV cache...", section "Il metodo
TurboQuant, in breve":
1. rotate the vector at random;
2. quantize every rotated coordinate on its own with the optimal scalar
   quantizer for the post-rotation law;
3. (second stage) the MSE-optimal quantizer biases inner products, so a 1-bit
   quantized JL sketch of the residual is kept to make the inner-product
   estimate unbiased.
The codebook is built for a unit vector, so the norm is stored separately and
the unit vector is what gets rotated and quantized.  Same page: 3.5 and 2.5
bits per channel are quoted; the 3.5-bit mix is read as rotated coordinates
0..63 at 4 bits and 64..127 at 3 bits.

Readings (the page is silent on these):
* the norm is the float64 Euclidean norm of the stored input value, kept as
  fp32 rounded to nearest even; with fp16 norms (a storage option of this
  library that the pages do not describe; the port they discuss only brings
  the cache back to float16 for attention, noze.it page, section "Cosa
  aggiunge turboquant-mlx") that fp32 value is rounded once more, to
  binary16, nearest even, saturating at the largest finite value 65504 (a
  norm that would round to infinity is stored as 65504);
* a zero vector quantizes y = 0 and stores norm 0;
* index = number of thresholds strictly below y (exact ties go to the lower
  index);
* QJL residual r = y - yhat in the rotated unit-norm domain, gamma = ||r||
  kept as fp32, sign bit j = 1 iff (S r)_j >= 0.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .codebook import lloyd_max
from .rotation import hadamard_rotation, rotation, sketch

F16_MAX = 65504.0   # largest finite binary16 value


@dataclass(frozen=True)
class Spec:
    d: int = 128
    bits_lo: int = 4      # bits of rotated coordinates i < split
    bits_hi: int = 4      # bits of rotated coordinates i >= split
    split: int = 128      # d for a uniform width
    qjl_m: int = 0        # QJL sketch rows (0 = no QJL stage)
    rot_seed: int = 0
    qjl_seed: int = 1
    rotation: str = "haar"  # "haar" or "hadamard"
    norm_f16: bool = False  # norms stored as fp16 (rounded from the fp32 norm)

    def bits_of(self) -> np.ndarray:
        """Bit width of every rotated coordinate."""
        b = np.full(self.d, self.bits_hi, dtype=np.int64)
        b[: self.split] = self.bits_lo
        return b

    @property
    def code_bits(self) -> int:
        return int(self.bits_of().sum())


def rotation_of(spec: Spec) -> np.ndarray:
    if spec.rotation == "hadamard":
        return hadamard_rotation(spec.rot_seed, spec.d)
    if spec.rotation != "haar":
        raise ValueError(f"unknown rotation {spec.rotation!r}")
    return rotation(spec.rot_seed, spec.d)


def sketch_of(spec: Spec) -> np.ndarray:
    return sketch(spec.qjl_seed, spec.qjl_m, spec.d)


def scalar_quantize(y: np.ndarray, spec: Spec) -> np.ndarray:
    """idx[..., i] = #{j : t_j < y[..., i]} with coordinate i's codebook."""
    idx = np.empty(y.shape, dtype=np.int64)
    lo = lloyd_max(spec.d, spec.bits_lo).boundaries
    hi = lloyd_max(spec.d, spec.bits_hi).boundaries
    s = spec.split
    idx[..., :s] = np.searchsorted(lo, y[..., :s], side="left")
    idx[..., s:] = np.searchsorted(hi, y[..., s:], side="left")
    return idx


def dequantize_rotated(idx: np.ndarray, spec: Spec) -> np.ndarray:
    """yhat[..., i] = c[idx[..., i]] (rotated, unit-norm domain, float64)."""
    lo = lloyd_max(spec.d, spec.bits_lo).centroids
    hi = lloyd_max(spec.d, spec.bits_hi).centroids
    s = spec.split
    out = np.empty(idx.shape, dtype=np.float64)
    out[..., :s] = lo[idx[..., :s]]
    out[..., s:] = hi[idx[..., s:]]
    return out


@dataclass
class Quantized:
    idx: np.ndarray        # [n, d] int64 codes
    norms: np.ndarray      # [n] float32 (stored), float16 with spec.norm_f16
    norms64: np.ndarray    # [n] float64 (exact)
    y: np.ndarray          # [n, d] float64 rotated unit vectors
    qjl_bits: np.ndarray | None = None   # [n, m] bool, True iff (S r)_j >= 0
    qjl_proj: np.ndarray | None = None   # [n, m] float64, S r
    rnorms: np.ndarray | None = None     # [n] float32 gamma = ||r||


def quantize(x: np.ndarray, spec: Spec, pi: np.ndarray | None = None,
             s_mat: np.ndarray | None = None) -> Quantized:
    """Quantize rows of ``x`` ([n, d], any float dtype, read exactly as float64)."""
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2 or x.shape[1] != spec.d:
        raise ValueError("x must be [n, d]")
    pi = rotation_of(spec) if pi is None else pi
    nrm = np.sqrt(np.sum(x * x, axis=1))
    y = x @ pi.T
    nz = nrm > 0
    y[nz] /= nrm[nz, None]
    y[~nz] = 0.0
    idx = scalar_quantize(y, spec)
    stored = nrm.astype(np.float32)
    if spec.norm_f16:
        # saturate at the largest finite binary16 value rather than round to +inf
        stored = np.minimum(stored, np.float32(F16_MAX)).astype(np.float16)
    out = Quantized(idx=idx, norms=stored, norms64=nrm, y=y)
    if spec.qjl_m:
        s_mat = sketch_of(spec) if s_mat is None else s_mat
        r = y - dequantize_rotated(idx, spec)
        proj = r @ s_mat.T
        out.qjl_proj = proj
        out.qjl_bits = proj >= 0.0
        out.rnorms = np.sqrt(np.sum(r * r, axis=1)).astype(np.float32)
    return out


def qjl_inner_estimate(q_rot: np.ndarray, s_mat: np.ndarray, bits: np.ndarray,
                       gamma: np.ndarray) -> np.ndarray:
    """Estimate <q_rot, r> from the sign sketch: sqrt(pi/2)/m * gamma * <S q_rot, z>.

    z_j = +1 if the stored bit is set else -1.  For a Gaussian row s,
    E[<s, q> sign<s, r>] = sqrt(2/pi) <q, r> / ||r||, hence the constant.
    """
    m = s_mat.shape[0]
    u = s_mat @ q_rot
    z = np.where(bits, 1.0, -1.0)
    return np.sqrt(np.pi / 2.0) / m * np.asarray(gamma, dtype=np.float64) * (z @ u)
