"""Single-query decode attention over the packed cache (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What is computed, per sequence b and query head h (KV head kh = h // G with
G = Hq / Hkv, contiguous groups):

* the query is rotated once: qr = Pi q (all dequantized keys live in the
  rotated domain, and Pi is orthogonal, so <q, Pi^T khat> = <qr, khat>);
* compressed token t (cache row t - sink) has score
      s_t = scale * n_t * ( <qr, c[idx_t]> + QJL_t ),
      QJL_t = sqrt(pi/2)/m * gamma_t * <S qr, z_t>   (only with a QJL stage)
  (noze.it "TurboQuant-MLX: ...", section "Il metodo TurboQuant, in breve":
  codebook scores plus the 1-bit sketch correction that makes the inner
  product estimate unbiased; the estimate of <qr, r_t> for the residual r_t
  of the unit vector, so it is scaled by the norm n_t like the codebook part);
* sink tokens t < sink are kept raw and scored s_t = scale * <q, k_t>
  (GitHub issue "Greetings from TurboQuant-MLX...", item 1: the first ~128
  tokens stay uncompressed);
* w = softmax(s) over all tokens of the sequence (sink and compressed jointly);
* out = Pi^T sum_{t compressed, w_t >= eps} w_t n^V_t c_V[idx^V_t]
        + sum_{t sink} w_t v_t,
  where tokens below the threshold eps are dropped without renormalising
  (same issue, item 3: V dequantization is skipped for attention weight
  below 1e-6; eps = 0 disables the rule).

Readings: scale = 1/sqrt(d); q and out are float; the weight compared with eps
is the final normalised softmax weight.
"""
from __future__ import annotations

import numpy as np

from .quantize import Spec, dequantize_rotated, qjl_inner_estimate, rotation_of, sketch_of


def compressed_scores(qr: np.ndarray, khat: np.ndarray, k_norm: np.ndarray,
                      qjl_dots: np.ndarray | None, scale: float) -> np.ndarray:
    """s_t = scale * n_t * (<qr, khat_t> + qjl_t) for the compressed tokens.

    khat [T, d] rotated unit-norm keys (centroids), qjl_dots [T] the sketch's
    estimate of <qr, r_t> (or None).  Both parts estimate inner products with
    the unit vector, so the norm multiplies their sum.
    """
    dots = khat @ qr
    if qjl_dots is not None:
        dots = dots + qjl_dots
    return scale * np.asarray(k_norm, np.float64) * dots


def attend_rotated(q: np.ndarray, qr: np.ndarray, khat: np.ndarray, k_norm: np.ndarray,
                   vhat: np.ndarray, v_norm: np.ndarray, pi_v: np.ndarray, *,
                   qjl_dots: np.ndarray | None = None, sink_k: np.ndarray | None = None,
                   sink_v: np.ndarray | None = None, scale: float, v_skip: float = 0.0):
    """Softmax attention with keys/values given as unit vectors in the rotated domain.

    khat/vhat [T, d] rotated unit-norm vectors (centroids for the cache, or the
    exact rotated vectors in the identity tests); qjl_dots [T] the optional
    sketch correction already in inner-product units.  Returns
    (out, w, keep, s): s holds the scores, sink tokens first.
    """
    s_comp = compressed_scores(qr, khat, k_norm, qjl_dots, scale)
    n_sink = 0 if sink_k is None else sink_k.shape[0]
    s_sink = scale * (np.asarray(sink_k, np.float64) @ q) if n_sink else np.zeros(0)
    s = np.concatenate((s_sink, s_comp))
    if s.size == 0:
        # a sequence with no tokens attends to nothing: the output is zero
        return np.zeros(pi_v.shape[1]), s, np.zeros(0, dtype=bool), s
    w = np.exp(s - s.max())
    w /= w.sum()
    w_sink, w_comp = w[:n_sink], w[n_sink:]
    keep = w_comp >= v_skip if v_skip > 0 else np.ones(w_comp.shape, dtype=bool)
    acc_rot = (w_comp[keep] * np.asarray(v_norm, np.float64)[keep]) @ vhat[keep]
    out = pi_v.T @ acc_rot
    if n_sink:
        out = out + w_sink @ np.asarray(sink_v, np.float64)
    return out, w, keep, s


def attend_group(qs: np.ndarray, kspec: Spec, k_idx: np.ndarray, k_norm: np.ndarray,
                 vspec: Spec, v_idx: np.ndarray, v_norm: np.ndarray, *,
                 k_bits: np.ndarray | None = None, k_gamma: np.ndarray | None = None,
                 sink_k: np.ndarray | None = None, sink_v: np.ndarray | None = None,
                 scale: float | None = None, v_skip: float = 0.0,
                 pi_k: np.ndarray | None = None, pi_v: np.ndarray | None = None,
                 s_mat: np.ndarray | None = None, return_details: bool = False):
    """Attention outputs of the query heads qs [G, d] that read one KV stream.

    k_idx/v_idx [T, d] codes of the stream's compressed tokens, norms [T];
    k_bits [T, m] bool and k_gamma [T] for a key spec with the QJL stage;
    sink_k/sink_v [S, d] raw.  The stream is dequantized once for the group.
    Returns out [G, d] (float64), and with return_details the per-head lists
    of (w, keep, s) as well.
    """
    d = kspec.d
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    qs = np.atleast_2d(np.asarray(qs, dtype=np.float64))
    pi_k = rotation_of(kspec) if pi_k is None else pi_k
    pi_v = rotation_of(vspec) if pi_v is None else pi_v
    khat = dequantize_rotated(np.asarray(k_idx), kspec)
    vhat = dequantize_rotated(np.asarray(v_idx), vspec)
    if kspec.qjl_m:
        s_mat = sketch_of(kspec) if s_mat is None else s_mat
    outs, details = [], []
    for q in qs:
        qr = pi_k @ q
        qjl = None
        if kspec.qjl_m:
            qjl = qjl_inner_estimate(qr, s_mat, np.asarray(k_bits, dtype=bool), k_gamma)
        out, w, keep, s = attend_rotated(q, qr, khat, k_norm, vhat, v_norm, pi_v, qjl_dots=qjl,
                                         sink_k=sink_k, sink_v=sink_v, scale=scale, v_skip=v_skip)
        outs.append(out)
        details.append((w, keep, s))
    out = np.stack(outs)
    return (out, details) if return_details else out


def attend_one(q: np.ndarray, kspec: Spec, k_idx: np.ndarray, k_norm: np.ndarray,
               vspec: Spec, v_idx: np.ndarray, v_norm: np.ndarray, *,
               k_bits: np.ndarray | None = None, k_gamma: np.ndarray | None = None,
               sink_k: np.ndarray | None = None, sink_v: np.ndarray | None = None,
               scale: float | None = None, v_skip: float = 0.0,
               pi_k: np.ndarray | None = None, pi_v: np.ndarray | None = None,
               s_mat: np.ndarray | None = None, return_weights: bool = False,
               return_scores: bool = False):
    """Attention output for one query head over one KV stream (float64).

    q [d]; k_idx/v_idx [T, d] codes of the compressed tokens; norms [T];
    k_bits [T, m] bool and k_gamma [T] for QJL; sink_k/sink_v [S, d] raw.
    return_weights adds (w, keep); return_scores adds the scores s (sink
    tokens first).
    """
    out, det = attend_group(np.asarray(q)[None, :], kspec, k_idx, k_norm, vspec, v_idx, v_norm,
                            k_bits=k_bits, k_gamma=k_gamma, sink_k=sink_k, sink_v=sink_v, scale=scale,
                            v_skip=v_skip, pi_k=pi_k, pi_v=pi_v, s_mat=s_mat, return_details=True)
    w, keep, s = det[0]
    res = (out[0],)
    if return_weights:
        res += (w, keep)
    if return_scores:
        res += (s,)
    return res if len(res) > 1 else res[0]


def attend(q: np.ndarray, kspec: Spec, vspec: Spec, seq_lens, k_idx, k_norm, v_idx, v_norm,
           *, k_bits=None, k_gamma=None, sink_k=None, sink_v=None, sink: int = 0,
           scale: float | None = None, v_skip: float = 0.0, heads=None) -> np.ndarray:
    """Batched decode attention.

    q [B, Hq, d]; seq_lens [B] (sink included); per (b, kh) the compressed
    arrays are indexed ``k_idx[b][kh]`` -> [L_b - sink, d] (lists or arrays;
    entries of streams no requested head reads may be None);
    sink_k/sink_v [B][Hkv] -> [sink, d].  heads: optional (b, h) pairs to
    evaluate, the other rows are NaN.  Returns out [B, Hq, d] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = len(k_idx[0])
    G = Hq // Hkv
    pi_k, pi_v = rotation_of(kspec), rotation_of(vspec)
    s_mat = sketch_of(kspec) if kspec.qjl_m else None
    want = None if heads is None else set(heads)
    out = np.full((B, Hq, d), np.nan) if want is not None else np.zeros((B, Hq, d))
    for b in range(B):
        L = int(seq_lens[b])
        ns = min(sink, L)
        nc = L - ns
        for kh in range(Hkv):
            hs = [h for h in range(kh * G, (kh + 1) * G) if want is None or (b, h) in want]
            if not hs:
                continue
            out[b, hs] = attend_group(
                q[b, hs], kspec, k_idx[b][kh][:nc], k_norm[b][kh][:nc],
                vspec, v_idx[b][kh][:nc], v_norm[b][kh][:nc],
                k_bits=None if k_bits is None else k_bits[b][kh][:nc],
                k_gamma=None if k_gamma is None else k_gamma[b][kh][:nc],
                sink_k=None if not ns else sink_k[b][kh][:ns],
                sink_v=None if not ns else sink_v[b][kh][:ns],
                scale=scale, v_skip=v_skip, pi_k=pi_k, pi_v=pi_v, s_mat=s_mat)
    return out
