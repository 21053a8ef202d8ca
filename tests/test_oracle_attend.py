"""Pins of the oracle's decode attention (CPU only)."""
import math

import numpy as np
import pytest

from oracle import attend as at
from oracle import quantize as qz
from oracle.rotation import sketch


def sdpa(q, K, V, scale):
    s = scale * (K @ q)
    w = np.exp(s - s.max())
    w /= w.sum()
    return w @ V, w


def _data(T=300, seed=0, d=128):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(d), rng.standard_normal((T, d)), rng.standard_normal((T, d))


def test_identity_dequantize_then_textbook_sdpa():
    # Attending in the rotated domain equals textbook SDPA over explicitly
    # dequantized keys/values Khat = n Pi^T c[idx] (Pi orthogonal).
    q, K, V = _data()
    ks, vs = qz.Spec(bits_lo=4, bits_hi=4), qz.Spec(bits_lo=3, bits_hi=3)
    qk, qv = qz.quantize(K, ks), qz.quantize(V, vs)
    out = at.attend_one(q, ks, qk.idx, qk.norms, vs, qv.idx, qv.norms)
    pi = qz.rotation_of(ks)
    Kh = qk.norms.astype(np.float64)[:, None] * (qz.dequantize_rotated(qk.idx, ks) @ pi)
    Vh = qv.norms.astype(np.float64)[:, None] * (qz.dequantize_rotated(qv.idx, vs) @ pi)
    ref, _ = sdpa(q, Kh, Vh, 1 / math.sqrt(128))
    assert np.max(np.abs(out - ref)) < 1e-12


def test_identity_exact_rotation_gives_plain_attention():
    # Feeding the exact rotated unit vectors instead of centroids recovers
    # softmax(q K^T / sqrt(d)) V on the original data.
    q, K, V = _data(seed=1)
    spec = qz.Spec()
    pi = qz.rotation_of(spec)
    nk, nv = np.linalg.norm(K, axis=1), np.linalg.norm(V, axis=1)
    yk, yv = (K @ pi.T) / nk[:, None], (V @ pi.T) / nv[:, None]
    out, _, _, _ = at.attend_rotated(q, pi @ q, yk, nk, yv, nv, pi, scale=1 / math.sqrt(128))
    ref, _ = sdpa(q, K, V, 1 / math.sqrt(128))
    assert np.max(np.abs(out - ref)) < 1e-12


def test_sink_tokens_join_the_softmax_raw():
    q, K, V = _data(T=200, seed=2)
    ks = vs = qz.Spec(bits_lo=4, bits_hi=4)
    n_sink = 16
    qk, qv = qz.quantize(K[n_sink:], ks), qz.quantize(V[n_sink:], vs)
    out = at.attend_one(q, ks, qk.idx, qk.norms, vs, qv.idx, qv.norms,
                        sink_k=K[:n_sink], sink_v=V[:n_sink])
    pi = qz.rotation_of(ks)
    Kh = np.concatenate([K[:n_sink], qk.norms.astype(np.float64)[:, None] * (qz.dequantize_rotated(qk.idx, ks) @ pi)])
    Vh = np.concatenate([V[:n_sink], qv.norms.astype(np.float64)[:, None] * (qz.dequantize_rotated(qv.idx, vs) @ pi)])
    ref, _ = sdpa(q, Kh, Vh, 1 / math.sqrt(128))
    assert np.max(np.abs(out - ref)) < 1e-12


def test_v_skip_bound_and_no_renormalisation():
    q, K, V = _data(T=2000, seed=3)
    q = q * 6.0                                     # peaked scores so the rule fires
    ks = vs = qz.Spec(bits_lo=4, bits_hi=4)
    qk, qv = qz.quantize(K, ks), qz.quantize(V, vs)
    o0, w, _ = at.attend_one(q, ks, qk.idx, qk.norms, vs, qv.idx, qv.norms, return_weights=True)
    oe, _, keep = at.attend_one(q, ks, qk.idx, qk.norms, vs, qv.idx, qv.norms, v_skip=1e-6,
                                return_weights=True)
    skipped = ~keep
    assert skipped.sum() > 10 and np.all(w[skipped] < 1e-6) and np.all(w[keep] >= 1e-6)
    vhat_norm = qv.norms.astype(np.float64)      # ||n c[idx]|| <= n since ||c[idx]|| < 1
    bound = np.sum(w[skipped] * vhat_norm[skipped])
    assert 0 < np.linalg.norm(oe - o0) <= bound
    # dropping is not renormalised: out_eps = out_0 - sum_skipped w_t vhat_t exactly
    pi = qz.rotation_of(vs)
    vh = qv.norms.astype(np.float64)[:, None] * (qz.dequantize_rotated(qv.idx, vs) @ pi)
    assert np.max(np.abs((o0 - w[skipped] @ vh[skipped]) - oe)) < 1e-13


def test_gqa_head_mapping():
    rng = np.random.default_rng(4)
    B, Hq, Hkv, T = 2, 8, 2, 64
    ks = vs = qz.Spec(bits_lo=3, bits_hi=3)
    q = rng.standard_normal((B, Hq, 128))
    kidx, knorm, vidx, vnorm = [], [], [], []
    for b in range(B):
        kb, vb = [], []
        for h in range(Hkv):
            kb.append(qz.quantize(rng.standard_normal((T, 128)), ks))
            vb.append(qz.quantize(rng.standard_normal((T, 128)), vs))
        kidx.append([x.idx for x in kb]); knorm.append([x.norms for x in kb])
        vidx.append([x.idx for x in vb]); vnorm.append([x.norms for x in vb])
    lens = [T, T - 7]
    out = at.attend(q, ks, vs, lens, kidx, knorm, vidx, vnorm)
    for b in range(B):
        for h in range(Hq):
            kh = h // (Hq // Hkv)
            L = lens[b]
            ref = at.attend_one(q[b, h], ks, kidx[b][kh][:L], knorm[b][kh][:L],
                                vs, vidx[b][kh][:L], vnorm[b][kh][:L])
            assert np.array_equal(out[b, h], ref)


def test_qjl_scores_unbiased_over_seeds():
    # The sketch-corrected score n(<qr, c[idx]> + estimate) averages to the exact
    # <q, k> over QJL seeds (the rotation, hence the residual, stays fixed).
    rng = np.random.default_rng(9)
    qv, k = rng.standard_normal(128), rng.standard_normal(128)
    exact = qv @ k
    vals, plain = [], []
    for s in range(1500):
        spec = qz.Spec(bits_lo=2, bits_hi=2, qjl_m=128, qjl_seed=500 + s)
        S = sketch(spec.qjl_seed, 128, 128)
        qq = qz.quantize(k[None, :], spec, s_mat=S)
        pi = qz.rotation_of(spec)
        qr = pi @ qv
        base = qz.dequantize_rotated(qq.idx, spec)[0] @ qr
        corr = qz.qjl_inner_estimate(qr, S, qq.qjl_bits[0], qq.rnorms[0])
        n = float(qq.norms64[0])
        vals.append(n * (base + corr))
        plain.append(n * base)
    vals = np.array(vals)
    se = vals.std() / math.sqrt(len(vals))
    assert abs(vals.mean() - exact) < 4 * se


def test_empty_sequence_gives_zero_output():
    d = 128
    pi = np.eye(d)
    empty = np.zeros((0, d))
    q = np.ones(d)
    out, w, keep, s = at.attend_rotated(q, q, empty, np.zeros(0), empty, np.zeros(0), pi, scale=0.1)
    assert out.shape == (d,) and np.all(out == 0.0) and w.size == 0 and keep.size == 0


# ---- the sketch branch of the attention oracle ------------------------------
#
# noze.it "TurboQuant-MLX: ...", section "Il metodo TurboQuant, in breve": the
# 1-bit sketch of the residual makes the inner-product estimate unbiased.  In
# attention that means the compressed token's score, averaged over sketch
# seeds, is scale * <q, k>.  The scores are taken from the oracle's own
# attention path (attend_one), and the query is aimed along the residual so
# that the sketch term is large: a dropped gamma, a flipped sign, a wrong
# constant or a missing norm factor then moves the mean by hundreds of
# standard errors.

def _qjl_score_zscore(n_seeds=1200):
    """z-score of the mean compressed-token score over sketch seeds against
    the exact scale * <q, k> (one sink token joins the softmax)."""
    rng = np.random.default_rng(21)
    k = rng.standard_normal(128)
    base = qz.Spec(bits_lo=2, bits_hi=2, qjl_m=128, qjl_seed=0)
    pi = qz.rotation_of(base)
    q0 = qz.quantize(k[None, :], base)
    r = q0.y[0] - qz.dequantize_rotated(q0.idx, base)[0]      # residual: independent of the sketch seed
    q = 3.0 * (pi.T @ (r / np.linalg.norm(r))) + 0.2 * rng.standard_normal(128)
    vs = qz.Spec(bits_lo=3, bits_hi=3)
    v = qz.quantize(rng.standard_normal((1, 128)), vs)
    sink_k, sink_v = rng.standard_normal((1, 128)), rng.standard_normal((1, 128))
    scale = 1 / math.sqrt(128)
    vals = []
    for s in range(n_seeds):
        spec = qz.Spec(bits_lo=2, bits_hi=2, qjl_m=128, qjl_seed=1000 + s)
        kq = qz.quantize(k[None, :], spec, pi=pi)
        _, sc = at.attend_one(q, spec, kq.idx, kq.norms, vs, v.idx, v.norms, k_bits=kq.qjl_bits,
                              k_gamma=kq.rnorms, sink_k=sink_k, sink_v=sink_v, scale=scale, pi_k=pi,
                              return_scores=True)
        assert sc.shape == (2,) and abs(sc[0] - scale * (sink_k[0] @ q)) < 1e-12
        vals.append(sc[1])
    vals = np.array(vals)
    exact = scale * float(q @ k)
    return (vals.mean() - exact) / (vals.std() / math.sqrt(len(vals)))


def test_qjl_attention_scores_unbiased_over_seeds():
    z = _qjl_score_zscore()
    assert abs(z) < 4.0, z


def _scaled_estimate(factor=1.0, sign=1.0, drop_gamma=False):
    orig = qz.qjl_inner_estimate

    def est(qr, s_mat, bits, gamma):
        g = np.ones_like(np.asarray(gamma, np.float64)) if drop_gamma else gamma
        return sign * factor * orig(qr, s_mat, bits, g)
    return est


@pytest.mark.parametrize("mistake", ["z_sign", "no_gamma", "constant", "no_norm"])
def test_qjl_attention_pin_catches_planted_mistakes(monkeypatch, mistake):
    """Mistakes planted in the oracle's sketch branch (on the CPU) must fail
    the unbiasedness pin above."""
    if mistake == "z_sign":
        monkeypatch.setattr(at, "qjl_inner_estimate", _scaled_estimate(sign=-1.0))
    elif mistake == "no_gamma":
        monkeypatch.setattr(at, "qjl_inner_estimate", _scaled_estimate(drop_gamma=True))
    elif mistake == "constant":   # sqrt(2/pi)/m instead of sqrt(pi/2)/m
        monkeypatch.setattr(at, "qjl_inner_estimate", _scaled_estimate(factor=2.0 / math.pi))
    else:                         # the sketch term added outside the norm factor
        def scores(qr, khat, k_norm, qjl_dots, scale):
            return scale * (np.asarray(k_norm, np.float64) * (khat @ qr) + qjl_dots)
        monkeypatch.setattr(at, "compressed_scores", scores)
    z = _qjl_score_zscore(n_seeds=300)
    assert abs(z) > 8.0, (mistake, z)


def test_gqa_head_mapping_with_sketch_and_sink():
    """The batched oracle with the QJL stage and sink tokens equals the
    single-head path on every head (brute-force loop)."""
    rng = np.random.default_rng(6)
    B, Hq, Hkv, T, S = 2, 8, 2, 40, 5
    ks = qz.Spec(bits_lo=2, bits_hi=2, qjl_m=128, qjl_seed=3)
    vs = qz.Spec(bits_lo=3, bits_hi=3)
    q = rng.standard_normal((B, Hq, 128))
    kidx, knorm, vidx, vnorm, kbits, kgam, skk, svv = ([] for _ in range(8))
    for b in range(B):
        rows = [[] for _ in range(8)]
        for h in range(Hkv):
            kq = qz.quantize(rng.standard_normal((T, 128)), ks)
            vq = qz.quantize(rng.standard_normal((T, 128)), vs)
            for lst, val in zip(rows, (kq.idx, kq.norms, vq.idx, vq.norms, kq.qjl_bits, kq.rnorms,
                                       rng.standard_normal((S, 128)), rng.standard_normal((S, 128)))):
                lst.append(val)
        for dst, src in zip((kidx, knorm, vidx, vnorm, kbits, kgam, skk, svv), rows):
            dst.append(src)
    lens = [S + T, S + T - 9]
    out = at.attend(q, ks, vs, lens, kidx, knorm, vidx, vnorm, k_bits=kbits, k_gamma=kgam, sink_k=skk,
                    sink_v=svv, sink=S)
    part = at.attend(q, ks, vs, lens, kidx, knorm, vidx, vnorm, k_bits=kbits, k_gamma=kgam, sink_k=skk,
                     sink_v=svv, sink=S, heads=[(1, 5)])
    for b in range(B):
        nc = lens[b] - S
        for h in range(Hq):
            kh = h // (Hq // Hkv)
            ref = at.attend_one(q[b, h], ks, kidx[b][kh][:nc], knorm[b][kh][:nc], vs, vidx[b][kh][:nc],
                                vnorm[b][kh][:nc], k_bits=kbits[b][kh][:nc], k_gamma=kgam[b][kh][:nc],
                                sink_k=skk[b][kh], sink_v=svv[b][kh])
            assert np.array_equal(out[b, h], ref)
    assert np.array_equal(part[1, 5], out[1, 5]) and np.isnan(part[0]).all()
