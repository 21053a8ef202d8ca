"""The quantize kernels' squared-norm scheme over the whole bf16 range, on
the CPU (host logic, no GPU): a numpy model of the fast form and of its
fallback, held to the exact norm.

Fast form: every square of a bf16 element is exact in fp32; the squares go
into fp32 chains (modelled with a rounding after every addition, and with
squares below fp32's normal range flushed to zero, the least favourable
reading of the hardware), the chains are combined in fp64.  A total outside
[2^-60, inf) takes the fallback: the elements are scaled by 2^70 (small
total) or 2^-70 (infinite total) before squaring, and the result is scaled
back in fp64.  The claim the kernels rely on: the fp32 rounding of the
square root is within 1 ulp of the correctly rounded norm, for finite
vectors whose norm is below FLT_MAX.
"""
import numpy as np

from compressed_kv_cache_tq_amd import workloads

F32_TINY = np.float32(2.0 ** -126)


def _chains(x32: np.ndarray, scale: np.float32) -> float:
    """Sum of (x s)^2 in four fp32 chains of 32 elements each, combined in fp64."""
    with np.errstate(over="ignore", under="ignore", invalid="ignore"):
        y = (x32 * scale).astype(np.float32)
        sq = (y * y).astype(np.float32)
        sq[np.abs(sq) < F32_TINY] = np.float32(0.0)  # flushed
        total = 0.0
        for c in range(4):
            acc = np.float32(0.0)
            for v in sq[32 * c:32 * (c + 1)]:
                acc = np.float32(acc + v)
            total += float(acc)
    return total


def _kernel_norm(x32: np.ndarray) -> np.float32:
    ss = _chains(x32, np.float32(1.0))
    if not (ss >= 2.0 ** -60 and ss < np.inf):
        s = np.float32(2.0 ** 70) if ss < 2.0 ** -60 else np.float32(2.0 ** -70)
        ss = _chains(x32, s) / (float(s) * float(s))
    return np.float32(np.sqrt(ss))


def _exact_norm(x32: np.ndarray) -> np.float32:
    x = x32.astype(np.float64)
    m = np.max(np.abs(x))
    if m == 0.0:
        return np.float32(0.0)
    with np.errstate(over="ignore"):
        return np.float32(m * np.sqrt(np.sum((x / m) ** 2)))  # inf past FLT_MAX (skipped)


def test_norm_scheme_within_one_ulp_over_the_bf16_range():
    rng = np.random.default_rng(11)
    worst = 0.0
    for e in list(range(-130, 126, 5)) + [-133, 60, 62, 63, 64, 65, 66]:
        x = rng.standard_normal((6, 128)).astype(np.float32) * np.float32(2.0 ** e)
        x = workloads.bf16_to_f32(workloads.bf16_bits(x))
        for v in x:
            exact = _exact_norm(v)
            if not np.isfinite(exact) or exact == 0.0:
                continue
            got = _kernel_norm(v)
            ulps = abs(float(got) - float(exact)) / float(np.spacing(exact))
            worst = max(worst, ulps)
            assert ulps <= 1.0, f"2^{e}: {got} vs {exact} ({ulps} ulp)"
    assert worst <= 1.0


def test_fast_form_alone_fails_outside_its_range():
    """Without the fallback the fast form loses such vectors: all squares of
    elements near 2^-80 flush to zero, and squares of elements near 2^70
    overflow; that is what the range check catches."""
    rng = np.random.default_rng(12)
    tiny = workloads.bf16_to_f32(workloads.bf16_bits(rng.standard_normal(128).astype(np.float32) * np.float32(2.0 ** -80)))
    huge = workloads.bf16_to_f32(workloads.bf16_bits(rng.standard_normal(128).astype(np.float32) * np.float32(2.0 ** 70)))
    assert _chains(tiny, np.float32(1.0)) == 0.0
    assert _chains(huge, np.float32(1.0)) == np.inf
    assert _kernel_norm(tiny) == _exact_norm(tiny) or abs(float(_kernel_norm(tiny)) - float(_exact_norm(tiny))) <= float(np.spacing(_exact_norm(tiny)))
    assert abs(float(_kernel_norm(huge)) - float(_exact_norm(huge))) <= float(np.spacing(_exact_norm(huge)))
