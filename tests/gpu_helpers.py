"""Shared helpers of the GPU tests: host <-> device transport of exact bit
patterns and error statistics.  Expected values always come from the
oracle, never from the library under test."""

import numpy as np
import torch

from workloads import bf16_bits_to_f32

BF16_TOL = 2e-2      # max-abs error, bf16 inputs, fp32 accumulation, unit-variance data
BF16_REL_RMS = 2e-2  # RMS error relative to the RMS of the exact output
F32_TOL = 1e-5       # max-abs error, fp32 end to end


def dev(a):
    """numpy -> device tensor with identical bits (bf16 travels as int16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host(t, like):
    """device tensor -> numpy with the dtype of `like`."""
    a = t.cpu().numpy()
    return a.view(like.dtype) if a.dtype != like.dtype else a


def as_f64(a):
    return (bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)


def errors(got, want):
    """max-abs, max-abs relative to max |want|, and relative RMS."""
    err = np.abs(got - want)
    scale = max(float(np.abs(want).max()), 1e-30)
    rms_w = max(float(np.sqrt((want ** 2).mean())), 1e-30)
    return {"max_abs": float(err.max()), "rel_max": float(err.max()) / scale,
            "rel_rms": float(np.sqrt((err ** 2).mean())) / rms_w}


def assert_close(got, want, dtype, what=""):
    e = errors(got, want)
    print(f"{what} max_abs={e['max_abs']:.3e} rel_max={e['rel_max']:.3e} rel_rms={e['rel_rms']:.3e}",
          flush=True)
    if dtype == "f32":
        assert e["max_abs"] <= F32_TOL, e
    else:
        assert e["max_abs"] <= BF16_TOL, e
        assert e["rel_rms"] <= BF16_REL_RMS, e
    return e


def lse_bound(q_rows, k_max_norm, n_kept, d, scale, dtype, lse_ref):
    """Per-row bound on |LSE_gpu - LSE_exact| from the kernels' arithmetic.

    - Scores are fp32 dot products of d terms: |error| <= d 2^-24 s |q| |k|
      (Cauchy-Schwarz), and LSE moves by at most the largest score error.
    - The row sum adds n_kept positive fp32 terms: relative error
      <= n_kept 2^-24, i.e. that much in LSE.
    - On the bf16 path each probability is rounded to bf16 before it is
      summed: round-to-nearest to an 8-bit significand moves each term by
      at most 2^-8 of itself, so the sum (all terms positive) moves by at
      most 2^-8 of itself and LSE = ln(sum) by at most ln(1 + 2^-8) < 2^-8.
      The same rounded values weight V.
    - exp2/log2 and the final scaling: a few ulp of max(1, |LSE|)."""
    u = 2.0 ** -24
    qn = np.linalg.norm(q_rows, axis=-1)
    t = d * u * scale * qn * k_max_norm + n_kept * u + 8 * u * np.maximum(1.0, np.abs(lse_ref))
    if dtype == "bf16":
        t = t + 2.0 ** -8
    return t + 1e-7


def assert_lse_close(got, want, bound, what=""):
    """-inf exactly where the oracle has -inf; elsewhere within the bound."""
    inf_w = np.isneginf(want)
    assert np.array_equal(np.isneginf(got), inf_w), what
    fin = ~inf_w
    assert np.all(np.isfinite(got[fin])), what
    err = np.abs(got[fin] - want[fin])
    worst = float((err / bound[fin]).max()) if fin.any() else 0.0
    print(f"{what} lse max_abs={float(err.max()) if fin.any() else 0.0:.3e} "
          f"max err/bound={worst:.3f}", flush=True)
    assert worst <= 1.0, what


def mass_bound(q, k, want, N):
    """Bound on |A_gpu - A_exact| for the tile mass, per entry: every term
    exp(s q.k - LSE) is positive, so A carries a relative error of at most
    the score error twice (d 2^-24 s |q| |k|, once in the score and once
    through the LSE) plus n 2^-24 for fp32 sums of n positive terms (N keys
    in the LSE, up to 128 x 128 terms per tile pair)."""
    u = 2.0 ** -24
    d = q.shape[-1]
    qn = max(np.linalg.norm(as_f64(q[h]), axis=-1).max() for h in range(q.shape[0]))
    kn = max(np.linalg.norm(as_f64(k[h]), axis=-1).max() for h in range(k.shape[0]))
    rel = 2 * d * u * qn * kn / np.sqrt(d) + (N + 128 * 128) * u
    return want * rel + 1e-12
