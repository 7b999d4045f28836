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
