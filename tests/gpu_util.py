"""Helpers for GPU parity tests: moving stored inputs to the device and comparing
against the float64 oracle at the stated tolerances.

Tolerances, per output tensor T in {out, lse, dq, dk, dv, dtable}:
  float32 inputs:  max |T_gpu - T_ref| <= 1e-4
  bfloat16 inputs: max |T_gpu - T_ref| / rms(T_ref) <= 2e-2   (float32 accumulation);
                   a reference that is exactly zero is held to max |T_gpu| <= 1e-4
"""
import numpy as np
import torch

TOL_F32_ABS = 1e-4
TOL_BF16_REL = 2e-2


def dev(stored):
    """A workloads.Stored tensor on cuda:0 in its storage type."""
    if stored.dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(stored.raw)).cuda()
    bits = np.ascontiguousarray(stored.raw).view(np.int16)
    return torch.from_numpy(bits).cuda().view(torch.bfloat16)


def host64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def err(got, ref, dtype, bound=None):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    e = float(np.max(np.abs(got - ref))) if got.size else 0.0
    if dtype == "f32":
        return e, e <= (TOL_F32_ABS if bound is None else bound)
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    if rms == 0.0:
        # an exactly zero reference (N = 1: dq = dk = 0) has no RMS to scale by; the
        # float32 rounding of the GPU's arithmetic is held to the float32 bound instead
        return e, e <= TOL_F32_ABS
    return e / rms, e / rms <= (TOL_BF16_REL if bound is None else bound)


def check(name, got, ref, dtype, report=None, bound=None):
    """Compare at the stated tolerance, or at `bound` where a test derives a wider one
    from the oracle's own spread (the stacked bfloat16 model)."""
    e, ok = err(got, ref, dtype, bound)
    if report is not None:
        report[name] = e
    if bound is None:
        bound = TOL_F32_ABS if dtype == "f32" else TOL_BF16_REL
    kind = "max-abs" if dtype == "f32" else "max-abs/rms"
    assert ok, f"{name}: {kind} error {e:.3e} exceeds {bound:.1e}"
    return e
