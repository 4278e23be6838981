"""Shared pieces of the GPU parity tests: the oracle pipeline on host copies of
the seeded inputs, and the comparison metrics.

Tolerances (fixed by the target statement of this layer): NF4 codes, the 8-bit
constants, c2 and the mean bit-exact; dequantized weights within 1e-6
relative (they are bit-exact here by construction); bf16 products and
gradients within 2e-2 relative Frobenius error of the float64 oracle.  The
extra elementwise guard (max |err| <= 5% of the reference RMS) catches a
localised fault (one wrong block or tile) that a Frobenius norm could hide;
bf16 rounding of the operands and of the output moves an element by well
under 1% of the RMS.
"""
import numpy as np
import torch

import oracle
from workloads import bf16_bits, host_f32

FRO_TOL = 2e-2
ELEM_TOL = 5e-2


def rel_fro(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def max_err_over_rms(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref * ref)) if ref.size else 0.0
    return float(np.max(np.abs(got - ref)) / (rms if rms > 0 else 1.0)) if ref.size else 0.0


def assert_close(name, got, ref, fro_tol=FRO_TOL, elem_tol=ELEM_TOL):
    f = rel_fro(got, ref)
    e = max_err_over_rms(got, ref)
    assert f <= fro_tol and e <= elem_tol, "%s: rel_fro=%.3e max/rms=%.3e" % (name, f, e)
    return f, e


def oracle_weight(W: torch.Tensor):
    """Oracle quantize + double-quantize + dequantize of a host weight tensor."""
    if W.dtype == torch.bfloat16:
        w = bf16_bits(W).reshape(-1)
    else:
        w = host_f32(W).reshape(-1)
    codes, absmax = oracle.nf4_quantize(w)
    q, c2, mean = oracle.double_quantize(absmax)
    Wd = oracle.nf4_dequantize(codes, q, c2, mean, tuple(W.shape))
    return dict(codes=codes, absmax=absmax, q=q, c2=c2, mean=mean, Wd=Wd)


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy() if t.dtype != torch.bfloat16 else host_f32(t)
