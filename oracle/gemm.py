"""Block-scaled GEMM by its definition: FP64 product of dequantized operands.

Test infrastructure only (see oracle/__init__.py).

NVFP4 pretraining post, data-flow paragraph after Figure 1: FPROP, DGRAD and
WGRAD consume NVFP4 inputs and emit BF16 outputs.  HN page opcode84: MXFP8 /
MXFP4 GEMMs with the block scale applied inside the matrix unit.

Convention: C[M, N] = alpha * sum_k deq(A)[m, k] * deq(B)[n, k]; both
operands are K-major (quantized along K).
* NVFP4: deq = e2m1(code) * e4m3(S_block); alpha = s_dec(A) * s_dec(B) with
  s_dec the float32 per-tensor decode scale of each operand.
* MX:    deq = element(code) * 2**(E - 127); alpha = 1.
* FP8 per-tensor (the post's FP8 baseline, oracle/quantize.py): deq =
  e4m3(code); alpha = s_dec(A) * s_dec(B) with the float32 FP8 decode scales.

Tolerance (a reading): the GPU result is BF16, whose own rounding is up to
half a BF16 ulp, which at these output sizes already exceeds 1e-2 * rms by
itself.  So the test passes when
    max_i ( |C_gpu - C_ref| - ulp_bf16(max(|C_gpu|, |C_ref|)) / 2 ) <= 1e-2 * rms(C_ref).
"""

import numpy as np

from . import formats as F
from .quantize import fp8_scale_dec, nvfp4_scale_dec


def dequant_nvfp4(codes, scales):
    """[M, K/2] packed E2M1 + [M, K/16] E4M3 -> float64 [M, K] (per-tensor scale not applied)."""
    vals = F.e2m1_decode(F.unpack_e2m1(codes)).astype(np.float64)
    M, K = vals.shape
    s = F.e4m3_decode(scales).astype(np.float64)
    return (vals.reshape(M, K // 16, 16) * s[:, :, None]).reshape(M, K)


def dequant_mx(codes, scales, fmt):
    """MX codes + E8M0 scales -> float64 [M, K]."""
    if fmt == "mxfp4":
        vals = F.e2m1_decode(F.unpack_e2m1(codes)).astype(np.float64)
    else:
        vals = F.e4m3_decode(codes).astype(np.float64)
    M, K = vals.shape
    s = F.e8m0_decode(scales)
    return (vals.reshape(M, K // 32, 32) * s[:, :, None]).reshape(M, K)


def nvfp4_alpha(a_amax, b_amax):
    """alpha = s_dec(A) * s_dec(B), the product of the two float32 decode scales, in float64."""
    return np.float64(nvfp4_scale_dec(a_amax)) * np.float64(nvfp4_scale_dec(b_amax))


def gemm_nvfp4(a_codes, a_scales, a_amax, b_codes, b_scales, b_amax):
    A = dequant_nvfp4(a_codes, a_scales)
    B = dequant_nvfp4(b_codes, b_scales)
    return nvfp4_alpha(a_amax, b_amax) * (A @ B.T)


def gemm_mx(a_codes, a_scales, b_codes, b_scales, fmt):
    A = dequant_mx(a_codes, a_scales, fmt)
    B = dequant_mx(b_codes, b_scales, fmt)
    return A @ B.T


def ulp_bf16(y):
    """BF16 unit in the last place at magnitude |y| (float64)."""
    y = np.abs(np.asarray(y, dtype=np.float64))
    _, e = np.frexp(np.maximum(y, np.ldexp(1.0, -126)))
    return np.ldexp(1.0, e - 8)


def tolerance_report(c_gpu, c_ref):
    """Compare a BF16 GPU result (as float64) with the FP64 reference."""
    c_gpu = np.asarray(c_gpu, dtype=np.float64)
    c_ref = np.asarray(c_ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(c_ref ** 2))) if c_ref.size else 0.0
    err = np.abs(c_gpu - c_ref)
    allow = 0.5 * ulp_bf16(np.maximum(np.abs(c_gpu), np.abs(c_ref)))
    excess = float(np.max(err - allow)) if err.size else 0.0
    return dict(
        rms=rms,
        max_err=float(err.max()) if err.size else 0.0,
        max_err_over_rms=(float(err.max()) / rms) if rms > 0 else 0.0,
        excess_over_rms=(excess / rms) if rms > 0 else excess,
        frac_equal_rne=float(np.mean(c_gpu == F.f64_to_bf16_rne(c_ref))) if c_ref.size else 1.0,
        passed=bool(excess <= 1e-2 * rms) if c_ref.size else True,
    )


def fp8_alpha(a_amax, b_amax):
    """alpha = s_dec(A) * s_dec(B) of two per-tensor FP8 operands, in float64."""
    return np.float64(fp8_scale_dec(a_amax)) * np.float64(fp8_scale_dec(b_amax))


def gemm_fp8(a_codes, a_amax, b_codes, b_amax):
    A = F.e4m3_decode(a_codes).astype(np.float64)
    B = F.e4m3_decode(b_codes).astype(np.float64)
    return fp8_alpha(a_amax, b_amax) * (A @ B.T)
