"""Block-scaled (NVFP4 / MXFP4 / MXFP8) quantize + GEMM on MI355X, with the
per-tensor FP8 baseline (format "fp8") for comparison.

Thin Python binding over the C ABI of libbsq.so (include/bsq.h): argument
marshalling only.  PyTorch supplies device memory and the current stream;
every step of the computation runs in the HIP kernels of libbsq.so.  If the
library has not been built (python -m fp8_quantized_gemm_amd._build), every
entry point raises; there is no fallback.
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbsq.so")

BSQ_OK, BSQ_EINVAL, BSQ_EUNSUPPORTED, BSQ_EHIP = 0, 1, 2, 3
FORMATS = {"nvfp4": 0, "mxfp4": 1, "mxfp8": 2, "fp8": 3}
ROUNDING = {"rne": 0, "sr": 1}
ABI_SYMBOLS = ("nvfp4_quantize", "mx_quantize", "quantize_transpose", "quantize_transpose_amax",
               "fp8_quantize_transpose", "swiglu_amax", "swiglu_backward_amax",
               "master_weight_update", "nvfp4_expand", "bs_gemm", "bs_gemm_noalloc",
               "bs_gemm_nvfp4_bx", "bsq_status_string")


class BsqError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed: {msg}")
        self.status = status


_lib = None


def lib():
    """Load libbsq.so (once).  Raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m fp8_quantized_gemm_amd._build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I, U64, U32, U16 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                    ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint16)
        L.nvfp4_quantize.argtypes = [P, I64, I64, I, I, U64, U32, I, U16, P, P, P, P, P]
        L.mx_quantize.argtypes = [P, I64, I64, I, I, U64, U32, P, P, P]
        L.quantize_transpose.argtypes = [P, I64, I64, I, I, I, U64, U32, I, U16,
                                         P, P, P, P, P, P, P]
        L.quantize_transpose_amax.argtypes = [P, I64, I64, I, I, U64, U32, I, U16,
                                              P, P, P, P, P, P, P]
        L.fp8_quantize_transpose.argtypes = [P, I64, I64, P, P, P, P]
        L.swiglu_amax.argtypes = [P, I64, I64, I, U16, P, P, P, P]
        L.swiglu_backward_amax.argtypes = [P, P, I64, I64, I, U16, P, P, P, P]
        L.master_weight_update.argtypes = [P, P, I64, ctypes.c_float, P, P, P]
        L.bs_gemm.argtypes = [I, I64, I64, I64, P, P, P, P, P, P, P, I64, P]
        L.bs_gemm_noalloc.argtypes = [I, I64, I64, I64, P, P, P, P, P, P, P, I64, P]
        L.nvfp4_expand.argtypes = [P, P, I64, I64, P, P]
        L.bs_gemm_nvfp4_bx.argtypes = [I64, I64, I64, P, P, P, P, P, P, I64, P]
        for fn in ABI_SYMBOLS[:-1]:
            getattr(L, fn).restype = I
        L.bsq_status_string.argtypes = [I]
        L.bsq_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status):
    return lib().bsq_status_string(int(status)).decode()


def _check(fn, status):
    if status != BSQ_OK:
        raise BsqError(fn, status, status_string(status))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_device(*tensors, out=None):
    """Every given tensor (None skipped) is a contiguous CUDA tensor on one device,
    and `out` a CUDA matrix with unit column stride (its row stride becomes ldc):
    the library dereferences the raw pointers on the GPU."""
    dev = None
    for t in tensors + ((out,) if out is not None else ()):
        if t is None:
            continue
        ok = isinstance(t, torch.Tensor) and t.is_cuda
        if t is out:
            ok = ok and t.dim() == 2 and (t.stride(1) == 1 or t.shape[1] <= 1)
        else:
            ok = ok and t.is_contiguous()
        if not ok:
            raise ValueError("operands must be contiguous CUDA tensors (out: rows with unit stride)")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("operands must be on one device")


def _check_amax(*amaxes):
    """Each given amax is a float32 tensor of at least one element."""
    for a in amaxes:
        if a is not None and not (isinstance(a, torch.Tensor) and a.dtype == torch.float32
                                  and a.numel() >= 1):
            raise ValueError("amax arguments must be float32 tensors of at least one element")


def _check_operand(what, codes, scales, K, fmt):
    """codes (uint8 [rows, K / elements-per-byte]) and scales (uint8 [rows, K /
    block], None for per-tensor FP8) of one K-major GEMM operand.  The library
    takes the row strides from K, so the widths must match exactly."""
    per_byte = 1 if fmt in ("mxfp8", "fp8") else 2
    blk = {"nvfp4": 16, "mxfp4": 32, "mxfp8": 32, "fp8": None}[fmt]
    if not (isinstance(codes, torch.Tensor) and codes.dtype == torch.uint8 and codes.dim() == 2):
        raise ValueError(f"{what} codes must be a 2-D uint8 tensor")
    if K < 0 or K % per_byte or codes.shape[1] != K // per_byte:
        raise ValueError(f"{what} codes are [{codes.shape[0]}, {codes.shape[1]}]; "
                         f"K = {K} needs [rows, {K // per_byte}]")
    if blk is None:
        return
    if not (isinstance(scales, torch.Tensor) and scales.dtype == torch.uint8 and scales.dim() == 2
            and scales.shape[0] == codes.shape[0] and scales.shape[1] == K // blk):
        raise ValueError(f"{what} scales must be uint8 [{codes.shape[0]}, {K // blk}]")


def _check_out(out, M, N, dtype):
    if out.dtype != dtype or tuple(out.shape) != (M, N):
        raise ValueError(f"out must be a {dtype} [{M}, {N}] tensor")


def _check_input(x):
    if not (isinstance(x, torch.Tensor) and x.is_cuda and x.dtype == torch.bfloat16 and x.dim() == 2):
        raise ValueError("x must be a 2-D bfloat16 CUDA tensor")
    return x.contiguous()


def _u8(shape, device):
    return torch.empty(shape, dtype=torch.uint8, device=device)


def nvfp4_quantize(x, block_rows=1, rnd="rne", seed=0, offset=0, rht=False, rht_signs=0,
                   amax=None):
    """Rowwise NVFP4 of x [R, C] -> (codes uint8 [R, C/2], scales uint8 [R, C/16], amax f32 [1])."""
    x = _check_input(x)
    _check_device(x, amax)
    _check_amax(amax)
    R, C = x.shape
    codes = _u8((R, C // 2), x.device)
    scales = _u8((R, max(C // 16, 0)), x.device)
    amax_out = torch.empty(1, dtype=torch.float32, device=x.device)
    st = lib().nvfp4_quantize(_ptr(x), R, C, int(block_rows), ROUNDING[rnd], int(seed), int(offset),
                              1 if rht else 0, int(rht_signs) & 0xFFFF, _ptr(amax),
                              _ptr(codes), _ptr(scales), _ptr(amax_out), _stream(x.device))
    _check("nvfp4_quantize", st)
    return codes, scales, amax_out


def mx_quantize(x, fmt="mxfp4", rnd="rne", seed=0, offset=0):
    """Rowwise MXFP4 / MXFP8 of x [R, C] -> (codes, scales E8M0 [R, C/32])."""
    x = _check_input(x)
    R, C = x.shape
    codes = _u8((R, C // 2 if fmt == "mxfp4" else C), x.device)
    scales = _u8((R, C // 32), x.device)
    st = lib().mx_quantize(_ptr(x), R, C, FORMATS[fmt], ROUNDING[rnd], int(seed), int(offset),
                           _ptr(codes), _ptr(scales), _stream(x.device))
    _check("mx_quantize", st)
    return codes, scales


def quantize_transpose(x, fmt="nvfp4", block_rows=1, rnd="rne", seed=0, offset=0,
                       rht_col=False, rht_signs=0, row=True, col=True):
    """Row (quantize(x)) and column (quantize(x^T)) outputs from one read of x [R, C].

    Returns a dict with row_codes, row_scales, row_amax, col_codes, col_scales,
    col_amax (entries of a skipped orientation, and amax for MX, are None)."""
    x = _check_input(x)
    R, C = x.shape
    blk = 16 if fmt == "nvfp4" else 32
    w = 1 if fmt == "mxfp8" else 2
    out = dict(row_codes=None, row_scales=None, row_amax=None,
               col_codes=None, col_scales=None, col_amax=None)
    if row:
        out["row_codes"] = _u8((R, C // w), x.device)
        out["row_scales"] = _u8((R, C // blk), x.device)
        if fmt == "nvfp4":
            out["row_amax"] = torch.empty(1, dtype=torch.float32, device=x.device)
    if col:
        out["col_codes"] = _u8((C, R // w), x.device)
        out["col_scales"] = _u8((C, R // blk), x.device)
        if fmt == "nvfp4":
            out["col_amax"] = torch.empty(1, dtype=torch.float32, device=x.device)
    st = lib().quantize_transpose(
        _ptr(x), R, C, FORMATS[fmt], int(block_rows), ROUNDING[rnd], int(seed), int(offset),
        1 if rht_col else 0, int(rht_signs) & 0xFFFF,
        _ptr(out["row_codes"]), _ptr(out["row_scales"]), _ptr(out["row_amax"]),
        _ptr(out["col_codes"]), _ptr(out["col_scales"]), _ptr(out["col_amax"]), _stream(x.device))
    _check("quantize_transpose", st)
    return out


def quantize_transpose_amax(x, amax_row, amax_col, block_rows=1, rnd="rne", seed=0, offset=0,
                            rht_col=False, rht_signs=0, row=True, col=True):
    """NVFP4 row and column outputs of x [R, C] under the given device amaxes
    (f32 [1] each; the one of a skipped side may be None).

    Returns a dict with row_codes, row_scales, col_codes, col_scales (None when skipped)."""
    x = _check_input(x)
    _check_device(x, amax_row, amax_col)
    _check_amax(amax_row, amax_col)
    R, C = x.shape
    out = dict(row_codes=None, row_scales=None, col_codes=None, col_scales=None)
    if row:
        out["row_codes"] = _u8((R, C // 2), x.device)
        out["row_scales"] = _u8((R, C // 16), x.device)
    if col:
        out["col_codes"] = _u8((C, R // 2), x.device)
        out["col_scales"] = _u8((C, R // 16), x.device)
    st = lib().quantize_transpose_amax(
        _ptr(x), R, C, int(block_rows), ROUNDING[rnd], int(seed), int(offset),
        1 if rht_col else 0, int(rht_signs) & 0xFFFF, _ptr(amax_row), _ptr(amax_col),
        _ptr(out["row_codes"]), _ptr(out["row_scales"]), _ptr(out["col_codes"]),
        _ptr(out["col_scales"]), _stream(x.device))
    _check("quantize_transpose_amax", st)
    return out


def swiglu(y_gu, rht_col=False, rht_signs=0, amax=True, out=None):
    """H [T, F] = silu(G) * U of y_gu = [G | U] [T, 2F] (bf16), with amax_row =
    max|H| and amax_col (the column RHT amax with rht_col, else max|H|).

    Returns dict(h, amax_row, amax_col); the amaxes are None with amax=False."""
    y = _check_input(y_gu)
    T, F2 = y.shape
    h = torch.empty((T, F2 // 2), dtype=torch.bfloat16, device=y.device) if out is None else out
    _check_device(y, h)
    if h.dtype != torch.bfloat16 or h.shape != (T, F2 // 2):
        raise ValueError("out must be a bfloat16 [T, F] tensor")
    ar = torch.empty(1, dtype=torch.float32, device=y.device) if amax else None
    ac = torch.empty(1, dtype=torch.float32, device=y.device) if amax else None
    st = lib().swiglu_amax(_ptr(y), T, F2 // 2, 1 if rht_col else 0, int(rht_signs) & 0xFFFF,
                           _ptr(h), _ptr(ar), _ptr(ac), _stream(y.device))
    _check("swiglu_amax", st)
    return dict(h=h, amax_row=ar, amax_col=ac)


def swiglu_backward(y_gu, d_h, rht_col=False, rht_signs=0, amax=True, out=None):
    """dY_gu [T, 2F] = [dG | dU] from y_gu = [G | U] [T, 2F] and d_h [T, F]
    (bf16), with the amaxes of dY_gu as for swiglu.

    Returns dict(d_y_gu, amax_row, amax_col)."""
    y = _check_input(y_gu)
    d = _check_input(d_h)
    T, F2 = y.shape
    if d.shape != (T, F2 // 2):
        raise ValueError("d_h must be [T, F] for y_gu [T, 2F]")
    dy = torch.empty((T, F2), dtype=torch.bfloat16, device=y.device) if out is None else out
    _check_device(y, d, dy)
    if dy.dtype != torch.bfloat16 or dy.shape != (T, F2):
        raise ValueError("out must be a bfloat16 [T, 2F] tensor")
    ar = torch.empty(1, dtype=torch.float32, device=y.device) if amax else None
    ac = torch.empty(1, dtype=torch.float32, device=y.device) if amax else None
    st = lib().swiglu_backward_amax(_ptr(y), _ptr(d), T, F2 // 2, 1 if rht_col else 0,
                                    int(rht_signs) & 0xFFFF, _ptr(dy), _ptr(ar), _ptr(ac),
                                    _stream(y.device))
    _check("swiglu_backward_amax", st)
    return dict(d_y_gu=dy, amax_row=ar, amax_col=ac)


def master_weight_update(w32, grad, lr, w_bf16=None, amax=True):
    """In place w32 <- w32 - lr * grad (FP32 master weight, BF16 gradient of the
    same shape); returns dict(w_bf16, amax) with the BF16 working copy and its
    amax (None with amax=False)."""
    if not (isinstance(w32, torch.Tensor) and w32.is_cuda and w32.dtype == torch.float32
            and w32.is_contiguous()):
        raise ValueError("w32 must be a contiguous float32 CUDA tensor (updated in place)")
    if not (isinstance(grad, torch.Tensor) and grad.is_cuda and grad.dtype == torch.bfloat16
            and grad.shape == w32.shape):
        raise ValueError("grad must be a bfloat16 CUDA tensor shaped like w32")
    g = grad.contiguous()
    wb = torch.empty(w32.shape, dtype=torch.bfloat16, device=w32.device) if w_bf16 is None else w_bf16
    _check_device(w32, g, wb)
    if wb.dtype != torch.bfloat16 or wb.numel() != w32.numel():
        raise ValueError("w_bf16 must be a bfloat16 tensor with w32's element count")
    a = torch.empty(1, dtype=torch.float32, device=w32.device) if amax else None
    st = lib().master_weight_update(_ptr(w32), _ptr(g), w32.numel(), float(lr), _ptr(wb), _ptr(a),
                                    _stream(w32.device))
    _check("master_weight_update", st)
    return dict(w_bf16=wb, amax=a)


def fp8_quantize_transpose(x, row=True, col=True):
    """Per-tensor FP8 (E4M3, s_enc = 448 / amax) of x [R, C] and of x^T.

    Returns a dict with row_codes [R, C], col_codes [C, R] (None when skipped)
    and amax (f32 [1])."""
    x = _check_input(x)
    R, C = x.shape
    rc = _u8((R, C), x.device) if row else None
    cc = _u8((C, R), x.device) if col else None
    amax = torch.empty(1, dtype=torch.float32, device=x.device)
    st = lib().fp8_quantize_transpose(_ptr(x), R, C, _ptr(rc), _ptr(cc), _ptr(amax), _stream(x.device))
    _check("fp8_quantize_transpose", st)
    return dict(row_codes=rc, col_codes=cc, amax=amax)


def bs_gemm(fmt, a_codes, a_scales, b_codes, b_scales, a_amax=None, b_amax=None, K=None, out=None):
    """C [M, N] bf16 = alpha * deq(A) . deq(B)^T with A, B K-major block-scaled operands
    (per-tensor "fp8": scales None, amaxes required)."""
    if fmt not in FORMATS:
        raise ValueError(f"unknown format {fmt!r}")
    if K is None and isinstance(a_codes, torch.Tensor) and a_codes.dim() == 2:
        K = a_codes.shape[1] * (1 if fmt in ("mxfp8", "fp8") else 2)
    K = int(K)
    _check_operand("A", a_codes, a_scales, K, fmt)
    _check_operand("B", b_codes, b_scales, K, fmt)
    if fmt in ("nvfp4", "fp8") and (a_amax is None or b_amax is None):
        raise ValueError(f"{fmt} needs both per-tensor amaxes")
    _check_amax(a_amax, b_amax)
    M, N = a_codes.shape[0], b_codes.shape[0]
    if out is not None:
        _check_out(out, M, N, torch.bfloat16)
    _check_device(a_codes, a_scales, b_codes, b_scales, a_amax, b_amax, out=out)
    dev = a_codes.device
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ldc = out.stride(0) if out.dim() == 2 else N
    st = lib().bs_gemm(FORMATS[fmt], M, N, int(K), _ptr(a_codes), _ptr(a_scales), _ptr(a_amax),
                       _ptr(b_codes), _ptr(b_scales), _ptr(b_amax), _ptr(out), ldc, _stream(dev))
    _check("bs_gemm", st)
    return out


def bs_gemm_noalloc(fmt, a_codes, a_scales, b_codes, b_scales, a_amax, b_amax, out, K=None):
    """bs_gemm into a caller-provided `out`, through the entry point that
    allocates no device memory (its NVFP4 workspace is the library's static
    per-device array; overlapping calls on one device race)."""
    if fmt not in FORMATS:
        raise ValueError(f"unknown format {fmt!r}")
    if K is None and isinstance(a_codes, torch.Tensor) and a_codes.dim() == 2:
        K = a_codes.shape[1] * (1 if fmt in ("mxfp8", "fp8") else 2)
    K = int(K)
    _check_operand("A", a_codes, a_scales, K, fmt)
    _check_operand("B", b_codes, b_scales, K, fmt)
    if fmt in ("nvfp4", "fp8") and (a_amax is None or b_amax is None):
        raise ValueError(f"{fmt} needs both per-tensor amaxes")
    _check_amax(a_amax, b_amax)
    M, N = a_codes.shape[0], b_codes.shape[0]
    _check_out(out, M, N, torch.bfloat16)
    _check_device(a_codes, a_scales, b_codes, b_scales, a_amax, b_amax, out=out)
    ldc = out.stride(0) if out.dim() == 2 else N
    st = lib().bs_gemm_noalloc(FORMATS[fmt], M, N, K, _ptr(a_codes), _ptr(a_scales), _ptr(a_amax),
                               _ptr(b_codes), _ptr(b_scales), _ptr(b_amax), _ptr(out), ldc,
                               _stream(out.device))
    _check("bs_gemm_noalloc", st)
    return out


# Largest FP16 B operand worth pre-expanding.  Zero: since the register-
# expansion GEMM (K % 256 == 0) expands in the tile faster than the
# pre-expanded-B kernel streams FP16, no Llama MLP GEMM gains from it
# (measured in the 8B step: FPROP_down 1549 against 1345 TF/s, DGRAD_down
# 1437 against 1264).  bs_gemm_nvfp4_bx stays available for callers that keep
# an expanded weight anyway.
BX_MAX_BYTES = 0


def bx_pays(N, K):
    """Whether a GEMM should take its B operand pre-expanded (nvfp4_expand +
    bs_gemm_nvfp4_bx) rather than expand it inside every output tile: when the
    FP16 copy of B is at most BX_MAX_BYTES (see there; currently never)."""
    return N * K * 2 <= BX_MAX_BYTES and K % 128 == 0


def nvfp4_expand(codes, scales, K=None, out=None):
    """FP16 [R, K] expansion v * S * 2^-7 of NVFP4 codes [R, K/2] + scales [R, K/16]."""
    if K is None and isinstance(codes, torch.Tensor) and codes.dim() == 2:
        K = codes.shape[1] * 2
    K = int(K)
    _check_operand("expand", codes, scales, K, "nvfp4")
    R = codes.shape[0]
    if out is not None:
        _check_out(out, R, K, torch.float16)
    _check_device(codes, scales, out)
    if out is None:
        out = torch.empty((R, K), dtype=torch.float16, device=codes.device)
    st = lib().nvfp4_expand(_ptr(codes), _ptr(scales), R, int(K), _ptr(out), _stream(codes.device))
    _check("nvfp4_expand", st)
    return out


def bs_gemm_nvfp4_bx(a_codes, a_scales, a_amax, b_x, b_amax, out=None):
    """C [M, N] bf16 of NVFP4 A (codes, scales, amax) and FP16-expanded B [N, K]."""
    if not (isinstance(b_x, torch.Tensor) and b_x.dtype == torch.float16 and b_x.dim() == 2):
        raise ValueError("b_x must be a 2-D float16 tensor (nvfp4_expand of B)")
    N, K = b_x.shape
    _check_operand("A", a_codes, a_scales, K, "nvfp4")
    if a_amax is None or b_amax is None:
        raise ValueError("nvfp4 needs both per-tensor amaxes")
    _check_amax(a_amax, b_amax)
    M = a_codes.shape[0]
    if out is not None:
        _check_out(out, M, N, torch.bfloat16)
    _check_device(a_codes, a_scales, a_amax, b_x, b_amax, out=out)
    dev = a_codes.device
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ldc = out.stride(0) if out.dim() == 2 else N
    st = lib().bs_gemm_nvfp4_bx(M, N, int(K), _ptr(a_codes), _ptr(a_scales), _ptr(a_amax), _ptr(b_x),
                                _ptr(b_amax), _ptr(out), ldc, _stream(dev))
    _check("bs_gemm_nvfp4_bx", st)
    return out
