"""GPU parity of the per-tensor FP8 baseline (E4M3 under s_enc = 448 / amax):
fp8_quantize_transpose bit for bit against the oracle (codes of x and of x^T,
amax), and bs_gemm("fp8") against the oracle's FP64 product within
max(|err| - ulp_bf16/2) <= 1e-2 * rms(C_ref).  The oracle quantizes the same
BF16 inputs itself; nothing it consumes comes from the GPU."""

import numpy as np
import pytest
import torch

import fp8_quantized_gemm_amd as bsq
from fp8_quantized_gemm_amd import synth
from oracle import gemm as G
from oracle import quantize as Q

from _gpu import announce, assert_bytes_equal, bits, f32, gpu, u8

pytestmark = gpu


def _check(c_gpu, c_ref, what):
    rep = G.tolerance_report(c_gpu.float().cpu().numpy().astype(np.float64), c_ref)
    print(what, {k: (round(v, 6) if isinstance(v, float) else v) for k, v in rep.items()})
    assert rep["passed"], (what, rep)


# (rows, cols, sigma, outliers): 256-multiples take the tile kernel, the rest the flat one
@pytest.mark.parametrize("R,C,sigma,outl", [(256, 256, 1.0, True), (512, 768, 1e-3, False),
                                            (48, 80, 1.0, True), (272, 528, 30.0, True),
                                            (256, 512, 1e-30, False), (16, 16, 1.0, False)])
def test_fp8_quantize_transpose(R, C, sigma, outl):
    announce("fp8 qt", R, C, sigma)
    x = synth.bf16_tensor((R, C), 7000 + R + C, sigma, outl, device="cuda")
    d = bsq.fp8_quantize_transpose(x)
    torch.cuda.synchronize()
    ref = Q.fp8_quantize_transpose(bits(x))
    assert f32(d["amax"])[0] == ref["amax"]
    assert_bytes_equal(u8(d["row_codes"]), ref["row_codes"], "row codes")
    assert_bytes_equal(u8(d["col_codes"]), ref["col_codes"], "col codes")


@pytest.mark.parametrize("row,col", [(True, False), (False, True)])
def test_fp8_quantize_one_orientation(row, col):
    announce("fp8 qt one side", row, col)
    x = synth.bf16_tensor((256, 512), 7101, device="cuda")
    d = bsq.fp8_quantize_transpose(x, row=row, col=col)
    torch.cuda.synchronize()
    ref = Q.fp8_quantize_transpose(bits(x))
    assert f32(d["amax"])[0] == ref["amax"]
    if row:
        assert d["col_codes"] is None
        assert_bytes_equal(u8(d["row_codes"]), ref["row_codes"], "row codes")
    else:
        assert d["row_codes"] is None
        assert_bytes_equal(u8(d["col_codes"]), ref["col_codes"], "col codes")


# (M, N, K): K % 64 == 0 takes the ping-pong kernel, other multiples of 32 the generic one
@pytest.mark.parametrize("M,N,K", [(256, 256, 512), (304, 208, 64), (512, 768, 1024),
                                   (64, 48, 4096), (128, 96, 96), (48, 272, 160)])
def test_fp8_gemm(M, N, K):
    announce("fp8 gemm", M, N, K)
    A = synth.bf16_tensor((M, K), 7200 + M + K, device="cuda")
    B = synth.bf16_tensor((N, K), 7300 + N + K, 0.02, False, device="cuda")
    a = bsq.fp8_quantize_transpose(A, col=False)
    b = bsq.fp8_quantize_transpose(B, col=False)
    C = bsq.bs_gemm("fp8", a["row_codes"], None, b["row_codes"], None, a["amax"], b["amax"], K=K)
    torch.cuda.synchronize()
    ra = Q.fp8_quantize_transpose(bits(A))
    rb = Q.fp8_quantize_transpose(bits(B))
    _check(C, G.gemm_fp8(ra["row_codes"], ra["amax"], rb["row_codes"], rb["amax"]), f"fp8 {M}x{N}x{K}")


def test_fp8_zero_tensor_and_empty_k():
    """All-zero input: amax 0, s_enc 1, all codes 0 (the oracle agrees); a GEMM
    with K = 0 writes zeros."""
    announce("fp8 zero / K=0")
    x = torch.zeros((256, 256), dtype=torch.bfloat16, device="cuda")
    d = bsq.fp8_quantize_transpose(x)
    torch.cuda.synchronize()
    ref = Q.fp8_quantize_transpose(bits(x))
    assert f32(d["amax"])[0] == 0.0 == ref["amax"]
    assert_bytes_equal(u8(d["row_codes"]), ref["row_codes"], "row codes")
    assert not u8(d["col_codes"]).any()
    c0 = torch.full((32, 48), 3.0, dtype=torch.bfloat16, device="cuda")
    codes = torch.zeros((48, 0), dtype=torch.uint8, device="cuda")
    out = bsq.bs_gemm("fp8", codes[:32], None, codes, None, d["amax"], d["amax"], K=0, out=c0)
    torch.cuda.synchronize()
    assert not out.float().any()


def test_fp8_wgrad_from_column_outputs():
    """WGRAD-shaped use: both operands from the column (x^T) outputs."""
    announce("fp8 wgrad")
    T, Fo, H = 512, 384, 256
    dY = synth.bf16_tensor((T, Fo), 7401, 1e-3, False, device="cuda")
    X = synth.bf16_tensor((T, H), 7402, device="cuda")
    a = bsq.fp8_quantize_transpose(dY, row=False)
    b = bsq.fp8_quantize_transpose(X, row=False)
    C = bsq.bs_gemm("fp8", a["col_codes"], None, b["col_codes"], None, a["amax"], b["amax"], K=T)
    torch.cuda.synchronize()
    ra = Q.fp8_quantize_transpose(bits(dY))
    rb = Q.fp8_quantize_transpose(bits(X))
    _check(C, G.gemm_fp8(ra["col_codes"], ra["amax"], rb["col_codes"], rb["amax"]), "fp8 wgrad")


def test_fp8_gemm_8b_fprop_gu_sampled():
    """The 8B FPROP_gu shape (32768 x 28672 x 4096) at full size; the oracle
    recomputes 128 sampled output rows across every column (every N tile)."""
    announce("fp8 8b FPROP_gu sampled")
    X = synth.workload_tensor("8b", "X", "cuda")
    W = synth.workload_tensor("8b", "W_gu", "cuda")
    a = bsq.fp8_quantize_transpose(X, col=False)
    b = bsq.fp8_quantize_transpose(W, col=False)
    C = bsq.bs_gemm("fp8", a["row_codes"], None, b["row_codes"], None, a["amax"], b["amax"])
    torch.cuda.synchronize()
    xb = X.cpu().view(torch.int16).numpy().view(np.uint16)
    wb = W.cpu().view(torch.int16).numpy().view(np.uint16)
    ax, aw = Q.tensor_amax(Q.as_f32(xb)), Q.tensor_amax(Q.as_f32(wb))
    assert f32(a["amax"])[0] == ax and f32(b["amax"])[0] == aw
    rows = np.sort(np.random.default_rng(11).choice(X.shape[0], 128, replace=False))
    xr, _ = Q.fp8_quantize(xb[rows], ax)
    wall, _ = Q.fp8_quantize(wb, aw)
    ridx = torch.from_numpy(rows).cuda()
    assert_bytes_equal(u8(a["row_codes"][ridx]), xr, "X sampled rows")
    assert_bytes_equal(u8(b["row_codes"]), wall, "W codes")
    _check(C[ridx], G.gemm_fp8(xr, ax, wall, aw), "fp8 8b FPROP_gu sampled rows")
