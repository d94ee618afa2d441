"""GPU parity of bs_gemm against the oracle's FP64 product of dequantized
operands, within max(|err| - ulp_bf16/2) <= 1e-2 * rms(C_ref).

The oracle always quantizes the same BF16 inputs itself (or reads the same
seeded random code bytes); nothing it consumes comes from the GPU."""

import numpy as np
import pytest
import torch

import fp8_quantized_gemm_amd as bsq
from fp8_quantized_gemm_amd import synth
from oracle import gemm as G
from oracle import quantize as Q

from _gpu import announce, assert_bytes_equal, bits, gpu, u8

pytestmark = gpu

TOL = 1e-2


def _c64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _check(c_gpu, c_ref, what):
    rep = G.tolerance_report(_c64(c_gpu), c_ref)
    print(what, {k: (round(v, 6) if isinstance(v, float) else v) for k, v in rep.items()})
    assert rep["passed"], (what, rep)
    return rep


def test_tiny_nvfp4_fprop_pipeline():
    """A [256, 256] 1x16 RNE, W [256, 256] 16x16, C = A . W^T."""
    announce("tiny nvfp4 fprop")
    A = synth.workload_tensor("tiny", "A", "cuda")
    W = synth.workload_tensor("tiny", "W", "cuda")
    ac, as_, aa = bsq.nvfp4_quantize(A, 1)
    wc, ws, wa = bsq.nvfp4_quantize(W, 16)
    C = bsq.bs_gemm("nvfp4", ac, as_, wc, ws, aa, wa)
    torch.cuda.synchronize()
    oac, oas, oaa = Q.nvfp4_quantize(bits(A), 1)
    owc, ows, owa = Q.nvfp4_quantize(bits(W), 16)
    assert_bytes_equal(u8(ac), oac, "A codes")
    assert_bytes_equal(u8(wc), owc, "W codes")
    ref = G.gemm_nvfp4(oac, oas, oaa, owc, ows, owa)
    rep = _check(C, ref, "tiny")
    assert rep["frac_equal_rne"] > 0.99


@pytest.mark.parametrize("M", [16, 48, 256, 300])
@pytest.mark.parametrize("N", [16, 48, 256, 272])
@pytest.mark.parametrize("K", [32, 64, 128, 160, 256, 384, 512, 4096])
def test_nvfp4_shape_sweep(M, N, K):
    announce("nvfp4 sweep", M, N, K)
    A = synth.bf16_tensor((M, K), 1000 + M + K, device="cuda")
    B = synth.bf16_tensor((N, K), 2000 + N + K, sigma=0.02, outliers=False, device="cuda")
    ac, as_, aa = bsq.nvfp4_quantize(A, 1)
    bc, bs, ba = bsq.nvfp4_quantize(B, 1)
    C = bsq.bs_gemm("nvfp4", ac, as_, bc, bs, aa, ba)
    torch.cuda.synchronize()
    oac, oas, oaa = Q.nvfp4_quantize(bits(A), 1)
    obc, obs, oba = Q.nvfp4_quantize(bits(B), 1)
    _check(C, G.gemm_nvfp4(oac, oas, oaa, obc, obs, oba), f"nvfp4 {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(300, 520, 768), (512, 272, 1280), (560, 768, 1792)])
def test_nvfp4_odd_pair_counts(M, N, K):
    """K = 768, 1280, 1792: 3, 5 and 7 pairs of 128-element K units, so the
    register-expansion kernel's last pair lands in the other of its two pair
    buffers than with the even pair counts of the other shapes; several
    waves of ragged tiles; run twice, bit-identical."""
    announce("nvfp4 odd pairs", M, N, K)
    A = synth.bf16_tensor((M, K), 3000 + M + K, device="cuda")
    B = synth.bf16_tensor((N, K), 4000 + N + K, sigma=0.02, outliers=False, device="cuda")
    ac, as_, aa = bsq.nvfp4_quantize(A, 1)
    bc, bs, ba = bsq.nvfp4_quantize(B, 1)
    C = bsq.bs_gemm("nvfp4", ac, as_, bc, bs, aa, ba)
    C2 = bsq.bs_gemm("nvfp4", ac, as_, bc, bs, aa, ba)
    torch.cuda.synchronize()
    assert torch.equal(C.view(torch.int16), C2.view(torch.int16))
    oac, oas, oaa = Q.nvfp4_quantize(bits(A), 1)
    obc, obs, oba = Q.nvfp4_quantize(bits(B), 1)
    _check(C, G.gemm_nvfp4(oac, oas, oaa, obc, obs, oba), f"nvfp4 {M}x{N}x{K}")


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("M,N,K", [(16, 16, 32), (48, 272, 96), (256, 256, 256), (512, 768, 384),
                                   (300, 48, 4096),
                                   # staged kernel (K % 512 == 0): fewest stages (one scale
                                   # period), ragged tiles, and an odd number of periods
                                   (256, 256, 512), (520, 300, 512), (768, 1024, 1536)])
def test_mx_shape_sweep(fmt, M, N, K):
    announce("mx sweep", fmt, M, N, K)
    A = synth.bf16_tensor((M, K), 3000 + M + K, device="cuda")
    B = synth.bf16_tensor((N, K), 4000 + N + K, device="cuda")
    ac, as_ = bsq.mx_quantize(A, fmt)
    bc, bs = bsq.mx_quantize(B, fmt)
    C = bsq.bs_gemm(fmt, ac, as_, bc, bs, K=K)
    torch.cuda.synchronize()
    oac, oas = Q.mx_quantize(bits(A), fmt)
    obc, obs = Q.mx_quantize(bits(B), fmt)
    _check(C, G.gemm_mx(oac, oas, obc, obs, fmt), f"{fmt} {M}x{N}x{K}")


def test_nvfp4_all_codes_and_scales():
    """Seeded random code bytes with every E2M1 code and every finite E4M3 scale."""
    announce("nvfp4 all codes/scales")
    rng = np.random.default_rng(42)
    M, N, K = 256, 256, 2048
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    bc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    as_ = rng.integers(0, 0x7F, (M, K // 16), dtype=np.uint8)       # 0 .. 0x7E
    bs = rng.integers(0, 0x7F, (N, K // 16), dtype=np.uint8)
    aa, ba = np.float32(2.5), np.float32(0.75)
    d = lambda a: torch.from_numpy(a).cuda()
    C = bsq.bs_gemm("nvfp4", d(ac), d(as_), d(bc), d(bs), d(np.array([aa])), d(np.array([ba])))
    torch.cuda.synchronize()
    _check(C, G.gemm_nvfp4(ac, as_, aa, bc, bs, ba), "nvfp4 all codes")


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_mx_all_codes(fmt):
    announce("mx all codes", fmt)
    rng = np.random.default_rng(43)
    M, N, K = 256, 256, 2048
    w = 2 if fmt == "mxfp4" else 1
    ac = rng.integers(0, 256, (M, K // w), dtype=np.uint8)
    bc = rng.integers(0, 256, (N, K // w), dtype=np.uint8)
    if fmt == "mxfp8":                      # no NaN codes
        ac[(ac & 0x7F) == 0x7F] = 0
        bc[(bc & 0x7F) == 0x7F] = 0
    as_ = rng.integers(117, 138, (M, K // 32), dtype=np.uint8)
    bs = rng.integers(117, 138, (N, K // 32), dtype=np.uint8)
    d = lambda a: torch.from_numpy(a).cuda()
    C = bsq.bs_gemm(fmt, d(ac), d(as_), d(bc), d(bs), K=K)
    torch.cuda.synchronize()
    _check(C, G.gemm_mx(ac, as_, bc, bs, fmt), f"{fmt} all codes")


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_mx_square_4096(fmt):
    """MX square GEMM, M = N = K = 4096, N(0,1) with 0.1% outliers x50."""
    announce("mx 4096^3", fmt)
    A = synth.workload_tensor("mx", "A", "cuda")
    B = synth.workload_tensor("mx", "B", "cuda")
    ac, as_ = bsq.mx_quantize(A, fmt)
    bc, bs = bsq.mx_quantize(B, fmt)
    C = bsq.bs_gemm(fmt, ac, as_, bc, bs, K=4096)
    torch.cuda.synchronize()
    oac, oas = Q.mx_quantize(bits(A), fmt)
    obc, obs = Q.mx_quantize(bits(B), fmt)
    assert_bytes_equal(u8(as_), oas, "A scales")
    assert_bytes_equal(u8(ac), oac, "A codes")
    rep = _check(C, G.gemm_mx(oac, oas, obc, obs, fmt), f"{fmt} 4096^3")
    # FP32 accumulation over K = 4096 wide-range products flips a few BF16 roundings
    assert rep["frac_equal_rne"] > 0.95


def test_nvfp4_split_last_wave():
    """A GEMM whose last wave of 256 x 256 tiles would leave most compute
    units idle: 16 tile rows and one tile column more than a wave, so the
    last wave holds 16 tiles, each computed as two K halves and joined
    (ragged M and N: the edge tiles are among them).  Whole output against
    the oracle, and a second launch must give the same bits."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tiles_n = cus // 16 + 1
    M, N, K = 16 * 256 - 24, tiles_n * 256 - 40, 4096
    announce("nvfp4 split last wave", M, N, K, "cus", cus)
    A = synth.bf16_tensor((M, K), 4100, device="cuda")
    B = synth.bf16_tensor((N, K), 4101, sigma=0.02, outliers=False, device="cuda")
    ac, as_, aa = bsq.nvfp4_quantize(A, 1)
    bc, bs, ba = bsq.nvfp4_quantize(B, 1)
    C = bsq.bs_gemm("nvfp4", ac, as_, bc, bs, aa, ba)
    C2 = bsq.bs_gemm("nvfp4", ac, as_, bc, bs, aa, ba)
    torch.cuda.synchronize()
    assert torch.equal(C.view(torch.int16), C2.view(torch.int16)), "second launch differs"
    oac, oas, oaa = Q.nvfp4_quantize(bits(A), 1)
    obc, obs, oba = Q.nvfp4_quantize(bits(B), 1)
    rep = _check(C, G.gemm_nvfp4(oac, oas, oaa, obc, obs, oba), f"nvfp4 split {M}x{N}x{K}")
    assert rep["frac_equal_rne"] > 0.95


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4", "mxfp8"])
def test_multi_wave_odd_row_stride(fmt):
    """More tiles than one wave, written into a column slice of a wider
    tensor (row stride N + 3, so every epilogue takes its element-wise store
    path): NVFP4 with a split last wave (its join too), MX on the four-wave
    kernel.  Whole output against the oracle; the three padding columns keep
    their value."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if fmt == "nvfp4":
        M, N, K = 16 * 256 - 24, (cus // 16 + 1) * 256 - 40, 4096
    else:
        M, N, K = 17 * 256 - 8, 17 * 256 - 24, 1024
    announce("multi-wave odd ldc", fmt, M, N, K)
    A = synth.bf16_tensor((M, K), 4200 + M, device="cuda")
    B = synth.bf16_tensor((N, K), 4300 + N, sigma=0.02, outliers=False, device="cuda")
    wide = torch.full((M, N + 3), 5.0, dtype=torch.bfloat16, device="cuda")
    out = wide[:, :N]
    if fmt == "nvfp4":
        ac, as_, aa = bsq.nvfp4_quantize(A, 1)
        bc, bs, ba = bsq.nvfp4_quantize(B, 1)
        bsq.bs_gemm("nvfp4", ac, as_, bc, bs, aa, ba, out=out)
        oac, oas, oaa = Q.nvfp4_quantize(bits(A), 1)
        obc, obs, oba = Q.nvfp4_quantize(bits(B), 1)
        ref = G.gemm_nvfp4(oac, oas, oaa, obc, obs, oba)
    else:
        ac, as_ = bsq.mx_quantize(A, fmt)
        bc, bs = bsq.mx_quantize(B, fmt)
        bsq.bs_gemm(fmt, ac, as_, bc, bs, K=K, out=out)
        oac, oas = Q.mx_quantize(bits(A), fmt)
        obc, obs = Q.mx_quantize(bits(B), fmt)
        ref = G.gemm_mx(oac, oas, obc, obs, fmt)
    torch.cuda.synchronize()
    assert bool((wide[:, N:] == 5.0).all()), "padding columns written"
    _check(out, ref, f"{fmt} {M}x{N}x{K} ldc {N + 3}")


def test_ldc_and_k_zero():
    announce("ldc / K=0")
    A = synth.bf16_tensor((64, 64), 5, device="cuda")
    ac, as_, aa = bsq.nvfp4_quantize(A)
    big = torch.full((64, 100), 7.0, dtype=torch.bfloat16, device="cuda")
    bsq.bs_gemm("nvfp4", ac, as_, ac, as_, aa, aa, out=big[:, 10:74])
    z = torch.full((8, 8), 7.0, dtype=torch.bfloat16, device="cuda")
    e = torch.empty((8, 0), dtype=torch.uint8, device="cuda")
    bsq.bs_gemm("nvfp4", e, e, e, e, aa, aa, K=0, out=z)
    torch.cuda.synchronize()
    oc, os_, oa = Q.nvfp4_quantize(bits(A))
    ref = G.gemm_nvfp4(oc, os_, oa, oc, os_, oa)
    _check(big[:, 10:74], ref, "ldc")
    assert bool((big[:, :10] == 7.0).all()) and bool((big[:, 74:] == 7.0).all())
    assert bool((z == 0).all())


def test_nvfp4_tiny_scales_subnormal_products():
    """E4M3 scales 2^-9 .. 2^-5: the exact FP16 products inside the GEMM are FP16
    subnormals; they must not be flushed."""
    announce("nvfp4 tiny scales")
    rng = np.random.default_rng(44)
    M, N, K = 64, 64, 512
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    bc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    as_ = rng.integers(1, 0x10, (M, K // 16), dtype=np.uint8)     # subnormal and smallest normal E4M3
    bs = rng.integers(1, 0x10, (N, K // 16), dtype=np.uint8)
    aa = ba = np.float32(2688.0)                                    # s_dec = 1
    d = lambda a: torch.from_numpy(a).cuda()
    C = bsq.bs_gemm("nvfp4", d(ac), d(as_), d(bc), d(bs), d(np.array([aa])), d(np.array([ba])))
    torch.cuda.synchronize()
    ref = G.gemm_nvfp4(ac, as_, aa, bc, bs, ba)
    rep = _check(C, ref, "nvfp4 tiny scales")
    assert rep["frac_equal_rne"] > 0.99


@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (1, 5, 48), (7, 1, 128), (3, 300, 16), (257, 1, 512)])
@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4", "mxfp8"])
def test_degenerate_shapes(fmt, M, N, K):
    """Single rows or columns and the smallest K of each format (one block)."""
    if fmt != "nvfp4" and K % 32 != 0:
        K = 32
    announce("degenerate", fmt, M, N, K)
    A = synth.bf16_tensor((M, K), 3000 + M + K, device="cuda")
    B = synth.bf16_tensor((N, K), 4000 + N + K, sigma=0.02, outliers=False, device="cuda")
    if fmt == "nvfp4":
        ac, as_, aa = bsq.nvfp4_quantize(A, 1)
        bc, bs, ba = bsq.nvfp4_quantize(B, 1)
        C = bsq.bs_gemm(fmt, ac, as_, bc, bs, aa, ba)
        oac, oas, oaa = Q.nvfp4_quantize(bits(A), 1)
        obc, obs, oba = Q.nvfp4_quantize(bits(B), 1)
        ref = G.gemm_nvfp4(oac, oas, oaa, obc, obs, oba)
    else:
        ac, as_ = bsq.mx_quantize(A, fmt)
        bc, bs = bsq.mx_quantize(B, fmt)
        C = bsq.bs_gemm(fmt, ac, as_, bc, bs, K=K)
        oac, oas = Q.mx_quantize(bits(A), fmt)
        obc, obs = Q.mx_quantize(bits(B), fmt)
        ref = G.gemm_mx(oac, oas, obc, obs, fmt)
    torch.cuda.synchronize()
    assert C.shape == (M, N)
    _check(C, ref, f"{fmt} {M}x{N}x{K}")
