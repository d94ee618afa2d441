"""The entry point that allocates no device memory (bs_gemm_noalloc) against
bs_gemm on the same operands, through the C ABI: two calls in a row, the
second on smaller operands, both NVFP4 GEMMs whose last wave of tiles is
split over K (so the library's static workspace is used and reused).  Same
kernels and split, so the outputs must be equal bit for bit."""

import torch

import fp8_quantized_gemm_amd as bsq
from fp8_quantized_gemm_amd import synth

from _gpu import announce, gpu

pytestmark = gpu


def _operands(M, N, K, seed):
    A = synth.bf16_tensor((M, K), seed, device="cuda")
    B = synth.bf16_tensor((N, K), seed + 1, sigma=0.02, outliers=False, device="cuda")
    return bsq.nvfp4_quantize(A, 1), bsq.nvfp4_quantize(B, 1)


def test_noalloc_gemm_matches_bs_gemm_twice():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    # 16 tile rows x (cus / 16 + 1) tile columns: a last wave of 16 split tiles;
    # then 8 x (cus / 8 + 1): 8 split tiles, fewer operand bytes, smaller K
    shapes = [(16 * 256 - 24, (cus // 16 + 1) * 256 - 40, 8192),
              (8 * 256 - 8, (cus // 8 + 1) * 256 - 8, 4096)]
    assert shapes[1][0] * shapes[1][2] + shapes[1][1] * shapes[1][2] < \
        shapes[0][0] * shapes[0][2] + shapes[0][1] * shapes[0][2]
    for i, (M, N, K) in enumerate(shapes):
        announce("gemm noalloc", i, M, N, K, "cus", cus)
        (ac, as_, aa), (bc, bs, ba) = _operands(M, N, K, 5200 + i)
        ref = bsq.bs_gemm("nvfp4", ac, as_, bc, bs, aa, ba)
        out = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda")
        bsq.bs_gemm_noalloc("nvfp4", ac, as_, bc, bs, aa, ba, out)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), (M, N, K)
        assert torch.isfinite(out.float()).all()
