"""GPU parity of the pre-expanded-B NVFP4 GEMM route.

* nvfp4_expand of the oracle's NVFP4 bytes against the oracle's dequantized
  values: out = v * S * 2^-7, exact in FP16, so bit for bit.
* bs_gemm_nvfp4_bx bit for bit against bs_gemm("nvfp4") on the same operands
  (the oracle's NVFP4 bytes)
  (the same FP16 values meet the same MFMA sequence), ragged M and N included,
  and within the GEMM tolerance rule against the oracle's FP64 product; the
  full 8B FPROP_gu shape compared whole against bs_gemm.
"""

import numpy as np
import pytest
import torch

import fp8_quantized_gemm_amd as bsq
from fp8_quantized_gemm_amd import synth
from oracle import gemm as G
from oracle import quantize as Q

from _gpu import announce, bits, gpu

pytestmark = gpu


@pytest.mark.parametrize("R,K,br", [(16, 16, 1), (64, 272, 1), (256, 4096, 16), (48, 1024, 16)])
def test_nvfp4_expand_exact(R, K, br):
    announce("nvfp4 expand", R, K, br)
    x = synth.bf16_tensor((R, K), 9500 + R + K, 0.02 if br == 16 else 1.0, br == 1)
    codes, scales, _ = Q.nvfp4_quantize(bits(x), br)            # the oracle's operand bytes
    out = bsq.nvfp4_expand(_dev(codes), _dev(scales))
    torch.cuda.synchronize()
    deq = G.dequant_nvfp4(codes, scales)
    want = (deq * 2.0 ** -7).astype(np.float16)
    assert np.array_equal(want.astype(np.float64) * 2.0 ** 7, deq)   # exact in FP16
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint16), want.view(np.uint16))


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _operands(M, N, K, seed):
    """NVFP4 operands quantized by the oracle (A 1x16, B 16x16 when N % 16 == 0),
    as numpy arrays and as device tensors."""
    A = synth.bf16_tensor((M, K), seed, 1.0, True)
    B = synth.bf16_tensor((N, K), seed + 1, 0.02, False)
    a = Q.nvfp4_quantize(bits(A), 1)
    b = Q.nvfp4_quantize(bits(B), 16 if N % 16 == 0 else 1)
    dev = lambda q: (_dev(q[0]), _dev(q[1]), _dev(np.array([q[2]], dtype=np.float32)))
    return a, b, dev(a), dev(b)


@pytest.mark.parametrize("M,N,K", [(256, 256, 128), (512, 768, 1024), (304, 520, 256),
                                   (64, 48, 4096), (1024, 256, 640)])
def test_gemm_bx_equals_gemm(M, N, K):
    announce("gemm bx", M, N, K)
    a, b, (ac, as_, aa), (bc, bs, ba) = _operands(M, N, K, 9600 + M + N + K)
    c_ref = bsq.bs_gemm("nvfp4", ac, as_, bc, bs, aa, ba)
    bx = bsq.nvfp4_expand(bc, bs)
    c = bsq.bs_gemm_nvfp4_bx(ac, as_, aa, bx, ba)
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int16), c_ref.view(torch.int16))
    rep = G.tolerance_report(c.double().cpu().numpy(), G.gemm_nvfp4(a[0], a[1], a[2], b[0], b[1], b[2]))
    print(M, N, K, rep)
    assert rep["passed"], rep


def test_gemm_bx_rejects_unsupported_k():
    announce("gemm bx unsupported K")
    _, _, (ac, as_, aa), (bc, bs, ba) = _operands(64, 64, 96, 9700)
    bx = bsq.nvfp4_expand(bc, bs)
    with pytest.raises(bsq.BsqError) as e:
        bsq.bs_gemm_nvfp4_bx(ac, as_, aa, bx, ba)
    assert e.value.status == bsq.BSQ_EUNSUPPORTED


def test_gemm_bx_8b_fprop_gu_full_size():
    """FPROP_gu of the 8B MLP (32768 x 28672 x 4096) with the weight
    pre-expanded: the whole output equals bs_gemm's bit for bit."""
    announce("gemm bx 8b FPROP_gu")
    X = synth.workload_tensor("8b", "X", "cuda")
    W = synth.workload_tensor("8b", "W_gu", "cuda")
    qx = bsq.quantize_transpose(X, rht_col=False, col=False)
    qw = bsq.quantize_transpose(W, block_rows=16, col=False)
    c_ref = bsq.bs_gemm("nvfp4", qx["row_codes"], qx["row_scales"], qw["row_codes"], qw["row_scales"],
                        qx["row_amax"], qw["row_amax"])
    wx = bsq.nvfp4_expand(qw["row_codes"], qw["row_scales"])
    c = bsq.bs_gemm_nvfp4_bx(qx["row_codes"], qx["row_scales"], qx["row_amax"], wx, qw["row_amax"])
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int16), c_ref.view(torch.int16))
