"""Exhaustive and dense checks of the hardware converts the kernels rely on,
and the non-finite-input contract of include/bsq.h.

* nvfp4_expand on every code byte under every finite E4M3 scale, bit for bit
  against the oracle's dequantized values times 2^-7 (exact in FP16).
* The FP32 -> E2M1 and FP32 -> E4M3 converts, reached through the public
  quantizers and compared byte for byte with the oracle:
  - MXFP4 / MXFP8 on every finite BF16 value below the block maximum (with a
    block exponent of 0 the converted value is the input itself, so every
    BF16 value, the E2M1 / E4M3 ties included, meets the convert);
  - NVFP4 on a dense, stratified sweep: block amaxes log-uniform over 24
    binades below the tensor amax (the scale convert sees its whole range,
    subnormal E4M3 scales included), elements uniform in the block and
    clustered around every E2M1 decision point after scaling, under several
    tensor amaxes (so the encode factor takes many FP32 mantissas), RNE and
    stochastic rounding, row and column outputs.
* NaN and Inf inputs: every entry point returns BSQ_OK without a fault and a
  later call on finite data still matches the oracle.
"""

import numpy as np
import pytest
import torch

import fp8_quantized_gemm_amd as bsq
from oracle import formats as F
from oracle import gemm as G
from oracle import quantize as Q

from _gpu import announce, assert_bytes_equal, bits, f32, from_bits, gpu, u8

pytestmark = gpu


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _finite_bf16(max_bits):
    """Every finite BF16 bit pattern with magnitude bits <= max_bits, both signs."""
    mag = np.arange(0, max_bits + 1, dtype=np.uint16)
    return np.concatenate([mag, mag | np.uint16(0x8000)])


# ---------------------------------------------------------------- FP4 -> FP16 expansion

def test_nvfp4_expand_every_code_and_scale():
    """127 rows (one per finite E4M3 scale code 0..0x7E) x 512 elements: the
    256 code bytes in order, twice; every 16-element block of row r carries
    scale code r."""
    announce("nvfp4_expand exhaustive")
    codes = np.tile(np.arange(256, dtype=np.uint8), (127, 2))          # [127, 512] bytes
    scales = np.repeat(np.arange(127, dtype=np.uint8)[:, None], 1024 // 16, axis=1)
    out = bsq.nvfp4_expand(_dev(codes), _dev(scales))
    torch.cuda.synchronize()
    deq = G.dequant_nvfp4(codes, scales)
    want = (deq * 2.0 ** -7).astype(np.float16)
    assert np.array_equal(want.astype(np.float64) * 2.0 ** 7, deq)     # exact in FP16
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint16), want.view(np.uint16))


# ---------------------------------------------------------------- MX: every BF16 value

def _mx_blocks(vals, max_bits, rng):
    """Rows of 32-element blocks: the block maximum (max_bits) at a random
    position, 31 values from `vals` (shuffled, padded by repetition)."""
    vals = rng.permutation(vals)
    n = -(-len(vals) // 31) * 31
    vals = np.resize(vals, n).reshape(-1, 31)
    pos = rng.integers(0, 32, len(vals))
    out = np.empty((len(vals), 32), dtype=np.uint16)
    for i in range(len(vals)):
        out[i] = np.insert(vals[i], pos[i], np.uint16(max_bits))
    rows = -(-out.size // 256)
    flat = np.resize(out.ravel(), rows * 256)                 # whole 32-blocks (256 = 8 x 32)
    return flat.reshape(rows, 256)


@pytest.mark.parametrize("fmt,rnd,max_bits", [("mxfp4", "rne", 0x40FF), ("mxfp4", "sr", 0x40FF),
                                              ("mxfp8", "rne", 0x43F0)])
def test_mx_convert_every_bf16_value(fmt, rnd, max_bits):
    """Block maximum 7.97 (E2M1, emax 2) or 480 (E4M3, emax 8): the block
    exponent is 0, so v = x for every BF16 x up to that maximum."""
    announce("mx convert sweep", fmt, rnd)
    rng = np.random.default_rng(0x5EED + max_bits)
    xb = _mx_blocks(_finite_bf16(max_bits), max_bits, rng)
    oc, os_ = Q.mx_quantize(xb, fmt, rnd, seed=77, offset=2)
    assert np.all(os_ == 127)                                  # exponent 0 everywhere
    codes, scales = bsq.mx_quantize(from_bits(xb), fmt, rnd, seed=77, offset=2)
    torch.cuda.synchronize()
    assert_bytes_equal(u8(scales), os_, f"{fmt} scales")
    assert_bytes_equal(u8(codes), oc, f"{fmt} codes")


# ---------------------------------------------------------------- NVFP4: dense FP32 sweep

E2M1_DECISIONS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def _nvfp4_sweep(amax_bits, rows, cols, seed):
    """BF16 bits [rows, cols]: per 16-block an amax a_b = bf16(G * 2^-24w), w
    uniform in [0, 1]; the block's other 15 elements are a_b * u with u half
    uniform in (0, 1], half within 2^-6 (relative) of a decision point of
    E2M1 after the block scale (6 u near one of E2M1_DECISIONS); random
    signs; the tensor amax G placed once."""
    rng = np.random.default_rng(seed)
    g = F.bf16_bits_to_f32(np.array([amax_bits], dtype=np.uint16))[0]
    nblk = rows * cols // 16
    ab = g * np.exp2(-24.0 * rng.random(nblk))
    uni = rng.random((nblk, 15))
    near = E2M1_DECISIONS[rng.integers(0, 7, (nblk, 15))] / 6 * (1 + (rng.random((nblk, 15)) - 0.5) * 2 ** -5)
    u = np.where(rng.random((nblk, 15)) < 0.5, uni, np.minimum(near, 1.0))
    x = np.concatenate([ab[:, None], ab[:, None] * u], axis=1)
    x *= np.where(rng.random(x.shape) < 0.5, -1.0, 1.0)
    perm = rng.permuted(np.tile(np.arange(16), (nblk, 1)), axis=1)      # amax position per block
    x = np.take_along_axis(x, perm, axis=1)
    xb = torch.from_numpy(x.astype(np.float32).reshape(rows, cols)).to(torch.bfloat16)
    xb = xb.view(torch.int16).numpy().view(np.uint16).copy()
    xb[rows // 2, cols // 2] = amax_bits
    return xb


@pytest.mark.parametrize("amax_bits", [0x3F80, 0x4049, 0x42C7, 0x3A83, 0x4F12, 0x2E5B])
def test_nvfp4_convert_dense_sweep(amax_bits):
    """Rowwise RNE and SR through nvfp4_quantize, and both orientations
    (column SR with RHT) through quantize_transpose, against the oracle."""
    announce("nvfp4 convert sweep", hex(amax_bits))
    xb = _nvfp4_sweep(amax_bits, 512, 1024, amax_bits)
    x = from_bits(xb)
    for rnd in ("rne", "sr"):
        codes, scales, amax = bsq.nvfp4_quantize(x, 1, rnd, seed=amax_bits, offset=9)
        torch.cuda.synchronize()
        oc, os_, oa = Q.nvfp4_quantize(xb, 1, rnd, amax_bits, 9)
        assert f32(amax)[0] == oa
        assert_bytes_equal(u8(scales), os_, f"{rnd} scales")
        assert_bytes_equal(u8(codes), oc, f"{rnd} codes")
    q = bsq.quantize_transpose(x, "nvfp4", 1, "sr", seed=5, offset=1, rht_col=True, rht_signs=0x6A5C)
    torch.cuda.synchronize()
    ref = Q.quantize_transpose(xb, "nvfp4", 1, "sr", 5, 1, rht_col=True, rht_signs=0x6A5C)
    for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
        assert_bytes_equal(u8(q[k]), ref[k], k)
    assert f32(q["col_amax"])[0] == ref["col_amax"]


def test_nvfp4_2d_convert_dense_sweep():
    announce("nvfp4 2D convert sweep")
    xb = _nvfp4_sweep(0x3C23, 512, 512, 91)
    codes, scales, amax = bsq.nvfp4_quantize(from_bits(xb), 16)
    torch.cuda.synchronize()
    oc, os_, oa = Q.nvfp4_quantize(xb, 16)
    assert f32(amax)[0] == oa
    assert_bytes_equal(u8(scales), os_, "scales")
    assert_bytes_equal(u8(codes), oc, "codes")


# ---------------------------------------------------------------- NaN / Inf inputs

NONFINITE = np.array([0x7FC0, 0x7F81, 0x7F80, 0xFF80, 0xFFC1, 0xFFFF], dtype=np.uint16)


def _with_nonfinite(shape, seed):
    rng = np.random.default_rng(seed)
    x = bits(torch.randn(shape, generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16))
    x = x.copy()
    idx = rng.choice(x.size, 64, replace=False)
    x.ravel()[idx] = NONFINITE[rng.integers(0, len(NONFINITE), 64)]
    return x


@pytest.mark.parametrize("shape", [(256, 512), (48, 160)])
def test_nonfinite_inputs_never_fault(shape):
    """How non-finite values flow through the kernels (read from the code):
    * amax passes and fused amaxes take an unsigned max of the magnitude
      bits, so a NaN or Inf input makes the per-tensor amax NaN or Inf; the
      encode factor s_enc = min(2688 / amax, FLT_MAX) is then FLT_MAX or 0;
    * the E4M3 block-scale code is the hardware convert of min(sf, 448) and
      is masked to 7 bits, so the 128-entry table of encode factors is always
      indexed in bounds;
    * the MX exponent is clamped to [-127, 127] before use;
    * the GEMMs and the expansion only convert bytes and multiply.
    Each call must return BSQ_OK (the binding raises otherwise), and a later
    call on finite data must still match the oracle."""
    announce("non-finite inputs", shape)
    R, C = shape
    x = from_bits(_with_nonfinite(shape, R + C))
    nan1 = torch.tensor([float("nan")], device="cuda")
    inf1 = torch.tensor([float("inf")], device="cuda")
    outs = []
    outs.append(bsq.nvfp4_quantize(x, 1))
    outs.append(bsq.nvfp4_quantize(x, 1, "sr", seed=3, rht=True, rht_signs=0x1357))
    outs.append(bsq.nvfp4_quantize(x, 16))
    outs.append(bsq.nvfp4_quantize(x, 1, amax=nan1))
    outs.append(bsq.nvfp4_quantize(x, 1, amax=inf1))
    outs.append(bsq.mx_quantize(x, "mxfp4"))
    outs.append(bsq.mx_quantize(x, "mxfp4", "sr", seed=4))
    outs.append(bsq.mx_quantize(x, "mxfp8"))
    q1 = bsq.quantize_transpose(x, "nvfp4", 1, "sr", seed=6, rht_col=True, rht_signs=0x2468)
    q2 = bsq.quantize_transpose(x, "nvfp4", 16)
    if R % 32 == 0:
        bsq.quantize_transpose(x, "mxfp4")
        bsq.quantize_transpose(x, "mxfp8")
    bsq.quantize_transpose_amax(x, nan1, inf1, 1, "sr", rht_col=True, rht_signs=0x11)
    bsq.quantize_transpose_amax(x, inf1, inf1, 16)
    f8 = bsq.fp8_quantize_transpose(x)
    y = from_bits(_with_nonfinite((R, 2 * C), R + 2 * C))
    bsq.swiglu(y, rht_col=True, rht_signs=0x0F0F)
    bsq.swiglu_backward(y, x, rht_col=True, rht_signs=0x0F0F)
    w32 = torch.zeros(R * C, dtype=torch.float32, device="cuda")
    bsq.master_weight_update(w32, x.reshape(-1), 0.5)
    # GEMMs on the codes, scales and amaxes made from non-finite inputs
    bsq.bs_gemm("nvfp4", q1["row_codes"], q1["row_scales"], q1["row_codes"], q1["row_scales"],
                q1["row_amax"], q1["row_amax"])
    bsq.bs_gemm("nvfp4", q1["col_codes"], q1["col_scales"], q2["col_codes"], q2["col_scales"],
                q1["col_amax"], nan1)
    mc, ms = outs[5]
    bsq.bs_gemm("mxfp4", mc, ms, mc, ms)
    mc8, ms8 = outs[7]
    bsq.bs_gemm("mxfp8", mc8, ms8, mc8, ms8)
    bsq.bs_gemm("fp8", f8["row_codes"], None, f8["row_codes"], None, f8["amax"], f8["amax"])
    if C % 128 == 0:
        bx = bsq.nvfp4_expand(q2["row_codes"], q2["row_scales"])
        bsq.bs_gemm_nvfp4_bx(q1["row_codes"], q1["row_scales"], inf1, bx, q2["row_amax"])
    torch.cuda.synchronize()
    assert not np.isfinite(f32(outs[0][2])[0])                  # the amax saw a non-finite value
    # the library still computes correctly afterwards
    z = torch.randn((R, C), generator=torch.Generator().manual_seed(1)).to(torch.bfloat16).cuda()
    ac, as_, aa = bsq.nvfp4_quantize(z, 1)
    c = bsq.bs_gemm("nvfp4", ac, as_, ac, as_, aa, aa)
    torch.cuda.synchronize()
    oc, os_, oa = Q.nvfp4_quantize(bits(z), 1)
    assert_bytes_equal(u8(ac), oc, "codes after non-finite calls")
    rep = G.tolerance_report(c.double().cpu().numpy(), G.gemm_nvfp4(oc, os_, oa, oc, os_, oa))
    assert rep["passed"], rep
