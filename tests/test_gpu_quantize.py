"""GPU parity of the quantizers against the CPU oracle: packed codes, scales
and amax must be bit-exact (stochastic rounding included) on seeded inputs
that span several tiles and ragged edges, plus special values."""

import numpy as np
import pytest
import torch

import fp8_quantized_gemm_amd as bsq
from fp8_quantized_gemm_amd import synth
from oracle import formats as F
from oracle import quantize as Q

from _gpu import announce, assert_bytes_equal, bits, f32, from_bits, gpu, u8

pytestmark = gpu

SHAPES_1x16 = [(1, 16), (16, 16), (37, 48), (256, 256), (130, 1040), (1024, 4096)]


@pytest.mark.parametrize("shape", SHAPES_1x16)
@pytest.mark.parametrize("rnd", ["rne", "sr"])
@pytest.mark.parametrize("rht", [False, True])
def test_nvfp4_rowwise(shape, rnd, rht):
    announce("nvfp4_quantize", shape, rnd, rht)
    x = synth.bf16_tensor(shape, 7 + shape[0], device="cuda")
    codes, scales, amax = bsq.nvfp4_quantize(x, 1, rnd, seed=0xDEADBEEF12, offset=3, rht=rht,
                                             rht_signs=0xB38E)
    torch.cuda.synchronize()
    oc, os_, oa = Q.nvfp4_quantize(bits(x), 1, rnd, 0xDEADBEEF12, 3, rht=rht, rht_signs=0xB38E)
    assert f32(amax)[0] == oa
    assert_bytes_equal(u8(scales), os_, "scales")
    assert_bytes_equal(u8(codes), oc, "codes")


@pytest.mark.parametrize("shape", [(16, 16), (48, 160), (256, 256), (1024, 4096)])
def test_nvfp4_2d(shape):
    announce("nvfp4_quantize 2D", shape)
    x = synth.bf16_tensor(shape, 11 + shape[1], sigma=0.02, outliers=False, device="cuda")
    codes, scales, amax = bsq.nvfp4_quantize(x, 16)
    torch.cuda.synchronize()
    oc, os_, oa = Q.nvfp4_quantize(bits(x), 16)
    assert f32(amax)[0] == oa
    assert_bytes_equal(u8(scales), os_, "scales")
    assert_bytes_equal(u8(codes), oc, "codes")


def test_nvfp4_amax_in():
    announce("nvfp4_quantize amax_in")
    x = synth.bf16_tensor((64, 128), 5, device="cuda")
    amax = torch.tensor([3.5], dtype=torch.float32, device="cuda")
    codes, scales, amax_out = bsq.nvfp4_quantize(x, amax=amax)
    torch.cuda.synchronize()
    oc, os_, _ = Q.nvfp4_quantize(bits(x), amax=np.float32(3.5))
    assert f32(amax_out)[0] == np.float32(3.5)
    assert_bytes_equal(u8(scales), os_, "scales")
    assert_bytes_equal(u8(codes), oc, "codes")


@pytest.mark.parametrize("shape", [(1, 32), (37, 64), (256, 256), (512, 4096)])
@pytest.mark.parametrize("fmt,rnd", [("mxfp4", "rne"), ("mxfp4", "sr"), ("mxfp8", "rne")])
def test_mx_rowwise(shape, fmt, rnd):
    announce("mx_quantize", shape, fmt, rnd)
    x = synth.bf16_tensor(shape, 9 + shape[0], device="cuda")
    codes, scales = bsq.mx_quantize(x, fmt, rnd, seed=77, offset=1)
    torch.cuda.synchronize()
    oc, os_ = Q.mx_quantize(bits(x), fmt, rnd, 77, 1)
    assert_bytes_equal(u8(scales), os_, "scales")
    assert_bytes_equal(u8(codes), oc, "codes")


QT_CASES = [
    # fmt, block_rows, rnd, rht_col
    ("nvfp4", 1, "rne", False), ("nvfp4", 1, "rne", True),
    ("nvfp4", 1, "sr", False), ("nvfp4", 1, "sr", True),
    ("nvfp4", 16, "rne", False),
    ("mxfp4", 1, "rne", False), ("mxfp4", 1, "sr", False), ("mxfp8", 1, "rne", False),
]


@pytest.mark.parametrize("shape", [(32, 32), (64, 96), (256, 256), (1024, 544), (4096, 1024)])
@pytest.mark.parametrize("case", QT_CASES)
def test_quantize_transpose(shape, case):
    fmt, br, rnd, rht = case
    announce("quantize_transpose", shape, case)
    sigma = 0.02 if br == 16 else 1.0
    x = synth.bf16_tensor(shape, 13 + shape[0] + shape[1], sigma=sigma, device="cuda")
    out = bsq.quantize_transpose(x, fmt, br, rnd, seed=2 ** 40 + 5, offset=9, rht_col=rht,
                                 rht_signs=0x5AC3)
    torch.cuda.synchronize()
    ref = Q.quantize_transpose(bits(x), fmt, br, rnd, 2 ** 40 + 5, 9, rht_col=rht, rht_signs=0x5AC3)
    for k in ("row", "col"):
        if fmt == "nvfp4":
            assert f32(out[k + "_amax"])[0] == ref[k + "_amax"], k
        assert_bytes_equal(u8(out[k + "_scales"]), ref[k + "_scales"], k + " scales")
        assert_bytes_equal(u8(out[k + "_codes"]), ref[k + "_codes"], k + " codes")


# (512, 256) runs the 256 x 256 tiled kernel, (128, 64) the general one.
@pytest.mark.parametrize("shape", [(128, 64), (512, 256)])
@pytest.mark.parametrize("row,col", [(True, False), (False, True)])
def test_quantize_transpose_one_orientation(row, col, shape):
    announce("quantize_transpose one side", row, col, shape)
    x = synth.bf16_tensor(shape, 21, device="cuda")
    out = bsq.quantize_transpose(x, "nvfp4", 1, "sr", 3, 0, rht_col=True, rht_signs=0x1234,
                                 row=row, col=col)
    torch.cuda.synchronize()
    ref = Q.quantize_transpose(bits(x), "nvfp4", 1, "sr", 3, 0, rht_col=True, rht_signs=0x1234)
    k = "row" if row else "col"
    assert out[("col" if row else "row") + "_codes"] is None
    assert f32(out[k + "_amax"])[0] == ref[k + "_amax"]
    assert_bytes_equal(u8(out[k + "_codes"]), ref[k + "_codes"], k)
    assert_bytes_equal(u8(out[k + "_scales"]), ref[k + "_scales"], k)


def _special_bits(R, C, seed):
    """BF16 bits with zeros, -0, BF16 subnormals, huge values, E2M1 midpoints."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((R, C)).astype(np.float32)
    b = (v.view(np.uint32) >> 16).astype(np.uint16)
    b[0, :16] = 0                                  # an all-zero block
    b[1, :16] = 0x8000                             # all -0
    b[2, :16] = rng.integers(1, 0x80, 16)          # positive subnormals
    b[2, 16:32] = rng.integers(0x8001, 0x8080, 16)  # negative subnormals
    b[3, :] = np.where(rng.random(C) < 0.5, 0x7C00, 0xFC00)   # +-2.7e36 (16x stays finite)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], dtype=np.float32)
    b[4, :] = (np.resize(mids, C).view(np.uint32) >> 16).astype(np.uint16)
    b[5, :] = 0x0001                               # the smallest subnormal everywhere
    b[16:32, :8] = 0                               # all-zero column blocks (scale 0, encode factor 0)
    return b


@pytest.mark.parametrize("shape", [(32, 64), (256, 256)])
@pytest.mark.parametrize("rnd", ["rne", "sr"])
def test_special_values_nvfp4(rnd, shape):
    announce("special values nvfp4", rnd, shape)
    b = _special_bits(*shape, 1)
    x = from_bits(b)
    out = bsq.quantize_transpose(x, "nvfp4", 1, rnd, 5, 0, rht_col=True, rht_signs=0xFFFF)
    c, s, a = bsq.nvfp4_quantize(x, 1, rnd, 5, 0)
    # a tensor of only tiny values exercises the FLT_MAX clamps
    tiny = np.zeros((16, 32), dtype=np.uint16)
    tiny[3, 5] = 0x0001
    tiny[7, 9] = 0x8003
    ct, st, at = bsq.nvfp4_quantize(from_bits(tiny), 1, rnd, 5, 0)
    torch.cuda.synchronize()
    ref = Q.quantize_transpose(b, "nvfp4", 1, rnd, 5, 0, rht_col=True, rht_signs=0xFFFF)
    for k in ("row", "col"):
        assert f32(out[k + "_amax"])[0] == ref[k + "_amax"]
        assert_bytes_equal(u8(out[k + "_codes"]), ref[k + "_codes"], k)
        assert_bytes_equal(u8(out[k + "_scales"]), ref[k + "_scales"], k)
    oc, os_, _ = Q.nvfp4_quantize(b, 1, rnd, 5, 0)
    assert_bytes_equal(u8(c), oc, "rowwise codes")
    assert_bytes_equal(u8(s), os_, "rowwise scales")
    tc, ts, ta = Q.nvfp4_quantize(tiny, 1, rnd, 5, 0)
    assert f32(at)[0] == ta
    assert_bytes_equal(u8(ct), tc, "tiny codes")
    assert_bytes_equal(u8(st), ts, "tiny scales")


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_special_values_mx(fmt):
    announce("special values mx", fmt)
    b = _special_bits(64, 64, 2)
    x = from_bits(b)
    c, s = bsq.mx_quantize(x, fmt)
    out = bsq.quantize_transpose(x, fmt)
    torch.cuda.synchronize()
    oc, os_ = Q.mx_quantize(b, fmt)
    assert_bytes_equal(u8(c), oc, "codes")
    assert_bytes_equal(u8(s), os_, "scales")
    ref = Q.quantize_transpose(b, fmt)
    for k in ("row", "col"):
        assert_bytes_equal(u8(out[k + "_codes"]), ref[k + "_codes"], k)
        assert_bytes_equal(u8(out[k + "_scales"]), ref[k + "_scales"], k)


def test_empty_inputs():
    announce("empty inputs")
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    c, s, a = bsq.nvfp4_quantize(x)
    out = bsq.quantize_transpose(x)
    cm, sm = bsq.mx_quantize(x)
    torch.cuda.synchronize()
    assert c.numel() == 0 and s.numel() == 0 and f32(a)[0] == 0.0
    assert f32(out["row_amax"])[0] == 0.0 and f32(out["col_amax"])[0] == 0.0


def test_deterministic_and_stream_ordered():
    announce("determinism + side stream")
    x = synth.bf16_tensor((2048, 2048), 31, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        r1 = bsq.quantize_transpose(x, "nvfp4", 1, "sr", 8, 0, rht_col=True, rht_signs=7)
        r2 = bsq.quantize_transpose(x, "nvfp4", 1, "sr", 8, 0, rht_col=True, rht_signs=7)
    s.synchronize()
    for k in ("row_codes", "row_scales", "row_amax", "col_codes", "col_scales", "col_amax"):
        assert torch.equal(r1[k], r2[k]), k


def test_argument_error_leaves_outputs_untouched():
    announce("argument error")
    x = synth.bf16_tensor((32, 48), 3, device="cuda")     # cols % 32 != 0 for MX
    codes = torch.full((32, 24), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.full((32, 1), 0xCD, dtype=torch.uint8, device="cuda")
    st = bsq.lib().mx_quantize(x.data_ptr(), 32, 48, 1, 0, 0, 0, codes.data_ptr(),
                               scales.data_ptr(), None)
    torch.cuda.synchronize()
    assert st == bsq.BSQ_EINVAL
    assert bool((codes == 0xAB).all()) and bool((scales == 0xCD).all())
