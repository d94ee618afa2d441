"""GPU parity of the SwiGLU producers and of the quantizer that takes their
amaxes.

* swiglu_amax / swiglu_backward_amax against the oracle (float64, one BF16
  rounding): every element within one BF16 ulp (the kernels evaluate the
  logistic function in FP32 with v_exp / v_rcp, a few FP32 ulps of relative
  error, so only values that close to a BF16 rounding boundary can round the
  other way), and at most 0.2% of the elements off by that ulp.
* Their amaxes: bit-equal to the ones quantize_transpose computes on the same
  BF16 output (plain max and the column RHT max), and equal to the oracle's
  amaxes of its own output whenever the two outputs agree bit for bit (else
  within one BF16 ulp, relative).
* quantize_transpose_amax: bit-equal to the oracle's quantize_transpose given
  the oracle's amaxes, and to quantize_transpose given the GPU amaxes
  (RNE, SR, with and without the column RHT, 2D tiles).
* The fused route swiglu_amax -> quantize_transpose_amax gives the same bytes
  as swiglu -> quantize_transpose.
"""

import numpy as np
import pytest
import torch

import fp8_quantized_gemm_amd as bsq
from fp8_quantized_gemm_amd import synth
from oracle import mlp as M
from oracle import quantize as Q

from _gpu import announce, assert_bytes_equal, bits, f32, from_bits, gpu, u8

pytestmark = gpu

SIGNS = 0xB3C5
MAX_OFF_FRACTION = 2e-3


def _key(b):
    """BF16 bits -> integers ordered like the values (+0 and -0 both 0)."""
    b = np.asarray(b).astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def assert_within_one_ulp(got, want, what, max_off_fraction=MAX_OFF_FRACTION):
    got, want = np.asarray(got), np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    d = np.abs(_key(got) - _key(want))
    off = int((d != 0).sum())
    print(what, f"elements one ulp off: {off} of {d.size}")
    assert d.max(initial=0) <= 1, (what, int(d.max()), tuple(np.argwhere(d > 1)[0]))
    assert off <= max_off_fraction * d.size, (what, off, d.size)
    return off


# Gates spread over [-120, 120].  The exponential's argument is range-reduced,
# so its error no longer grows with |g|; what remains off by one BF16 ulp:
# for 17 < g < 40 the FP32 sigmoid rounds to exactly 1, so H = g * u, a
# product of two BF16 values, can sit exactly on a BF16 tie that the exact
# value lies just below (about one element in 256 of that band); for
# |g| > 87 exp(-|g|) is an FP32 denormal with fewer significant bits.
# Measured 53 of 32768 (H) and 21 of 32768 (dY_gu); the bound keeps margin.
EXTREME_OFF_FRACTION = 5e-3


def _amax_ref(h_bits, rht):
    r = Q.quantize_transpose(h_bits, "nvfp4", 1, "rne", rht_col=rht, rht_signs=SIGNS)
    return np.float32(r["row_amax"]), np.float32(r["col_amax"])


def _check_amaxes(d, out, h_ref, rht, exact_match, what):
    """Fused amaxes = quantize_transpose's on the same output (bitwise), and the
    oracle's on its own output (bitwise when the outputs agree)."""
    q = bsq.quantize_transpose(out, rht_col=rht, rht_signs=SIGNS)
    torch.cuda.synchronize()
    ar, ac = f32(d["amax_row"])[0], f32(d["amax_col"])[0]
    assert ar == f32(q["row_amax"])[0], (what, "row amax vs quantize_transpose", ar, f32(q["row_amax"])[0])
    assert ac == f32(q["col_amax"])[0], (what, "col amax vs quantize_transpose", ac, f32(q["col_amax"])[0])
    rr, rc = _amax_ref(h_ref, rht)
    if exact_match:
        assert (ar, ac) == (rr, rc), (what, (ar, ac), (rr, rc))
    else:
        assert abs(ar - rr) <= rr * 2.0 ** -7 and abs(ac - rc) <= rc * 2.0 ** -7, (what, (ar, ac), (rr, rc))


# (rows, f, sigma): f = 272 and 16 leave part of the last 256-column group empty
@pytest.mark.parametrize("R,F,sigma", [(16, 16, 1.0), (32, 272, 2.0), (64, 1024, 1.0),
                                       (256, 528, 4.0), (48, 256, 1e-3)])
@pytest.mark.parametrize("rht", [True, False])
def test_swiglu_forward(R, F, sigma, rht):
    announce("swiglu fwd", R, F, sigma, rht)
    y = synth.bf16_tensor((R, 2 * F), 8000 + R + F, sigma, True, device="cuda")
    d = bsq.swiglu(y, rht_col=rht, rht_signs=SIGNS)
    torch.cuda.synchronize()
    h_ref = M.swiglu(bits(y))
    off = assert_within_one_ulp(bits(d["h"]), h_ref, f"H {R}x{F}")
    _check_amaxes(d, d["h"], h_ref, rht, off == 0, f"H {R}x{F}")
    if not rht:
        assert f32(d["amax_row"])[0] == f32(d["amax_col"])[0]


def test_swiglu_without_amax_writes_the_same_output():
    announce("swiglu no amax")
    y = synth.bf16_tensor((128, 1536), 8101, 1.0, True, device="cuda")
    a = bsq.swiglu(y, rht_col=True, rht_signs=SIGNS)
    b = bsq.swiglu(y, amax=False)
    torch.cuda.synchronize()
    assert b["amax_row"] is None and b["amax_col"] is None
    assert_bytes_equal(bits(b["h"]), bits(a["h"]), "H without amax")


def test_swiglu_extreme_gates():
    """Gates over [-120, 120]: exp(-|g|) underflows to FP32 denormals and then
    zero, sigmoid saturates; every element still within one BF16 ulp."""
    announce("swiglu extreme gates")
    R, F = 64, 512
    g = np.linspace(-120.0, 120.0, R * F).reshape(R, F)
    u = np.random.default_rng(8102).standard_normal((R, F)) * 100.0
    yb = torch.tensor(np.concatenate([g, u], axis=1), dtype=torch.float32).to(torch.bfloat16)
    y = yb.cuda()
    d = bsq.swiglu(y, rht_col=True, rht_signs=SIGNS)
    torch.cuda.synchronize()
    h_ref = M.swiglu(bits(yb))
    off = assert_within_one_ulp(bits(d["h"]), h_ref, "H extreme", EXTREME_OFF_FRACTION)
    _check_amaxes(d, d["h"], h_ref, True, off == 0, "H extreme")


@pytest.mark.parametrize("R,F,sigma", [(16, 16, 1.0), (32, 272, 2.0), (128, 768, 1.0),
                                       (256, 528, 4.0)])
@pytest.mark.parametrize("rht", [True, False])
def test_swiglu_backward(R, F, sigma, rht):
    announce("swiglu bwd", R, F, sigma, rht)
    y = synth.bf16_tensor((R, 2 * F), 8200 + R + F, sigma, True, device="cuda")
    dh = synth.bf16_tensor((R, F), 8300 + R + F, 1e-3, False, device="cuda")
    d = bsq.swiglu_backward(y, dh, rht_col=rht, rht_signs=SIGNS)
    torch.cuda.synchronize()
    ref = M.swiglu_backward(bits(y), bits(dh))
    off = assert_within_one_ulp(bits(d["d_y_gu"]), ref, f"dY_gu {R}x{F}")
    _check_amaxes(d, d["d_y_gu"], ref, rht, off == 0, f"dY_gu {R}x{F}")


def test_swiglu_backward_extreme_gates():
    announce("swiglu bwd extreme gates")
    R, F = 32, 512
    g = np.linspace(-120.0, 120.0, R * F).reshape(R, F)
    rng = np.random.default_rng(8301)
    u = rng.standard_normal((R, F)) * 10.0
    yb = torch.tensor(np.concatenate([g, u], axis=1), dtype=torch.float32).to(torch.bfloat16)
    dhb = torch.tensor(rng.standard_normal((R, F)), dtype=torch.float32).to(torch.bfloat16)
    d = bsq.swiglu_backward(yb.cuda(), dhb.cuda(), rht_col=True, rht_signs=SIGNS)
    torch.cuda.synchronize()
    ref = M.swiglu_backward(bits(yb), bits(dhb))
    off = assert_within_one_ulp(bits(d["d_y_gu"]), ref, "dY_gu extreme", EXTREME_OFF_FRACTION)
    _check_amaxes(d, d["d_y_gu"], ref, True, off == 0, "dY_gu extreme")


def test_swiglu_empty():
    announce("swiglu empty")
    y = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    d = bsq.swiglu(y, rht_col=True)
    b = bsq.swiglu_backward(y, torch.empty((0, 32), dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    assert d["h"].shape == (0, 32) and b["d_y_gu"].shape == (0, 64)
    for t in (d["amax_row"], d["amax_col"], b["amax_row"], b["amax_col"]):
        assert f32(t)[0] == 0.0


# (rows, cols, block_rows, rnd, rht): the tile kernel (256-multiples) and the
# general one, every option of the column side
QTA_CASES = [(256, 512, 1, "rne", True), (256, 256, 1, "sr", True), (96, 160, 1, "rne", False),
             (48, 272, 1, "sr", True), (256, 512, 16, "rne", False), (64, 96, 16, "rne", False)]


@pytest.mark.parametrize("R,C,br,rnd,rht", QTA_CASES)
def test_quantize_transpose_amax_against_oracle(R, C, br, rnd, rht):
    announce("qt amax vs oracle", R, C, br, rnd, rht)
    x = synth.bf16_tensor((R, C), 8400 + R + C, 1.0, br == 1, device="cuda")
    seed, offset = 0x5EED0000 + R, 3
    ref = Q.quantize_transpose(bits(x), "nvfp4", br, rnd, seed, offset, rht, SIGNS)
    ar = torch.tensor([ref["row_amax"]], dtype=torch.float32, device="cuda")
    ac = torch.tensor([ref["col_amax"]], dtype=torch.float32, device="cuda")
    if br == 16:       # 16x16 tiles: one amax for both sides, passed once
        with pytest.raises(bsq.BsqError) as e:
            bsq.quantize_transpose_amax(x, ar, ac, br, rnd, seed, offset, rht, SIGNS)
        assert e.value.status == bsq.BSQ_EINVAL
        ac = ar
    d = bsq.quantize_transpose_amax(x, ar, ac, br, rnd, seed, offset, rht, SIGNS)
    torch.cuda.synchronize()
    for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
        assert_bytes_equal(u8(d[k]), ref[k], k)


@pytest.mark.parametrize("R,C,br,rnd,rht", QTA_CASES)
def test_quantize_transpose_amax_matches_quantize_transpose(R, C, br, rnd, rht):
    announce("qt amax vs qt", R, C, br, rnd, rht)
    x = synth.bf16_tensor((R, C), 8500 + R + C, 1.0, br == 1, device="cuda")
    q = bsq.quantize_transpose(x, "nvfp4", br, rnd, 77, 5, rht, SIGNS)
    d = bsq.quantize_transpose_amax(x, q["row_amax"], q["row_amax"] if br == 16 else q["col_amax"],
                                    br, rnd, 77, 5, rht, SIGNS)
    one_row = bsq.quantize_transpose_amax(x, q["row_amax"], None, br, rnd, 77, 5, rht, SIGNS, col=False)
    one_col = bsq.quantize_transpose_amax(x, None, q["col_amax"], br, rnd, 77, 5, rht, SIGNS, row=False)
    torch.cuda.synchronize()
    for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
        assert_bytes_equal(u8(d[k]), u8(q[k]), k)
    assert_bytes_equal(u8(one_row["row_codes"]), u8(q["row_codes"]), "row only")
    assert_bytes_equal(u8(one_col["col_scales"]), u8(q["col_scales"]), "col only")
    assert one_row["col_codes"] is None and one_col["row_codes"] is None


@pytest.mark.parametrize("rnd", ["rne", "sr"])
def test_fused_route_equals_unfused(rnd):
    """swiglu_amax -> quantize_transpose_amax == swiglu -> quantize_transpose."""
    announce("fused vs unfused", rnd)
    y = synth.bf16_tensor((512, 2 * 1280), 8601, 1.0, True, device="cuda")
    f = bsq.swiglu(y, rht_col=True, rht_signs=SIGNS)
    qa = bsq.quantize_transpose_amax(f["h"], f["amax_row"], f["amax_col"], 1, rnd, 9, 1, True, SIGNS)
    h = bsq.swiglu(y, amax=False)["h"]
    q = bsq.quantize_transpose(h, "nvfp4", 1, rnd, 9, 1, True, SIGNS)
    torch.cuda.synchronize()
    for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
        assert_bytes_equal(u8(qa[k]), u8(q[k]), k)


def _sample_rows(T, n, seed):
    return np.sort(np.random.default_rng(seed).choice(T, n, replace=False))


@pytest.mark.parametrize("T,F", [(32768, 14336), (8192, 53248)], ids=["8b", "405b"])
def test_swiglu_full_size_sampled(T, F):
    """Llama 3 8B (T = 32768 tokens, F = 14336) and Llama 3.1 405B (T = 8192,
    F = 53248) MLP shapes: forward and backward at full size in the launch
    configuration the benchmark times; 48 sampled rows against the oracle,
    the amaxes against quantize_transpose on the whole output."""
    announce("swiglu full size", T, F)
    y = synth.bf16_tensor((T, 2 * F), 8701, 1.0, True, device="cuda")
    d = bsq.swiglu(y, rht_col=True, rht_signs=SIGNS)
    torch.cuda.synchronize()
    rows = _sample_rows(T, 48, 8702)
    yr = bits(y[torch.from_numpy(rows).cuda()])
    assert_within_one_ulp(bits(d["h"][torch.from_numpy(rows).cuda()]), M.swiglu(yr), "H sampled")
    q = bsq.quantize_transpose(d["h"], rht_col=True, rht_signs=SIGNS, row=True, col=True)
    torch.cuda.synchronize()
    assert f32(d["amax_row"])[0] == f32(q["row_amax"])[0]
    assert f32(d["amax_col"])[0] == f32(q["col_amax"])[0]
    del q
    dh = synth.bf16_tensor((T, F), 8703, 1e-3, False, device="cuda")
    b = bsq.swiglu_backward(y, dh, rht_col=True, rht_signs=SIGNS)
    torch.cuda.synchronize()
    ridx = torch.from_numpy(rows).cuda()
    assert_within_one_ulp(bits(b["d_y_gu"][ridx]), M.swiglu_backward(yr, bits(dh[ridx])), "dY_gu sampled")
    q = bsq.quantize_transpose(b["d_y_gu"], rnd="sr", rht_col=True, rht_signs=SIGNS)
    torch.cuda.synchronize()
    assert f32(b["amax_row"])[0] == f32(q["row_amax"])[0]
    assert f32(b["amax_col"])[0] == f32(q["col_amax"])[0]


def _random_shapes(seed, n, max_rows=40, max_cols=70):
    rng = np.random.default_rng(seed)
    return [(16 * int(rng.integers(1, max_rows)), 16 * int(rng.integers(1, max_cols))) for _ in range(n)]


@pytest.mark.parametrize("R,F", _random_shapes(8801, 6))
def test_swiglu_random_shapes(R, F):
    """Seeded random multiples of 16 (the last 256-column group partly empty
    in most of them): forward and backward with the column RHT amax."""
    announce("swiglu random", R, F)
    y = synth.bf16_tensor((R, 2 * F), 8900 + R + F, 1.5, True, device="cuda")
    dh = synth.bf16_tensor((R, F), 8950 + R + F, 1e-2, False, device="cuda")
    d = bsq.swiglu(y, rht_col=True, rht_signs=SIGNS)
    b = bsq.swiglu_backward(y, dh, rht_col=True, rht_signs=SIGNS)
    torch.cuda.synchronize()
    h_ref = M.swiglu(bits(y))
    off = assert_within_one_ulp(bits(d["h"]), h_ref, f"H {R}x{F}")
    _check_amaxes(d, d["h"], h_ref, True, off == 0, f"H {R}x{F}")
    g_ref = M.swiglu_backward(bits(y), bits(dh))
    off = assert_within_one_ulp(bits(b["d_y_gu"]), g_ref, f"dY_gu {R}x{F}")
    _check_amaxes(b, b["d_y_gu"], g_ref, True, off == 0, f"dY_gu {R}x{F}")


@pytest.mark.parametrize("R,C", _random_shapes(8802, 6))
@pytest.mark.parametrize("rnd", ["rne", "sr"])
def test_quantize_transpose_amax_random_shapes(R, C, rnd):
    announce("qt amax random", R, C, rnd)
    x = synth.bf16_tensor((R, C), 9000 + R + C, 1.0, True, device="cuda")
    ref = Q.quantize_transpose(bits(x), "nvfp4", 1, rnd, 0xABCDEF, 11, True, SIGNS)
    ar = torch.tensor([ref["row_amax"]], dtype=torch.float32, device="cuda")
    ac = torch.tensor([ref["col_amax"]], dtype=torch.float32, device="cuda")
    d = bsq.quantize_transpose_amax(x, ar, ac, 1, rnd, 0xABCDEF, 11, True, SIGNS)
    torch.cuda.synchronize()
    for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
        assert_bytes_equal(u8(d[k]), ref[k], k)
