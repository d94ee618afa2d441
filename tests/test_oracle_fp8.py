"""Pins of the per-tensor FP8 oracle (the NVFP4 post's FP8 baseline, read as
E4M3 under one float32 scale 448 / amax per tensor).

* The element encode equals torch's CPU float8_e4m3fn cast (a library RNE
  conversion) of x * s_enc formed by torch itself.
* Closed forms: the amax element encodes to +-448; an all-zero tensor has
  s_enc = 1 and all-zero codes; s_enc * amax is 448 within one rounding.
* Round trip from codes: x = e4m3(code) * 2^j with a code 0x7E present gives
  s_enc = 2^-j exactly, so quantization returns the codes.
* Transpose: the column output is the row output transposed.
* GEMM: exact rational arithmetic on a small case."""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import gemm as G
from oracle import quantize as Q


def _bf16_bits(v):
    return torch.tensor(np.asarray(v, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("seed,sigma", [(1, 1.0), (2, 1e-3), (3, 40.0), (4, 1e-30)])
def test_fp8_encode_matches_torch_cast(seed, sigma):
    rng = np.random.default_rng(seed)
    x = _bf16_bits(rng.standard_normal((64, 96)) * sigma)
    codes, amax = Q.fp8_quantize(x)
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).float()
    s = torch.tensor(float(Q.fp8_scale_enc(amax)), dtype=torch.float32)
    assert float(xt.abs().max()) == float(amax)
    want = (xt * s).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(codes, want)


def test_fp8_closed_forms():
    rng = np.random.default_rng(5)
    x = _bf16_bits(rng.standard_normal((32, 32)))
    codes, amax = Q.fp8_quantize(x)
    y = F.bf16_bits_to_f32(x)
    at = np.abs(y) == amax
    assert np.all((codes[at] & 0x7F) == 0x7E)
    s = Q.fp8_scale_enc(amax)
    assert abs(float(s) * float(amax) - 448.0) <= 448.0 * 2.0 ** -23
    assert Q.fp8_scale_dec(amax) == np.float32(1.0) / s
    z, za = Q.fp8_quantize(np.zeros((16, 16), dtype=np.uint16))
    assert za == 0 and Q.fp8_scale_enc(za) == 1 and not z.any()


@pytest.mark.parametrize("j", [-20, 0, 7])
def test_fp8_round_trip_from_codes(j):
    rng = np.random.default_rng(100 + j)
    codes = rng.integers(0, 256, (48, 64)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C          # no NaN codes
    codes[3, 5] = 0x7E                             # the amax, 448
    codes[(codes & 0x7F) > 0x7E] = 0x7E
    vals = F.e4m3_decode(codes).astype(np.float64) * 2.0 ** j
    x = _bf16_bits(vals)                           # E4M3 values are exact in BF16
    assert np.array_equal(F.bf16_bits_to_f32(x).astype(np.float64), vals)
    got, amax = Q.fp8_quantize(x)
    assert amax == np.float32(448.0 * 2.0 ** j)
    np.testing.assert_array_equal(got, codes)


def test_fp8_transpose_is_the_row_output_transposed():
    x = _bf16_bits(np.random.default_rng(7).standard_normal((48, 80)) * 3)
    d = Q.fp8_quantize_transpose(x)
    np.testing.assert_array_equal(d["col_codes"], d["row_codes"].T)


def test_fp8_gemm_exact_small_case():
    rng = np.random.default_rng(8)
    a = _bf16_bits(rng.standard_normal((4, 32)))
    b = _bf16_bits(rng.standard_normal((3, 32)) * 0.1)
    ac, aa = Q.fp8_quantize(a)
    bc, ba = Q.fp8_quantize(b)
    c = G.gemm_fp8(ac, aa, bc, ba)
    sa, sb = Fraction(float(Q.fp8_scale_dec(aa))), Fraction(float(Q.fp8_scale_dec(ba)))
    av = [[Fraction(float(v)) for v in row] for row in F.e4m3_decode(ac)]
    bv = [[Fraction(float(v)) for v in row] for row in F.e4m3_decode(bc)]
    for m in range(4):
        for n in range(3):
            exact = sa * sb * sum(p * q for p, q in zip(av[m], bv[n]))
            assert abs(Fraction(float(c[m, n])) - exact) <= abs(exact) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 200)
