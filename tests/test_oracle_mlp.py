"""Pins of the SwiGLU oracle.

* silu agrees with torch's float64 SiLU (a library routine) to 1e-15
  relative; silu(0) = 0 and silu(g) - silu(-g) = g (the logistic identity).
* The final BF16 rounding agrees with torch's float32 -> bfloat16 cast (RNE)
  on float32 inputs, and rounds float64 halfway cases to even.
* H = silu(G) * U on a small case equals an independent scalar evaluation.
"""

import math

import numpy as np
import torch

from oracle import formats as F
from oracle import mlp as M


def test_silu_matches_torch_and_identities():
    g = np.concatenate([np.linspace(-30, 30, 4001), np.random.default_rng(1).standard_normal(1000) * 5])
    s = M.silu_f64(g)
    t = torch.nn.functional.silu(torch.tensor(g, dtype=torch.float64)).numpy()
    np.testing.assert_allclose(s, t, rtol=1e-15, atol=1e-300)
    assert M.silu_f64(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(M.silu_f64(g) - M.silu_f64(-g), g, rtol=1e-14, atol=1e-14)


def test_bf16_rounding_matches_torch_cast():
    x = (np.random.default_rng(2).standard_normal(100000) * 10.0 ** np.random.default_rng(3).integers(-30, 30, 100000)).astype(np.float32)
    got = M.f64_to_bf16_bits(x.astype(np.float64))
    want = torch.tensor(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, want)
    # float64 halfway between two BF16 values rounds to the even one
    one_plus = 1.0 + 2.0 ** -8                      # halfway between 1 and 1 + 2^-7
    assert M.f64_to_bf16_bits(np.array([one_plus]))[0] == 0x3F80
    assert M.f64_to_bf16_bits(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 0x3F82


def _bits(v):
    return torch.tensor(np.asarray(v, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_swiglu_small_case_scalar():
    rng = np.random.default_rng(4)
    y = _bits(rng.standard_normal((3, 8)) * 3)
    h = M.swiglu(y)
    yf = F.bf16_bits_to_f32(y).astype(np.float64)
    for t in range(3):
        for j in range(4):
            g, u = float(yf[t, j]), float(yf[t, 4 + j])
            exact = g / (1.0 + math.exp(-g)) * u
            want = M.f64_to_bf16_bits(np.array([exact]))[0]
            assert h[t, j] == want, (t, j)
    assert not M.swiglu(_bits(np.concatenate([np.ones((2, 4)), np.zeros((2, 4))], axis=1))).view(np.int16).any()
