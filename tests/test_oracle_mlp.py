"""Pins of the SwiGLU oracle.

* silu agrees with torch's float64 SiLU (a library routine) to 1e-15
  relative; silu(0) = 0 and silu(g) - silu(-g) = g (the logistic identity).
* The final BF16 rounding agrees with torch's float32 -> bfloat16 cast (RNE)
  on float32 inputs, and rounds float64 halfway cases to even.
* H = silu(G) * U on a small case equals an independent scalar evaluation.
* Backward: silu' agrees with torch autograd's float64 derivative of SiLU
  and with a central finite difference of silu; dY_gu agrees with autograd's
  vector-Jacobian product of silu(G) * U (rounded once to BF16), keeps the
  [dG | dU] order, and reduces to dG = dH * U / 2, dU = 0 at G = 0.
* Master-weight update: lr = 0 and dW = 0 leave w unchanged; with lr a power
  of two the product is exact and w - lr * dW rounds once (checked against
  exact rational arithmetic); for a general lr the result lies within the
  two-rounding bound ulp(lr * dW) / 2 + ulp(w') / 2 of the exact value, and
  within ulp(lr * dW) + ulp(w') of torch.optim.SGD (no momentum), which
  rounds once (fused multiply-add) on the CPU; the BF16 copy equals torch's
  float32 -> bfloat16 cast and the amax is the largest magnitude.
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


def test_dsilu_matches_autograd_and_finite_difference():
    g = np.concatenate([np.linspace(-30, 30, 4001), np.random.default_rng(5).standard_normal(1000) * 5])
    gt = torch.tensor(g, dtype=torch.float64, requires_grad=True)
    torch.nn.functional.silu(gt).sum().backward()
    np.testing.assert_allclose(M.dsilu_f64(g), gt.grad.numpy(), rtol=1e-13, atol=1e-15)
    h = 1e-5
    fd = (M.silu_f64(g + h) - M.silu_f64(g - h)) / (2 * h)
    np.testing.assert_allclose(M.dsilu_f64(g), fd, rtol=1e-7, atol=1e-9)
    assert M.dsilu_f64(np.array([0.0]))[0] == 0.5


def test_swiglu_backward_matches_autograd_vjp():
    rng = np.random.default_rng(6)
    T, Fh = 7, 24
    y = _bits(rng.standard_normal((T, 2 * Fh)) * 2)
    dh = _bits(rng.standard_normal((T, Fh)) * 1e-3)
    got = M.swiglu_backward(y, dh)
    yt = torch.tensor(F.bf16_bits_to_f32(y).astype(np.float64), requires_grad=True)
    dht = torch.tensor(F.bf16_bits_to_f32(dh).astype(np.float64))
    (torch.nn.functional.silu(yt[:, :Fh]) * yt[:, Fh:]).backward(dht)
    want = yt.grad.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    # autograd's float64 result differs from the oracle's only in the last
    # float64 bits, which decide the BF16 rounding with probability ~2^-44
    np.testing.assert_array_equal(got, want)
    assert got.shape == (T, 2 * Fh)


def test_swiglu_backward_at_zero_gate():
    u = np.array([[1.5, -2.0, 0.25, 3.0]])
    y = _bits(np.concatenate([np.zeros((1, 4)), u], axis=1))
    dh = _bits(np.array([[2.0, 0.5, -4.0, 1.0]]))
    d = M.swiglu_backward(y, dh)
    np.testing.assert_array_equal(F.bf16_bits_to_f32(d[:, :4]).astype(np.float64), [[1.5, -0.5, -0.5, 1.5]])
    assert not (d[:, 4:] & 0x7FFF).any()


def _f32_ulp(x):
    x = np.abs(np.asarray(x, dtype=np.float32))
    return np.spacing(x).astype(np.float64)


def test_master_update_identities_and_exact_cases():
    from fractions import Fraction
    rng = np.random.default_rng(7)
    w = (rng.standard_normal(4096) * 0.02).astype(np.float32)
    g = _bits(rng.standard_normal(4096) * 1e-2)
    w0, b0, a0 = M.master_update(w, g, 0.0)
    np.testing.assert_array_equal(w0, w)
    wz, _, _ = M.master_update(w, np.zeros(4096, np.uint16), 0.5)
    np.testing.assert_array_equal(wz, w)
    # lr = 2^-7: lr * g is exact, so w - lr * g is rounded once
    wn, _, _ = M.master_update(w[:256], g[:256], 2.0 ** -7)
    gf = F.bf16_bits_to_f32(g[:256])
    for i in range(256):
        exact = Fraction(float(w[i])) - Fraction(2) ** -7 * Fraction(float(gf[i]))
        assert wn[i] == np.float32(float(exact)) or abs(Fraction(float(wn[i])) - exact) <= Fraction(float(_f32_ulp(wn[i]))) / 2
    # two roundings, not one: RN32(0.1f * 3) equals RN32(0.3), so the difference is exactly 0,
    # where a fused multiply-add would leave 0.3f - 0.1f * 3 = 7.45e-9
    w3, _, _ = M.master_update(np.array([0.3], np.float32), _bits([3.0]), np.float32(0.1))
    assert w3[0] == 0.0
    # BF16 copy and amax
    want = torch.tensor(w0).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(b0, want)
    assert a0 == np.float32(np.abs(torch.tensor(w0).to(torch.bfloat16).float().numpy()).max())


def test_master_update_matches_sgd():
    rng = np.random.default_rng(8)
    n, lr = 50000, 3e-4
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = _bits(rng.standard_normal(n) * 10.0 ** rng.integers(-6, 1, n))
    wn, bits, _ = M.master_update(w, g, lr)
    p = torch.nn.Parameter(torch.tensor(w))
    p.grad = torch.tensor(F.bf16_bits_to_f32(g))
    torch.optim.SGD([p], lr=lr).step()
    ref = p.detach().numpy().astype(np.float64)
    prod = np.float64(np.float32(lr)) * F.bf16_bits_to_f32(g).astype(np.float64)   # exact in float64
    exact = w.astype(np.float64) - prod
    bound = _f32_ulp(prod) / 2 + _f32_ulp(wn) / 2
    assert np.all(np.abs(wn.astype(np.float64) - exact) <= bound)
    assert np.all(np.abs(wn.astype(np.float64) - ref) <= 2 * bound + _f32_ulp(ref))
    # away from cancellation both routes round to the same value almost always
    assert np.mean(wn.astype(np.float64) == ref) > 0.99
