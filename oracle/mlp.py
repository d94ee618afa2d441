"""SwiGLU of the MLP whose GEMMs the workloads model.

Test infrastructure only (see oracle/__init__.py).

The NVFP4 post's "Performance results" measure Llama 3 8B and Llama 3.1 405B;
their MLP is gate/up projection -> SwiGLU -> down projection, so the BF16
input H of the down projection (and of its WGRAD) is SwiGLU of the fused
gate/up GEMM output.  The pages give no formula.  Readings:
* [G | U] = Y_gu [T, 2F]: the first F columns are the gate, the last F the up
  projection;
* H = silu(G) * U with silu(g) = g / (1 + exp(-g)), evaluated in float64 on
  the BF16 inputs and rounded once to BF16 (round to nearest even).
* Backward (the chain rule of H = silu(G) * U, nothing the pages add): from
  the BF16 gradient dH [T, F], dG = dH * U * silu'(G) and dU = dH * silu(G),
  silu'(g) = sigma(g) * (1 + g * (1 - sigma(g))), sigma the logistic
  function; each output is evaluated in float64 and rounded once to BF16, and
  dY_gu = [dG | dU] [T, 2F] keeps the forward's column order.
* Master-weight update: the data-flow paragraph after Figure 1 folds the
  BF16 GEMM outputs into an FP32 master weight on the optimizer step and
  names no optimizer.  The plainest fold is taken: w <- w - lr * dW, FP32
  product then FP32 difference (two round-to-nearest-even steps, no fused
  multiply-add), and the BF16 working copy the next step quantizes is
  RNE(w).  Its amax (max |BF16 copy|) is the per-tensor amax the next step's
  16x16 weight quantizer needs.
"""

import numpy as np

from . import formats as F


def silu_f64(g):
    g = np.asarray(g, dtype=np.float64)
    return g / (1.0 + np.exp(-g))


def f64_to_bf16_bits(x):
    """float64 -> BF16 bit patterns (uint16), round to nearest even."""
    v = F.f64_to_bf16_rne(x).astype(np.float32)            # exact: BF16 values are FP32 values
    return (v.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def swiglu(y_gu):
    """H [T, F] BF16 bits from Y_gu [T, 2F] BF16 bits."""
    y = F.bf16_bits_to_f32(y_gu).astype(np.float64)
    T, F2 = y.shape
    assert F2 % 2 == 0
    Fh = F2 // 2
    return f64_to_bf16_bits(silu_f64(y[:, :Fh]) * y[:, Fh:])


def sigmoid_f64(g):
    g = np.asarray(g, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-g))


def dsilu_f64(g):
    """d silu / d g = sigma(g) * (1 + g * (1 - sigma(g)))."""
    g = np.asarray(g, dtype=np.float64)
    s = sigmoid_f64(g)
    return s * (1.0 + g * (1.0 - s))


def swiglu_backward(y_gu, d_h):
    """dY_gu [T, 2F] BF16 bits from Y_gu [T, 2F] and dH [T, F] BF16 bits."""
    y = F.bf16_bits_to_f32(y_gu).astype(np.float64)
    dh = F.bf16_bits_to_f32(d_h).astype(np.float64)
    T, F2 = y.shape
    Fh = F2 // 2
    assert F2 % 2 == 0 and dh.shape == (T, Fh)
    g, u = y[:, :Fh], y[:, Fh:]
    return np.concatenate([f64_to_bf16_bits(dh * u * dsilu_f64(g)),
                           f64_to_bf16_bits(dh * silu_f64(g))], axis=1)


def f64_to_f32(x):
    """float64 -> nearest float32 (RNE), as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def master_update(w32, grad_bf16, lr):
    """FP32 master weight w32 (float32 array) and BF16 gradient bits ->
    (new w32 float32, BF16 bits of the new weight, amax of that copy as float32)."""
    w = np.asarray(w32, dtype=np.float32).astype(np.float64)
    g = F.bf16_bits_to_f32(grad_bf16).astype(np.float64)
    step = f64_to_f32(f64_to_f32(lr) * g)                  # FP32 product (exact in float64, then one rounding)
    w_new = f64_to_f32(w - step)                           # FP32 difference, one rounding
    bits = f64_to_bf16_bits(w_new)
    amax = np.float32(np.abs(F.bf16_bits_to_f32(bits)).max(initial=0.0))
    return w_new.astype(np.float32), bits, amax
