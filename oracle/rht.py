"""16-point Random Hadamard Transform on WGRAD operands.

Test infrastructure only (see oracle/__init__.py).

NVFP4 pretraining post, section "NVFP4 pretraining recipe", ingredient 3: a
Random Hadamard Transform is applied only to the inputs of the WGRAD GEMM to
spread outliers before 4-bit quantization; FPROP and DGRAD skip it, since
transforming them would also require transforming the weight and break 2D
scale consistency.

Readings (the pages give neither size nor construction):
* Size 16, applied to each aligned 16-element chunk along the blocked
  (token / reduction) dimension of a WGRAD operand.
* R = (1/4) * H16 * D, with D = diag(+-1) from a 16-bit sign mask (bit i set
  -> element i negated) and H16 the natural-order (Sylvester) Hadamard matrix
  H[i][j] = (-1)**popcount(i & j).  R is orthogonal.  Both WGRAD operands use
  the same mask, so (R A)^T (R B) = A^T B.
* Computed in float32: D first, then the butterfly for h = 1, 2, 4, 8 over
  every i with (i & h) == 0: (y_i, y_{i+h}) <- (y_i + y_{i+h}, y_i - y_{i+h}),
  then y <- 0.25 * y.  No BF16 re-rounding before quantization.
"""

import numpy as np


def rht16(chunks, signs):
    """chunks: float32 array [..., 16]; signs: int 0..65535.  Returns float32 [..., 16].

    Stage h pairs element i (with i & h == 0) with element i + h; viewing the
    last axis as [16 / (2h), 2, h] puts such pairs at [..., k, 0, j] and
    [..., k, 1, j], so each stage is one float32 add and one subtract over the
    whole array, in the same pairs and order as the scalar butterfly."""
    y = np.array(chunks, dtype=np.float32, copy=True)
    assert y.shape[-1] == 16
    signs = int(signs) & 0xFFFF
    d = np.array([-1.0 if (signs >> i) & 1 else 1.0 for i in range(16)], dtype=np.float32)
    y *= d                                   # exact sign flips (multiplication by +-1)
    lead = y.shape[:-1]
    h = 1
    while h < 16:
        v = y.reshape(lead + (16 // (2 * h), 2, h))
        a = v[..., 0, :]
        b = v[..., 1, :]
        y = np.stack([a + b, a - b], axis=-2).reshape(lead + (16,))
        h *= 2
    return (y * np.float32(0.25)).astype(np.float32)


def rht16_scalar(chunk, signs):
    """The same transform on one 16-element chunk, element by element (for pins)."""
    y = [np.float32(v) for v in chunk]
    for i in range(16):
        if (int(signs) >> i) & 1:
            y[i] = -y[i]
    h = 1
    while h < 16:
        for i in range(16):
            if i & h == 0:
                a, b = y[i], y[i + h]
                y[i], y[i + h] = np.float32(a + b), np.float32(a - b)
        h *= 2
    return np.array([np.float32(v * np.float32(0.25)) for v in y], dtype=np.float32)


def rht_matrix_f64(signs):
    """The 16x16 matrix R = 0.25 * H16 * D in float64 (for pins only)."""
    i = np.arange(16)
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i[:, None] & i[None, :])
    H = np.where(pc % 2 == 0, 1.0, -1.0)
    d = np.array([-1.0 if (int(signs) >> k) & 1 else 1.0 for k in range(16)])
    return 0.25 * H * d[None, :]


def rht_along_rows(x, signs):
    """Apply rht16 to every aligned 16-chunk along the last axis of a 2-D float32 array."""
    x = np.asarray(x, dtype=np.float32)
    R, C = x.shape
    assert C % 16 == 0
    return rht16(x.reshape(R, C // 16, 16), signs).reshape(R, C)
