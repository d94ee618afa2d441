"""Pins for the oracle's block quantizers (CPU only).

* Global-scale closed form: the block holding the tensor amax gets the E4M3
  scale 448 (0x7E) and its largest element code 7 (6.0).
* Round trips built from codes: inputs constructed as code value x block
  scale (exact in BF16) quantize back to the same bytes (NVFP4 1x16 and
  16x16; MXFP4 and MXFP8).
* 2D invariant: quantize(W)^T == quantize(W^T) bytewise.
* MX closed form: block max element lands in [2**emax, 2**(emax+1)).
* Brute-force scalar NVFP4 / MX block quantization on a few blocks, written
  with Python Fractions and explicit float32 rounding points.
"""

from fractions import Fraction

import numpy as np
import torch

from oracle import formats as F
from oracle import quantize as Q
from fp8_quantized_gemm_amd import synth


def bf16_bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def f32_to_bf16_bits_exact(x):
    """float32 values that are exactly BF16 -> BF16 bits (asserts exactness)."""
    x = np.asarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    assert np.all((b & 0xFFFF) == 0)
    return (b >> 16).astype(np.uint16)


def test_global_scale_closed_form():
    x = bf16_bits(synth.bf16_tensor((64, 256), 11))
    codes, S, amax = Q.nvfp4_quantize(x, block_rows=1)
    y = F.bf16_bits_to_f32(x)
    r, c = np.unravel_index(np.argmax(np.abs(y)), y.shape)
    assert amax == np.abs(y).max()
    assert S[r, c // 16] == 0x7E
    cd = F.unpack_e2m1(codes)
    assert (cd[r, c] & 7) == 7
    assert all(F.e4m3_decode(S).ravel() <= 448)
    # dequantized tensor max equals amax within E2M1/E4M3 rounding
    deq = F.e2m1_decode(cd).reshape(64, 16, 16) * F.e4m3_decode(S)[:, :, None]
    deq = deq.reshape(64, 256) * Q.nvfp4_scale_dec(amax)
    assert abs(np.abs(deq).max() - amax) <= amax * 2.0 ** -20


def test_scale_enc_special_values():
    assert Q.nvfp4_scale_enc(np.float32(0)) == 1.0
    assert Q.nvfp4_scale_enc(np.float32(2688)) == 1.0
    tiny = np.float32(2.0 ** -133)                          # smallest BF16 subnormal
    assert Q.nvfp4_scale_enc(tiny) == F.FLT_MAX
    z = np.zeros((16, 32), dtype=np.uint16)
    codes, S, amax = Q.nvfp4_quantize(z)
    assert amax == 0 and not codes.any() and not S.any()


def _codes_roundtrip_input(rng, R, C, block_rows, neg_zero=True):
    """Random codes and E4M3 scales with code 7 in every block and 448 in block 0."""
    codes = rng.integers(0, 16, (R, C), dtype=np.uint8)
    nbr = R // block_rows
    S = rng.integers(1, 0x7F, (nbr, C // 16), dtype=np.uint8)   # nonzero, non-NaN scales
    S[0, 0] = 0x7E
    for i in range(nbr):
        for j in range(C // 16):
            r0 = i * block_rows + rng.integers(0, block_rows)
            codes[r0, j * 16 + rng.integers(0, 16)] = 7 | (8 * rng.integers(0, 2))
    if not neg_zero:
        codes[codes == 8] = 0
    Sx = np.repeat(S, block_rows, axis=0)
    x = F.e2m1_decode(codes).reshape(R, C // 16, 16) * F.e4m3_decode(Sx)[:, :, None]
    return codes, Sx, f32_to_bf16_bits_exact(x.reshape(R, C).astype(np.float32))


def test_nvfp4_roundtrip_from_codes_1x16():
    rng = np.random.default_rng(5)
    codes, S, x = _codes_roundtrip_input(rng, 48, 128, 1)
    qc, qs, amax = Q.nvfp4_quantize(x, block_rows=1)
    assert amax == 2688.0
    assert np.array_equal(qs, S)
    assert np.array_equal(qc, F.pack_e2m1(codes))


def test_nvfp4_roundtrip_from_codes_16x16():
    rng = np.random.default_rng(6)
    codes, S, x = _codes_roundtrip_input(rng, 64, 96, 16)
    qc, qs, amax = Q.nvfp4_quantize(x, block_rows=16)
    assert np.array_equal(qs, S)
    assert np.array_equal(qc, F.pack_e2m1(codes))


def test_2d_transpose_invariant():
    w = bf16_bits(synth.bf16_tensor((128, 64), 12, sigma=0.02, outliers=False))
    r = Q.quantize_transpose(w, "nvfp4", block_rows=16)
    row = F.unpack_e2m1(r["row_codes"])
    col = F.unpack_e2m1(r["col_codes"])
    assert np.array_equal(row.T, col)
    assert r["row_amax"] == r["col_amax"]
    # compact 16x16 grid identical in both orientations
    assert np.array_equal(r["row_scales"][::16, :], r["col_scales"][::16, :].T)
    assert np.array_equal(np.repeat(r["row_scales"][::16, :], 16, axis=0), r["row_scales"])


def test_1x16_differs_from_2d():
    w = bf16_bits(synth.bf16_tensor((32, 32), 13))
    a = Q.nvfp4_quantize(w, block_rows=1)[1]
    b = Q.nvfp4_quantize(w, block_rows=16)[1]
    assert not np.array_equal(a, b)
    assert np.all(b >= a)            # a tile amax is never below its rows' block amax


def _f32(x):
    return Fraction(float(np.float32(x)))


def _fl(q):
    """Round a Fraction to float32 (RNE) via float64 (exact for these magnitudes)."""
    return Fraction(float(np.float32(float(q))))


def test_nvfp4_scalar_brute_force():
    """Per-element scalar recomputation with Fractions and explicit float32 rounding."""
    x = bf16_bits(synth.bf16_tensor((4, 64), 14))
    codes, S, amax = Q.nvfp4_quantize(x)
    y = F.bf16_bits_to_f32(x)
    e4 = [Fraction(float(v)) for v in F.e4m3_decode(np.arange(0x7F, dtype=np.uint8))]
    grid = [Fraction(g) for g in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]
    amax_q = max(abs(_f32(v)) for v in y.ravel())
    s_enc = _fl(Fraction(2688) / amax_q)
    cd = F.unpack_e2m1(codes)
    for r in range(4):
        for j in range(4):
            blk = [_f32(v) for v in y[r, j * 16:(j + 1) * 16]]
            ab = max(abs(v) for v in blk)
            sf = _fl(_fl(ab / 6) * s_enc)
            # nearest E4M3 value, ties to even code
            best = min(range(len(e4)), key=lambda k: (abs(e4[k] - sf), k % 2))
            if sf > 448:
                best = 0x7E
            assert S[r, j] == best
            enc = _fl(s_enc / e4[best])
            for i, v in enumerate(blk):
                a = abs(_fl(v * enc))
                m = min(range(8), key=lambda k: (abs(grid[k] - a), k % 2))
                if a > 6:
                    m = 7
                want = m | (8 if np.signbit(y[r, j * 16 + i]) else 0)
                assert cd[r, j * 16 + i] == want


def test_mx_closed_form_and_scalar():
    x = bf16_bits(synth.bf16_tensor((8, 128), 15))
    y = F.bf16_bits_to_f32(x).astype(np.float64)
    for fmt, emax in (("mxfp4", 2), ("mxfp8", 8)):
        codes, E = Q.mx_quantize(x, fmt)
        e = E.astype(np.int64) - 127
        bm = np.abs(y).reshape(8, 4, 32).max(axis=2)
        scaled = bm * 2.0 ** (-e)
        assert np.all((scaled >= 2.0 ** emax) & (scaled < 2.0 ** (emax + 1)))
        # scalar: v = x * 2**-e is exact; element code by brute force nearest
        vals = F.e2m1_decode(np.arange(16, dtype=np.uint8)) if fmt == "mxfp4" else \
            F.e4m3_decode(np.arange(256, dtype=np.uint8))
        dec = F.unpack_e2m1(codes) if fmt == "mxfp4" else codes
        for r in range(8):
            for c in range(0, 128, 7):
                v = y[r, c] * 2.0 ** (-e[r, c // 32])
                lim = 6.0 if fmt == "mxfp4" else 448.0
                vv = max(min(v, lim), -lim)
                cands = [k for k in range(len(vals)) if not np.isnan(vals[k])
                         and np.signbit(vals[k]) == np.signbit(v)]
                best = min(cands, key=lambda k: (abs(float(vals[k]) - vv), k % 2))
                assert dec[r, c] == best, (fmt, r, c, v)


def test_mx_roundtrip_from_codes():
    rng = np.random.default_rng(16)
    R, C = 16, 128
    for fmt in ("mxfp4", "mxfp8"):
        E = rng.integers(100, 150, (R, C // 32)).astype(np.int64)
        if fmt == "mxfp4":
            codes = rng.integers(0, 16, (R, C), dtype=np.uint8)
            vals = F.e2m1_decode(codes).astype(np.float64)
            for r in range(R):
                for j in range(C // 32):
                    codes[r, j * 32] = 6 + rng.integers(0, 2)      # block max 4 or 6
        else:
            codes = rng.integers(0, 0x7E, (R, C), dtype=np.uint8)
            codes[(codes & 0x7F) == 0x7F] = 0
            for r in range(R):
                for j in range(C // 32):
                    codes[r, j * 32] = 0x78 + rng.integers(0, 7)    # block max in [256, 448]
        vals = (F.e2m1_decode(codes) if fmt == "mxfp4" else F.e4m3_decode(codes)).astype(np.float64)
        x = vals.reshape(R, C // 32, 32) * np.ldexp(1.0, E - 127)[:, :, None]
        xb = f32_to_bf16_bits_exact(x.reshape(R, C).astype(np.float32))
        qc, qs = Q.mx_quantize(xb, fmt)
        assert np.array_equal(qs.astype(np.int64), E - 127 + 127)
        want = F.pack_e2m1(codes) if fmt == "mxfp4" else codes
        assert np.array_equal(qc, want)


def test_mx_zero_block_and_clamp():
    x = np.zeros((1, 64), dtype=np.uint16)
    x[0, 32] = f32_to_bf16_bits_exact(np.float32(2.0 ** 127))[()]
    c, e = Q.mx_quantize(x, "mxfp4")
    assert e[0, 0] == 0 and e[0, 1] == 127 + 125


def test_quantize_transpose_col_equals_rowwise_of_transpose():
    x = bf16_bits(synth.bf16_tensor((64, 48), 17))
    r = Q.quantize_transpose(x, "nvfp4", 1, "sr", seed=9, offset=3, rht_col=True, rht_signs=0xA5C3)
    c2, s2, a2 = Q.nvfp4_quantize(np.ascontiguousarray(x.T), 1, "sr", 9, 3, stream=1,
                                  rht=True, rht_signs=0xA5C3)
    assert np.array_equal(r["col_codes"], c2) and np.array_equal(r["col_scales"], s2)
    assert r["col_amax"] == a2
    r1, s1, a1 = Q.nvfp4_quantize(x, 1, "sr", 9, 3, stream=0)
    assert np.array_equal(r["row_codes"], r1) and r["row_amax"] == a1


def test_row_subset_matches_full_and_chunked_rht_amax():
    x = bf16_bits(synth.bf16_tensor((64, 96), 18))
    full = Q.quantize_transpose(x, "nvfp4", 1, "sr", seed=4, offset=2, rht_col=True, rht_signs=0x3C5A)
    ids = np.array([3, 17, 50, 95])
    xt = np.ascontiguousarray(x.T)[ids]
    c, s, _ = Q.nvfp4_quantize(xt, 1, "sr", 4, 2, stream=1, rht=True, rht_signs=0x3C5A,
                               amax=full["col_amax"], row_ids=ids)
    assert np.array_equal(c, full["col_codes"][ids]) and np.array_equal(s, full["col_scales"][ids])
    assert Q.tensor_amax_rht_cols(x, 0x3C5A, chunk_rows=32) == full["col_amax"]
