"""Block quantizers: NVFP4 (1x16 and 16x16), MXFP4 / MXFP8 (1x32), both orientations.

Test infrastructure only (see oracle/__init__.py).

Sources:
* NVFP4 pretraining post, "NVFP4 pretraining recipe":
  - ingredient 1: 16-element micro-blocks along the reduction dimension;
  - ingredient 2: E4M3 block scale factors under a per-tensor FP32 scale;
  - ingredient 3: RHT on WGRAD inputs only (oracle/rht.py);
  - ingredient 4: one FP8 scale per 16x16 weight block, so FPROP and its
    transposed DGRAD see the same values; activations and gradients keep 1x16;
  - ingredient 5: RNE for weights and activations, stochastic rounding for
    gradients.
* HN page opcode84: MXFP8 / MXFP4 block-scaled formats (OCP MX spec: 32
  elements share one E8M0 power-of-two scale).

Readings (the pages give no formulas):
* Per-tensor scale: amax = max|x| (after the RHT when it applies);
  s_enc = 2688 / amax in float32 (2688 = 448 * 6, the largest E4M3 scale times
  the largest E2M1 value), 1 if amax == 0, clamped to FLT_MAX;
  s_dec = 1 / s_enc in float32, used by consumers.
* Block step, in this float32 order: a_b = block amax; sf = (a_b / 6) * s_enc;
  S = E4M3_RNE_sat(sf); sfq = decode(S);
  enc = 0 if sfq == 0 else min(s_enc / sfq, FLT_MAX); v = x * enc;
  code = E2M1(v) by RNE or stochastic rounding.
  (The min(.., FLT_MAX) keeps enc finite for blocks of denormal-range inputs.)
* MX block (OCP floor rule): a_b = block amax; e = floor(log2 a_b) - emax with
  emax = 2 (E2M1) or 8 (E4M3); e = -127 for an all-zero block; e is clamped
  to [-127, 127] and stored as the E8M0 code e + 127; v = x * 2**-e (float32);
  element = E2M1_RNE / E2M1_SR (saturate at 6) or E4M3_RNE (saturate at 448).
* Layouts: rowwise codes [R, C/2] (FP4) or [R, C] (FP8), scales [R, C/B].
  Columnwise = the rowwise quantization of x^T ([C, R]).  2D 16x16 scales are
  stored expanded in both: row scales[r, j] = S[r//16, j], column
  scales[c, i] = S[i, c//16].
* Stochastic rounding streams: rowwise outputs use stream 0, columnwise
  outputs stream 1 (oracle/philox.py).
"""

import numpy as np

from . import formats as F
from .philox import sr_random16_grid, STREAM_ROW, STREAM_COL
from .rht import rht_along_rows, rht16

NVFP4_BLOCK = 16
MX_BLOCK = 32


def as_f32(x):
    """Accept BF16 bit patterns (uint16) or float32 values; return float32."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return F.bf16_bits_to_f32(x)
    assert x.dtype == np.float32
    return x


# --------------------------------------------------------------------------
# NVFP4
# --------------------------------------------------------------------------

def tensor_amax(y):
    """max |y| over the whole tensor (float32, exact)."""
    y = np.asarray(y, dtype=np.float32)
    if y.size == 0:
        return np.float32(0.0)
    return np.float32(np.max(np.abs(y)))


def nvfp4_scale_enc(amax):
    """Per-tensor encode scale s_enc = 2688 / amax (float32), 1 for amax == 0."""
    amax = np.float32(amax)
    if amax == 0:
        return np.float32(1.0)
    with np.errstate(over="ignore", divide="ignore"):
        s = np.float32(2688.0) / amax
    return np.float32(min(s, F.FLT_MAX))


def nvfp4_scale_dec(amax):
    """Per-tensor decode scale s_dec = 1 / s_enc (float32)."""
    return np.float32(np.float32(1.0) / nvfp4_scale_enc(amax))


def nvfp4_block_amax(y, block_rows):
    """Block amax [R, C/16]: 1x16 blocks, or 16x16 tiles expanded to every row."""
    R, C = y.shape
    a = np.abs(y).reshape(R, C // 16, 16).max(axis=2)
    if block_rows == 16:
        t = a.reshape(R // 16, 16, C // 16).max(axis=1)     # [R/16, C/16]
        a = np.repeat(t, 16, axis=0)
    return a.astype(np.float32)


def nvfp4_encode_blocks(y, block_amax, s_enc, rnd, r16=None):
    """Encode float32 values y [R, C] given their block amax [R, C/16]."""
    R, C = y.shape
    sf = (block_amax / np.float32(6.0)) * np.float32(s_enc)       # two float32 ops
    S = F.e4m3_encode_rne(sf.astype(np.float32))
    sfq = F.e4m3_decode(S)
    with np.errstate(over="ignore", divide="ignore", invalid="ignore"):
        enc = np.where(sfq == 0, np.float32(0.0),
                       np.minimum(np.float32(s_enc) / sfq, F.FLT_MAX)).astype(np.float32)
    v = (y.reshape(R, C // 16, 16) * enc[:, :, None]).reshape(R, C).astype(np.float32)
    if rnd == "rne":
        codes = F.e2m1_encode_rne(v)
    else:
        codes = F.e2m1_encode_sr(v, r16)
    return F.pack_e2m1(codes), S


def nvfp4_quantize(x, block_rows=1, rnd="rne", seed=0, offset=0, stream=STREAM_ROW,
                   rht=False, rht_signs=0, amax=None, row_ids=None):
    """Rowwise NVFP4 of x [R, C] (blocks along C).

    Returns (codes uint8 [R, C/2], scales uint8 [R, C/16], amax float32).
    With rht=True the RHT is applied along C first and amax is taken over the
    transformed values.  `amax` may be supplied (it is then used as given).
    row_ids: when x holds only some rows of a larger tensor (whole 16-row tiles
    for block_rows=16), their global row indices; they place the stochastic
    rounding stream.  amax must then be given.
    """
    y = as_f32(x)
    R, C = y.shape
    assert C % 16 == 0 and block_rows in (1, 16)
    if block_rows == 16:
        assert R % 16 == 0
    if rht:
        y = rht_along_rows(y, rht_signs)
    if amax is None:
        amax = tensor_amax(y)
    s_enc = nvfp4_scale_enc(amax)
    if row_ids is not None:
        assert amax is not None and len(row_ids) == R
    r16 = sr_random16_grid(R, C, seed, offset, stream, row_ids) if rnd == "sr" else None
    codes, S = nvfp4_encode_blocks(y, nvfp4_block_amax(y, block_rows), s_enc, rnd, r16)
    return codes, S, np.float32(amax)


def tensor_amax_rht_cols(x, rht_signs, chunk_rows=2048):
    """max |RHT(x^T)| over a whole tensor x [R, C]: the RHT runs along R (the
    blocked dimension of x^T).  Same definition as tensor_amax(rht_along_rows(x^T)),
    evaluated over 16-row slabs of x at a time to bound memory."""
    R, C = x.shape
    assert R % 16 == 0 and chunk_rows % 16 == 0
    m = np.float32(0.0)
    for r0 in range(0, R, chunk_rows):
        y = as_f32(x[r0:r0 + chunk_rows])
        n = y.shape[0] // 16
        chunks = np.ascontiguousarray(y.reshape(n, 16, C).transpose(0, 2, 1))   # [n, C, 16]
        m = max(m, tensor_amax(rht16(chunks, rht_signs)))
    return np.float32(m)


# --------------------------------------------------------------------------
# MX (MXFP4 / MXFP8)
# --------------------------------------------------------------------------

MX_EMAX = {"mxfp4": 2, "mxfp8": 8}


def mx_scale_exponent(block_amax, fmt):
    """Shared exponent e per 32-block (int64), OCP floor rule, clamped to [-127, 127]."""
    a = np.asarray(block_amax, dtype=np.float32)
    e = np.full(a.shape, -127, dtype=np.int64)
    nz = a > 0
    e[nz] = F.floor_log2(a[nz]) - MX_EMAX[fmt]
    return np.clip(e, -127, 127)


def mx_quantize(x, fmt="mxfp4", rnd="rne", seed=0, offset=0, stream=STREAM_ROW, row_ids=None):
    """Rowwise MX quantization of x [R, C] (blocks of 32 along C).

    Returns (codes, scales): codes uint8 [R, C/2] (mxfp4) or [R, C] (mxfp8),
    scales uint8 [R, C/32] (E8M0 codes)."""
    y = as_f32(x)
    R, C = y.shape
    assert C % MX_BLOCK == 0
    blocks = y.reshape(R, C // 32, 32)
    e = mx_scale_exponent(np.abs(blocks).max(axis=2), fmt)
    mult = np.ldexp(np.float32(1.0), (-e).astype(np.int32)).astype(np.float32)  # 2**-e, exact
    v = (blocks * mult[:, :, None]).reshape(R, C).astype(np.float32)
    if fmt == "mxfp4":
        if rnd == "rne":
            codes = F.e2m1_encode_rne(v)
        else:
            codes = F.e2m1_encode_sr(v, sr_random16_grid(R, C, seed, offset, stream, row_ids))
        codes = F.pack_e2m1(codes)
    else:
        assert rnd == "rne"
        codes = F.e4m3_encode_rne(v)
    return codes, (e + 127).astype(np.uint8)


# --------------------------------------------------------------------------
# Both orientations
# --------------------------------------------------------------------------

def quantize_transpose(x, fmt="nvfp4", block_rows=1, rnd="rne", seed=0, offset=0,
                       rht_col=False, rht_signs=0):
    """Row and column quantizations of x [R, C].

    row = quantize(x) (stream 0, never rotated); col = quantize(x^T) (stream 1;
    with rht_col the RHT runs along R, the blocked dimension of x^T).
    Returns dict with row_codes, row_scales, row_amax, col_codes, col_scales,
    col_amax (amax entries are None for MX formats)."""
    y = as_f32(x)
    yt = np.ascontiguousarray(y.T)
    if fmt == "nvfp4":
        rc, rs, ra = nvfp4_quantize(y, block_rows, rnd, seed, offset, STREAM_ROW)
        cc, cs, ca = nvfp4_quantize(yt, block_rows, rnd, seed, offset, STREAM_COL,
                                    rht=rht_col, rht_signs=rht_signs)
    else:
        assert block_rows == 1 and not rht_col
        rc, rs = mx_quantize(y, fmt, rnd, seed, offset, STREAM_ROW)
        cc, cs = mx_quantize(yt, fmt, rnd, seed, offset, STREAM_COL)
        ra = ca = None
    return dict(row_codes=rc, row_scales=rs, row_amax=ra,
                col_codes=cc, col_scales=cs, col_amax=ca)


# --------------------------------------------------------------------------
# Per-tensor FP8: the FP8 baseline the NVFP4 post measures against
# --------------------------------------------------------------------------
#
# NVFP4 pretraining post: the paragraph after the example script names the
# FP8 baseline run (MaxText quantization=te_fp8_delayedscaling), and section
# "Performance results" (Table 1, Figure 2) compares NVFP4 with it.  The pages
# give no formula.  Readings: every tensor is E4M3 (OCP E4M3FN) under one
# float32 per-tensor scale taken from the tensor's own amax (the amax history
# of delayed scaling, which spans training steps, is left out):
#     s_enc = 448 / amax (1 if amax == 0, at most FLT_MAX), s_dec = 1 / s_enc,
#     code  = E4M3_RNE_sat(x * s_enc)      (one float32 multiply),
# and the column output is the same rule applied to x^T (same amax).

FP8_MAX = 448.0


def fp8_scale_enc(amax):
    """Per-tensor FP8 encode scale 448 / amax (float32), 1 for amax == 0."""
    amax = np.float32(amax)
    if amax == 0:
        return np.float32(1.0)
    with np.errstate(over="ignore", divide="ignore"):
        s = np.float32(FP8_MAX) / amax
    return np.float32(min(s, F.FLT_MAX))


def fp8_scale_dec(amax):
    """Per-tensor FP8 decode scale 1 / s_enc (float32)."""
    return np.float32(np.float32(1.0) / fp8_scale_enc(amax))


def fp8_quantize(x, amax=None):
    """Per-tensor FP8 of x [R, C]: (codes uint8 [R, C] E4M3, amax float32)."""
    y = as_f32(x)
    if amax is None:
        amax = tensor_amax(y)
    v = (y * fp8_scale_enc(amax)).astype(np.float32)
    return F.e4m3_encode_rne(v), np.float32(amax)


def fp8_quantize_transpose(x):
    """Row (x) and column (x^T) per-tensor FP8 outputs under one amax."""
    y = as_f32(x)
    rc, amax = fp8_quantize(y)
    cc, _ = fp8_quantize(np.ascontiguousarray(y.T), amax)
    return dict(row_codes=rc, col_codes=cc, amax=amax)
