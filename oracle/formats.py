"""Element and scale formats: E2M1, E4M3 (OCP E4M3FN), E8M0, BF16.

Test infrastructure only (see oracle/__init__.py).

Definitions follow the OCP Microscaling Formats spec linked from the
"HN page opcode84" (E2M1 elements, E4M3 elements, E8M0 scales) and the
"NVFP4 pretraining post", section "NVFP4 pretraining recipe", ingredient 2
(E4M3 block scale factors with mantissa bits) and ingredient 5 (round to
nearest even for weights and activations, stochastic rounding for gradients).

Readings where the pages are silent:
* E2M1 magnitudes are {0, 0.5, 1, 1.5, 2, 3, 4, 6}; no Inf/NaN; anything
  above the top grid point saturates to 6 (code 7).  RNE ties go to the even
  code.  The sign bit (0x8) is kept, so -0 and small negatives become 0x8.
* Two E2M1 codes per byte, the element with the even index in the low nibble.
* E4M3 is OCP E4M3FN: bias 7, subnormals kept, max 448, 0x7F/0xFF are NaN and
  are never produced; values above 448 saturate to 448 (0x7E).
* Stochastic rounding uses 16 random bits per element: with lo <= a < hi the
  neighbouring grid points and frac = (a - lo) / (hi - lo), the element rounds
  up iff r16 < floor(frac * 2**16).
"""

import numpy as np

FLT_MAX = np.float32(np.finfo(np.float32).max)

# E2M1 magnitude by 3-bit magnitude code.
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)
E2M1_MAX = np.float32(6.0)
E4M3_MAX = np.float32(448.0)


# --------------------------------------------------------------------------
# BF16
# --------------------------------------------------------------------------

def bf16_bits_to_f32(bits):
    """BF16 bit patterns (uint16) -> float32 values (exact widening)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f64_to_bf16_rne(x):
    """float64 -> nearest BF16 value (ties to even), returned as float64.

    Used only to report how many GEMM outputs equal the correctly rounded
    reference.  Rounds directly from float64 (no float32 double rounding).
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = (x != 0) & np.isfinite(x)
    f, e = np.frexp(x[nz])               # x = f * 2**e, 0.5 <= |f| < 1
    e = np.maximum(e, -125)               # below 2**-126 the BF16 quantum is fixed at 2**-133
    q = np.rint(np.ldexp(x[nz], 8 - e))   # 8 significant bits, RNE
    out[nz] = np.ldexp(q, e - 8)
    out[~np.isfinite(x)] = x[~np.isfinite(x)]
    return out


# --------------------------------------------------------------------------
# E2M1 (4-bit elements)
# --------------------------------------------------------------------------

def e2m1_decode(codes):
    """4-bit codes -> float32 values (sign bit 0x8)."""
    codes = np.asarray(codes, dtype=np.uint8)
    mag = E2M1_MAGNITUDES[codes & 7]
    return np.where((codes & 8) != 0, -mag, mag).astype(np.float32)


def e2m1_encode_rne(v):
    """float32 -> 4-bit codes by round-to-nearest, ties to the even code,
    saturating at 6.

    The magnitude code is read off the decision table on a = |v|:
    a <= 0.25 -> 0, a < 0.75 -> 1, a <= 1.25 -> 2, a < 1.75 -> 3,
    a <= 2.5 -> 4, a < 3.5 -> 5, a <= 5 -> 6, otherwise 7.
    The thresholds are the midpoints of neighbouring grid values; whether the
    midpoint itself goes down (<=) or up (<) is fixed by which neighbour has
    the even code.
    """
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v)
    m = np.full(a.shape, 7, dtype=np.uint8)
    m[a <= 5.0] = 6
    m[a < 3.5] = 5
    m[a <= 2.5] = 4
    m[a < 1.75] = 3
    m[a <= 1.25] = 2
    m[a < 0.75] = 1
    m[a <= 0.25] = 0
    sign = np.signbit(v).astype(np.uint8) << 3
    return (m | sign).astype(np.uint8)


def e2m1_encode_sr(v, r16):
    """float32 -> 4-bit codes by stochastic rounding with 16-bit random words.

    a = |v|.  If a >= 6 the magnitude code is 7.  Otherwise lo <= a < hi are
    the neighbouring grid magnitudes (their gap is 0.5, 1 or 2, a power of
    two, so frac = (a - lo) / (hi - lo) is exact in float32) and the element
    rounds up to hi iff r16 < floor(frac * 2**16).  Grid points never move;
    P(up) = floor(frac * 2**16) / 2**16.
    """
    v = np.asarray(v, dtype=np.float32)
    r16 = np.asarray(r16, dtype=np.uint32)
    a = np.abs(v)
    # index of the largest grid magnitude <= a (a < 6 here)
    lo_idx = np.searchsorted(E2M1_MAGNITUDES, a, side="right").astype(np.int64) - 1
    lo_idx = np.clip(lo_idx, 0, 6)
    lo = E2M1_MAGNITUDES[lo_idx]
    hi = E2M1_MAGNITUDES[lo_idx + 1]
    frac = (a - lo) / (hi - lo)                                   # float32, exact
    frac = np.where(a >= E2M1_MAX, np.float32(0.0), frac)         # saturated below
    t = np.floor(frac * np.float32(65536.0)).astype(np.uint32)   # 0 .. 65535
    up = r16 < t
    m = (lo_idx + up).astype(np.uint8)
    m = np.where(a >= E2M1_MAX, np.uint8(7), m).astype(np.uint8)
    sign = np.signbit(v).astype(np.uint8) << 3
    return (m | sign).astype(np.uint8)


def pack_e2m1(codes):
    """[..., 2n] 4-bit codes -> [..., n] bytes, even index in the low nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    assert codes.shape[-1] % 2 == 0
    lo = codes[..., 0::2]
    hi = codes[..., 1::2]
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_e2m1(packed):
    """[..., n] bytes -> [..., 2n] 4-bit codes."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0x0F
    out[..., 1::2] = packed >> 4
    return out


# --------------------------------------------------------------------------
# E4M3 (OCP E4M3FN): NVFP4 block scales and MXFP8 elements
# --------------------------------------------------------------------------

def e4m3_decode(codes):
    """8-bit E4M3FN codes -> float32 (0x7F/0xFF decode to NaN)."""
    codes = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (codes >> 7) & 1
    e = (codes >> 3) & 0xF
    m = codes & 7
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64), -9),
                   np.ldexp((8 + m).astype(np.float64), e - 10))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag).astype(np.float32)


def e4m3_encode_rne(s):
    """float32 -> E4M3FN code, round to nearest even, saturating at 448.

    For a = |s|:
    * a > 448            -> 0x7E (448)
    * a < 2**-6          -> subnormal: q = rint(a * 2**9), code q (q = 8 is
                            the smallest normal, which the encoding gives
                            naturally)
    * otherwise          -> e = floor(log2 a), m = rint(a * 2**(3 - e));
                            if m == 16 then e += 1, m = 8;
                            code = ((e + 7) << 3) | (m - 8)
    The sign bit is taken from the sign of s (so -0 -> 0x80).  All steps are
    exact in float64 except the two rint() calls, which are the rounding.
    """
    s = np.asarray(s, dtype=np.float32)
    a = np.abs(s).astype(np.float64)
    code = np.zeros(a.shape, dtype=np.int64)

    sub = a < 2.0 ** -6
    code[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)

    nrm = ~sub & (a <= 448.0)
    f, ex = np.frexp(a[nrm])            # a = f * 2**ex, 0.5 <= f < 1
    e = ex - 1                          # floor(log2 a)
    m = np.rint(np.ldexp(a[nrm], 3 - e)).astype(np.int64)
    carry = m == 16
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 8, m)
    code[nrm] = ((e + 7) << 3) | (m - 8)

    code[a > 448.0] = 0x7E
    code = code | (np.signbit(s).astype(np.int64) << 7)
    return code.astype(np.uint8)


# --------------------------------------------------------------------------
# E8M0 power-of-two scales (MX formats)
# --------------------------------------------------------------------------

def e8m0_decode(codes):
    """E8M0 code -> float64 2**(code - 127) (code 255 is NaN, never produced)."""
    codes = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    out = np.ldexp(1.0, codes - 127)
    return np.where(codes == 255, np.nan, out)


def floor_log2(a):
    """floor(log2 a) for finite a > 0 (float32 or float64 input), exact via frexp."""
    _, ex = np.frexp(np.asarray(a, dtype=np.float64))
    return ex.astype(np.int64) - 1
