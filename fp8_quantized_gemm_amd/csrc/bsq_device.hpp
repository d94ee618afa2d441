// Device-side codecs for the block quantizers (gfx950).
//
// E2M1 / E4M3 / E8M0 encoders, the NVFP4 block-scale step, the 16-point
// Hadamard butterfly and Philox4x32-10.  Every function reproduces the
// numerical contract stated in include/bsq.h bit for bit: IEEE float32 RNE
// operations, denormals kept (the default gfx950 float mode), and this file
// is compiled with -ffp-contract=off so no multiply-add is fused.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsq {

constexpr float kFltMax = 3.40282346638528859812e+38f;

__device__ __forceinline__ uint32_t f2u(float f) { return __float_as_uint(f); }
__device__ __forceinline__ float u2f(uint32_t u) { return __uint_as_float(u); }

// BF16 halves of a packed dword -> float32 (exact widening).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return u2f(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return u2f(w & 0xFFFF0000u); }

// Two FP32 values -> a packed BF16 pair (lo in bits 0-15), rounded to nearest
// even by the hardware pack: the same bits as the integer rounding rule for
// every non-NaN input, denormals and ties included; NaN stays NaN.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------- E2M1
// Magnitude code (0..7) of a = |v| by round-to-nearest, ties to the even code,
// saturating at 6 (OCP MX E2M1 element).
//  * a < 1: the grid is {0, 0.5, 1}; the code is (a > 0.25) + (a >= 0.75).
//  * a >= 1: E2M1 is a float with one significand bit, so rounding the FP32
//    significand to one bit (add 0x1FFFFF plus the kept bit, then drop 22
//    bits) gives ((exp - 127) * 2 + mantissa bit), offset so 1.0 -> code 2.
// For finite a >= 0 float ordering equals unsigned ordering of the bits.
__device__ __forceinline__ uint32_t e2m1_rne_mag(float a) {
  const uint32_t b = f2u(a);
  const uint32_t lo = (b > 0x3E800000u ? 1u : 0u) + (b >= 0x3F400000u ? 1u : 0u);
  const uint32_t r = (b + 0x1FFFFFu + ((b >> 22) & 1u)) >> 22;
  const uint32_t hi = min(r - 252u, 7u);
  return b < 0x3F800000u ? lo : hi;
}

// ---------------------------------------------------------------- E4M3
// OCP E4M3FN code (0..0x7E) of a >= 0 by RNE, saturating at 448, subnormals
// kept.  Normal range: round the FP32 significand to 3 bits (drop 20 bits with
// the ties-to-even bias) and rebias the exponent (127 - 7) << 3 = 960;
// a significand carry increments the exponent field by itself.
__device__ __forceinline__ uint32_t e4m3_rne_mag(float a) {
  const uint32_t b = f2u(a);
  if (b > 0x43E00000u) return 0x7Eu;                 // > 448 (and Inf / NaN)
  if (b < 0x3C800000u)                                // < 2^-6: grid 2^-9
    return (uint32_t)__builtin_rintf(a * 512.0f);    // 0..8 (8 = min normal)
  const uint32_t r = b + 0x7FFFFu + ((b >> 20) & 1u);
  return (r >> 20) - 960u;
}

// Decode an unsigned E4M3 code (0..0x7E) exactly.
__device__ __forceinline__ float e4m3_decode_mag(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  return e ? u2f(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
}

// ---------------------------------------------------------------- NVFP4 scales
// Per-tensor encode scale: 2688 / amax (2688 = 448 * 6), 1 for amax == 0,
// at most FLT_MAX.
__device__ __forceinline__ float nvfp4_s_enc(float amax) {
  if (amax == 0.0f) return 1.0f;
  return fminf(2688.0f / amax, kFltMax);
}

// Correctly rounded a / 6 for a >= 0.  For a >= 2^-120 the quotient is a
// normal float and one FMA correction step on a * RN(1/6) gives the IEEE
// result (checked against IEEE division on every FP32 input on gfx950);
// below that, plain IEEE division.
__device__ __forceinline__ float div6(float a) {
  if (a < 0x1p-120f) return a / 6.0f;
  const float y = 1.0f / 6.0f;
  const float q = a * y;
  const float r = __builtin_fmaf(-q, 6.0f, a);
  return __builtin_fmaf(r, y, q);
}

// E4M3 code (0..0x7E) of the block scale sf = (a_b / 6) * s_enc, RNE and
// saturating at 448.  The hardware FP32 -> E4M3 convert rounds to nearest
// even and agrees with e4m3_rne_mag on [0, 464) (checked exhaustively); the
// clamp maps everything above 448 (reachable only with a caller-supplied
// amax below the true one) to 448, as e4m3_rne_mag does.  sf is never
// negative, so the code fits 7 bits; the mask keeps it below 128 even for
// non-finite inputs, where it indexes the 128-entry encode-factor tables.
__device__ __forceinline__ uint32_t nvfp4_scale_code(float a_b, float s_enc) {
  const float sf = fminf(div6(a_b) * s_enc, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sf, 0.0f, 0, false) & 0x7Fu;
}

// Encode factor for every E4M3 scale code: enc = s_enc / S (0 for S == 0),
// clamped to FLT_MAX.  Filled once per workgroup into LDS (128 entries).
__device__ __forceinline__ float nvfp4_enc_of_code(uint32_t c, float s_enc) {
  if (c == 0) return 0.0f;
  return fminf(s_enc / e4m3_decode_mag(c), kFltMax);
}

// Reference block step (one IEEE division), kept for the generic paths.
struct BlockScale {
  uint32_t code;
  float enc;
};
__device__ __forceinline__ BlockScale nvfp4_block_scale(float a_b, float s_enc) {
  BlockScale bs;
  bs.code = nvfp4_scale_code(a_b, s_enc);
  bs.enc = nvfp4_enc_of_code(bs.code, s_enc);
  return bs;
}

// ---------------------------------------------------------------- E2M1 (hardware pack)
// Eight FP32 values -> eight E2M1 codes, RNE, packed low nibble first.  The
// gfx950 packed convert (scale 1.0) implements exactly the E2M1 RNE rule of
// e2m1_rne_mag plus the sign bit, on every FP32 input (checked
// exhaustively); byte k of the result holds elements 2k (low) and 2k+1.
__device__ __forceinline__ uint32_t fp4x8_rne(const float (&v)[8]) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], 1.0f, 3);
  return w;
}

// ---------------------------------------------------------------- E8M0 (MX)
// floor(log2 a) for finite a > 0, including FP32 subnormals.
__device__ __forceinline__ int floor_log2(float a) {
  const uint32_t b = f2u(a);
  if (b >= 0x00800000u) return (int)(b >> 23) - 127;
  return (31 - (int)__builtin_clz(b)) - 149;
}

// Shared MX exponent of a block with amax a_b: floor(log2 a_b) - emax, -127 for
// a zero block, clamped to [-127, 127].
__device__ __forceinline__ int mx_exponent(float a_b, int emax) {
  if (a_b == 0.0f) return -127;
  const int e = floor_log2(a_b) - emax;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// 2^-e as an exact float32 (2^-127 is the subnormal 0x00400000).
__device__ __forceinline__ float exp2_neg(int e) {
  const int k = 127 - e;                 // biased exponent of 2^-e
  return k >= 1 ? u2f((uint32_t)k << 23) : u2f(0x00400000u);
}

// ---------------------------------------------------------------- RHT
// y <- H16 * D * y on 16 values held in one thread (natural-order Sylvester
// H16; bit i of signs negates element i first), without the 1/4.
__device__ __forceinline__ void rht16_unscaled(float (&y)[16], uint32_t signs) {
#pragma unroll
  for (int i = 0; i < 16; ++i) y[i] = u2f(f2u(y[i]) ^ (((signs >> i) & 1u) << 31));
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((i & h) == 0) {
        const float a = y[i], b = y[i + h];
        y[i] = a + b;
        y[i + h] = a - b;
      }
    }
  }
}

// y <- 0.25 * H16 * D * y.
__device__ __forceinline__ void rht16(float (&y)[16], uint32_t signs) {
  rht16_unscaled(y, signs);
#pragma unroll
  for (int i = 0; i < 16; ++i) y[i] = y[i] * 0.25f;
}

// ---------------------------------------------------------------- cross-lane
// quad_perm DPP moves: lane ^ 1 and lane ^ 2 within each group of four lanes.
__device__ __forceinline__ uint32_t dpp_xor1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t dpp_xor2(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
}
__device__ __forceinline__ float dpp_xor1f(float v) { return u2f(dpp_xor1(f2u(v))); }

// ---------------------------------------------------------------- Philox4x32-10
// Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"
// (SC'11).  Ten rounds; multipliers 0xD2511F53 / 0xCD9E8D57; Weyl key bumps
// 0x9E3779B9 / 0xBB67AE85.
struct U4 {
  uint32_t x, y, z, w;
};
__device__ __forceinline__ void philox_round(uint32_t& c0, uint32_t& c1, uint32_t& c2, uint32_t& c3,
                                             uint32_t k0, uint32_t k1) {
  const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
  const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
  // three-input XORs as single v_bitop3_b32 (truth table 0x96)
  const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
  const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
  c0 = n0;
  c1 = (uint32_t)p1;
  c2 = n2;
  c3 = (uint32_t)p0;
}

// The four output words, each bitwise complemented (~x, ~y, ~z, ~w): the
// stochastic-rounding pack below takes 65535 - r16 = ~r16, and the last
// round's three-input XORs give ~x and ~z at no cost (truth table 0x69).
__device__ __forceinline__ U4 philox10_not(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                           uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 9; ++r) {
    philox_round(c0, c1, c2, c3, k0, k1);
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
  const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
  const uint32_t nx = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x69);
  const uint32_t nz = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x69);
  return U4{nx, ~(uint32_t)p1, nz, ~(uint32_t)p0};
}

// Eight 16-bit random words for elements idx = 8*grp + j, j = 0..7 (Philox
// output word j>>1, low half for even j), held complemented: nw[k] = ~word k,
// so the half of element j is 65535 - r16(j).
struct R16x8 {
  uint32_t nw[4];
};
__device__ __forceinline__ R16x8 sr_words(uint64_t grp, uint64_t seed, uint32_t offset, uint32_t stream) {
  const U4 r = philox10_not((uint32_t)grp, (uint32_t)(grp >> 32), offset, stream,
                            (uint32_t)seed, (uint32_t)(seed >> 32));
  R16x8 o;
  o.nw[0] = r.x;
  o.nw[1] = r.y;
  o.nw[2] = r.z;
  o.nw[3] = r.w;
  return o;
}

// ---------------------------------------------------------------- E2M1 (stochastic rounding)
// Eight FP32 values -> eight E2M1 codes by stochastic rounding, packed low
// nibble first.  The rule: with lo <= |v| < hi the neighbouring E2M1
// magnitudes and r16 the element's 16-bit random word, round up to hi iff
// r16 < floor((|v| - lo) / (hi - lo) * 65536); |v| >= 6 gives 6; the sign is
// kept.
// gfx950's stochastic FP4 pack (scale 1.0) rounds |v| up iff
// floor(frac * 2^22) + R >= 2^22, with frac the same position between the two
// magnitudes and R bits 31..10 of its random operand for the first value of the
// pair (bits 30..9 for the second), saturating at 6 and keeping the sign
// (measured on 2^21 random inputs against that formula, no mismatch).  With
// R = (65535 - r16) << 6 the carry happens iff r16 < floor(frac * 2^16), which
// is the rule above bit for bit.  The two random fields of one instruction
// overlap, so each pair is converted twice: once with the even element's
// 65535 - r16 in bits 31..16 (bits 15..0 zero), once with the odd element's
// in bits 30..15 (bits 14..0 zero).  The instruction writes only the byte its
// op_sel names and keeps the other three, so pair k's two conversions go to
// byte k of two words, e (even nibbles valid) and o (odd nibbles valid), and
// one bitwise select merges them.  Written as inline assembly with the words
// as tied operands: the compiler's builtin does not tie the kept bytes.  The
// s_nop after each conversion gives the wait state a VALU read of a
// byte-selected destination needs, which the compiler cannot insert for
// inline assembly.
template <int K>
__device__ __forceinline__ void sr_pk_fp4_byte(uint32_t& dst, float a, float b, uint32_t rnd) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  const f2 pr = {a, b};
  if constexpr (K == 0)   // bytes 1-3 are written by the later conversions
    asm volatile("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0\n\ts_nop 0" : "=v"(dst) : "v"(pr), "v"(rnd));
  else if constexpr (K == 1)
    asm volatile("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0 op_sel:[0,0,1,0]\n\ts_nop 0"
                 : "+v"(dst) : "v"(pr), "v"(rnd));
  else if constexpr (K == 2)
    asm volatile("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0 op_sel:[0,0,0,1]\n\ts_nop 0"
                 : "+v"(dst) : "v"(pr), "v"(rnd));
  else
    asm volatile("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0 op_sel:[0,0,1,1]\n\ts_nop 0"
                 : "+v"(dst) : "v"(pr), "v"(rnd));
}

template <int K = 0>
__device__ __forceinline__ void fp4x8_sr_pairs(const float (&v)[8], const R16x8& rnd, uint32_t& e,
                                               uint32_t& o) {
  if constexpr (K < 4) {
    const uint32_t nw = rnd.nw[K];
    sr_pk_fp4_byte<K>(e, v[2 * K], v[2 * K + 1], nw << 16);
    sr_pk_fp4_byte<K>(o, v[2 * K], v[2 * K + 1], (nw >> 1) & 0x7FFF8000u);
    fp4x8_sr_pairs<K + 1>(v, rnd, e, o);
  }
}

__device__ __forceinline__ uint32_t fp4x8_sr(const float (&v)[8], const R16x8& rnd) {
  uint32_t e, o;
  fp4x8_sr_pairs<0>(v, rnd, e, o);
  return (e & 0x0F0F0F0Fu) | (o & 0xF0F0F0F0u);   // one bitfield insert
}

}  // namespace bsq
