// Pieces shared by the block-scaled GEMM kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsq {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;     // NaN stays NaN
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// E4M3 byte SEL of w -> float (exact; OCP E4M3FN on gfx950).
template <int SEL>
__device__ __forceinline__ float e4m3_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8((int)w, SEL);
}

// Block scale S (E4M3 byte SEL of w) as the FP16 pair {S * 2^7, S * 2^7}
// (exact: S * 2^7 lies in [2^-2, 57344]).
template <int SEL>
__device__ __forceinline__ halfx2 nvfp4_scale_pair(uint32_t w) {
  const float s = e4m3_to_f32<SEL>(w) * 128.0f;
  return __builtin_bit_cast(halfx2, __builtin_amdgcn_cvt_pkrtz(s, s));
}

// 8 E2M1 codes (nibble i = element i of one dword) times a block scale, as 8
// FP16 values v * S * 2^-7 (exact), in element order.
// E2M1 is a 1-sign / 2-exponent / 1-mantissa float, so an FP16 whose high byte
// is (sign << 7) | (magnitude bits << 1) and whose low byte is 0 equals
// exactly v * 2^-14 (code 1, 0.5, lands on the FP16 subnormal 0.5 * 2^-14).
// The high bytes of the even and odd nibbles are built four at a time, then
// byte permutes pair them with zero low bytes.  The packed FP16 multiply by
// S * 2^7 is exact: v * S has at most 6 significant bits and its lowest bit is
// >= 2^-10, so v * S * 2^-7 is representable (FP16 denormals are kept).  The
// MFMA products carry 2^-14 per operand pair, undone in the epilogue.
__device__ __forceinline__ halfx8 dequant8(uint32_t w, halfx2 s2) {
  const uint32_t he = ((w & 0x07070707u) << 1) | ((w << 4) & 0x80808080u);          // nibbles 0,2,4,6
  const uint32_t ho = (((w >> 4) & 0x07070707u) << 1) | (w & 0x80808080u);          // nibbles 1,3,5,7
  // dword k = FP16 {element 2k, element 2k+1}: bytes {0, he.k, 0, ho.k}
  const uint32_t d0 = __builtin_amdgcn_perm(ho, he, 0x040C000Cu);
  const uint32_t d1 = __builtin_amdgcn_perm(ho, he, 0x050C010Cu);
  const uint32_t d2 = __builtin_amdgcn_perm(ho, he, 0x060C020Cu);
  const uint32_t d3 = __builtin_amdgcn_perm(ho, he, 0x070C030Cu);
  const halfx2 p0 = __builtin_bit_cast(halfx2, d0) * s2;
  const halfx2 p1 = __builtin_bit_cast(halfx2, d1) * s2;
  const halfx2 p2 = __builtin_bit_cast(halfx2, d2) * s2;
  const halfx2 p3 = __builtin_bit_cast(halfx2, d3) * s2;
  return __builtin_bit_cast(halfx8, make_uint4(__builtin_bit_cast(uint32_t, p0),
                                               __builtin_bit_cast(uint32_t, p1),
                                               __builtin_bit_cast(uint32_t, p2),
                                               __builtin_bit_cast(uint32_t, p3)));
}

__device__ __forceinline__ float nvfp4_s_dec(float amax) {
  const float s_enc = amax == 0.0f ? 1.0f : fminf(2688.0f / amax, 3.40282346638528859812e+38f);
  return 1.0f / s_enc;
}

// Output tile of block `pid`.  Workgroups are dealt round-robin to the 8 XCDs
// (each with its own L2), so block pid runs on XCD pid % 8; the remap gives
// every XCD one contiguous run of the tile order, and the tile order sweeps
// GROUP_M tile rows at a time so neighbouring tiles share A rows and B rows.
__device__ __forceinline__ void tile_of_block(int pid, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int kXcd = 8, kGroupM = 8;
  const int nt = tiles_m * tiles_n;
  const int q = nt / kXcd, r = nt % kXcd;
  const int x = pid % kXcd, i = pid / kXcd;
  const int t = x * q + (x < r ? x : r) + i;
  const int group_size = kGroupM * tiles_n;
  const int first_m = (t / group_size) * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  tm = first_m + (t % group_size) % gm;
  tn = (t % group_size) / gm;
}

}  // namespace bsq
