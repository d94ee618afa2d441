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
// gfx950's FP4 -> FP16 pair convert turns byte k of the dword (elements 2k and
// 2k + 1, low nibble first) into two FP16 values multiplied by the power of
// two of its scale operand; with 2^-14 it yields v * 2^-14 exactly, FP16
// subnormals and signed zeros included (checked on every byte value at scales
// 1, 2^-7, 2^-14 and 2^-20).  The packed FP16 multiply by S * 2^7 is exact:
// v * S has at most 6 significant bits and its lowest bit is >= 2^-10, so
// v * S * 2^-7 is representable (FP16 denormals are kept).  The MFMA products
// carry 2^-14 per operand pair, undone in the epilogue.
__device__ __forceinline__ halfx8 dequant8(uint32_t w, halfx2 s2) {
  const float k = 0x1p-14f;
  const halfx2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, k, 0) * s2;
  const halfx2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, k, 1) * s2;
  const halfx2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, k, 2) * s2;
  const halfx2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, k, 3) * s2;
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
