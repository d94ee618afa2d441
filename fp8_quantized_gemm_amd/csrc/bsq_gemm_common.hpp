// Pieces shared by the block-scaled GEMM kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsq_device.hpp"   // pack_bf16x2

namespace bsq {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx2 __attribute__((ext_vector_type(2)));

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

// Block scales of E4M3 bytes 2H and 2H + 1 of w as the FP16 pair
// {S0 * 2^7, S1 * 2^7} in one scaled convert (the scale operand contributes
// its power of two; exact for the same reason).
template <int H>
__device__ __forceinline__ halfx2 nvfp4_scale_pairs2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 128.0f, H != 0);
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

// Per-tensor FP8 decode scale: 1 / (448 / amax), 1 for amax == 0.
__device__ __forceinline__ float fp8_s_dec(float amax) {
  const float s_enc = amax == 0.0f ? 1.0f : fminf(448.0f / amax, 3.40282346638528859812e+38f);
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

// ---------------------------------------------------------------- shared GEMM pieces

// Epilogue of a 512-thread, 256 x 256 tile whose 8 waves (2 x 4) each hold a
// 128 x 64 accumulator as 4 x 2 MFMA tiles of 32 x 32 in the D = B . A^T
// layout: alpha * acc -> BF16 (RNE), staged per wave through LDS so that global
// stores are whole 128-byte row segments.  Lane holds output row
// m = 32 mi + l32 and columns n = 32 ni + 8 q + 4 h + e (e = 0..3) of the wave
// tile.  The caller has passed a barrier after the last LDS read of its main
// loop; the staging needs kEpiLds bytes of LDS.
constexpr int kEpiRowB = 144;                        // LDS bytes per staged 64-wide BF16 row
constexpr int kEpiLds = 8 * 128 * kEpiRowB;          // 147456
__device__ __forceinline__ void store_tile_bf16(const floatx16 (&acc)[4][2], uint8_t* smem,
                                                float alpha, uint16_t* c, int64_t ldc, int64_t M,
                                                int64_t N, int64_t m0, int64_t n0, int wm, int wn,
                                                int lane, int vec_store) {
  const int h = lane >> 5, l32 = lane & 31, wave = threadIdx.x >> 6;
  uint8_t* E = smem + wave * (128 * kEpiRowB);
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const floatx16& a = acc[mi][ni];
        *reinterpret_cast<uint2*>(E + (mi * 32 + l32) * kEpiRowB + (ni * 32 + q * 8 + h * 4) * 2) =
            make_uint2(pack_bf16x2(a[4 * q] * alpha, a[4 * q + 1] * alpha),
                       pack_bf16x2(a[4 * q + 2] * alpha, a[4 * q + 3] * alpha));
      }
  __syncthreads();
  const int64_t gm0 = m0 + wm * 128, gn = n0 + wn * 64 + (lane & 7) * 8;
#pragma unroll 4
  for (int it = 0; it < 16; ++it) {
    const int row = it * 8 + (lane >> 3);
    const int64_t gm = gm0 + row;
    if (gm >= M) continue;
    const uint4 v = *reinterpret_cast<const uint4*>(E + row * kEpiRowB + (lane & 7) * 16);
    uint16_t* dst = c + gm * ldc + gn;
    if (vec_store && gn + 7 < N) {
      // streaming store: the output (GB-sized) is not kept in L2 / MALL, so
      // the next kernel does not pay for writing it back
      typedef uint32_t u32x4n __attribute__((ext_vector_type(4)));
      __builtin_nontemporal_store(u32x4n{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4n*>(dst));
    } else {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (gn + e < N) dst[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
    }
  }
}


// One global -> LDS direct load: each lane reads BYTES (4 or 16) at base + voff
// into LDS address lds + lane * BYTES; M0 holds the wave-uniform LDS address.
// Written as inline assembly so that the compiler neither waits for it at
// workgroup fences nor before unrelated LDS reads; wait_vmcnt orders the
// reads of the staged data.
template <int BYTES>
__device__ __forceinline__ void dma_to_lds(const uint8_t* base, uint32_t voff, uint32_t lds) {
  if (BYTES == 16)
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" :: "v"(voff), "s"(base), "s"(lds) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" :: "v"(voff), "s"(base), "s"(lds) : "memory", "m0");
}

// Wait until at most N of this wave's vector-memory operations (here: direct
// loads) are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  if (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Workgroup barrier that waits only for this wave's LDS operations: direct
// loads in flight are not waited for (a workgroup release fence would wait
// for them).  The memory clobber keeps the compiler from moving LDS accesses
// across it; the scheduling barriers keep register-only work (MFMAs) on its
// side of it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

}  // namespace bsq
