// Inner-loop ceilings of the NVFP4 GEMM routes on gfx950 (measurement
// kernels, built into libbsq_ceiling.so, not part of the libbsq ABI).
//
// NVFP4 operands carry an E4M3 scale per 16 K-elements (NVFP4 pretraining
// post, recipe ingredients 1-2), which no scaled MFMA of gfx950 takes (its
// scales are E8M0, one per 32 K-elements).  Two routes keep the arithmetic
// exact:
//  (a) per-16-K partial accumulation: one MFMA per 16-block on the unscaled
//      E2M1 values (a fresh product), then acc += (sA(row) * sB(col)) * P on
//      the VALU (16 multiplies and 16 multiply-adds per lane and MFMA);
//  (b) exact expansion of E2M1 x E4M3 to FP16 before the MFMA, which then
//      accumulates directly (the library's GEMM).
// MODE 0 runs (a)'s inner loop on the FP16 32x32x16 MFMA, MODE 1 the same
// MFMAs accumulating directly (route (b)'s MFMA-only ceiling), MODE 2 (a)'s
// inner loop on the scaled FP4 MFMA v_mfma_scale_f32_32x32x64_f8f6f4: each
// instruction carries one 16-block of E2M1 codes (the other 48 K positions
// zero, unit E8M0 scales) into a fresh accumulator, followed by the same
// VALU rescale, and MODE 3 that FP4 instruction with all 64 K positions
// filled, accumulating directly (the MXFP4 MFMA-only ceiling, which an
// NVFP4 GEMM cannot use as is).  MODE 4 is route (b) on the FP16 16x16x32
// MFMA the library's GEMM uses, accumulating directly, and MODE 5 the same
// with one expansion pair (an FP4 -> FP16 convert and a packed FP16 multiply
// by a block-scale pair) after every MFMA, written in one assembly block with
// it as in the GEMM: the ceiling of that GEMM's inner loop, which has exactly
// this instruction mix plus its loads, reads and waits.  Operands live in registers: no memory, no
// LDS, no code conversion inside the loop, so each figure is an upper bound
// for its route.  512 threads (8 waves) per workgroup, four independent
// accumulator chains per wave, values drawn from the E2M1 grid and scale
// mantissas from the E4M3 set 1 + m/8 (operand bit patterns set the MFMA's
// power draw, and with it the clock).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int intx8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t mix(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// Value of a 4-bit E2M1 code (sign in bit 3), computed rather than looked up.
__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const uint32_t e = (c >> 1) & 3, m = c & 1;
  const float mag = e == 0 ? 0.5f * (float)m : __builtin_ldexpf(1.0f + 0.5f * (float)m, (int)e - 1);
  return (c & 8) ? -mag : mag;
}

template <int MODE>
__global__ void __launch_bounds__(512) k_route_ceiling(float* sink, int iters) {
  const int t = threadIdx.x;
  halfx8 a[8], b[8];
  intx8 qa[8], qb[8];
  float sa[16], sb[8];
  for (int s = 0; s < 8; ++s) {
    for (int i = 0; i < 8; ++i) {
      const uint32_t r = mix(blockIdx.x * 4096u + t * 64u + s * 8u + i);
      a[s][i] = (_Float16)e2m1_value(r & 15);
      b[s][i] = (_Float16)e2m1_value((r >> 4) & 15);
      // FP4 operands of the scaled MFMA: lane half h carries K 32 h .. 32 h + 31
      // in dwords 0-3 (eight codes per dword).  MODE 2: one 16-block (lane half
      // 0, dwords 0-1), everything else zero; MODE 3: all 64 K positions.
      const uint32_t ca = mix(r ^ 0x5bd1e995u), cb = mix(r ^ 0x27d4eb2fu);
      const bool used = MODE == 3 ? i < 4 : (i < 2 && (t & 63) < 32);
      qa[s][i] = used ? (int)ca : 0;
      qb[s][i] = used ? (int)cb : 0;
    }
  }
  for (int s = 0; s < 8; ++s) sb[s] = 1.0f + (float)(mix(t * 7u + s) & 7) * 0.125f;
  for (int e = 0; e < 16; ++e) sa[e] = 1.0f + (float)(mix(t * 131u + e) & 7) * 0.125f;
  floatx16 acc[4] = {};
  const floatx16 zero = {};
  for (int it = 0; it < iters; ++it) {
    // operands and block scales are opaque to the compiler from trip to trip
    // (no instructions): every trip issues all 8 MFMAs and forms the 16 scale
    // products of each block, as a GEMM walking K does
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (MODE == 0 || MODE == 1) asm volatile("" : "+v"(a[s]), "+v"(b[s]));
      else asm volatile("" : "+v"(qa[s]), "+v"(qb[s]));
      asm volatile("" : "+v"(sb[s]));
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (MODE == 1) {
        acc[s & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[s], b[s], acc[s & 3], 0, 0, 0);
      } else if (MODE == 3) {
        // format 4 = E2M1 for both operands, E8M0 scale 127 = 1.0
        acc[s & 3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[s], qb[s], acc[s & 3], 4, 4, 0, 127, 0, 127);
      } else {
        const floatx16 p =
            MODE == 0 ? __builtin_amdgcn_mfma_f32_32x32x16_f16(a[s], b[s], zero, 0, 0, 0)
                      : __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[s], qb[s], zero, 4, 4, 0, 127, 0, 127);
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[s & 3][e] = __builtin_fmaf(sa[e] * sb[s], p[e], acc[s & 3][e]);
      }
    }
  }
  float sum = 0.f;
  for (int q = 0; q < 4; ++q)
    for (int e = 0; e < 16; ++e) sum += acc[q][e];
  sink[(int64_t)blockIdx.x * 512 + t] = sum;   // keeps the loop live
}

// Route (b) on the 16x16x32 FP16 MFMA: eight accumulator chains per wave;
// PAIR: one expansion pair after each MFMA, in the same assembly block.
template <bool PAIR>
__global__ void __launch_bounds__(512) k_route_ceiling16(float* sink, int iters) {
  const int t = threadIdx.x;
  halfx8 a[8], b[8];
  uint32_t cw[8];
  halfx2 sp[8];
  for (int s = 0; s < 8; ++s) {
    for (int i = 0; i < 8; ++i) {
      const uint32_t r = mix(blockIdx.x * 4096u + t * 64u + s * 8u + i);
      a[s][i] = (_Float16)e2m1_value(r & 15);
      b[s][i] = (_Float16)e2m1_value((r >> 4) & 15);
    }
    cw[s] = mix(t * 977u + s);
    const float m = 1.0f + (float)(mix(t * 7u + s) & 7) * 0.125f;
    sp[s] = halfx2{(_Float16)m, (_Float16)m};
  }
  floatx4 acc[8] = {};
  uint32_t out[8] = {};
  const float k = 0x1p-14f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < 8; ++s) asm volatile("" : "+v"(a[s]), "+v"(b[s]), "+v"(cw[s]), "+v"(sp[s]));
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (PAIR)
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %2, %3, %0\n\t"
                     "v_cvt_scalef32_pk_f16_fp4 %1, %4, %5 op_sel:[1,0,0]\n\t"
                     "v_pk_mul_f16 %1, %6, %1 op_sel_hi:[0,1]"
                     : "+a"(acc[s]), "=&v"(out[s])
                     : "v"(b[s]), "v"(a[s]), "v"(cw[s]), "s"(k), "v"(sp[s]));
      else
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc[s]) : "v"(b[s]), "v"(a[s]));
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) asm volatile("" : "+v"(out[s]));
  }
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  float sum = 0.f;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    asm volatile("" : "+a"(acc[q]));
    sum += acc[q][0] + acc[q][3] + (float)(out[q] & 1u);
  }
  sink[(int64_t)blockIdx.x * 512 + t] = sum;   // keeps the loop live
}

}  // namespace

// Launches `blocks` workgroups of 512 threads, each running `iters` trips of
// 8 MFMAs per wave (modes 0-2: 2 * 32 * 32 * 16 useful flops each; mode 3:
// 2 * 32 * 32 * 64; modes 4-5: 2 * 16 * 16 * 32).  sink: device float
// [blocks * 512].  mode 0: route (a) on the FP16 MFMA; 1: route (b)
// MFMA-only; 2: route (a) on the scaled FP4 MFMA; 3: scaled FP4 MFMA-only;
// 4: route (b) on the 16x16x32 FP16 MFMA; 5: mode 4 with one expansion pair
// per MFMA.  Returns 0, or -1 for bad arguments, or the HIP error code of
// the launch.
extern "C" int bsq_route_ceiling(int mode, float* sink, int iters, int blocks, void* stream) {
  if (mode < 0 || mode > 5 || !sink || iters < 0 || blocks < 1) return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (mode) {
    case 0: hipLaunchKernelGGL(k_route_ceiling<0>, dim3(blocks), dim3(512), 0, s, sink, iters); break;
    case 1: hipLaunchKernelGGL(k_route_ceiling<1>, dim3(blocks), dim3(512), 0, s, sink, iters); break;
    case 2: hipLaunchKernelGGL(k_route_ceiling<2>, dim3(blocks), dim3(512), 0, s, sink, iters); break;
    case 3: hipLaunchKernelGGL(k_route_ceiling<3>, dim3(blocks), dim3(512), 0, s, sink, iters); break;
    case 4: hipLaunchKernelGGL(k_route_ceiling16<false>, dim3(blocks), dim3(512), 0, s, sink, iters); break;
    default: hipLaunchKernelGGL(k_route_ceiling16<true>, dim3(blocks), dim3(512), 0, s, sink, iters); break;
  }
  return (int)hipGetLastError();
}
