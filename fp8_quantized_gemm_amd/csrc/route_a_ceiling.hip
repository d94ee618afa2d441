// Inner-loop ceilings of the two NVFP4 GEMM routes on gfx950 (measurement
// kernels, built into libbsq_ceiling.so, not part of the libbsq ABI).
//
// NVFP4 operands carry an E4M3 scale per 16 K-elements (NVFP4 pretraining
// post, recipe ingredients 1-2), which no scaled MFMA of gfx950 takes.  Two
// routes keep the arithmetic exact:
//  (a) per-16-K partial accumulation: one FP16 32x32x16 MFMA per 16-block on
//      the unscaled E2M1 values (a fresh product), then
//      acc += (sA(row) * sB(col)) * P on the VALU (16 multiplies and 16
//      multiply-adds per lane and MFMA);
//  (b) exact expansion of E2M1 x E4M3 to FP16 before the MFMA, which then
//      accumulates directly (the library's GEMM).
// MODE 0 runs (a)'s inner loop, MODE 1 the same MFMAs accumulating directly
// (route (b)'s MFMA-only ceiling).  Operands live in registers: no memory,
// no LDS, no code conversion inside the loop, so each figure is an upper
// bound for its route.  512 threads (8 waves) per workgroup, four
// independent accumulator chains per wave, values drawn from the E2M1 grid
// and scale mantissas from the E4M3 set 1 + m/8 (operand bit patterns set
// the MFMA's power draw, and with it the clock).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

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
  halfx8 a[4], b[4];
  float sa[16], sb[8];
  for (int s = 0; s < 4; ++s) {
    for (int i = 0; i < 8; ++i) {
      const uint32_t r = mix(blockIdx.x * 4096u + t * 64u + s * 8u + i);
      a[s][i] = (_Float16)e2m1_value(r & 15);
      b[s][i] = (_Float16)e2m1_value((r >> 4) & 15);
    }
  }
  for (int s = 0; s < 8; ++s) sb[s] = 1.0f + (float)(mix(t * 7u + s) & 7) * 0.125f;
  for (int e = 0; e < 16; ++e) sa[e] = 1.0f + (float)(mix(t * 131u + e) & 7) * 0.125f;
  floatx16 acc[4] = {};
  const floatx16 zero = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (MODE == 1) {
        acc[s & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[s & 3], b[(s + 1) & 3], acc[s & 3], 0, 0, 0);
      } else {
        const floatx16 p = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[s & 3], b[(s + 1) & 3], zero, 0, 0, 0);
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

}  // namespace

// Launches `blocks` workgroups of 512 threads, each running `iters` trips of
// 8 MFMAs per wave (2 * 32 * 32 * 16 flops each).  sink: device float
// [blocks * 512].  mode 0: route (a) loop; 1: route (b) MFMA-only loop.
// Returns 0, or -1 for bad arguments, or the HIP error code of the launch.
extern "C" int bsq_route_ceiling(int mode, float* sink, int iters, int blocks, void* stream) {
  if ((mode != 0 && mode != 1) || !sink || iters < 0 || blocks < 1) return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (mode == 0)
    hipLaunchKernelGGL(k_route_ceiling<0>, dim3(blocks), dim3(512), 0, s, sink, iters);
  else
    hipLaunchKernelGGL(k_route_ceiling<1>, dim3(blocks), dim3(512), 0, s, sink, iters);
  return (int)hipGetLastError();
}
