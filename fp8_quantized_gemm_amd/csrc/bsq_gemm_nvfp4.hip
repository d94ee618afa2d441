// NVFP4 block-scaled GEMM for gfx950: C[M, N] (BF16) = alpha * A[M, K] . B[N, K]^T
// with A and B as packed E2M1 codes plus one E4M3 scale per 16 K-elements and
// a per-tensor FP32 scale each (alpha = s_dec(A) * s_dec(B)).
//
// NVFP4 pretraining post, data-flow paragraph after Figure 1: FPROP, DGRAD and
// WGRAD consume NVFP4 operands and emit BF16; recipe ingredients 1-2 define
// the operand format.
//
// Route on CDNA4: the E4M3 per-16 scale is not a scale type of the scaled
// MFMA, but E2M1 x E4M3 is exact in FP16, so each operand element is expanded
// exactly to FP16 (dequant8) and fed to v_mfma_f32_32x32x16_f16 with FP32
// accumulation.
//
// Work split per 512-thread workgroup (8 waves, 2 x 4, wave tile 128 x 64),
// output tile 256 x 256, K stage of 64:
//  * each thread loads one 32-element chunk (16 code bytes + 2 scale bytes)
//    of A and one of B per stage, two stages ahead of use;
//  * the chunks of stage k+1 are expanded to FP16 once per workgroup and
//    written to LDS while the MFMAs of stage k run (four slices, one per
//    16-wide K step), so each element is dequantized once, not once per wave;
//  * LDS holds two FP16 stages (rows padded to 144 bytes: 16-byte fragment
//    reads of 16 consecutive rows hit distinct banks), one barrier per stage;
//  * the epilogue stages each wave's BF16 tile through LDS so that global
//    stores are whole 128-byte row segments.
#include "bsq_gemm_common.hpp"
#include "bsq_internal.hpp"

namespace bsq {

namespace {

constexpr int kNvThreads = 512;
constexpr int kNvRowB = 144;                      // LDS bytes per FP16 row (64 + 8 halves)
constexpr int kNvOpB = 256 * kNvRowB;             // one operand, one stage
constexpr int kNvStageB = 2 * kNvOpB;
constexpr int kNvLds = 2 * kNvStageB;             // 147456 bytes
constexpr int kNvEpiRowB = 144;                   // LDS bytes per row of a wave's 128 x 64 BF16 tile
static_assert(8 * 128 * kNvEpiRowB <= kNvLds, "epilogue staging must fit in the stage buffers");

// 32 consecutive K-elements of one operand row (two 16-element blocks).
struct NvChunk {
  uint4 codes;
  uint32_t scales;          // block scale bytes in bits 0..7 and 8..15
};

// FP16 scale pairs of a chunk's two blocks.
struct NvScales {
  halfx2 s0, s1;
};
__device__ __forceinline__ NvScales nv_scales(const NvChunk& c) {
  return NvScales{nvfp4_scale_pair<0>(c.scales), nvfp4_scale_pair<1>(c.scales)};
}

// Chunk of thread t for stage kt: row t/2 of the 256-row tile, half t%2 of
// the stage's 64 elements.  Rows past the end re-read the last row (their
// results are never stored).  FAST: whole chunks in bounds and aligned.
template <bool FAST>
__device__ __forceinline__ void nv_load(NvChunk& c, const uint8_t* codes,
                                        const uint8_t* scales, int64_t rows,
                                        int64_t row0, int64_t kt, int64_t code_ld,
                                        int64_t scale_ld) {
  const int t = threadIdx.x;
  int64_t gr = row0 + (t >> 1);
  gr = gr < rows ? gr : rows - 1;
  const int64_t kb = kt * 32 + (t & 1) * 16;      // code byte offset in the row
  const int64_t sb = kt * 4 + (t & 1) * 2;        // scale byte offset in the row
  if constexpr (FAST) {
    c.codes = *reinterpret_cast<const uint4*>(codes + gr * code_ld + kb);
    c.scales = *reinterpret_cast<const uint16_t*>(scales + gr * scale_ld + sb);
  } else {
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (kb + j < code_ld) w[j >> 2] |= (uint32_t)codes[gr * code_ld + kb + j] << (8 * (j & 3));
    c.codes = make_uint4(w[0], w[1], w[2], w[3]);
    c.scales = 0;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (sb + j < scale_ld) c.scales |= (uint32_t)scales[gr * scale_ld + sb + j] << (8 * j);
  }
}

// Expand group G (8 elements) of a chunk to FP16 and store it to the LDS tile.
template <int G>
__device__ __forceinline__ void nv_store_group(const NvChunk& c, const NvScales& sc,
                                               uint8_t* lds_op) {
  const int t = threadIdx.x;
  const uint32_t w = G == 0 ? c.codes.x : G == 1 ? c.codes.y : G == 2 ? c.codes.z : c.codes.w;
  *reinterpret_cast<halfx8*>(lds_op + (t >> 1) * kNvRowB + (t & 1) * 64 + G * 16) =
      dequant8(w, G < 2 ? sc.s0 : sc.s1);
}

template <int G>
__device__ __forceinline__ void nv_store_group2(const NvChunk& a, const NvScales& sa,
                                                const NvChunk& b, const NvScales& sb,
                                                uint8_t* la, uint8_t* lb) {
  nv_store_group<G>(a, sa, la);
  nv_store_group<G>(b, sb, lb);
}

// Fragments of one 16-wide K step: 4 A tiles and 2 B tiles of 32 rows.
struct NvFrags {
  halfx8 a[4], b[2];
};
__device__ __forceinline__ void nv_frags(NvFrags& f, const uint8_t* La, const uint8_t* Lb, int s,
                                         int wm, int wn, int h, int l32) {
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
    f.a[mi] = *reinterpret_cast<const halfx8*>(La + (wm * 128 + mi * 32 + l32) * kNvRowB + s * 32 + h * 16);
#pragma unroll
  for (int ni = 0; ni < 2; ++ni)
    f.b[ni] = *reinterpret_cast<const halfx8*>(Lb + (wn * 64 + ni * 32 + l32) * kNvRowB + s * 32 + h * 16);
}

// One K stage, straight-line: MFMAs on LDS buffer `buf` (stage kt) while the
// chunks of stage kt+1 (ca, cb) are expanded into the other buffer and the
// loads of stage kt+2 go into (na, nb).  Fragments of the next 16-wide K step
// are read while the current step's MFMAs run; scheduling groups interleave
// MFMA, LDS and VALU work.  At the last stages the prefetch re-reads the last
// stage and the expansion writes an unused buffer (never read before the
// final barrier), which keeps the code branch-free.
template <bool FAST>
__device__ __forceinline__ void nv_stage(floatx16 (&acc)[4][2], uint8_t* smem, int64_t kt,
                                         int64_t KT, const NvChunk& ca, const NvChunk& cb,
                                         NvChunk& na, NvChunk& nb, const uint8_t* a_codes,
                                         const uint8_t* a_scales, const uint8_t* b_codes,
                                         const uint8_t* b_scales, int64_t M, int64_t N,
                                         int64_t m0, int64_t n0, int64_t code_ld,
                                         int64_t scale_ld, int wm, int wn, int h, int l32) {
  const int buf = (int)(kt & 1);
  const int64_t kp = kt + 2 < KT ? kt + 2 : KT - 1;
  nv_load<FAST>(na, a_codes, a_scales, M, m0, kp, code_ld, scale_ld);
  nv_load<FAST>(nb, b_codes, b_scales, N, n0, kp, code_ld, scale_ld);
  // keep the prefetch here (the operand pointers are deliberately not
  // __restrict__, so these loads cannot be sunk towards their use in the next
  // stage, where they would then have to be waited for)
  asm volatile("" ::: "memory");
  const uint8_t* La = smem + buf * kNvStageB;
  const uint8_t* Lb = La + kNvOpB;
  uint8_t* Na = smem + (buf ^ 1) * kNvStageB;
  uint8_t* Nb = Na + kNvOpB;
  const NvScales sa = nv_scales(ca), sb = nv_scales(cb);
  NvFrags f[2];
  nv_frags(f[0], La, Lb, 0, wm, wn, h, l32);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    NvFrags& cur = f[s & 1];
    if (s < 3) nv_frags(f[(s + 1) & 1], La, Lb, s + 1, wm, wn, h, l32);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(cur.b[ni], cur.a[mi], acc[mi][ni], 0, 0, 0);
    if (s == 0) nv_store_group2<0>(ca, sa, cb, sb, Na, Nb);
    if (s == 1) nv_store_group2<1>(ca, sa, cb, sb, Na, Nb);
    if (s == 2) nv_store_group2<2>(ca, sa, cb, sb, Na, Nb);
    if (s == 3) nv_store_group2<3>(ca, sa, cb, sb, Na, Nb);
    // 8 MFMAs, each followed by one fragment read (6) and ~4 VALU ops of the
    // expansion; the two LDS writes of the expanded group last.
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              // MFMA
      if (s < 3 && i < 6) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);              // VALU
    }
    __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);                // DS write
  }
  __syncthreads();
}

template <bool FAST>
__global__ __launch_bounds__(kNvThreads) void k_gemm_nvfp4(
    int64_t M, int64_t N, int64_t K, const uint8_t* a_codes, const uint8_t* a_scales,
    const float* __restrict__ a_amax, const uint8_t* b_codes, const uint8_t* b_scales,
    const float* __restrict__ b_amax, uint16_t* __restrict__ c, int64_t ldc, int tiles_m,
    int tiles_n, int vec_store) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int tm, tn;
  tile_of_block(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * 256, n0 = (int64_t)tn * 256;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t code_ld = K / 2, scale_ld = K / 16;
  const int64_t KT = (K + 63) / 64;

  floatx16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  NvChunk xa, xb, ya, yb;                          // two register sets, used alternately
  if (KT > 0) {
    NvChunk a0, b0;
    nv_load<FAST>(a0, a_codes, a_scales, M, m0, 0, code_ld, scale_ld);
    nv_load<FAST>(b0, b_codes, b_scales, N, n0, 0, code_ld, scale_ld);
    const NvScales sa = nv_scales(a0), sb = nv_scales(b0);
    nv_store_group2<0>(a0, sa, b0, sb, smem, smem + kNvOpB);
    nv_store_group2<1>(a0, sa, b0, sb, smem, smem + kNvOpB);
    nv_store_group2<2>(a0, sa, b0, sb, smem, smem + kNvOpB);
    nv_store_group2<3>(a0, sa, b0, sb, smem, smem + kNvOpB);
  }
  if (KT > 1) {
    nv_load<FAST>(xa, a_codes, a_scales, M, m0, 1, code_ld, scale_ld);
    nv_load<FAST>(xb, b_codes, b_scales, N, n0, 1, code_ld, scale_ld);
  }
  __syncthreads();

  for (int64_t kt = 0; kt < KT; kt += 2) {
    nv_stage<FAST>(acc, smem, kt, KT, xa, xb, ya, yb, a_codes, a_scales, b_codes, b_scales, M, N,
                   m0, n0, code_ld, scale_ld, wm, wn, h, l32);
    if (kt + 1 < KT)
      nv_stage<FAST>(acc, smem, kt + 1, KT, ya, yb, xa, xb, a_codes, a_scales, b_codes, b_scales,
                     M, N, m0, n0, code_ld, scale_ld, wm, wn, h, l32);
  }

  // ---- epilogue: alpha * acc -> BF16, staged per wave through LDS.
  // Lane holds output row m = 32 mi + l32 and columns n = 32 ni + 8 q + 4 h + e
  // (e = 0..3) of the wave tile (D = B_tile . A_tile^T layout).
  const float alpha = nvfp4_s_dec(*a_amax) * nvfp4_s_dec(*b_amax) * 16384.0f;   // undo 2^-7 per operand
  uint8_t* E = smem + wave * (128 * kNvEpiRowB);
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t b[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) b[e] = f32_to_bf16_rne(acc[mi][ni][4 * q + e] * alpha);
        *reinterpret_cast<uint2*>(E + (mi * 32 + l32) * kNvEpiRowB + (ni * 32 + q * 8 + h * 4) * 2) =
            make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
      }
  __syncthreads();
  const int64_t gm0 = m0 + wm * 128, gn = n0 + wn * 64 + (lane & 7) * 8;
#pragma unroll 4
  for (int it = 0; it < 16; ++it) {
    const int row = it * 8 + (lane >> 3);
    const int64_t gm = gm0 + row;
    if (gm >= M) continue;
    const uint4 v = *reinterpret_cast<const uint4*>(E + row * kNvEpiRowB + (lane & 7) * 16);
    uint16_t* dst = c + gm * ldc + gn;
    if (vec_store && gn + 7 < N) {
      *reinterpret_cast<uint4*>(dst) = v;
    } else {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (gn + e < N) dst[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
    }
  }
}

}  // namespace

hipError_t launch_gemm_nvfp4(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                             const float* aa, const uint8_t* bc, const uint8_t* bs,
                             const float* ba, void* c, int64_t ldc, hipStream_t s) {
  const int tiles_m = (int)((M + 255) / 256), tiles_n = (int)((N + 255) / 256);
  const auto al = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; };
  const bool fast = (K % 64 == 0) && al(ac, 16) && al(bc, 16) && al(as, 2) && al(bs, 2);
  const bool vec_store = (ldc % 8 == 0) && al(c, 16);
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_nvfp4<true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kNvLds) != hipSuccess ||
        hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_nvfp4<false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kNvLds) != hipSuccess)
      return hipErrorInvalidConfiguration;
    attr_set = true;
  }
  const dim3 grid((unsigned)(tiles_m * tiles_n)), block(kNvThreads);
  uint16_t* cp = static_cast<uint16_t*>(c);
  if (fast)
    hipLaunchKernelGGL(k_gemm_nvfp4<true>, grid, block, kNvLds, s, M, N, K, ac, as, aa, bc, bs, ba,
                       cp, ldc, tiles_m, tiles_n, vec_store ? 1 : 0);
  else
    hipLaunchKernelGGL(k_gemm_nvfp4<false>, grid, block, kNvLds, s, M, N, K, ac, as, aa, bc, bs, ba,
                       cp, ldc, tiles_m, tiles_n, vec_store ? 1 : 0);
  return hipGetLastError();
}

}  // namespace bsq
