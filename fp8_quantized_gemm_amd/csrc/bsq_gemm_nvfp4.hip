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
static_assert(kEpiLds <= kNvLds, "epilogue staging must fit in the stage buffers");

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

// Epilogue of both NVFP4 kernels: alpha = s_dec(A) * s_dec(B), times 2^14 to
// undo the 2^-7 each expanded operand carries.
__device__ __forceinline__ void nv_epilogue(const floatx16 (&acc)[4][2], uint8_t* smem,
                                            const float* a_amax, const float* b_amax, uint16_t* c,
                                            int64_t ldc, int64_t M, int64_t N, int64_t m0,
                                            int64_t n0, int wm, int wn, int lane, int vec_store) {
  const float alpha = nvfp4_s_dec(*a_amax) * nvfp4_s_dec(*b_amax) * 16384.0f;
  store_tile_bf16(acc, smem, alpha, c, ldc, M, N, m0, n0, wm, wn, lane, vec_store);
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

  nv_epilogue(acc, smem, a_amax, b_amax, c, ldc, M, N, m0, n0, wm, wn, lane, vec_store);
}

// ---------------------------------------------------------------- ping-pong kernel
//
// Same 256 x 256 output tile, wave tiles and FP16 dequant route, scheduled so
// that the MFMA pipe of every SIMD is fed by one wave while its sibling wave
// does the memory work.  The two waves of a SIMD belong to different groups
// (waves 0-3 and 4-7 share SIMDs pairwise); time is cut into slots separated
// by workgroup barriers.  In each slot one group runs the 16 MFMAs of a
// 32-wide K half-stage on fragments already in registers and, in the shadow of
// those MFMAs, expands one operand's 256 rows of a later half-stage to FP16 in
// LDS (group 0 the A rows, group 1 the B rows; 32 elements per thread, from
// raw codes and scales its own wave staged in LDS), while the other group
//  * reads all its fragments for its next half-stage from LDS,
//  * reads the raw chunk its next MFMA slot expands, and
//  * every fourth turn, stages the raw data of four more half-stages with
//    global -> LDS direct loads.
// Group 0 computes half-stage j on slot 2j and expands A(j + 1) there; group 1
// computes j on slot 2j + 1 and expands B(j + 2) there.  So A(j) is complete
// at slot 2j - 2 and B(j) at slot 2j - 3, before group 0 reads half-stage j
// (slot 2j - 1) and group 1 reads it (slot 2j), and two FP16 buffers suffice.
// Past the last half-stage the staging loads and expansions are clamped to
// it: those writes land where nobody reads again.
constexpr int kPpRowB = 80;                      // LDS bytes per row: 32 halves + 16 pad
constexpr int kPpOpB = 256 * kPpRowB;            // one operand, one half-stage
constexpr int kPpBufB = 2 * kPpOpB;              // 40960

// Raw operand staging.  Each group stages its operand's 256 rows in LDS, four
// half-stages (64 code bytes and 8 scale bytes per row) at a time, with
// global -> LDS direct loads: four lanes cover one row's 64 contiguous code
// bytes, so a wave instruction touches 16 row segments instead of 64 lines.
// A wave loads exactly the rows its own threads expand, so only its own
// vmcnt orders the staging writes and reads.  The 16-byte chunk c of row r sits
// in slot c ^ ((r >> 2) & 3), which keeps the per-turn reads (one chunk of 64
// consecutive rows) free of bank conflicts.
constexpr int kPpStCodeB = 256 * 64;                 // codes of one staged quad
constexpr int kPpStB = kPpStCodeB + 256 * 8;         // plus scales
constexpr int kPpStOff = 2 * kPpBufB;                // staging after the FP16 buffers
constexpr int kPpLds = kPpStOff + 4 * kPpStB;        // 2 groups x 2 staging buffers
static_assert(2 * kPpBufB <= kNvLds, "two half-stage buffers must fit in the LDS allocation");
static_assert(kPpLds >= kEpiLds && kPpLds <= 160 * 1024, "ping-pong LDS plan");

// Issue the 6 direct loads of quad `qd` (half-stages 4 qd .. 4 qd + 3) of the
// 256 operand rows starting at `base` into the staging buffer at LDS address
// `st`: 4 of codes (16 rows x 64 bytes each), 2 of scales (32 rows x 8 bytes).
// Rows past `rows` re-read the last row (their results are never stored).
// The per-lane offsets are formed here, in 32 bits (the operand arrays are
// below 4 GiB), rather than kept in registers across the loop.
__device__ __forceinline__ void pp_stage(const uint8_t* codes, const uint8_t* scales,
                                         int64_t base, int64_t rows, int64_t code_ld,
                                         int64_t scale_ld, int64_t qd, uint32_t st, int w,
                                         int lane) {
  const uint8_t* cq = codes + qd * 64;
  const uint8_t* sq = scales + qd * 8;
  const uint32_t b32 = (uint32_t)base, last = (uint32_t)(rows - 1);
  const uint32_t chunk = (uint32_t)((lane & 3) ^ ((lane >> 4) & 3));   // slot c ^ ((r >> 2) & 3)
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t gr = min(b32 + (uint32_t)(w * 64 + q * 16 + (lane >> 2)), last);
    dma_to_lds<16>(cq, gr * (uint32_t)code_ld + chunk * 16, st + (w * 64 + q * 16) * 64);
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const uint32_t gr = min(b32 + (uint32_t)(w * 64 + p * 32 + (lane >> 1)), last);
    dma_to_lds<4>(sq, gr * (uint32_t)scale_ld + (uint32_t)(lane & 1) * 4, st + kPpStCodeB + (w * 64 + p * 32) * 8);
  }
}

// Chunk C (0..3) of this thread's staged row: codes and the scale dword.
struct PpRaw {
  uint4 codes;
  uint32_t sw;
};
template <int C>
__device__ __forceinline__ PpRaw pp_raw(const uint8_t* st, int r) {
  PpRaw x;
  x.codes = *reinterpret_cast<const uint4*>(st + r * 64 + ((C ^ ((r >> 2) & 3)) << 4));
  x.sw = *reinterpret_cast<const uint32_t*>(st + kPpStCodeB + r * 8 + (C >> 1) * 4);
  return x;
}

// Expand a staged chunk (half-stage parity Q selects its scale bytes) into an
// FP16 LDS row (prologue only; the main loop interleaves it with MFMAs).
template <int Q>
__device__ __forceinline__ void pp_expand(const PpRaw& x, uint8_t* row) {
  const halfx2 s0 = nvfp4_scale_pair<2 * Q>(x.sw), s1 = nvfp4_scale_pair<2 * Q + 1>(x.sw);
  *reinterpret_cast<halfx8*>(row + 0) = dequant8(x.codes.x, s0);
  *reinterpret_cast<halfx8*>(row + 16) = dequant8(x.codes.y, s0);
  *reinterpret_cast<halfx8*>(row + 32) = dequant8(x.codes.z, s1);
  *reinterpret_cast<halfx8*>(row + 48) = dequant8(x.codes.w, s1);
}

// Fragments of one half-stage: 4 A tiles and 2 B tiles of 32 rows, 2 K steps.
struct PpFrags {
  halfx8 a[2][4], b[2][2];
};

// Fragment reads of K step S: A tiles (PART & 1) and/or B tiles (PART & 2).
template <int S, int PART>
__device__ __forceinline__ void pp_frags(PpFrags& f, const uint8_t* buf, int wm, int wn, int h,
                                         int l32) {
  const uint8_t* La = buf;
  const uint8_t* Lb = buf + kPpOpB;
  if (PART & 1) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
      f.a[S][mi] = *reinterpret_cast<const halfx8*>(La + (wm * 128 + mi * 32 + l32) * kPpRowB + S * 32 + h * 16);
  }
  if (PART & 2) {
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
      f.b[S][ni] = *reinterpret_cast<const halfx8*>(Lb + (wn * 64 + ni * 32 + l32) * kPpRowB + S * 32 + h * 16);
  }
}

// One FP16 pair of the expansion: byte SEL of `w` (two E2M1 codes) times the
// scale pair `s` (see dequant8).
template <int SEL>
__device__ __forceinline__ uint32_t pp_pk(uint32_t w, halfx2 s) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 0x1p-14f, SEL) * s);
}
__device__ __forceinline__ uint32_t pp_pk_sel(uint32_t w, int sel, halfx2 s) {
  switch (sel) {
    case 0: return pp_pk<0>(w, s);
    case 1: return pp_pk<1>(w, s);
    case 2: return pp_pk<2>(w, s);
    default: return pp_pk<3>(w, s);
  }
}

// Pairs of the expansion issued after MFMA k of a slot: pairs [lo(k), lo(k+1)),
// spread over MFMAs 2..13 (the scale pairs are formed after MFMA 0).
__host__ __device__ constexpr int pp_pk_lo(int k) {
  return k < 2 ? 0 : (((k - 2) * 16 + 11) / 12 > 16 ? 16 : ((k - 2) * 16 + 11) / 12);
}

// MFMA slot: the 16 MFMAs of a half-stage with the expansion of one staged
// chunk (half-stage parity Q) into the FP16 row `row`, interleaved in program
// order and pinned there by scheduling barriers, so that the expansion's VALU
// work issues in the MFMA shadow of the same wave; each 16-byte row write
// leaves as soon as its 8 values exist, early enough to complete before the
// slot's barrier.  The wave raises its priority for the slot, so that the
// SIMD's issue arbiter serves it before its memory-slot sibling (+2% over the
// six 8B GEMMs, bit-identical output).
template <int Q>
__device__ __forceinline__ void pp_mfma_slot(floatx16 (&acc)[4][2], const PpFrags& f,
                                             const PpRaw& raw, uint8_t* row) {
  const uint32_t cw[4] = {raw.codes.x, raw.codes.y, raw.codes.z, raw.codes.w};
  halfx2 s0 = {}, s1 = {};
  uint32_t o[16];
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int st = k >> 3, mi = (k & 7) >> 1, ni = k & 1;
    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.b[st][ni], f.a[st][mi], acc[mi][ni], 0, 0, 0);
    if (k == 0) {
      const halfx2 ss = nvfp4_scale_pairs2<Q>(raw.sw);   // both block scales of the chunk
      s0 = halfx2{ss.x, ss.x};
      s1 = halfx2{ss.y, ss.y};
    }
    const int lo = pp_pk_lo(k), hi = pp_pk_lo(k + 1);
#pragma unroll
    for (int p = 0; p < 16; ++p)
      if (p >= lo && p < hi) o[p] = pp_pk_sel(cw[p >> 2], p & 3, p < 8 ? s0 : s1);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * i + 3 >= lo && 4 * i + 3 < hi)
        *reinterpret_cast<uint4*>(row + 16 * i) = make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_setprio(0);
}

// Memory slot reads: the raw chunk C that the next MFMA slot expands, then all
// fragments (both K steps) of the half-stage in FP16 buffer `fbuf`.
template <int C>
__device__ __forceinline__ void pp_mem_reads(PpFrags& f, PpRaw& raw, const uint8_t* fbuf,
                                             const uint8_t* st, int r, int wm, int wn, int h,
                                             int l32) {
  raw = pp_raw<C>(st, r);
  pp_frags<0, 3>(f, fbuf, wm, wn, h, l32);
  pp_frags<1, 3>(f, fbuf, wm, wn, h, l32);
}

// Workgroup barrier for the ping-pong loops (see lds_barrier).  Each group
// runs its own loop (selected by a scalar branch, so no barrier ever sits in
// an exec-masked region) and both loops pass the same number of barriers per
// half-stage.  The direct staging loads still in flight are read by their own
// wave alone, after its explicit vmcnt wait.
__device__ __forceinline__ void pp_sync() { lds_barrier(); }

template <int N>
__device__ __forceinline__ void pp_wait_staged() { wait_vmcnt<N>(); }

// Where a group's staging loads come from (all wave-uniform).
struct PpSrc {
  const uint8_t* codes;
  const uint8_t* scales;
  int64_t base, rows, code_ld, scale_ld;   // the group's 256 operand rows start at `base`
  int64_t NQ;                              // staged quads (K / 128)
  uint32_t st_lds;                         // this group's two staging buffers (LDS address)
  const uint8_t* st;                       // the same, generic pointer
  int w;                                   // wave within the group
};

// Staging at U == 2 of quad J: quad J + 2 (clamped to the last) goes into the
// buffer that held quad J, whose four chunks have been read by now.
__device__ __forceinline__ void pp_stage_ahead(const PpSrc& s, int64_t J, int lane) {
  const int64_t qd = J + 2 < s.NQ ? J + 2 : s.NQ - 1;
  pp_stage(s.codes, s.scales, s.base, s.rows, s.code_ld, s.scale_ld, qd,
           s.st_lds + (uint32_t)(J & 1) * kPpStB, s.w, lane);
}

// Group 0, half-stage j = 4 J + U.  Slot 2j: MFMAs of j while expanding
// A(j + 1) (raw chunk read in the previous slot) into buffer (j + 1) & 1.
// Slot 2j + 1: fragments of j + 1 (A of j + 1 written in slot 2j, B of j + 1
// by group 1 in slot 2j - 1) and the raw chunk of A(j + 2); at U == 2 the
// first chunk of quad J + 1 is read (staged four turns ago) and quad J + 2 is
// staged.
template <int U>
__device__ __forceinline__ void pp_turn0(floatx16 (&acc)[4][2], PpFrags& f, PpRaw& raw,
                                         uint8_t* smem, const PpSrc& s, int64_t J, int r,
                                         int dst_off, int wm, int wn, int h, int l32, int lane) {
  pp_mfma_slot<(U + 1) & 1>(acc, f, raw, smem + ((U + 1) & 1) * kPpBufB + dst_off);
  pp_sync();
  if (U == 2) pp_wait_staged<0>();
  pp_mem_reads<(U + 2) & 3>(f, raw, smem + ((U + 1) & 1) * kPpBufB,
                            s.st + ((J + ((U + 2) >> 2)) & 1) * kPpStB, r, wm, wn, h, l32);
  if (U == 2) pp_stage_ahead(s, J, lane);
  pp_sync();
}

// Group 1, half-stage j = 4 J + U.  Slot 2j: fragments of j (A of j written by
// group 0 in slot 2j - 2, B of j by group 1 in slot 2j - 3) and the raw chunk
// of B(j + 2), with the same staging rule as group 0.  Slot 2j + 1: MFMAs of
// j while expanding B(j + 2) into buffer j & 1 (whose B(j) both groups have
// read by then).
template <int U>
__device__ __forceinline__ void pp_turn1(floatx16 (&acc)[4][2], PpFrags& f, PpRaw& raw,
                                         uint8_t* smem, const PpSrc& s, int64_t J, int r,
                                         int dst_off, int wm, int wn, int h, int l32, int lane) {
  if (U == 2) pp_wait_staged<0>();
  pp_mem_reads<(U + 2) & 3>(f, raw, smem + (U & 1) * kPpBufB,
                            s.st + ((J + ((U + 2) >> 2)) & 1) * kPpStB, r, wm, wn, h, l32);
  if (U == 2) pp_stage_ahead(s, J, lane);
  pp_sync();
  pp_mfma_slot<U & 1>(acc, f, raw, smem + (U & 1) * kPpBufB + dst_off);
  pp_sync();
}

__global__ __launch_bounds__(kNvThreads) void k_gemm_nvfp4_pp(
    int64_t M, int64_t N, int64_t K, const uint8_t* a_codes, const uint8_t* a_scales,
    const float* __restrict__ a_amax, const uint8_t* b_codes, const uint8_t* b_scales,
    const float* __restrict__ b_amax, uint16_t* __restrict__ c, int64_t ldc, int tiles_m,
    int tiles_n, int vec_store) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int tm, tn;
  tile_of_block(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * 256, n0 = (int64_t)tn * 256;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int g = wave >> 2;
  const int wm = g, wn = wave & 3;
  const int h = lane >> 5, l32 = lane & 31;

  // the operand and row this thread expands; its wave stages that row itself
  // (group and wave index made scalar: they address the direct loads)
  const int gs = __builtin_amdgcn_readfirstlane(g);
  const int r = t & 255, w = __builtin_amdgcn_readfirstlane((t >> 6) & 3);
  const int dst_off = gs * kPpOpB + r * kPpRowB;
  const uint32_t smem_lds = (uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t*)smem;
  PpSrc s;
  s.codes = gs == 0 ? a_codes : b_codes;
  s.scales = gs == 0 ? a_scales : b_scales;
  s.base = gs == 0 ? m0 : n0;
  s.rows = gs == 0 ? M : N;
  s.code_ld = K / 2;
  s.scale_ld = K / 16;
  s.NQ = K / 128;
  s.w = w;
  s.st = smem + kPpStOff + 2 * gs * kPpStB;
  s.st_lds = smem_lds + kPpStOff + 2 * (uint32_t)gs * kPpStB;

  floatx16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jn = 0; jn < 2; ++jn)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][jn][e] = 0.0f;

  PpFrags f;
  PpRaw raw;
  pp_stage(s.codes, s.scales, s.base, s.rows, s.code_ld, s.scale_ld, 0, s.st_lds, w, lane);
  pp_stage(s.codes, s.scales, s.base, s.rows, s.code_ld, s.scale_ld, s.NQ > 1 ? 1 : 0,
           s.st_lds + kPpStB, w, lane);
  pp_wait_staged<6>();                                            // quad 0 in (quad 1 may be in flight)
  if (gs == 0) {
    pp_expand<0>(pp_raw<0>(s.st, r), smem + dst_off);             // A(0)
    pp_sync();
    raw = pp_raw<1>(s.st, r);                                     // A(1), expanded in slot 0
    pp_frags<0, 3>(f, smem, wm, wn, h, l32);
    pp_frags<1, 3>(f, smem, wm, wn, h, l32);
    for (int64_t J = 0; J < s.NQ; ++J) {
      pp_turn0<0>(acc, f, raw, smem, s, J, r, dst_off, wm, wn, h, l32, lane);
      pp_turn0<1>(acc, f, raw, smem, s, J, r, dst_off, wm, wn, h, l32, lane);
      pp_turn0<2>(acc, f, raw, smem, s, J, r, dst_off, wm, wn, h, l32, lane);
      pp_turn0<3>(acc, f, raw, smem, s, J, r, dst_off, wm, wn, h, l32, lane);
    }
  } else {
    pp_expand<0>(pp_raw<0>(s.st, r), smem + dst_off);             // B(0)
    pp_expand<1>(pp_raw<1>(s.st, r), smem + kPpBufB + dst_off);   // B(1)
    pp_sync();
    for (int64_t J = 0; J < s.NQ; ++J) {
      pp_turn1<0>(acc, f, raw, smem, s, J, r, dst_off, wm, wn, h, l32, lane);
      pp_turn1<1>(acc, f, raw, smem, s, J, r, dst_off, wm, wn, h, l32, lane);
      pp_turn1<2>(acc, f, raw, smem, s, J, r, dst_off, wm, wn, h, l32, lane);
      pp_turn1<3>(acc, f, raw, smem, s, J, r, dst_off, wm, wn, h, l32, lane);
    }
  }
  // the last staged loads (clamped re-reads) land in LDS the epilogue reuses
  pp_wait_staged<0>();
  pp_sync();

  nv_epilogue(acc, smem, a_amax, b_amax, c, ldc, M, N, m0, n0, wm, wn, lane, vec_store);
}

// ---------------------------------------------------------------- pre-expanded B operand
// The same ping-pong kernel with B handed over already expanded: an FP16
// matrix Bx [N, K] holding v * S * 2^-7 for every element (the exact values
// the in-kernel expansion produces, written once by k_nvfp4_expand).  Group 1
// then expands nothing: in its memory slot it copies B half-stages from Bx
// into a ring of LDS buffers with global -> LDS direct loads, D half-stages
// ahead, and its MFMA slot holds the 16 MFMAs alone.  Group 0 is unchanged
// (it stages and expands A), except that it reads B fragments from the ring.
// Ring buffers hold 256 rows x 64 bytes (one half-stage); 16-byte chunk c of
// row r sits in slot c ^ ((r >> 2) & 3), so both the direct loads (16 rows of
// 64 contiguous bytes per instruction) and the fragment reads (one chunk of 16
// consecutive rows per 16 lanes) avoid bank conflicts.
constexpr int kPxRingB = 256 * 64;                       // one B half-stage
constexpr int kPxD = 4;                                  // B half-stages issued ahead
constexpr int kPxNB = kPxD + 1;                          // ring buffers
constexpr int kPxABufB = kPpOpB;                         // one A half-stage (80-byte rows)
constexpr int kPxStOff = 2 * kPxABufB;                   // A staging after the two A buffers
constexpr int kPxRingOff = kPxStOff + 2 * kPpStB;        // B ring after the A staging
constexpr int kPxLds = kPxRingOff + kPxNB * kPxRingB;    // 159744
static_assert(kPxLds >= kEpiLds && kPxLds <= 160 * 1024, "pre-expanded-B LDS plan");

// Direct loads of B half-stage `hs` (FP16, rows n0 .. n0 + 255 of Bx) into the
// ring buffer at LDS address `dst`: wave w of group 1 copies rows 64 w .. 64 w
// + 63, four instructions of 16 rows x 64 bytes.  Rows past N re-read the last
// row (their results are never stored).  32-bit offsets: N * K * 2 < 2^32.
__device__ __forceinline__ void px_stage_b(const uint8_t* bx, int64_t n0, int64_t N, int64_t K,
                                           int64_t hs, uint32_t dst, int w, int lane) {
  const uint8_t* src = bx + hs * 64;                     // K offset of the half-stage, in bytes
  const uint32_t row_b = (uint32_t)K * 2u, last = (uint32_t)(N - 1), b32 = (uint32_t)n0;
  const uint32_t chunk = (uint32_t)((lane & 3) ^ ((lane >> 4) & 3));
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t gr = min(b32 + (uint32_t)(w * 64 + q * 16 + (lane >> 2)), last);
    dma_to_lds<16>(src, gr * row_b + chunk * 16, dst + (w * 64 + q * 16) * 64);
  }
}

// Fragment reads of one half-stage: A from its 80-byte-row buffer, B from a
// ring buffer.
template <int S>
__device__ __forceinline__ void px_frags(PpFrags& f, const uint8_t* abuf, const uint8_t* ring,
                                         int wm, int wn, int h, int l32) {
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
    f.a[S][mi] = *reinterpret_cast<const halfx8*>(abuf + (wm * 128 + mi * 32 + l32) * kPpRowB + S * 32 + h * 16);
#pragma unroll
  for (int ni = 0; ni < 2; ++ni) {
    const int r = wn * 64 + ni * 32 + l32;
    f.b[S][ni] = *reinterpret_cast<const halfx8*>(ring + r * 64 + (((2 * S + h) ^ ((r >> 2) & 3)) << 4));
  }
}

__device__ __forceinline__ void px_pin_acc(floatx16 (&acc)[4][2]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(acc[i][0]), "+v"(acc[i][1]));
}

// Group 1's MFMA slot: the 16 MFMAs of a half-stage and nothing else.
__device__ __forceinline__ void px_mfma_only(floatx16 (&acc)[4][2], const PpFrags& f) {
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int st = k >> 3, mi = (k & 7) >> 1, ni = k & 1;
    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.b[st][ni], f.a[st][mi], acc[mi][ni], 0, 0, 0);
  }
  __builtin_amdgcn_s_setprio(0);
}

// Group 0, half-stage j = 4 J + U (as pp_turn0, B fragments from the ring).
template <int U>
__device__ __forceinline__ void px_turn0(floatx16 (&acc)[4][2], PpFrags& f, PpRaw& raw,
                                         uint8_t* smem, const PpSrc& s, int64_t J, int r,
                                         int dst_off, int wm, int wn, int h, int l32, int lane) {
  const int64_t j = 4 * J + U;
  pp_mfma_slot<(U + 1) & 1>(acc, f, raw, smem + ((U + 1) & 1) * kPxABufB + dst_off);
  pp_sync();
  if (U == 2) pp_wait_staged<0>();
  raw = pp_raw<(U + 2) & 3>(s.st + ((J + ((U + 2) >> 2)) & 1) * kPpStB, r);
  const uint8_t* ring = smem + kPxRingOff + (int)((j + 1) % kPxNB) * kPxRingB;
  px_frags<0>(f, smem + ((U + 1) & 1) * kPxABufB, ring, wm, wn, h, l32);
  px_frags<1>(f, smem + ((U + 1) & 1) * kPxABufB, ring, wm, wn, h, l32);
  if (U == 2) pp_stage_ahead(s, J, lane);
  pp_sync();
}

// Group 1, half-stage j: slot 2j reads the fragments of j, issues B(j + D) and
// waits for B(j + 1) (read by group 0 in slot 2j + 1); slot 2j + 1 runs the
// MFMAs of j.  B(j + D) goes into the ring buffer of B(j - 1), which both
// groups finished reading by slot 2j - 2.
__device__ __forceinline__ void px_turn1(floatx16 (&acc)[4][2], PpFrags& f, uint8_t* smem,
                                         uint32_t ring_lds, const uint8_t* bx, int64_t n0,
                                         int64_t N, int64_t K, int64_t NH, int64_t j, int w,
                                         int wm, int wn, int h, int l32, int lane) {
  const uint8_t* ring = smem + kPxRingOff + (int)(j % kPxNB) * kPxRingB;
  px_frags<0>(f, smem + (int)(j & 1) * kPxABufB, ring, wm, wn, h, l32);
  px_frags<1>(f, smem + (int)(j & 1) * kPxABufB, ring, wm, wn, h, l32);
  const int64_t hs = j + kPxD < NH ? j + kPxD : NH - 1;
  px_stage_b(bx, n0, N, K, hs, ring_lds + (uint32_t)((j + kPxD) % kPxNB) * kPxRingB, w, lane);
  pp_wait_staged<4 * (kPxD - 1)>();                     // B(j + 1) has landed
  pp_sync();
  px_mfma_only(acc, f);
  px_pin_acc(acc);
  pp_sync();
}

__global__ __launch_bounds__(kNvThreads) void k_gemm_nvfp4_px(
    int64_t M, int64_t N, int64_t K, const uint8_t* a_codes, const uint8_t* a_scales,
    const float* __restrict__ a_amax, const uint8_t* bx, const float* __restrict__ b_amax,
    uint16_t* __restrict__ c, int64_t ldc, int tiles_m, int tiles_n, int vec_store) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int tm, tn;
  tile_of_block(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * 256, n0 = (int64_t)tn * 256;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int g = wave >> 2;
  const int wm = g, wn = wave & 3;
  const int h = lane >> 5, l32 = lane & 31;
  const int gs = __builtin_amdgcn_readfirstlane(g);
  const int r = t & 255, w = __builtin_amdgcn_readfirstlane((t >> 6) & 3);
  const uint32_t smem_lds = (uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t*)smem;
  const int64_t NH = K / 32;

  floatx16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jn = 0; jn < 2; ++jn)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][jn][e] = 0.0f;

  PpFrags f;
  if (gs == 0) {
    PpSrc s;
    s.codes = a_codes;
    s.scales = a_scales;
    s.base = m0;
    s.rows = M;
    s.code_ld = K / 2;
    s.scale_ld = K / 16;
    s.NQ = K / 128;
    s.w = w;
    s.st = smem + kPxStOff;
    s.st_lds = smem_lds + kPxStOff;
    const int dst_off = r * kPpRowB;
    PpRaw raw;
    pp_stage(s.codes, s.scales, s.base, s.rows, s.code_ld, s.scale_ld, 0, s.st_lds, w, lane);
    pp_stage(s.codes, s.scales, s.base, s.rows, s.code_ld, s.scale_ld, s.NQ > 1 ? 1 : 0,
             s.st_lds + kPpStB, w, lane);
    pp_wait_staged<6>();                                          // quad 0 in
    pp_expand<0>(pp_raw<0>(s.st, r), smem + dst_off);             // A(0)
    pp_sync();                                                    // A(0) and B(0) visible
    raw = pp_raw<1>(s.st, r);
    px_frags<0>(f, smem, smem + kPxRingOff, wm, wn, h, l32);
    px_frags<1>(f, smem, smem + kPxRingOff, wm, wn, h, l32);
    for (int64_t J = 0; J < s.NQ; ++J) {
      px_turn0<0>(acc, f, raw, smem, s, J, r, dst_off, wm, wn, h, l32, lane);
      px_turn0<1>(acc, f, raw, smem, s, J, r, dst_off, wm, wn, h, l32, lane);
      px_turn0<2>(acc, f, raw, smem, s, J, r, dst_off, wm, wn, h, l32, lane);
      px_turn0<3>(acc, f, raw, smem, s, J, r, dst_off, wm, wn, h, l32, lane);
    }
  } else {
    const uint32_t ring_lds = smem_lds + kPxRingOff;
#pragma unroll
    for (int i = 0; i < kPxD; ++i)
      px_stage_b(bx, n0, N, K, i < NH ? i : NH - 1, ring_lds + (uint32_t)i * kPxRingB, w, lane);
    pp_wait_staged<4 * (kPxD - 1)>();                             // B(0) has landed
    pp_sync();
    for (int64_t j = 0; j < NH; ++j)
      px_turn1(acc, f, smem, ring_lds, bx, n0, N, K, NH, j, w, wm, wn, h, l32, lane);
  }
  pp_wait_staged<0>();                                            // clamped tail loads landed
  pp_sync();
  nv_epilogue(acc, smem, a_amax, b_amax, c, ldc, M, N, m0, n0, wm, wn, lane, vec_store);
}

// FP16 expansion of an NVFP4 operand: out [R, K] = v * S * 2^-7 (exact), the
// values the GEMM's in-kernel expansion produces.  A thread expands one
// 16-element block per trip (8 code bytes, one scale byte, 32 output bytes).
__global__ __launch_bounds__(256) void k_nvfp4_expand(const uint2* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales,
                                                      int64_t nblk, uint4* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblk; b += stride) {
    const uint2 cw = codes[b];
    const halfx2 s = nvfp4_scale_pair<0>((uint32_t)scales[b]);
    out[2 * b] = __builtin_bit_cast(uint4, dequant8(cw.x, s));
    out[2 * b + 1] = __builtin_bit_cast(uint4, dequant8(cw.y, s));
  }
}

}  // namespace

hipError_t launch_gemm_nvfp4(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                             const float* aa, const uint8_t* bc, const uint8_t* bs,
                             const float* ba, void* c, int64_t ldc, void* scratch,
                             size_t scratch_bytes, hipStream_t s) {
  const int tiles_m = (int)((M + 255) / 256), tiles_n = (int)((N + 255) / 256);
  const auto al = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; };
  // the register-expansion kernel where it applies (13-14% faster on the
  // Llama MLP shapes), its last wave split over K when it would leave more
  // than half the compute units idle; the ping-pong kernel for K % 256 == 128
  if (gemm_nvfp4_rx_fits(M, N, K, ac, as, bc, bs)) {
    const int tail = gemm_nvfp4_rx_split(M, N, K, device_cus());
    if (tail == 0) return launch_gemm_nvfp4_rx(M, N, K, ac, as, aa, bc, bs, ba, c, ldc, 0, nullptr, s);
    const size_t bytes = (size_t)tail * kRxSplitTileBytes;
    if (scratch != nullptr) {
      if (scratch_bytes < bytes) return hipErrorInvalidValue;
      return launch_gemm_nvfp4_rx(M, N, K, ac, as, aa, bc, bs, ba, c, ldc, tail, scratch, s);
    }
    void* part = nullptr;
    hipError_t e = hipMallocAsync(&part, bytes, s);
    if (e != hipSuccess) return e;
    e = launch_gemm_nvfp4_rx(M, N, K, ac, as, aa, bc, bs, ba, c, ldc, tail, part, s);
    const hipError_t f = hipFreeAsync(part, s);
    return e != hipSuccess ? e : f;
  }
  // the ping-pong kernel stages 64 code bytes and 8 scale bytes per row and four
  // half-stages, runs its loop in groups of four half-stages, and addresses
  // each operand with 32-bit byte offsets
  const bool fast = K > 0 && (K % 128 == 0) && al(ac, 16) && al(bc, 16) && al(as, 4) && al(bs, 4) &&
                    M * (K / 2) < ((int64_t)1 << 32) && N * (K / 2) < ((int64_t)1 << 32);
  const bool vec_store = (ldc % 8 == 0) && al(c, 16);
  if (set_lds_limit(reinterpret_cast<const void*>(&k_gemm_nvfp4_pp), kPpLds) != hipSuccess ||
      set_lds_limit(reinterpret_cast<const void*>(&k_gemm_nvfp4<false>), kNvLds) != hipSuccess)
    return hipErrorInvalidConfiguration;
  uint16_t* cp = static_cast<uint16_t*>(c);
  const dim3 grid((unsigned)(tiles_m * tiles_n)), block(kNvThreads);
  if (fast)
    hipLaunchKernelGGL(k_gemm_nvfp4_pp, grid, block, kPpLds, s, M, N, K, ac, as, aa, bc, bs, ba,
                       cp, ldc, tiles_m, tiles_n, vec_store ? 1 : 0);
  else
    hipLaunchKernelGGL(k_gemm_nvfp4<false>, grid, block, kNvLds, s, M, N, K, ac, as, aa, bc, bs, ba,
                       cp, ldc, tiles_m, tiles_n, vec_store ? 1 : 0);
  return hipGetLastError();
}

}  // namespace bsq

namespace bsq {

hipError_t launch_gemm_nvfp4_bx(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                                const float* aa, const void* bx, const float* ba, void* c,
                                int64_t ldc, hipStream_t s) {
  const int tiles_m = (int)((M + 255) / 256), tiles_n = (int)((N + 255) / 256);
  const auto al = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; };
  if (!(K > 0 && K % 128 == 0 && al(ac, 16) && al(as, 4) && al(bx, 16) &&
        M * (K / 2) < ((int64_t)1 << 32) && N * K * 2 < ((int64_t)1 << 32)))
    return hipErrorNotSupported;
  const bool vec_store = (ldc % 8 == 0) && al(c, 16);
  if (set_lds_limit(reinterpret_cast<const void*>(&k_gemm_nvfp4_px), kPxLds) != hipSuccess)
    return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(k_gemm_nvfp4_px, dim3((unsigned)(tiles_m * tiles_n)), dim3(kNvThreads), kPxLds, s,
                     M, N, K, ac, as, aa, static_cast<const uint8_t*>(bx), ba,
                     static_cast<uint16_t*>(c), ldc, tiles_m, tiles_n, vec_store ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_nvfp4_expand(const uint8_t* codes, const uint8_t* scales, int64_t R, int64_t K,
                               void* out, hipStream_t s) {
  const int64_t nblk = R * (K / 16);
  int64_t g = (nblk + 255) / 256;
  g = g < 1 ? 1 : (g > 4096 ? 4096 : g);
  hipLaunchKernelGGL(k_nvfp4_expand, dim3((unsigned)g), dim3(256), 0, s,
                     reinterpret_cast<const uint2*>(codes), scales, nblk, static_cast<uint4*>(out));
  return hipGetLastError();
}

size_t gemm_nvfp4_scratch_bytes(int64_t M, int64_t N, int64_t K, const uint8_t* ac,
                                const uint8_t* as, const uint8_t* bc, const uint8_t* bs) {
  if (!gemm_nvfp4_rx_fits(M, N, K, ac, as, bc, bs)) return 0;
  return (size_t)gemm_nvfp4_rx_split(M, N, K, device_cus()) * kRxSplitTileBytes;
}

}  // namespace bsq
