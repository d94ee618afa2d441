// MX block-scaled GEMM for gfx950: C[M, N] (BF16) = A[M, K] . B[N, K]^T with
// MXFP8 (E4M3) or MXFP4 (E2M1) codes and one E8M0 scale per 32 K-elements;
// the same kernels run the per-tensor FP8 baseline (E4M3 codes, unit block
// scales, alpha = s_dec(A) * s_dec(B) from the two amaxes).
//
// HN page opcode84 (MXFP8 / MXFP4 GEMMs on the OCP Microscaling formats): the
// block scale is applied inside the matrix unit.  On CDNA4,
// v_mfma_scale_f32_32x32x64_f8f6f4 takes one E8M0 scale per lane per 32-element
// K block, which is exactly the MX block, so codes go from LDS straight into
// the MFMA (operand layouts at MxFrag below).  The NVFP4 GEMM lives in
// bsq_gemm_nvfp4.hip.
//
// Tiling: 256 x 256 output tile per 512-thread workgroup (8 waves as 2 x 4,
// each 128 (M) x 64 (N) = 4 x 2 MFMA tiles of 32 x 32); each wave computes
// D = B_tile . A_tile^T so that every lane holds consecutive output columns.
//  * k_gemm_mx_pp (K % 512 == 0, aligned operands): 64 code bytes per row per
//    stage (K 64 for MXFP8, 128 for MXFP4) staged in LDS by global -> LDS
//    direct loads four stages ahead, scales 16 bytes per row per period of
//    8 / 4 stages; the two waves of each SIMD alternate between the MFMAs of
//    one stage and the fragment reads of the next (layout and schedule below).
//  * k_gemm (any K): the general path, register-staged, one stage ahead.
//  * where K % 512 == 0 the four-wave kernel k_gemm_mx_rx
//    (bsq_gemm_mx_rx.hip) takes precedence: same K order, same bits.
//
// K order inside a stage: an MFMA only needs A and B to agree on which K index
// sits in which slot, so lane half h takes one contiguous run of the stage.
#include "bsq_gemm_common.hpp"
#include "bsq_internal.hpp"

namespace bsq {

namespace {

constexpr int kBM = 256, kBN = 256, kThreads = 512;

template <int FMT>
struct Cfg {
  static constexpr int BK = FMT == kMXFP4 ? 256 : 128;                 // K elements per stage
  static constexpr int RB = fp8_elems(FMT) ? BK : BK / 2;              // code bytes per row per stage
  static constexpr int SB = FMT == kNVFP4 ? BK / 16 : BK / 32;         // scale bytes per row per stage
  static constexpr int LDR = RB + 16;                                  // padded LDS row stride
  static constexpr int CODE_BYTES = kBM * LDR;                         // per operand per stage
  static constexpr int SCALE_BYTES = kBM * SB;
  static constexpr int STAGE_BYTES = 2 * CODE_BYTES + 2 * SCALE_BYTES;
  static constexpr int CHUNKS = kBM * RB / 16;                         // 16B code chunks per operand
  static constexpr int CPT = CHUNKS / kThreads;                        // per thread
  static constexpr int STEPS = FMT == kNVFP4 ? BK / 16 : BK / 64;      // MFMA K steps per stage
};

// Scaled MFMA with the scale byte chosen by the K step (the byte select must be
// an immediate).
template <int FMTC>
__device__ __forceinline__ floatx16 mfma_mx(int step, const intx8& a, const intx8& b,
                                            const floatx16& c, uint32_t sa, uint32_t sb) {
  switch (step) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FMTC, FMTC, 0, (int)sa, 0, (int)sb);
    case 1: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FMTC, FMTC, 1, (int)sa, 1, (int)sb);
    case 2: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FMTC, FMTC, 2, (int)sa, 2, (int)sb);
    default: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FMTC, FMTC, 3, (int)sa, 3, (int)sb);
  }
}

// Global -> register staging of one stage of one operand (codes + scales).
template <int FMT>
struct Stage {
  uint4 code[Cfg<FMT>::CPT];
  uint32_t scale[2];          // this thread's share of the scale rows (8 bytes max)
};

// Load stage kt of an operand with rows [row0, row0+256) of a [rows, K] matrix.
// Fast path: whole 16-byte chunks and whole scale words (K % BK == 0 and
// aligned pointers).  Generic path: byte loads with K bounds (zeros past K).
template <int FMT, bool FAST>
__device__ __forceinline__ void load_stage(Stage<FMT>& st, const uint8_t* __restrict__ codes,
                                           const uint8_t* __restrict__ scales, int64_t rows,
                                           int64_t row0, int64_t kt, int64_t code_ld,
                                           int64_t scale_ld) {
  using C = Cfg<FMT>;
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < C::CPT; ++i) {
    const int ch = t + i * kThreads;
    const int r = ch / (C::RB / 16), c16 = ch % (C::RB / 16);
    int64_t gr = row0 + r;
    gr = gr < rows ? gr : rows - 1;
    const int64_t kb = kt * C::RB + c16 * 16;            // byte offset along K
    if constexpr (FAST) {
      st.code[i] = *reinterpret_cast<const uint4*>(codes + gr * code_ld + kb);
    } else {
      uint8_t b[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) b[j] = (kb + j < code_ld) ? codes[gr * code_ld + kb + j] : 0;
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = b[4 * j] | (b[4 * j + 1] << 8) | (b[4 * j + 2] << 16) | ((uint32_t)b[4 * j + 3] << 24);
      st.code[i] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
  // scales: thread t < 256 loads row t's SB bytes (SB is 4 or 8); per-tensor
  // FP8 has none and uses the E8M0 unit scale (127) for every block
  st.scale[0] = st.scale[1] = FMT == kFP8 ? 0x7F7F7F7Fu : 0u;
  if (FMT != kFP8 && t < kBM) {
    int64_t gr = row0 + t;
    gr = gr < rows ? gr : rows - 1;
    const int64_t sb = kt * C::SB;
    if constexpr (FAST) {
      if (C::SB == 8) {
        const uint2 v = *reinterpret_cast<const uint2*>(scales + gr * scale_ld + sb);
        st.scale[0] = v.x;
        st.scale[1] = v.y;
      } else {
        st.scale[0] = *reinterpret_cast<const uint32_t*>(scales + gr * scale_ld + sb);
      }
    } else {
#pragma unroll
      for (int j = 0; j < C::SB; ++j) {
        const uint32_t b = (sb + j < scale_ld) ? scales[gr * scale_ld + sb + j] : 0;
        st.scale[j >> 2] |= b << (8 * (j & 3));
      }
    }
  }
}

template <int FMT>
__device__ __forceinline__ void store_stage(const Stage<FMT>& st, uint8_t* lds_codes,
                                            uint8_t* lds_scales) {
  using C = Cfg<FMT>;
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < C::CPT; ++i) {
    const int ch = t + i * kThreads;
    const int r = ch / (C::RB / 16), c16 = ch % (C::RB / 16);
    *reinterpret_cast<uint4*>(lds_codes + r * C::LDR + c16 * 16) = st.code[i];
  }
  if (t < kBM) {
    if (C::SB == 8)
      *reinterpret_cast<uint2*>(lds_scales + t * 8) = make_uint2(st.scale[0], st.scale[1]);
    else
      *reinterpret_cast<uint32_t*>(lds_scales + t * 4) = st.scale[0];
  }
}

template <int FMT, bool FAST>
__global__ __launch_bounds__(kThreads) void k_gemm(
    int64_t M, int64_t N, int64_t K, const uint8_t* __restrict__ a_codes,
    const uint8_t* __restrict__ a_scales, const float* __restrict__ a_amax,
    const uint8_t* __restrict__ b_codes, const uint8_t* __restrict__ b_scales,
    const float* __restrict__ b_amax, uint16_t* __restrict__ c, int64_t ldc, int tiles_m,
    int tiles_n, int vec_store) {
  using C = Cfg<FMT>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  // grouped tile order: 8 M-tiles share each sweep over N for L2 reuse
  const int pid = blockIdx.x;
  constexpr int GROUP = 8;
  const int group_size = GROUP * tiles_n;
  const int gid = pid / group_size;
  const int first_m = gid * GROUP;
  const int gm = min(tiles_m - first_m, GROUP);
  const int tm = first_m + (pid % group_size) % gm;
  const int tn = (pid % group_size) / gm;
  const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN;

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 2, wn = wave & 3;            // 2 x 4 waves
  const int h = lane >> 5, l32 = lane & 31;

  const int64_t code_ld = fp8_elems(FMT) ? K : K / 2;
  const int64_t scale_ld = FMT == kNVFP4 ? K / 16 : K / 32;
  const int64_t KT = (K + C::BK - 1) / C::BK;

  floatx16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  auto lds_a = [&](int buf) { return smem + buf * C::STAGE_BYTES; };
  auto lds_b = [&](int buf) { return smem + buf * C::STAGE_BYTES + C::CODE_BYTES; };
  auto lds_sa = [&](int buf) { return smem + buf * C::STAGE_BYTES + 2 * C::CODE_BYTES; };
  auto lds_sb = [&](int buf) {
    return smem + buf * C::STAGE_BYTES + 2 * C::CODE_BYTES + C::SCALE_BYTES;
  };

  Stage<FMT> sa, sb;
  if (KT > 0) {
    load_stage<FMT, FAST>(sa, a_codes, a_scales, M, m0, 0, code_ld, scale_ld);
    load_stage<FMT, FAST>(sb, b_codes, b_scales, N, n0, 0, code_ld, scale_ld);
    store_stage<FMT>(sa, lds_a(0), lds_sa(0));
    store_stage<FMT>(sb, lds_b(0), lds_sb(0));
  }
  __syncthreads();

  for (int64_t kt = 0; kt < KT; ++kt) {
    const int buf = (int)(kt & 1);
    const bool more = kt + 1 < KT;
    if (more) {
      load_stage<FMT, FAST>(sa, a_codes, a_scales, M, m0, kt + 1, code_ld, scale_ld);
      load_stage<FMT, FAST>(sb, b_codes, b_scales, N, n0, kt + 1, code_ld, scale_ld);
    }
    const uint8_t* La = lds_a(buf);
    const uint8_t* Lb = lds_b(buf);
    const uint8_t* LSa = lds_sa(buf);
    const uint8_t* LSb = lds_sb(buf);

    {
      // MX operand layouts of v_mfma_scale_f32_32x32x64_f8f6f4 (K = 64 = two
      // 32-element MX blocks per instruction; block b's E8M0 scale comes from
      // lane half b):
      //  * FP4: lane half h supplies one whole block (32 codes, 16 bytes); here
      //    step s of the stage uses block h*STEPS + s for lane half h.
      //  * FP8: bytes 0-15 of every lane belong to the first block of the
      //    instruction and bytes 16-31 to the second, each block split over the
      //    two lane halves; here step s uses blocks 2s and 2s+1, lane half h
      //    taking elements [16h, 16h+16) of each.
      constexpr int FMTC = fp8_elems(FMT) ? 0 : 4;    // cbsz / blgp operand type
      uint32_t sca[4], scb[2];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int row = wm * 128 + mi * 32 + l32;
        sca[mi] = fp8_elems(FMT) ? (*reinterpret_cast<const uint32_t*>(LSa + row * 4) >> (8 * h))
                                : *reinterpret_cast<const uint32_t*>(LSa + row * 8 + 4 * h);
      }
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int row = wn * 64 + ni * 32 + l32;
        scb[ni] = fp8_elems(FMT) ? (*reinterpret_cast<const uint32_t*>(LSb + row * 4) >> (8 * h))
                                : *reinterpret_cast<const uint32_t*>(LSb + row * 8 + 4 * h);
      }
      auto frag = [&](const uint8_t* base, int row, int s) {
        const uint8_t* p = base + row * C::LDR;
        uint4 lo, hi = make_uint4(0, 0, 0, 0);
        if (fp8_elems(FMT)) {
          lo = *reinterpret_cast<const uint4*>(p + (2 * s) * 32 + 16 * h);
          hi = *reinterpret_cast<const uint4*>(p + (2 * s + 1) * 32 + 16 * h);
        } else {
          lo = *reinterpret_cast<const uint4*>(p + (h * C::STEPS + s) * 16);
        }
        return intx8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                     (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      };
#pragma unroll
      for (int s = 0; s < C::STEPS; ++s) {
        const int sel = fp8_elems(FMT) ? 2 * s : s;   // scale byte of this lane's block
        intx8 fa[4], fb[2];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) fa[mi] = frag(La, wm * 128 + mi * 32 + l32, s);
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) fb[ni] = frag(Lb, wn * 64 + ni * 32 + l32, s);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
          for (int ni = 0; ni < 2; ++ni)
            acc[mi][ni] = mfma_mx<FMTC>(sel, fb[ni], fa[mi], acc[mi][ni], scb[ni], sca[mi]);
        __builtin_amdgcn_sched_barrier(0);      // keep each step's fragments short-lived
      }
    }

    if (more) {
      store_stage<FMT>(sa, lds_a(buf ^ 1), lds_sa(buf ^ 1));
      store_stage<FMT>(sb, lds_b(buf ^ 1), lds_sb(buf ^ 1));
    }
    __syncthreads();
  }

  // epilogue: alpha * acc -> BF16 (RNE).  Lane holds column m = l32 of D = C^T,
  // rows n = 8*(r/4) + 4*h + r%4 of each 32x32 tile.
  const float alpha = FMT == kFP8 ? fp8_s_dec(*a_amax) * fp8_s_dec(*b_amax) : 1.0f;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int64_t m = m0 + wm * 128 + mi * 32 + l32;
    if (m >= M) continue;
    uint16_t* crow = c + m * ldc;
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t n = n0 + wn * 64 + ni * 32 + 8 * q + 4 * h;
        const floatx16& a = acc[mi][ni];
        const uint32_t w0 = pack_bf16x2(a[4 * q] * alpha, a[4 * q + 1] * alpha);
        const uint32_t w1 = pack_bf16x2(a[4 * q + 2] * alpha, a[4 * q + 3] * alpha);
        if (vec_store && n + 3 < N) {
          *reinterpret_cast<uint2*>(crow + n) = make_uint2(w0, w1);
        } else {
          const uint16_t b[4] = {(uint16_t)w0, (uint16_t)(w0 >> 16), (uint16_t)w1, (uint16_t)(w1 >> 16)};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < N) crow[n + e] = b[e];
        }
      }
    }
  }
}

// ---------------------------------------------------------------- staged kernel
//
// Stage layout in LDS: four code buffers of 32 KiB (A codes 256 rows x 64
// bytes, then B codes; 16-byte chunk c of row r in slot c ^ ((r >> 2) & 3),
// which keeps the fragment reads of 16 consecutive rows on distinct banks),
// then two scale buffers of 8 KiB (16 scale bytes of each of the 256 A rows
// and 256 B rows: four MXFP4 stages or eight MXFP8 stages).  A row's scales
// are fetched as one 16-byte piece per period instead of one dword per stage,
// which removes over a third of the L2 requests.
constexpr int kMxRowB = 64;
constexpr int kMxCodeB = 256 * kMxRowB;
constexpr int kMxStageB = 2 * kMxCodeB;                  // 32 KiB of codes per stage
constexpr int kMxStages = 4;
constexpr int kMxScOff = kMxStages * kMxStageB;          // scale buffers after the code buffers
constexpr int kMxScB = 2 * 256 * 16;                     // one scale period, both operands
constexpr int kMxLds = kMxScOff + 2 * kMxScB > kEpiLds ? kMxScOff + 2 * kMxScB : kEpiLds;
static_assert(kMxLds <= 160 * 1024, "MX staged LDS plan");

// Stages per scale period: 16 bytes of a row hold 4 MXFP4 stages (128 K
// each, 4 blocks) or 8 MXFP8 stages (64 K each, 2 blocks).
template <int FMT>
constexpr int mx_period() { return fp8_elems(FMT) ? 8 : 4; }

// Fragments and scale operands of one stage for one wave.  MXFP8: fa[0]/fa[1]
// are bytes 0-15 / 16-31 of the operand (chunks h and 2 + h); MXFP4: fa[s] is
// the operand of K step s (chunk 2h + s, upper half zero).  Scale operands are
// read as the byte (MXFP8) or byte pair (MXFP4, the K step selecting one) the
// instruction uses: lane half h carries block h of the instruction (MXFP8) or
// blocks 2h, 2h + 1 of the stage (MXFP4).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
struct MxFrag {
  u32x4 fa[2][4], fb[2][2];
  uint32_t sa[4], sb[2];
};

// Read number Q (0..17) of a stage's fragments: 8 A chunks, 4 B chunks, 4 A
// scales, 2 B scales.  sb0 = the stage's first scale byte within its period's
// 16 bytes (MXFP8: 2 x position, 2 blocks per stage; MXFP4: 4 x position).
template <int FMT, int Q>
__device__ __forceinline__ void mx_read(MxFrag& F, const uint8_t* buf, const uint8_t* sbuf, int sb0,
                                        int wm, int wn, int h, int l32) {
  const uint8_t* La = buf;
  const uint8_t* Lb = buf + kMxCodeB;
  const uint8_t* Sa = sbuf;
  const uint8_t* Sb = sbuf + 256 * 16;
  const auto chunk = [](const uint8_t* base, int row, int c) {
    return *reinterpret_cast<const u32x4*>(base + row * kMxRowB + ((c ^ ((row >> 2) & 3)) << 4));
  };
  if (Q < 8) {
    const int j = Q >> 2, mi = Q & 3, row = wm * 128 + mi * 32 + l32;
    F.fa[j][mi] = chunk(La, row, fp8_elems(FMT) ? (j == 0 ? h : 2 + h) : 2 * h + j);
  } else if (Q < 12) {
    const int j = (Q - 8) >> 1, ni = (Q - 8) & 1, row = wn * 64 + ni * 32 + l32;
    F.fb[j][ni] = chunk(Lb, row, fp8_elems(FMT) ? (j == 0 ? h : 2 + h) : 2 * h + j);
  } else if (FMT == kFP8) {                        // per-tensor: E8M0 unit scale
    if (Q < 16) F.sa[Q - 12] = 0x7Fu;
    else F.sb[Q - 16] = 0x7Fu;
  } else if (Q < 16) {
    const int mi = Q - 12, row = wm * 128 + mi * 32 + l32;
    F.sa[mi] = FMT == kMXFP8 ? (uint32_t)Sa[row * 16 + sb0 + h]
                             : (uint32_t)*reinterpret_cast<const uint16_t*>(Sa + row * 16 + sb0 + 2 * h);
  } else {
    const int ni = Q - 16, row = wn * 64 + ni * 32 + l32;
    F.sb[ni] = FMT == kMXFP8 ? (uint32_t)Sb[row * 16 + sb0 + h]
                             : (uint32_t)*reinterpret_cast<const uint16_t*>(Sb + row * 16 + sb0 + 2 * h);
  }
}

// MFMA number I of a stage (MXFP8: 8, mi = I / 2, ni = I % 2; MXFP4: 16, K step
// I / 8).
template <int FMT, int I>
__device__ __forceinline__ void mx_mfma(floatx16 (&acc)[4][2], const MxFrag& F) {
  constexpr int FMTC = fp8_elems(FMT) ? 0 : 4;           // cbsz / blgp operand type
  constexpr int s = fp8_elems(FMT) ? 0 : I >> 3;
  constexpr int mi = (I & 7) >> 1, ni = I & 1;
  const u32x4 z = {0u, 0u, 0u, 0u};
  const u32x4 al = F.fa[s][mi], bl = F.fb[s][ni];
  const u32x4 ah = fp8_elems(FMT) ? F.fa[1][mi] : z;
  const u32x4 bh = fp8_elems(FMT) ? F.fb[1][ni] : z;
  const intx8 a = __builtin_bit_cast(intx8, __builtin_shufflevector(al, ah, 0, 1, 2, 3, 4, 5, 6, 7));
  const intx8 b = __builtin_bit_cast(intx8, __builtin_shufflevector(bl, bh, 0, 1, 2, 3, 4, 5, 6, 7));
  acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, acc[mi][ni], FMTC, FMTC, s,
                                                                (int)F.sb[ni], s, (int)F.sa[mi]);
}

// ---------------------------------------------------------------- ping-pong kernel
//
// The matrix pipe of every SIMD is fed by one wave while its sibling wave
// reads fragments.  The two waves of a SIMD belong to different
// groups (waves 0-3 compute rows 0-127 of the tile, waves 4-7 rows 128-255);
// time is cut into slots separated by workgroup barriers.  Group 0 runs the
// MFMAs of stage j on slot 2j and reads all fragments of stage j + 1 on slot
// 2j + 1; group 1 reads stage j on slot 2j and runs its MFMAs on slot 2j + 1.
// Staging: on slot 2j + 1 both groups issue stage j + 4 into the buffer of
// stage j (read by group 0 on slot 2j - 1 and by group 1 on slot 2j), group 0
// the A rows and group 1 the B rows (wave w: rows 64 w .. 64 w + 63, four
// direct loads of 16 rows x 64 bytes), each with one scale load (the rows'
// 16 bytes of a scale period at the period's first stage, else lane 0
// reloading its own 16 bytes in place) so that every issue is five loads
// (four for per-tensor FP8, which has no scales).
// Stage j is issued on slot 2j - 7 and waited for by its issuing waves on slot
// 2j - 2 (their loads of stages j + 1 and j + 2 may stay in flight), before the
// barrier that precedes its first read on slot 2j - 1.  A scale period q is
// issued with code stage q P on slot 2 q P - 7 into the buffer of period q - 2,
// whose last read was on slot 2 q P - 2 P - 2 (P >= 4 stages per period).
// Loads per issued stage per wave: four code loads and the scale slot (none
// for per-tensor FP8).
template <int FMT>
constexpr int mx_pp_loads() { return FMT == kFP8 ? 4 : 5; }
static_assert(kMxStages == 4, "the stage ring is indexed with s & 3");

struct MxPpSrc {
  const uint8_t* codes;                                  // this group's operand
  const uint8_t* scales;
  uint32_t code_off[4];                                  // this lane's byte offsets (stage 0)
  uint32_t scale_off;
  uint32_t code_lds, scale_lds;                          // this wave's LDS rows (stage buffer 0, period buffer 0)
  int64_t KT, NP;
};

// Issue stage s (clamped to the last) and its scale slot.
template <int FMT>
__device__ __forceinline__ void mx_pp_issue(const MxPpSrc& x, int64_t s, int lane) {
  constexpr int PER = mx_period<FMT>();
  const int64_t cs = s < x.KT ? s : x.KT - 1;
  const uint32_t buf = x.code_lds + (uint32_t)(s & 3) * kMxStageB;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    dma_to_lds<16>(x.codes + cs * kMxRowB, x.code_off[i], buf + i * 16 * kMxRowB);
  if (FMT == kFP8) return;
  const int64_t q = s / PER, cq = q < x.NP ? q : x.NP - 1;
  if (s - q * PER == 0)
    dma_to_lds<16>(x.scales + cq * 16, x.scale_off, x.scale_lds + (uint32_t)(q & 1) * kMxScB);
  else if (lane == 0)
    dma_to_lds<16>(x.scales + cq * 16, x.scale_off, x.scale_lds + (uint32_t)(q & 1) * kMxScB);
}

// Slot boundaries for register-only work.  The barriers order memory accesses
// only, and the MFMAs touch no memory, so without these empty statements the
// compiler may move a slot's MFMAs across a barrier into the other slot.  An
// asm statement that reads and writes the accumulators (or the fragments)
// keeps the MFMAs that produce (or consume) them on its side.
__device__ __forceinline__ void pin_acc(floatx16 (&acc)[4][2]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    asm volatile("" : "+v"(acc[i][0]), "+v"(acc[i][1]));
}
__device__ __forceinline__ void pin_frag(MxFrag& F) {
#pragma unroll
  for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(F.fa[0][i]), "+v"(F.fa[1][i]), "+v"(F.sa[i]));
#pragma unroll
  for (int i = 0; i < 2; ++i) asm volatile("" : "+v"(F.fb[0][i]), "+v"(F.fb[1][i]), "+v"(F.sb[i]));
}

template <int FMT>
__device__ __forceinline__ void mx_pp_mfmas(floatx16 (&acc)[4][2], const MxFrag& F) {
  mx_mfma<FMT, 0>(acc, F);
  mx_mfma<FMT, 1>(acc, F);
  mx_mfma<FMT, 2>(acc, F);
  mx_mfma<FMT, 3>(acc, F);
  mx_mfma<FMT, 4>(acc, F);
  mx_mfma<FMT, 5>(acc, F);
  mx_mfma<FMT, 6>(acc, F);
  mx_mfma<FMT, 7>(acc, F);
  if (FMT == kMXFP4) {
    mx_mfma<FMT, 8>(acc, F);
    mx_mfma<FMT, 9>(acc, F);
    mx_mfma<FMT, 10>(acc, F);
    mx_mfma<FMT, 11>(acc, F);
    mx_mfma<FMT, 12>(acc, F);
    mx_mfma<FMT, 13>(acc, F);
    mx_mfma<FMT, 14>(acc, F);
    mx_mfma<FMT, 15>(acc, F);
  }
}

// All fragments and scale operands of stage s.
template <int FMT, int Q>
__device__ __forceinline__ void mx_pp_read_from(MxFrag& F, const uint8_t* buf, const uint8_t* sbuf,
                                                int sb0, int wm, int wn, int h, int l32) {
  mx_read<FMT, Q>(F, buf, sbuf, sb0, wm, wn, h, l32);
  if constexpr (Q + 1 < 18) mx_pp_read_from<FMT, Q + 1>(F, buf, sbuf, sb0, wm, wn, h, l32);
}
template <int FMT>
__device__ __forceinline__ void mx_pp_read(MxFrag& F, const uint8_t* smem, int64_t s, int wm, int wn,
                                           int h, int l32) {
  constexpr int PER = mx_period<FMT>();
  const int64_t q = s / PER;
  const int sb0 = (int)(s - q * PER) * (fp8_elems(FMT) ? 2 : 4);
  mx_pp_read_from<FMT, 0>(F, smem + (s & 3) * kMxStageB, smem + kMxScOff + (q & 1) * kMxScB, sb0,
                          wm, wn, h, l32);
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void k_gemm_mx_pp(
    int64_t M, int64_t N, int64_t K, const uint8_t* a_codes, const uint8_t* a_scales,
    const float* __restrict__ a_amax, const uint8_t* b_codes, const uint8_t* b_scales,
    const float* __restrict__ b_amax, uint16_t* __restrict__ c, int64_t ldc, int tiles_m,
    int tiles_n, int vec_store) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int tm, tn;
  tile_of_block(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int h = lane >> 5, l32 = lane & 31;
  // group and wave within the group, scalar: they address the direct loads
  const int gs = __builtin_amdgcn_readfirstlane(wave >> 2);
  const int w = __builtin_amdgcn_readfirstlane(wave & 3);
  const int64_t code_ld = fp8_elems(FMT) ? K : K / 2, scale_ld = K / 32;
  const uint32_t smem_lds = (uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t*)smem;
  MxPpSrc x;
  x.codes = gs == 0 ? a_codes : b_codes;
  x.scales = gs == 0 ? a_scales : b_scales;
  x.KT = code_ld / kMxRowB;
  x.NP = x.KT / mx_period<FMT>();                        // scale periods (none for per-tensor FP8)
  {
    const int64_t base = gs == 0 ? m0 : n0, rows = gs == 0 ? M : N;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = w * 64 + i * 16 + (lane >> 2);      // row within the tile
      const int64_t gr = base + rr < rows ? base + rr : rows - 1;
      x.code_off[i] = (uint32_t)(gr * code_ld + (((lane & 3) ^ ((rr >> 2) & 3)) << 4));
    }
    const int rr = w * 64 + lane;
    const int64_t gr = base + rr < rows ? base + rr : rows - 1;
    x.scale_off = (uint32_t)(gr * scale_ld);
  }
  x.code_lds = smem_lds + (uint32_t)gs * kMxCodeB + (uint32_t)(w * 64) * kMxRowB;
  x.scale_lds = smem_lds + kMxScOff + (uint32_t)gs * (256 * 16) + (uint32_t)(w * 64) * 16;

  floatx16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  mx_pp_issue<FMT>(x, 0, lane);
  mx_pp_issue<FMT>(x, 1, lane);
  mx_pp_issue<FMT>(x, 2, lane);
  mx_pp_issue<FMT>(x, 3, lane);
  wait_vmcnt<3 * mx_pp_loads<FMT>()>();                  // stage 0 and period 0 in
  lds_barrier();
  MxFrag F;
  if (gs == 0) {
    mx_pp_read<FMT>(F, smem, 0, wm, wn, h, l32);
    for (int64_t j = 0; j < x.KT; ++j) {
      pin_frag(F);
      mx_pp_mfmas<FMT>(acc, F);                          // slot 2j
      pin_acc(acc);
      wait_vmcnt<2 * mx_pp_loads<FMT>()>();              // stage j + 1 in
      lds_barrier();
      mx_pp_read<FMT>(F, smem, j + 1, wm, wn, h, l32);   // slot 2j + 1
      mx_pp_issue<FMT>(x, j + 4, lane);
      lds_barrier();
    }
  } else {
    for (int64_t j = 0; j < x.KT; ++j) {
      mx_pp_read<FMT>(F, smem, j, wm, wn, h, l32);       // slot 2j
      wait_vmcnt<2 * mx_pp_loads<FMT>()>();              // stage j + 1 in
      lds_barrier();
      pin_frag(F);
      mx_pp_issue<FMT>(x, j + 4, lane);                  // slot 2j + 1
      mx_pp_mfmas<FMT>(acc, F);
      pin_acc(acc);
      lds_barrier();
    }
  }
  wait_vmcnt<0>();                                       // the clamped tail loads land in LDS the epilogue reuses
  lds_barrier();
  const float alpha = FMT == kFP8 ? fp8_s_dec(*a_amax) * fp8_s_dec(*b_amax) : 1.0f;
  store_tile_bf16(acc, smem, alpha, c, ldc, M, N, m0, n0, wm, wn, lane, vec_store);
}

template <int FMT>
hipError_t launch_gemm_t(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                         const float* aa, const uint8_t* bc, const uint8_t* bs, const float* ba,
                         void* c, int64_t ldc, hipStream_t s) {
  using C = Cfg<FMT>;
  const int tiles_m = (int)((M + kBM - 1) / kBM), tiles_n = (int)((N + kBN - 1) / kBN);
  const auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  const int64_t code_ld = fp8_elems(FMT) ? K : K / 2;
  const int64_t scale_ld = FMT == kNVFP4 ? K / 16 : K / 32;
  const bool fast = (K % C::BK == 0) && al16(ac) && al16(bc) && (code_ld % 16 == 0) &&
                    ((scale_ld * 1) % C::SB == 0) &&
                    ((reinterpret_cast<uintptr_t>(as) | reinterpret_cast<uintptr_t>(bs)) % C::SB == 0);
  const bool vec_store = (ldc % 4 == 0) && ((reinterpret_cast<uintptr_t>(c) & 7) == 0);   // 8-byte stores
  const size_t lds = 2 * (size_t)C::STAGE_BYTES;
  if (set_lds_limit(reinterpret_cast<const void*>(&k_gemm<FMT, true>), (int)lds) != hipSuccess ||
      set_lds_limit(reinterpret_cast<const void*>(&k_gemm<FMT, false>), (int)lds) != hipSuccess)
    return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)(tiles_m * tiles_n)), block(kThreads);
  uint16_t* cp = static_cast<uint16_t*>(c);
  // staged kernel: whole 64-byte code segments per stage, 16-byte scale pieces
  // per scale period (K % 512 == 0 for both formats), 32-bit byte offsets
  // within each operand
  // (per-tensor FP8: 64-byte stages only, no scale periods and no scale arrays)
  const bool staged = K > 0 && (FMT == kFP8 ? K % 64 == 0 : K % 512 == 0) && al16(ac) && al16(bc) &&
                      (FMT == kFP8 || (al16(as) && al16(bs))) &&
                      M * code_ld < ((int64_t)1 << 32) && N * code_ld < ((int64_t)1 << 32);
  // the four-wave kernel (whole 16-byte scale periods, K % 512 == 0): the same
  // results bit for bit, 4-15% faster than the ping-pong kernel
  if (gemm_mx_rx_fits<FMT>(M, N, K, ac, as, bc, bs))
    return launch_gemm_mx_rx<FMT>(M, N, K, ac, as, aa, bc, bs, ba, c, ldc, s);
  if (staged) {
    if (set_lds_limit(reinterpret_cast<const void*>(&k_gemm_mx_pp<FMT>), kMxLds) != hipSuccess)
      return hipErrorInvalidConfiguration;
    // its epilogue writes 16-byte row pieces: ldc % 8 == 0 and a 16-byte aligned c
    const bool vec16 = (ldc % 8 == 0) && al16(c);
    hipLaunchKernelGGL((k_gemm_mx_pp<FMT>), grid, block, kMxLds, s, M, N, K, ac, as, aa, bc, bs, ba,
                       cp, ldc, tiles_m, tiles_n, vec16 ? 1 : 0);
    return hipGetLastError();
  }
  if (fast)
    hipLaunchKernelGGL((k_gemm<FMT, true>), grid, block, lds, s, M, N, K, ac, as, aa, bc, bs, ba,
                       cp, ldc, tiles_m, tiles_n, vec_store ? 1 : 0);
  else
    hipLaunchKernelGGL((k_gemm<FMT, false>), grid, block, lds, s, M, N, K, ac, as, aa, bc, bs, ba,
                       cp, ldc, tiles_m, tiles_n, vec_store ? 1 : 0);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(Fmt fmt, int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                       const uint8_t* a_scales, const float* a_amax, const uint8_t* b_codes,
                       const uint8_t* b_scales, const float* b_amax, void* c, int64_t ldc,
                       void* scratch, size_t scratch_bytes, hipStream_t s) {
  switch (fmt) {
    case kNVFP4:
      return launch_gemm_nvfp4(M, N, K, a_codes, a_scales, a_amax, b_codes, b_scales, b_amax, c,
                               ldc, scratch, scratch_bytes, s);
    case kMXFP4:
      return launch_gemm_t<kMXFP4>(M, N, K, a_codes, a_scales, a_amax, b_codes, b_scales, b_amax,
                                   c, ldc, s);
    case kFP8:
      return launch_gemm_t<kFP8>(M, N, K, a_codes, a_scales, a_amax, b_codes, b_scales, b_amax, c,
                                 ldc, s);
    default:
      return launch_gemm_t<kMXFP8>(M, N, K, a_codes, a_scales, a_amax, b_codes, b_scales, b_amax,
                                   c, ldc, s);
  }
}

}  // namespace bsq
