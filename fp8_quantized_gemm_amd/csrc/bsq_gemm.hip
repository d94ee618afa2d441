// MX block-scaled GEMM for gfx950: C[M, N] (BF16) = A[M, K] . B[N, K]^T with
// MXFP8 (E4M3) or MXFP4 (E2M1) codes and one E8M0 scale per 32 K-elements.
//
// HN page opcode84 (MXFP8 / MXFP4 GEMMs on the OCP Microscaling formats): the
// block scale is applied inside the matrix unit.  On CDNA4,
// v_mfma_scale_f32_32x32x64_f8f6f4 takes one E8M0 scale per lane per 32-element
// K block, which is exactly the MX block, so codes go from LDS straight into
// the MFMA (operand layouts in k_gemm_mx below).  The NVFP4 GEMM lives in
// bsq_gemm_nvfp4.hip.
//
// Tiling: 256 x 256 output tile per 512-thread workgroup (8 waves as 2 x 4,
// each 128 (M) x 64 (N) = 4 x 2 MFMA tiles of 32 x 32); each wave computes
// D = B_tile . A_tile^T so that every lane holds consecutive output columns.
//  * k_gemm_mx (K % 512 == 0, aligned operands): 64 code bytes per row per
//    stage (K 64 for MXFP8, 128 for MXFP4) staged in LDS by global -> LDS
//    direct loads four stages ahead (four stage buffers), scales 16 bytes per
//    row per period of 8 / 4 stages, one barrier per stage; each wave reads the
//    next stage's fragments into a second register set while the MFMAs of the
//    current stage run.
//  * k_gemm (any K): the general path, register-staged, one stage ahead.
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
  static constexpr int RB = FMT == kMXFP8 ? BK : BK / 2;               // code bytes per row per stage
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
  // scales: thread t < 256 loads row t's SB bytes (SB is 4 or 8)
  st.scale[0] = st.scale[1] = 0;
  if (t < kBM) {
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

  const int64_t code_ld = FMT == kMXFP8 ? K : K / 2;
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
      constexpr int FMTC = FMT == kMXFP8 ? 0 : 4;     // cbsz / blgp operand type
      uint32_t sca[4], scb[2];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int row = wm * 128 + mi * 32 + l32;
        sca[mi] = FMT == kMXFP8 ? (*reinterpret_cast<const uint32_t*>(LSa + row * 4) >> (8 * h))
                                : *reinterpret_cast<const uint32_t*>(LSa + row * 8 + 4 * h);
      }
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int row = wn * 64 + ni * 32 + l32;
        scb[ni] = FMT == kMXFP8 ? (*reinterpret_cast<const uint32_t*>(LSb + row * 4) >> (8 * h))
                                : *reinterpret_cast<const uint32_t*>(LSb + row * 8 + 4 * h);
      }
      auto frag = [&](const uint8_t* base, int row, int s) {
        const uint8_t* p = base + row * C::LDR;
        uint4 lo, hi = make_uint4(0, 0, 0, 0);
        if (FMT == kMXFP8) {
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
        const int sel = FMT == kMXFP8 ? 2 * s : s;    // scale byte of this lane's block
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
  const float alpha = 1.0f;
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
// and 256 B rows: four MXFP4 stages or eight MXFP8 stages).  Wave w stages rows
// 32 w .. 32 w + 31 of both operands' codes every stage (4 direct loads of 16
// rows x 64 bytes) and 64 rows of one operand's scales once per scale period
// (one direct load of 64 rows x 16 bytes).  The kernel is bound by the number
// of L2 requests, not bytes: a row's scales are fetched as one 16-byte piece
// per period instead of one dword per stage, which removes over a third of the
// requests.
constexpr int kMxRowB = 64;
constexpr int kMxCodeB = 256 * kMxRowB;
constexpr int kMxStageB = 2 * kMxCodeB;                  // 32 KiB of codes per stage
constexpr int kMxStages = 4;
constexpr int kMxScOff = kMxStages * kMxStageB;          // scale buffers after the code buffers
constexpr int kMxScB = 2 * 256 * 16;                     // one scale period, both operands
constexpr int kMxLds = kMxScOff + 2 * kMxScB > kEpiLds ? kMxScOff + 2 * kMxScB : kEpiLds;
constexpr int kMxDma = 4;                                // code loads per wave per stage
static_assert(kMxLds <= 160 * 1024, "MX staged LDS plan");

// Stages per scale period: 16 bytes of a row hold 4 MXFP4 stages (128 K
// each, 4 blocks) or 8 MXFP8 stages (64 K each, 2 blocks).
template <int FMT>
constexpr int mx_period() { return FMT == kMXFP8 ? 8 : 4; }

struct MxLoadMap {
  uint32_t code[4];                                      // byte offset of this lane's 16 bytes
  uint32_t scale;                                        // byte offset of this lane's scale row
};

template <int FMT>
__device__ __forceinline__ void mx_stage(const uint8_t* ac, const uint8_t* bc, const MxLoadMap& lm,
                                         int64_t kt, uint32_t st, int w) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint8_t* base = (i < 2 ? ac : bc) + kt * kMxRowB;
    dma_to_lds<16>(base, lm.code[i], st + (i >> 1) * kMxCodeB + (w * 32 + (i & 1) * 16) * kMxRowB);
  }
}

// Scale period q (16 bytes per row) into scale buffer `sb`.
__device__ __forceinline__ void mx_stage_scales(const uint8_t* as, const uint8_t* bs,
                                                const MxLoadMap& lm, int64_t q, uint32_t sb, int w) {
  dma_to_lds<16>((w < 4 ? as : bs) + q * 16, lm.scale, sb + (w >> 2) * (256 * 16) + (w & 3) * (64 * 16));
}

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
    F.fa[j][mi] = chunk(La, row, FMT == kMXFP8 ? (j == 0 ? h : 2 + h) : 2 * h + j);
  } else if (Q < 12) {
    const int j = (Q - 8) >> 1, ni = (Q - 8) & 1, row = wn * 64 + ni * 32 + l32;
    F.fb[j][ni] = chunk(Lb, row, FMT == kMXFP8 ? (j == 0 ? h : 2 + h) : 2 * h + j);
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
  constexpr int FMTC = FMT == kMXFP8 ? 0 : 4;            // cbsz / blgp operand type
  constexpr int s = FMT == kMXFP8 ? 0 : I >> 3;
  constexpr int mi = (I & 7) >> 1, ni = I & 1;
  const u32x4 z = {0u, 0u, 0u, 0u};
  const u32x4 al = F.fa[s][mi], bl = F.fb[s][ni];
  const u32x4 ah = FMT == kMXFP8 ? F.fa[1][mi] : z;
  const u32x4 bh = FMT == kMXFP8 ? F.fb[1][ni] : z;
  const intx8 a = __builtin_bit_cast(intx8, __builtin_shufflevector(al, ah, 0, 1, 2, 3, 4, 5, 6, 7));
  const intx8 b = __builtin_bit_cast(intx8, __builtin_shufflevector(bl, bh, 0, 1, 2, 3, 4, 5, 6, 7));
  acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, acc[mi][ni], FMTC, FMTC, s,
                                                                (int)F.sb[ni], s, (int)F.sa[mi]);
}

// Reads issued after MFMA I: [lo(I), lo(I + 1)), spread over the first 8 MFMAs
// (MXFP8) or the first 12 (MXFP4) so that they complete before the barrier.
template <int FMT>
__host__ __device__ constexpr int mx_rd_lo(int i) {
  return FMT == kMXFP8 ? (i * 18 + 7) / 8 > 18 ? 18 : (i * 18 + 7) / 8
                       : (i * 18 + 11) / 12 > 18 ? 18 : (i * 18 + 11) / 12;
}

template <int FMT, int I>
__device__ __forceinline__ void mx_step(floatx16 (&acc)[4][2], const MxFrag& C, MxFrag& N,
                                        const uint8_t* nbuf, const uint8_t* nsbuf, int nsb0, int wm,
                                        int wn, int h, int l32) {
  mx_mfma<FMT, I>(acc, C);
  constexpr int lo = mx_rd_lo<FMT>(I), hi = mx_rd_lo<FMT>(I + 1);
  if (lo + 0 < hi) mx_read<FMT, lo + 0 < 18 ? lo + 0 : 17>(N, nbuf, nsbuf, nsb0, wm, wn, h, l32);
  if (lo + 1 < hi) mx_read<FMT, lo + 1 < 18 ? lo + 1 : 17>(N, nbuf, nsbuf, nsb0, wm, wn, h, l32);
  if (lo + 2 < hi) mx_read<FMT, lo + 2 < 18 ? lo + 2 : 17>(N, nbuf, nsbuf, nsb0, wm, wn, h, l32);
  __builtin_amdgcn_sched_barrier(0);
}

// Everything a stage needs besides the fragments (wave-uniform).
struct MxCtx {
  const uint8_t* ac;
  const uint8_t* as;
  const uint8_t* bc;
  const uint8_t* bs;
  uint8_t* smem;
  uint32_t smem_lds;
  int64_t KT, NP;            // stages, scale periods
  int w;
};

// Scale slot of stage kt (one direct load every stage, so that this wave's
// load count per stage is fixed): at a period start (kt % period == 0) the
// scales of period q + 1 into its buffer; otherwise lane 0 reloads its own 16
// bytes of the current period into the place they already occupy (one L2
// request, same bytes).
__device__ __forceinline__ void mx_scale_slot(const MxCtx& x, const MxLoadMap& lm, int64_t q,
                                              int64_t ph, int lane) {
  if (ph == 0) {
    const int64_t nq = q + 1 < x.NP ? q + 1 : x.NP - 1;
    mx_stage_scales(x.as, x.bs, lm, nq, x.smem_lds + kMxScOff + (uint32_t)((q + 1) & 1) * kMxScB, x.w);
  } else if (lane == 0) {
    mx_stage_scales(x.as, x.bs, lm, q, x.smem_lds + kMxScOff + (uint32_t)(q & 1) * kMxScB, x.w);
  }
}

// Stage kt (P = kt & 1): wait until stage kt + 1 has landed (this wave's loads,
// then everyone's), the scale slot, stage kt + 4 into the buffer of stage kt
// (whose fragments are in registers), then the MFMAs of kt on C with the
// fragment reads of kt + 1 into N interleaved.  This wave's loads issued after
// stage kt + 1's are the scale slots and stages of kt + 2 and kt + 3, so at
// most 2 (1 + kMxDma) may remain.  A period's scales are issued before the
// code stage four ahead, which is waited for before that period's first read.
template <int FMT, int P>
__device__ __forceinline__ void mx_iter(floatx16 (&acc)[4][2], MxFrag& C, MxFrag& N,
                                        const MxCtx& x, const MxLoadMap& lm, int64_t kt, int wm,
                                        int wn, int h, int l32, int lane) {
  constexpr int PER = mx_period<FMT>();
  wait_vmcnt<2 * (1 + kMxDma)>();
  lds_barrier();                               // everyone's; all fragments of kt are in registers
  const int64_t q = kt / PER, ph = kt - q * PER;
  mx_scale_slot(x, lm, q, ph, lane);
  const int64_t nk = kt + 4 < x.KT ? kt + 4 : x.KT - 1;
  mx_stage<FMT>(x.ac, x.bc, lm, nk, x.smem_lds + (uint32_t)(kt & 3) * kMxStageB, x.w);
  const uint8_t* nbuf = x.smem + ((kt + 1) & 3) * kMxStageB;
  const int64_t nq = (kt + 1) / PER;
  const uint8_t* nsbuf = x.smem + kMxScOff + (nq & 1) * kMxScB;
  const int nsb0 = (int)(kt + 1 - nq * PER) * (FMT == kMXFP8 ? 2 : 4);
  mx_step<FMT, 0>(acc, C, N, nbuf, nsbuf, nsb0, wm, wn, h, l32);
  mx_step<FMT, 1>(acc, C, N, nbuf, nsbuf, nsb0, wm, wn, h, l32);
  mx_step<FMT, 2>(acc, C, N, nbuf, nsbuf, nsb0, wm, wn, h, l32);
  mx_step<FMT, 3>(acc, C, N, nbuf, nsbuf, nsb0, wm, wn, h, l32);
  mx_step<FMT, 4>(acc, C, N, nbuf, nsbuf, nsb0, wm, wn, h, l32);
  mx_step<FMT, 5>(acc, C, N, nbuf, nsbuf, nsb0, wm, wn, h, l32);
  mx_step<FMT, 6>(acc, C, N, nbuf, nsbuf, nsb0, wm, wn, h, l32);
  mx_step<FMT, 7>(acc, C, N, nbuf, nsbuf, nsb0, wm, wn, h, l32);
  if (FMT == kMXFP4) {
    mx_step<FMT, 8>(acc, C, N, nbuf, nsbuf, nsb0, wm, wn, h, l32);
    mx_step<FMT, 9>(acc, C, N, nbuf, nsbuf, nsb0, wm, wn, h, l32);
    mx_step<FMT, 10>(acc, C, N, nbuf, nsbuf, nsb0, wm, wn, h, l32);
    mx_step<FMT, 11>(acc, C, N, nbuf, nsbuf, nsb0, wm, wn, h, l32);
    mx_step<FMT, 12>(acc, C, N, nbuf, nsbuf, nsb0, wm, wn, h, l32);
    mx_step<FMT, 13>(acc, C, N, nbuf, nsbuf, nsb0, wm, wn, h, l32);
    mx_step<FMT, 14>(acc, C, N, nbuf, nsbuf, nsb0, wm, wn, h, l32);
    mx_step<FMT, 15>(acc, C, N, nbuf, nsbuf, nsb0, wm, wn, h, l32);
  }
}

template <int FMT, int Q>
__device__ __forceinline__ void mx_read_all(MxFrag& F, const uint8_t* buf, const uint8_t* sbuf,
                                            int wm, int wn, int h, int l32) {
  mx_read<FMT, Q>(F, buf, sbuf, 0, wm, wn, h, l32);
  if constexpr (Q + 1 < 18) mx_read_all<FMT, Q + 1>(F, buf, sbuf, wm, wn, h, l32);
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void k_gemm_mx(
    int64_t M, int64_t N, int64_t K, const uint8_t* a_codes, const uint8_t* a_scales,
    const uint8_t* b_codes, const uint8_t* b_scales, uint16_t* __restrict__ c, int64_t ldc,
    int tiles_m, int tiles_n, int vec_store) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int tm, tn;
  tile_of_block(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int h = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(wave);
  const int64_t code_ld = FMT == kMXFP8 ? K : K / 2, scale_ld = K / 32;
  constexpr int P = mx_period<FMT>();
  MxCtx x;
  x.ac = a_codes;
  x.as = a_scales;
  x.bc = b_codes;
  x.bs = b_scales;
  x.smem = smem;
  x.smem_lds = (uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t*)smem;
  x.KT = code_ld / kMxRowB;                              // stages (a multiple of the period)
  x.NP = x.KT / P;
  x.w = w;
  MxLoadMap lm;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = w * 32 + (i & 1) * 16 + (lane >> 2);  // row within the tile
    const int64_t base = i < 2 ? m0 : n0, rows = i < 2 ? M : N;
    const int64_t gr = base + rr < rows ? base + rr : rows - 1;
    lm.code[i] = (uint32_t)(gr * code_ld + (((lane & 3) ^ ((rr >> 2) & 3)) << 4));
  }
  {
    const int rr = (w & 3) * 64 + lane;
    const int64_t base = w < 4 ? m0 : n0, rows = w < 4 ? M : N;
    const int64_t gr = base + rr < rows ? base + rr : rows - 1;
    lm.scale = (uint32_t)(gr * scale_ld);
  }
  floatx16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // prologue: the scales of period 0 and the code stages 0..3, each stage
  // preceded by a scale slot's worth of loads so the per-stage count is fixed
  mx_stage_scales(a_scales, b_scales, lm, 0, x.smem_lds + kMxScOff, w);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (k > 0 && lane == 0) mx_stage_scales(a_scales, b_scales, lm, 0, x.smem_lds + kMxScOff, w);
    mx_stage<FMT>(a_codes, b_codes, lm, k < x.KT ? k : x.KT - 1, x.smem_lds + k * kMxStageB, w);
  }
  wait_vmcnt<3 * (1 + kMxDma)>();              // period-0 scales and stage 0 in
  lds_barrier();
  MxFrag F0, F1;
  mx_read_all<FMT, 0>(F0, smem, smem + kMxScOff, wm, wn, h, l32);
  for (int64_t kt = 0; kt < x.KT; kt += 2) {   // KT is even (a multiple of the period)
    mx_iter<FMT, 0>(acc, F0, F1, x, lm, kt, wm, wn, h, l32, lane);
    mx_iter<FMT, 1>(acc, F1, F0, x, lm, kt + 1, wm, wn, h, l32, lane);
  }
  wait_vmcnt<0>();                             // the clamped tail loads land in LDS the epilogue reuses
  lds_barrier();
  store_tile_bf16(acc, smem, 1.0f, c, ldc, M, N, m0, n0, wm, wn, lane, vec_store);
}

template <int FMT>
hipError_t launch_gemm_t(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                         const float* aa, const uint8_t* bc, const uint8_t* bs, const float* ba,
                         void* c, int64_t ldc, hipStream_t s) {
  using C = Cfg<FMT>;
  const int tiles_m = (int)((M + kBM - 1) / kBM), tiles_n = (int)((N + kBN - 1) / kBN);
  const auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  const int64_t code_ld = FMT == kMXFP8 ? K : K / 2;
  const int64_t scale_ld = FMT == kNVFP4 ? K / 16 : K / 32;
  const bool fast = (K % C::BK == 0) && al16(ac) && al16(bc) && (code_ld % 16 == 0) &&
                    ((scale_ld * 1) % C::SB == 0) &&
                    ((reinterpret_cast<uintptr_t>(as) | reinterpret_cast<uintptr_t>(bs)) % C::SB == 0);
  const bool vec_store = (ldc % 4 == 0) && ((reinterpret_cast<uintptr_t>(c) & 7) == 0);
  const size_t lds = 2 * (size_t)C::STAGE_BYTES;
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm<FMT, true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess ||
        hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm<FMT, false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return hipErrorInvalidConfiguration;
    attr_set = true;
  }
  const dim3 grid((unsigned)(tiles_m * tiles_n)), block(kThreads);
  uint16_t* cp = static_cast<uint16_t*>(c);
  // staged kernel: whole 64-byte code segments per stage, 16-byte scale pieces
  // per scale period (K % 512 == 0 for both formats), 32-bit byte offsets
  // within each operand
  const bool staged = K > 0 && K % 512 == 0 && al16(ac) && al16(bc) && al16(as) && al16(bs) &&
                      M * code_ld < ((int64_t)1 << 32) && N * code_ld < ((int64_t)1 << 32);
  static bool mx_attr_set = false;
  if (staged) {
    if (!mx_attr_set) {
      if (hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_mx<FMT>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, kMxLds) != hipSuccess)
        return hipErrorInvalidConfiguration;
      mx_attr_set = true;
    }
    hipLaunchKernelGGL((k_gemm_mx<FMT>), grid, block, kMxLds, s, M, N, K, ac, as, bc, bs, cp, ldc,
                       tiles_m, tiles_n, vec_store ? 1 : 0);
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
                       hipStream_t s) {
  switch (fmt) {
    case kNVFP4:
      return launch_gemm_nvfp4(M, N, K, a_codes, a_scales, a_amax, b_codes, b_scales, b_amax, c,
                               ldc, s);
    case kMXFP4:
      return launch_gemm_t<kMXFP4>(M, N, K, a_codes, a_scales, a_amax, b_codes, b_scales, b_amax,
                                   c, ldc, s);
    default:
      return launch_gemm_t<kMXFP8>(M, N, K, a_codes, a_scales, a_amax, b_codes, b_scales, b_amax,
                                   c, ldc, s);
  }
}

}  // namespace bsq
