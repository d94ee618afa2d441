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
//  * k_gemm_mx (K % 128 == 0, aligned operands): 64 code bytes per row per
//    stage (K 64 for MXFP8, 128 for MXFP4) staged in LDS by global -> LDS
//    direct loads three stages ahead (four stage buffers), one barrier per
//    stage.
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
        uint32_t b[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) b[e] = f32_to_bf16_rne(acc[mi][ni][4 * q + e] * alpha);
        if (vec_store && n + 3 < N) {
          *reinterpret_cast<uint2*>(crow + n) = make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < N) crow[n + e] = (uint16_t)b[e];
        }
      }
    }
  }
}

// ---------------------------------------------------------------- staged kernel
//
// Stage layout in LDS (34 KiB, four buffers): A codes 256 rows x 64 bytes, B
// codes the same (16-byte chunk c of row r in slot c ^ ((r >> 2) & 3), which
// keeps the fragment reads of 16 consecutive rows on distinct banks), then one
// scale dword per row of A and of B (MXFP8: the dword holding this stage's two
// scales and the next stage's; MXFP4: this stage's four).  Wave w stages rows
// 32 w .. 32 w + 31 of both operands' codes (4 direct loads of 16 rows x 64
// bytes) and the scale dwords of 64 rows of one operand (1 direct load).
constexpr int kMxRowB = 64;
constexpr int kMxCodeB = 256 * kMxRowB;
constexpr int kMxStageB = 2 * kMxCodeB + 2 * 256 * 4;
constexpr int kMxStages = 4;
constexpr int kMxLds = kMxStages * kMxStageB > kEpiLds ? kMxStages * kMxStageB : kEpiLds;
constexpr int kMxDma = 5;                                // direct loads per wave per stage
static_assert(kMxLds <= 160 * 1024, "MX staged LDS plan");

struct MxLoadMap {
  uint32_t code[4];                                      // byte offset of this lane's 16 bytes
  uint32_t scale;                                        // byte offset of this lane's scale row
};

template <int FMT>
__device__ __forceinline__ void mx_stage(const uint8_t* ac, const uint8_t* as, const uint8_t* bc,
                                         const uint8_t* bs, const MxLoadMap& lm, int64_t kt,
                                         uint32_t st, int w) {
  const int64_t sdw = FMT == kMXFP8 ? (kt >> 1) : kt;     // scale dword index along the row
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint8_t* base = (i < 2 ? ac : bc) + kt * kMxRowB;
    dma_to_lds<16>(base, lm.code[i], st + (i >> 1) * kMxCodeB + (w * 32 + (i & 1) * 16) * kMxRowB);
  }
  dma_to_lds<4>((w < 4 ? as : bs) + sdw * 4, lm.scale, st + 2 * kMxCodeB + (w >> 2) * 1024 + (w & 3) * 256);
}

// One stage of MFMAs from LDS buffer `buf`; P = stage parity (MXFP8 scale byte).
template <int FMT, int P>
__device__ __forceinline__ void mx_compute(floatx16 (&acc)[4][2], const uint8_t* buf, int wm,
                                           int wn, int h, int l32) {
  constexpr int FMTC = FMT == kMXFP8 ? 0 : 4;            // cbsz / blgp operand type
  const uint8_t* La = buf;
  const uint8_t* Lb = buf + kMxCodeB;
  const uint8_t* Sa = buf + 2 * kMxCodeB;
  const uint8_t* Sb = Sa + 1024;
  // scale operands: MXFP8 lane half h carries the scale of the instruction's
  // block h (stage block h, byte 2P + h); MXFP4 lane half h supplies stage
  // blocks 2h + s (byte 2h + s), selected below by the K step s
  uint32_t sca[4], scb[2];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
    sca[mi] = *reinterpret_cast<const uint32_t*>(Sa + (wm * 128 + mi * 32 + l32) * 4) >> (FMT == kMXFP8 ? 8 * h : 16 * h);
#pragma unroll
  for (int ni = 0; ni < 2; ++ni)
    scb[ni] = *reinterpret_cast<const uint32_t*>(Sb + (wn * 64 + ni * 32 + l32) * 4) >> (FMT == kMXFP8 ? 8 * h : 16 * h);
  const auto chunk = [](const uint8_t* base, int row, int c) {
    return *reinterpret_cast<const uint4*>(base + row * kMxRowB + ((c ^ ((row >> 2) & 3)) << 4));
  };
  constexpr int STEPS = FMT == kMXFP8 ? 1 : 2;
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    intx8 fa[4], fb[2];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int row = wm * 128 + mi * 32 + l32;
      // MXFP8: bytes 0-15 = elements [16h, 16h + 16) of block 0 (chunk h),
      // bytes 16-31 = the same of block 1 (chunk 2 + h); MXFP4: block 2h + s
      const uint4 lo = chunk(La, row, FMT == kMXFP8 ? h : 2 * h + s);
      const uint4 hi = FMT == kMXFP8 ? chunk(La, row, 2 + h) : make_uint4(0, 0, 0, 0);
      fa[mi] = intx8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int row = wn * 64 + ni * 32 + l32;
      const uint4 lo = chunk(Lb, row, FMT == kMXFP8 ? h : 2 * h + s);
      const uint4 hi = FMT == kMXFP8 ? chunk(Lb, row, 2 + h) : make_uint4(0, 0, 0, 0);
      fb[ni] = intx8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    constexpr int SEL = FMT == kMXFP8 ? 2 * P : 0;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        acc[mi][ni] = mfma_mx<FMTC>(FMT == kMXFP8 ? SEL : s, fb[ni], fa[mi], acc[mi][ni], scb[ni], sca[mi]);
  }
}

// One stage: wait for it, barrier, stage kt + 3, compute kt.  P = kt & 1
// (only MXFP8 uses it, to pick the scale bytes of its half of the dword).
template <int FMT, int P>
__device__ __forceinline__ void mx_iter(floatx16 (&acc)[4][2], uint8_t* smem, uint32_t smem_lds,
                                        const uint8_t* ac, const uint8_t* as, const uint8_t* bc,
                                        const uint8_t* bs, const MxLoadMap& lm, int64_t kt,
                                        int64_t KT, int w, int wm, int wn, int h, int l32) {
  wait_vmcnt<2 * kMxDma>();                    // this wave's loads of stage kt are in
  lds_barrier();                               // everyone's are; stage kt - 1 is read
  const int64_t nk = kt + 3 < KT ? kt + 3 : KT - 1;
  mx_stage<FMT>(ac, as, bc, bs, lm, nk, smem_lds + (uint32_t)((kt + 3) & 3) * kMxStageB, w);
  mx_compute<FMT, P>(acc, smem + (kt & 3) * kMxStageB, wm, wn, h, l32);
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
  const int64_t KT = code_ld / kMxRowB;                  // stages
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

  const uint32_t smem_lds = (uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t*)smem;
#pragma unroll
  for (int k = 0; k < 3; ++k)
    mx_stage<FMT>(a_codes, a_scales, b_codes, b_scales, lm, k < KT ? k : KT - 1,
                  smem_lds + k * kMxStageB, w);
  if (FMT == kMXFP8) {                         // KT is even (K % 128 == 0)
    for (int64_t kt = 0; kt < KT; kt += 2) {
      mx_iter<FMT, 0>(acc, smem, smem_lds, a_codes, a_scales, b_codes, b_scales, lm, kt, KT, w, wm, wn, h, l32);
      mx_iter<FMT, 1>(acc, smem, smem_lds, a_codes, a_scales, b_codes, b_scales, lm, kt + 1, KT, w, wm, wn, h, l32);
    }
  } else {
    for (int64_t kt = 0; kt < KT; ++kt)
      mx_iter<FMT, 0>(acc, smem, smem_lds, a_codes, a_scales, b_codes, b_scales, lm, kt, KT, w, wm, wn, h, l32);
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
  // staged kernel: whole 64-byte code segments and aligned scale dwords per
  // stage, 32-bit byte offsets within each operand
  const bool staged = K > 0 && K % 128 == 0 && al16(ac) && al16(bc) &&
                      ((reinterpret_cast<uintptr_t>(as) | reinterpret_cast<uintptr_t>(bs)) % 4 == 0) &&
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
