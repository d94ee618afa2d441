// MX block-scaled GEMM for gfx950, four-wave schedule:
// C[M, N] (BF16) = A[M, K] . B[N, K]^T with MXFP8 (E4M3) or MXFP4 (E2M1)
// codes and one E8M0 scale per 32 K-elements, or per-tensor FP8 (unit block
// scales, alpha from the two amaxes).
//
// HN page opcode84 (MXFP8 / MXFP4 GEMMs on the OCP Microscaling formats): the
// block scale is applied inside the matrix unit.  CDNA4's
// v_mfma_scale_f32_32x32x64_f8f6f4 takes one E8M0 scale per lane per 32-element
// K block, so codes go from LDS straight into the MFMA.
//
// Work split: one 256-thread workgroup (four waves, one per SIMD) per 256 x 256
// output tile; wave w owns the 128 x 128 quarter (w >> 1, w & 1) as 4 x 4
// accumulator tiles of 32 x 32 (256 FP32 accumulator registers, pinned by
// MFMAs written as inline assembly with tied operands).  Each MFMA computes
// D = B . A^T (B rows in the first operand), so a lane holds four consecutive
// output columns per register quad.  Against eight waves of 128 x 64, every
// A and B fragment is read from LDS by two waves instead of three on average,
// a third less LDS traffic per MFMA.
//
// Units: 128 code bytes per row (K 128 for FP8 codes, 256 for FP4), i.e. two
// (FP8) or four (FP4) K steps of 64, 16 MFMAs per wave each.  Raw units reach
// LDS by global -> LDS direct loads, two unit buffers; each wave loads A rows
// and B rows 64 w .. 64 w + 63 as eight 8-row code loads per operand (the
// eight lanes of a row read one whole 128-byte line: 64-byte pieces cost as
// many L2 requests as whole lines) and, per scale period (16 scale bytes per
// row: 4 FP8 units, 2 FP4 units), one 64-row scale load per operand.
// Fragments of K step k + 1 are read during step k into the other half of a
// double-buffered register set.  The last step of unit U first waits for
// unit U + 1 (the only loads in flight), then a workgroup barrier makes it
// visible and retires unit U's buffer (its last reads were issued in the
// step before), and the loads of unit U + 2 go into that buffer during the
// step.
//
// LDS code rows are 128 bytes; the 16-byte chunk c of row r sits at slot
// c ^ swz(r), swz(r) = (r >> 1) & 7: a 16-byte read is served sixteen lanes
// (sixteen consecutive rows, one chunk) per cycle by 64 four-byte banks, and
// rows of one parity start on the same bank.  FP8: lane half h takes chunks
// 4 j + h and 4 j + 2 + h for K step j; FP4: chunk 4 (j >> 1) + 2 h + (j & 1).
// A and B use the same map, so each MFMA contracts matching K indices.
//
// Loop: unrolled by one scale period (eight K steps in both formats) so that
// every load count and wait count is a compile-time constant and a K step is
// one basic block (the compiler does not see the MFMAs' operand timing and
// must not move work across a branch next to them).
#include "bsq_gemm_common.hpp"
#include "bsq_internal.hpp"

namespace bsq {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMrThreads = 256;
constexpr int kMrRowB = 128;                      // code bytes per row and unit
constexpr int kMrCodeB = 256 * kMrRowB;           // one operand's codes of a unit: 32 KiB
constexpr int kMrUnitB = 2 * kMrCodeB;            // A then B: 64 KiB
constexpr int kMrScOpB = 256 * 16;                // one operand's scale period
constexpr int kMrScOff = 2 * kMrUnitB;            // two unit buffers, then two periods
constexpr int kMrLds = kMrScOff + 2 * 2 * kMrScOpB;   // 147456
constexpr int kMrEpiRowB = 272;
static_assert(4 * 128 * kMrEpiRowB <= kMrLds, "epilogue staging must fit");
static_assert(kMrLds <= 160 * 1024, "LDS plan");

// K steps of 64 per unit, units per scale period (16 scale bytes per row)
template <int FMT>
constexpr int mr_ksteps() { return fp8_elems(FMT) ? 2 : 4; }
template <int FMT>
constexpr int mr_period() { return fp8_elems(FMT) ? 4 : 2; }

// 16 lanes (16 consecutive rows, one chunk) per cycle across 64 banks: rows of
// one parity must take distinct slots
__host__ __device__ constexpr int mr_swz(int r) { return (r >> 1) & 7; }

struct MrSrc {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const uint8_t* b_codes;
  const uint8_t* b_scales;
  uint32_t m0, n0, last_m, last_n;
  uint32_t code_ld, scale_ld;
};

// Load Q of a unit: Q 0-7 the A code rows 64 w + 8 Q .. + 7 of unit u (lane l
// fills row l >> 3, slot l & 7 with the chunk that belongs there: the eight
// lanes of a row read one whole 128-byte line), Q 8-15 the B rows; Q 16-17
// the A / B scales of period p, rows 64 w + l, into the period buffer `sc`.
template <int Q>
__device__ __forceinline__ void mr_load(const MrSrc& s, uint32_t u, uint32_t p, uint32_t raw,
                                        uint32_t sc, int w, int lane) {
  if constexpr (Q < 16) {
    constexpr int op = Q / 8, i = Q % 8;
    const uint32_t base = op ? s.n0 : s.m0, last = op ? s.last_n : s.last_m;
    const int rr = i * 8 + (lane >> 3);
    const int c = (lane & 7) ^ mr_swz(rr);
    const uint32_t gr = min(base + (uint32_t)(w * 64 + rr), last);
    dma_to_lds<16>((op ? s.b_codes : s.a_codes) + u * kMrRowB, gr * s.code_ld + (uint32_t)(c * 16),
                   raw + (uint32_t)(op * kMrCodeB + (w * 64 + i * 8) * kMrRowB));
  } else {
    constexpr int op = Q - 16;
    const uint32_t base = op ? s.n0 : s.m0, last = op ? s.last_n : s.last_m;
    const uint32_t gr = min(base + (uint32_t)(w * 64 + lane), last);
    dma_to_lds<16>((op ? s.b_scales : s.a_scales) + p * 16u, gr * s.scale_ld,
                   sc + (uint32_t)(op * kMrScOpB + w * 64 * 16));
  }
}

// Fragments of one K step: four A and four B tiles of 32 rows, and the lane's
// block scale byte per tile.  FP8: chunks 4 j + h and 4 j + 2 + h of the row
// (32 bytes, 8 registers); FP4: chunk 4 (j >> 1) + 2 h + (j & 1) (16 bytes, 4
// registers: steps 0-3 pair the unit's 32-element blocks as (0, 2), (1, 3),
// (4, 6), (5, 7)).
template <int FMT>
struct MrFrag {
  static constexpr bool kF8 = fp8_elems(FMT);
  intx8 a8[kF8 ? 4 : 1], b8[kF8 ? 4 : 1];
  u32x4 a4[kF8 ? 1 : 4], b4[kF8 ? 1 : 4];
  uint32_t sa[4], sb[4];
};

struct MrLane {
  int wm, wn, h, l32, w, lane;
};

// Read item Q (0-15) of K step j of a unit in buffer `buf` (scale bytes of
// the unit start at `sbyte` of a row's 16 in `sbuf`): Q 0-3 A tile Q, 4-7 B
// tile Q - 4, 8-11 A scales, 12-15 B scales.
template <int FMT, int Q>
__device__ __forceinline__ void mr_read(MrFrag<FMT>& F, const uint8_t* buf, const uint8_t* sbuf,
                                        int sbyte, int j, const MrLane& L) {
  const auto chunk = [](const uint8_t* base, int row, int c) {
    return *reinterpret_cast<const u32x4*>(base + row * kMrRowB + ((c ^ mr_swz(row)) << 4));
  };
  if constexpr (Q < 8) {
    constexpr int op = Q >> 2, t = Q & 3;
    const int row = (op ? L.wn : L.wm) * 128 + t * 32 + L.l32;
    const uint8_t* base = buf + op * kMrCodeB;
    if constexpr (fp8_elems(FMT)) {
      const u32x4 lo = chunk(base, row, 4 * j + L.h), hi = chunk(base, row, 4 * j + 2 + L.h);
      const intx8 v = __builtin_bit_cast(intx8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      if constexpr (op) F.b8[t] = v;
      else F.a8[t] = v;
    } else if constexpr (op) {
      F.b4[t] = chunk(base, row, 4 * (j >> 1) + 2 * L.h + (j & 1));
    } else {
      F.a4[t] = chunk(base, row, 4 * (j >> 1) + 2 * L.h + (j & 1));
    }
  } else if constexpr (FMT == kFP8) {
    if constexpr (Q < 12) F.sa[Q - 8] = 0x7Fu;
    else F.sb[Q - 12] = 0x7Fu;
  } else {
    constexpr int op = Q >= 12, t = Q & 3;
    const int row = (op ? L.wn : L.wm) * 128 + t * 32 + L.l32;
    const uint8_t* sp = sbuf + op * kMrScOpB + row * 16 + sbyte;
    const uint32_t v = (uint32_t)sp[fp8_elems(FMT) ? 2 * j + L.h : 4 * (j >> 1) + 2 * L.h + (j & 1)];
    if constexpr (op) F.sb[t] = v;
    else F.sa[t] = v;
  }
}

__device__ __forceinline__ void mr_mfma_f8(floatx16& acc, const intx8& b, const intx8& a, uint32_t sb,
                                           uint32_t sa) {
  asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
               : "+a"(acc) : "v"(b), "v"(a), "v"(sb), "v"(sa));
}
__device__ __forceinline__ void mr_mfma_f4(floatx16& acc, const u32x4& b, const u32x4& a, uint32_t sb,
                                           uint32_t sa) {
  asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0] cbsz:4 blgp:4"
               : "+a"(acc) : "v"(b), "v"(a), "v"(sb), "v"(sa));
}

template <int FMT, int MI, int NI>
__device__ __forceinline__ void mr_mfma(floatx16& acc, const MrFrag<FMT>& F) {
  if constexpr (fp8_elems(FMT)) mr_mfma_f8(acc, F.b8[NI], F.a8[MI], F.sb[NI], F.sa[MI]);
  else mr_mfma_f4(acc, F.b4[NI], F.a4[MI], F.sb[NI], F.sa[MI]);
}

// read item q after MFMA mr_rd_after(q) (from MFMA 1 on); load q of n after
// MFMA mr_ld_after(q, n)
__host__ __device__ constexpr int mr_rd_after(int q) { return 1 + (q * 13) / 15; }
__host__ __device__ constexpr int mr_ld_after(int q, int n) { return (q * 15) / n; }

template <int FMT, int K, int Q = 0>
__device__ __forceinline__ void mr_reads_at(MrFrag<FMT>& G, const uint8_t* nbuf, const uint8_t* nsbuf,
                                            int nsbyte, int nj, const MrLane& L) {
  if constexpr (Q < 16) {
    if constexpr (mr_rd_after(Q) == K) mr_read<FMT, Q>(G, nbuf, nsbuf, nsbyte, nj, L);
    mr_reads_at<FMT, K, Q + 1>(G, nbuf, nsbuf, nsbyte, nj, L);
  }
}
template <int K, int NLD, int Q = 0>
__device__ __forceinline__ void mr_loads_at(const MrSrc& s, uint32_t lu, uint32_t lp, uint32_t lraw,
                                            uint32_t lsc, const MrLane& L) {
  if constexpr (Q < NLD) {
    if constexpr (mr_ld_after(Q, NLD) == K) mr_load<Q>(s, lu, lp, lraw, lsc, L.w, L.lane);
    mr_loads_at<K, NLD, Q + 1>(s, lu, lp, lraw, lsc, L);
  }
}

// MFMA K (0-15) of a K step: A tile K >> 2, B tile K & 3; then the reads of
// the next K step and (NLD > 0) the loads placed after it.
template <int FMT, int NLD, int K>
__device__ __forceinline__ void mr_steps(floatx16 (&acc)[4][4], const MrFrag<FMT>& F, MrFrag<FMT>& G,
                                         const uint8_t* nbuf, const uint8_t* nsbuf, int nsbyte, int nj,
                                         const MrSrc& s, uint32_t lu, uint32_t lp, uint32_t lraw,
                                         uint32_t lsc, const MrLane& L) {
  if constexpr (K < 16) {
    constexpr int mi = K >> 2, ni = K & 3;
    mr_mfma<FMT, mi, ni>(acc[mi][ni], F);
    mr_reads_at<FMT, K>(G, nbuf, nsbuf, nsbyte, nj, L);
    mr_loads_at<K, NLD>(s, lu, lp, lraw, lsc, L);
    __builtin_amdgcn_sched_barrier(0);
    mr_steps<FMT, NLD, K + 1>(acc, F, G, nbuf, nsbuf, nsbyte, nj, s, lu, lp, lraw, lsc, L);
  }
}

// K step at position KP (0-7) of a scale period starting at unit U0: unit
// U0 + KP / S, step j = KP % S.  The last step of a unit first waits for the
// next unit (all of this wave's loads in flight belong to it), then a
// barrier (the next unit visible; every wave done with this unit's buffer,
// whose last reads were issued in the step before), then issues the loads of
// the unit two ahead into this unit's buffer (LD: unless past the end).
template <int FMT, int KP, bool LD>
__device__ __forceinline__ void mr_kstep(floatx16 (&acc)[4][4], const MrFrag<FMT>& F, MrFrag<FMT>& G,
                                         const uint8_t* smem, uint32_t smem_lds, const MrSrc& s, int U0,
                                         int NU, const MrLane& L) {
  constexpr int S = mr_ksteps<FMT>(), P = mr_period<FMT>();
  constexpr int I = KP / S, j = KP % S;
  constexpr bool last = j == S - 1;
  const int U = U0 + I;
  if constexpr (last) {
    wait_vmcnt<0>();
    lds_barrier();
    asm volatile("s_nop 4" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  }
  // the next K step: this unit's step j + 1, or step 0 of unit U + 1 (past the
  // last unit: its last unit again, whose buffer is not refilled)
  const int un = last ? (U + 1 < NU ? U + 1 : NU - 1) : U;
  constexpr int nj = last ? 0 : j + 1;
  const int unp = un / P;
  const uint8_t* nbuf = smem + (un & 1) * kMrUnitB;
  const uint8_t* nsbuf = smem + kMrScOff + (unp & 1) * (2 * kMrScOpB);
  const int nsbyte = (un - unp * P) * (fp8_elems(FMT) ? 4 : 8);
  // loads of unit U + 2 (with the scales of its period when it starts one)
  constexpr bool pstart = FMT != kFP8 && ((I + 2) % P) == 0;
  constexpr int NLD = (last && LD) ? (pstart ? 18 : 16) : 0;
  const uint32_t lu = (uint32_t)(U + 2), lp = lu / P;
  const uint32_t lraw = smem_lds + (uint32_t)((lu & 1) * kMrUnitB);
  const uint32_t lsc = smem_lds + kMrScOff + (uint32_t)((lp & 1) * (2 * kMrScOpB));
  mr_steps<FMT, NLD, 0>(acc, F, G, nbuf, nsbuf, nsbyte, nj, s, lu, lp, lraw, lsc, L);
}

template <int FMT, bool LAST, int KP = 0>
__device__ __forceinline__ void mr_period_body(floatx16 (&acc)[4][4], MrFrag<FMT>& F0, MrFrag<FMT>& F1,
                                               const uint8_t* smem, uint32_t smem_lds, const MrSrc& s,
                                               int U0, int NU, const MrLane& L) {
  constexpr int S = mr_ksteps<FMT>(), P = mr_period<FMT>();
  if constexpr (KP < S * P) {
    constexpr bool ld = !LAST || (KP / S) + 2 < P;
    if constexpr ((KP & 1) == 0) mr_kstep<FMT, KP, ld>(acc, F0, F1, smem, smem_lds, s, U0, NU, L);
    else mr_kstep<FMT, KP, ld>(acc, F1, F0, smem, smem_lds, s, U0, NU, L);
    mr_period_body<FMT, LAST, KP + 1>(acc, F0, F1, smem, smem_lds, s, U0, NU, L);
  }
}

template <int FMT, int Q = 0>
__device__ __forceinline__ void mr_issue(const MrSrc& s, uint32_t u, uint32_t smem_lds, const MrLane& L) {
  constexpr int P = mr_period<FMT>();
  if constexpr (Q < 18) {
    if constexpr (Q < 16) {
      mr_load<Q>(s, u, 0, smem_lds + (uint32_t)((u & 1) * kMrUnitB), 0, L.w, L.lane);
    } else if (FMT != kFP8 && u % P == 0) {
      mr_load<Q>(s, u, u / P, 0, smem_lds + kMrScOff + (uint32_t)(((u / P) & 1) * (2 * kMrScOpB)), L.w, L.lane);
    }
    mr_issue<FMT, Q + 1>(s, u, smem_lds, L);
  }
}

template <int FMT, int Q = 0>
__device__ __forceinline__ void mr_read_all(MrFrag<FMT>& F, const uint8_t* buf, const uint8_t* sbuf,
                                            const MrLane& L) {
  if constexpr (Q < 16) {
    mr_read<FMT, Q>(F, buf, sbuf, 0, 0, L);
    mr_read_all<FMT, Q + 1>(F, buf, sbuf, L);
  }
}

template <int FMT>
__global__ __launch_bounds__(kMrThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_gemm_mx_rx(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes, const uint8_t* a_scales,
                  const float* __restrict__ a_amax, const uint8_t* b_codes, const uint8_t* b_scales,
                  const float* __restrict__ b_amax, uint16_t* __restrict__ c, int64_t ldc, int tiles_m,
                  int tiles_n, int vec_store) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int P = mr_period<FMT>();
  int tm, tn;
  tile_of_block(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int t = threadIdx.x;
  MrLane L;
  L.lane = t & 63;
  L.w = __builtin_amdgcn_readfirstlane(t >> 6);
  L.wm = L.w >> 1;
  L.wn = L.w & 1;
  L.h = L.lane >> 5;
  L.l32 = L.lane & 31;
  const uint32_t smem_lds = (uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t*)smem;
  MrSrc s;
  s.a_codes = a_codes;
  s.a_scales = a_scales;
  s.b_codes = b_codes;
  s.b_scales = b_scales;
  s.m0 = (uint32_t)tm * 256u;
  s.n0 = (uint32_t)tn * 256u;
  s.last_m = (uint32_t)(M - 1);
  s.last_n = (uint32_t)(N - 1);
  s.code_ld = (uint32_t)(fp8_elems(FMT) ? K : K / 2);
  s.scale_ld = (uint32_t)(K / 32);
  const int NU = (int)(s.code_ld / kMrRowB);             // a multiple of P

  // accumulators zeroed here, fenced: an accumulator written by a VALU
  // operation needs wait states before an MFMA reads it, and the compiler
  // does not see into the MFMA assembly
  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
      asm volatile("" : "+a"(acc[i][j]));
    }
  __builtin_amdgcn_sched_barrier(0);

  // prologue: units 0 and 1 in flight; unit 0's first K step in registers
  mr_issue<FMT>(s, 0, smem_lds, L);
  mr_issue<FMT>(s, 1, smem_lds, L);
  wait_vmcnt<16>();                                      // unit 0 landed (unit 1: 16 code loads)
  lds_barrier();
  MrFrag<FMT> F0, F1;
  mr_read_all<FMT>(F0, smem, smem + kMrScOff, L);
  __builtin_amdgcn_sched_barrier(0);

  int U = 0;
  for (; U + P < NU; U += P) mr_period_body<FMT, false>(acc, F0, F1, smem, smem_lds, s, U, NU, L);
  mr_period_body<FMT, true>(acc, F0, F1, smem, smem_lds, s, U, NU, L);

  // every wave is done with the unit buffers (the epilogue reuses the LDS;
  // no load is in flight: the last two units issue none), and the last
  // MFMAs' results have reached the accumulator registers
  lds_barrier();
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  // the accumulators count as written here: no read of them moves above the
  // barrier and the wait states
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) asm volatile("" : "+a"(acc[i][j]));
  __builtin_amdgcn_sched_barrier(0);

  // epilogue: alpha * acc -> BF16 (RNE), staged per wave through LDS so that
  // global stores are 256-byte row segments.  acc[mi][ni] register r holds,
  // in lane l, row 32 mi + (l & 31) and column 32 ni + 8 (r >> 2) + 4 (l >> 5)
  // + (r & 3) of the wave's quarter.
  const float alpha = FMT == kFP8 ? fp8_s_dec(*a_amax) * fp8_s_dec(*b_amax) : 1.0f;
  uint8_t* E = smem + L.w * (128 * kMrEpiRowB);
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const floatx16 v = acc[mi][ni];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<uint2*>(E + (mi * 32 + L.l32) * kMrEpiRowB + (ni * 32 + 8 * q + 4 * L.h) * 2) =
            make_uint2(pack_bf16x2(v[4 * q] * alpha, v[4 * q + 1] * alpha),
                       pack_bf16x2(v[4 * q + 2] * alpha, v[4 * q + 3] * alpha));
    }
  __syncthreads();
  const int64_t gm0 = (int64_t)s.m0 + L.wm * 128, gn = (int64_t)s.n0 + L.wn * 128 + (L.lane & 15) * 8;
#pragma unroll 4
  for (int it = 0; it < 32; ++it) {
    const int row = it * 4 + (L.lane >> 4);
    const int64_t gm = gm0 + row;
    if (gm >= M) continue;
    const uint4 v = *reinterpret_cast<const uint4*>(E + row * kMrEpiRowB + (L.lane & 15) * 16);
    uint16_t* dst = c + gm * ldc + gn;
    if (vec_store && gn + 7 < N) {
      typedef uint32_t u32x4n __attribute__((ext_vector_type(4)));
      __builtin_nontemporal_store(u32x4n{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4n*>(dst));
    } else {
      const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (gn + e < N) dst[e] = (uint16_t)(wv[e >> 1] >> (16 * (e & 1)));
    }
  }
}

}  // namespace

// whole scale periods (16 scale bytes per row: K % 512 == 0), at least one
template <int FMT>
bool gemm_mx_rx_fits(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                     const uint8_t* bc, const uint8_t* bs) {
  const auto al = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; };
  const int64_t code_ld = fp8_elems(FMT) ? K : K / 2;
  return K >= 512 && K % 512 == 0 && al(ac, 16) && al(bc, 16) &&
         (FMT == kFP8 || (al(as, 16) && al(bs, 16))) && M * code_ld < ((int64_t)1 << 32) &&
         N * code_ld < ((int64_t)1 << 32) && M * (K / 32) < ((int64_t)1 << 32) &&
         N * (K / 32) < ((int64_t)1 << 32);
}

template <int FMT>
hipError_t launch_gemm_mx_rx(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                             const float* aa, const uint8_t* bc, const uint8_t* bs, const float* ba,
                             void* c, int64_t ldc, hipStream_t s) {
  const int tiles_m = (int)((M + 255) / 256), tiles_n = (int)((N + 255) / 256);
  const bool vec_store = (ldc % 8 == 0) && (reinterpret_cast<uintptr_t>(c) % 16 == 0);
  if (set_lds_limit(reinterpret_cast<const void*>(&k_gemm_mx_rx<FMT>), kMrLds) != hipSuccess)
    return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(k_gemm_mx_rx<FMT>, dim3((unsigned)(tiles_m * tiles_n)), dim3(kMrThreads), kMrLds, s,
                     M, N, K, ac, as, aa, bc, bs, ba, static_cast<uint16_t*>(c), ldc, tiles_m, tiles_n,
                     vec_store ? 1 : 0);
  return hipGetLastError();
}

#define BSQ_MX_RX(F)                                                                               \
  template bool gemm_mx_rx_fits<F>(int64_t, int64_t, int64_t, const uint8_t*, const uint8_t*,      \
                                   const uint8_t*, const uint8_t*);                                \
  template hipError_t launch_gemm_mx_rx<F>(int64_t, int64_t, int64_t, const uint8_t*,              \
                                           const uint8_t*, const float*, const uint8_t*,           \
                                           const uint8_t*, const float*, void*, int64_t, hipStream_t);
BSQ_MX_RX(kMXFP4)
BSQ_MX_RX(kMXFP8)
BSQ_MX_RX(kFP8)
#undef BSQ_MX_RX

}  // namespace bsq
