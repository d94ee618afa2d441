// NVFP4 block-scaled GEMM for gfx950, register-expansion schedule:
// C[M, N] (BF16) = alpha * A[M, K] . B[N, K]^T, A and B packed E2M1 codes with
// one E4M3 scale per 16 K-elements and a per-tensor FP32 scale each.
//
// NVFP4 pretraining post, data-flow paragraph after Figure 1: FPROP, DGRAD and
// WGRAD consume NVFP4 operands and emit BF16; recipe ingredients 1-2 define
// the operand format.  E2M1 x E4M3 is exact in FP16, so every operand element
// is expanded exactly to FP16 (v * S * 2^-7) and fed to the FP16 MFMA.
//
// Work split: one 256-thread workgroup (four waves, one per SIMD) per 256 x 256
// output tile; wave w owns the 128 x 128 quarter (w >> 1, w & 1) and keeps it
// as 8 x 8 accumulator tiles of 16 x 16 (v_mfma_f32_16x16x32_f16, 256 FP32
// accumulator registers pinned by inline assembly).
//
// Why registers and not LDS for the FP16 values: expanding each operand once
// per workgroup into LDS and reading FP16 fragments back costs more LDS
// traffic per MFMA than the LDS can serve at the MFMA rate.  Here each wave
// reads the packed codes (4 bits per element) and block scales of its own 128
// A rows and 128 B rows from LDS and expands them in registers, interleaved
// with its MFMAs.  Every A row is expanded by the two waves that share it
// (likewise B): two VALU operations per MFMA, and a quarter of the LDS
// traffic of FP16 fragments.
//
// K layout inside a 128-element unit of K: lane group g = lane >> 4 owns the
// 32 elements [32 g, 32 g + 32) of its row (16 code bytes, two block scales),
// and MFMA step ks (0..3) of the unit feeds it elements 32 g + 8 ks .. + 7.
// A and B use the same map, so each step contracts a quarter of the unit and
// the four steps together all of it (the sum over K is order-free; the
// accumulation order differs from a natural-order K walk only in FP32
// rounding).
//
// Pipeline per unit U (four steps of 64 MFMAs):
//  * raw units reach LDS by global -> LDS direct loads in pairs (units 2 p,
//    2 p + 1): per row 128 code bytes as eight 16-byte chunks, so the eight
//    lanes of a row read one whole 128-byte line (64-byte pieces cost as many
//    L2 requests as whole lines and halved the rate the tiles draw from the
//    L2), and 16 scale bytes; two pair buffers; wave w loads A rows and B
//    rows 64 w .. 64 w + 63; an odd unit U issues pair (U + 3) / 2, its 18
//    loads spread over the unit's 256 MFMAs (one every 14), into the buffer
//    of units U - 1 and U, whose codes and scales were read during the unit
//    before each; one workgroup barrier per pair (at odd units) makes a
//    landed pair visible to all waves;
//  * each tile's 16 code bytes for the unit (its four steps) are read from
//    LDS in one piece during steps 2-3 of the unit before, once that unit's
//    last expansion from them is done; the scales of U + 1 are read in step
//    0 of U and converted in step 1;
//  * during step ks: exactly one expansion pair (two VALU operations) after
//    each MFMA, written with the MFMA as one assembly block: the eight A
//    tiles and B tiles 0-6 of step ks + 1 (B tile n in place, once step ks
//    has read it), and B tile 7 of step ks itself (see rx_slot).
// Fragments are written and read inside inline assembly, so the compiler's
// hazard recognizer does not see those dependencies: every fragment is
// complete at least two MFMAs before its first reader and is rewritten no
// earlier than two MFMAs after its last.
// LDS code rows are 128 bytes (a pair): the 16-byte chunk c of row r sits at
// slot c ^ swz(r), swz(r) = (r >> 1) & 7.  A 16-byte read is served sixteen
// lanes (sixteen consecutive rows, one chunk) per cycle by 64 four-byte banks;
// rows of one parity start on the same bank, so their eight slots must differ.
#include "bsq_gemm_common.hpp"
#include "bsq_internal.hpp"

#include <mutex>

namespace bsq {

namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kRxThreads = 256;
// Units of 128 K (64 code bytes and 8 scale bytes per row) are staged in
// pairs: a pair buffer holds two consecutive units, each row's 128 code bytes
// and 16 scale bytes contiguous, so that every direct load reads whole
// 128-byte lines (code) or whole 16-byte scale pieces.
constexpr int kRxRowB = 128;                            // code bytes per row and pair
constexpr int kRxCodeB = 256 * kRxRowB;                 // one operand's codes of a pair: 32 KiB
constexpr int kRxOpB = kRxCodeB + 256 * 16;             // plus its scales: 36 KiB
constexpr int kRxUnitB = 2 * kRxOpB;                    // A then B: one pair buffer, 72 KiB
constexpr int kRxNBuf = 2;                              // pair buffers
constexpr int kRxLds = kRxNBuf * kRxUnitB;              // 147456
constexpr int kRxEpiRowB = 272;                         // epilogue: 128 BF16 + 16 bytes pad per row
constexpr int kRxLoadsPerPair = 18;                     // direct loads per wave and pair
static_assert(2 * kRxLoadsPerPair <= 63, "the wait counts of two pairs fit the load counter");
static_assert(4 * 128 * kRxEpiRowB <= kRxLds, "epilogue staging must fit");
static_assert(kRxLds <= 160 * 1024, "LDS plan");

// a 16-byte read is served 16 lanes (16 consecutive rows, one chunk) per
// cycle across 64 banks: the 128-byte rows of one parity take distinct slots
__host__ __device__ constexpr int rx_swz(int r) { return (r >> 1) & 7; }

// Where the operands come from (all wave-uniform).
struct RxSrc {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const uint8_t* b_codes;
  const uint8_t* b_scales;
  uint32_t m0, n0, last_m, last_n;     // tile origin; last valid row of each operand
  uint32_t code_ld, scale_ld;          // bytes per operand row
};

// Direct loads of pair `p` (units 2 p, 2 p + 1: K elements 256 p .. 256 p + 255)
// of A rows and B rows 64 w .. 64 w + 63 of the tile into the pair buffer at
// LDS address `raw`, load Q (0..17) of 18: Q / 9 picks the operand; Q % 9 < 8
// is a code load of 8 rows x 128 bytes, one 16-byte chunk per lane (lane l
// fills row l >> 3, slot l & 7 of the 8 rows with the chunk that belongs
// there: the eight lanes of a row read one whole line); Q % 9 == 8 the
// scales, 64 rows x 16 bytes.  Rows past the operand re-read its last row
// (their results are never stored).  32-bit offsets: operands are below 4 GiB.
// One direct load of 16 bytes per lane into LDS at M0 + 16 * lane, with M0
// formed by a single scalar add of a compile-time offset to an LDS base.
template <int IMM>
__device__ __forceinline__ void rx_dma16(const uint8_t* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_add_u32 m0, %2, %3\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(base), "s"(lds), "n"(IMM) : "memory", "m0", "scc");
}

template <int Q>
__device__ __forceinline__ void rx_stage_one(const RxSrc& s, uint32_t p, uint32_t raw, int w, int lane) {
  constexpr int op = Q / 9, i = Q % 9;
  const uint32_t base = op ? s.n0 : s.m0, last = op ? s.last_n : s.last_m;
  if constexpr (i < 8) {
    const uint8_t* cq = (op ? s.b_codes : s.a_codes) + p * kRxRowB;
    const int rr = i * 8 + (lane >> 3);                  // row within the wave's 64
    const int c = (lane & 7) ^ rx_swz(rr);               // chunk held at slot lane & 7
    const uint32_t gr = min(base + (uint32_t)(w * 64 + rr), last);
    rx_dma16<op * kRxOpB + i * 8 * kRxRowB>(cq, gr * s.code_ld + (uint32_t)(c * 16),
                                           raw + (uint32_t)(w * 64 * kRxRowB));
  } else {
    const uint8_t* sq = (op ? s.b_scales : s.a_scales) + p * 16;
    const uint32_t gr = min(base + (uint32_t)(w * 64 + lane), last);
    rx_dma16<op * kRxOpB + kRxCodeB>(sq, gr * s.scale_ld, raw + (uint32_t)(w * 64 * 16));
  }
}

// All 18 loads of a pair at once (prologue).
template <int Q = 0>
__device__ __forceinline__ void rx_stage(const RxSrc& s, uint32_t p, uint32_t raw, int w, int lane) {
  if constexpr (Q < 18) {
    rx_stage_one<Q>(s, p, raw, w, lane);
    rx_stage<Q + 1>(s, p, raw, w, lane);
  }
}

// Where in an odd unit (slot 64 ks + k of its 256) the 18 loads of the pair
// two ahead are issued: load Q at slot 14 Q + 10, spread out so that no slot
// waits for a burst of loads to be accepted.
__host__ __device__ constexpr int rx_ld_at(int KS, int K) {
  const int x = KS * 64 + K - 10;
  return (x >= 0 && x % 14 == 0 && x / 14 < 18) ? x / 14 : -1;
}

struct RxLd {
  const RxSrc* s;
  uint32_t u, raw;     // pair to load and its buffer
  int w, lane;
};

// Per-lane LDS offsets in a pair buffer, fixed for the kernel: tile T (0-7 A
// tiles of the wave's rows, 8-15 B tiles of its columns) adds (T & 7) * 2048
// to the code offsets and (T & 7) * 256 to the scale offsets (16 rows per
// tile); the second unit of the pair adds 8 to the scale offsets.
struct RxLane {
  int ca[2], cb[2];    // chunk 4 P + g of row (lane & 15) of A / B tile 0 for the unit of parity P
  int sa, sb;          // the two scale bytes 2 g, 2 g + 1 of those rows (first unit)
};

// Registers of the pipeline (indices are compile-time after unrolling).  The
// code dword of tile T for step ks sits in cw[T][ks]: the tile's 16 code
// bytes of one unit, read from LDS in one piece (see rx_reads).
struct RxRegs {
  uint32_t cw[16][4];        // code dwords (8 E2M1 codes) per tile and step
  uint32_t sraw[16];         // scale bytes 2 g, 2 g + 1 of the next unit, as read
  halfx2 pr[2][16];          // {S(2g), S(2g + 1)} * 2^7 per tile, units of parity 0 / 1
  halfx8 a[2][8];            // A fragments of the current step and the next
  halfx8 b[8];               // B fragments (tiles 0-6 rewritten for the next step once read)
  uint32_t o[2][4];          // pairs of the fragment being expanded: A stream, B stream
};

// Pair SEL (0-3) of the expansion of tile T for step s (= KS of a unit of
// parity UP): byte SEL of the step's code dword times the block scale of the
// step (block 2 g for steps 0-1, 2 g + 1 for steps 2-3), see dequant8.
template <int UP, int KS, int T, int SEL>
__device__ __forceinline__ uint32_t rx_pk(const RxRegs& r) {
  const halfx2 p = r.pr[UP][T];
  const halfx2 s = (KS >> 1) ? halfx2{p.y, p.y} : halfx2{p.x, p.x};
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(r.cw[T][KS], 0x1p-14f, SEL) * s);
}

template <int UP, int KS, int T, int SEL, int STREAM>
__device__ __forceinline__ void rx_pair_to(RxRegs& r, halfx8& dst) {
  uint32_t (&o)[4] = r.o[STREAM];
  o[SEL] = rx_pk<UP, KS, T, SEL>(r);
  if constexpr (SEL == 3) dst = __builtin_bit_cast(halfx8, make_uint4(o[0], o[1], o[2], o[3]));
}

// MFMA and expansion pair as one assembly block: acc += s0 . s1 (the MFMA's
// first operand is the B fragment, its second the A fragment), then
// out = pair SEL of the code dword cw (byte SEL: two E2M1 codes, times 2^-14)
// times the block scale, half H of p broadcast to both halves (the same two
// operations as rx_pk).  Written together so that the compiler can neither
// split the pair around the MFMA nor move it to another MFMA: left to
// itself it placed one VALU operation between some MFMAs and three between
// others, and a third operation between two MFMAs delays the second.
// The pair is formed in its own output register (early clobber: written
// before the scale is read), so that consecutive blocks share no register
// that one writes and the next touches; the compiler, which cannot see into
// the blocks, would otherwise put a wait state between them.
#define BSQ_RX_MP(CVT_SEL, MUL_SEL)                                                            \
  asm volatile("v_mfma_f32_16x16x32_f16 %0, %2, %3, %0\n\t"                                    \
               "v_cvt_scalef32_pk_f16_fp4 %1, %4, %5" CVT_SEL "\n\t"                           \
               "v_pk_mul_f16 %1, %6, %1" MUL_SEL                                                \
               : "+a"(acc), "=&v"(out)                                                          \
               : "v"(s0), "v"(s1), "v"(cw), "s"(k), "v"(p))
template <int SEL, int H>
__device__ __forceinline__ void rx_mfma_pair(floatx4& acc, const halfx8& s0, const halfx8& s1, uint32_t cw,
                                             halfx2 p, uint32_t& out) {
  const float k = 0x1p-14f;
  if constexpr (H == 0) {
    if constexpr (SEL == 0) BSQ_RX_MP("", " op_sel_hi:[0,1]");
    else if constexpr (SEL == 1) BSQ_RX_MP(" op_sel:[1,0,0]", " op_sel_hi:[0,1]");
    else if constexpr (SEL == 2) BSQ_RX_MP(" op_sel:[0,1,0]", " op_sel_hi:[0,1]");
    else BSQ_RX_MP(" op_sel:[1,1,0]", " op_sel_hi:[0,1]");
  } else {
    if constexpr (SEL == 0) BSQ_RX_MP("", " op_sel:[1,0]");
    else if constexpr (SEL == 1) BSQ_RX_MP(" op_sel:[1,0,0]", " op_sel:[1,0]");
    else if constexpr (SEL == 2) BSQ_RX_MP(" op_sel:[0,1,0]", " op_sel:[1,0]");
    else BSQ_RX_MP(" op_sel:[1,1,0]", " op_sel:[1,0]");
  }
}
#undef BSQ_RX_MP

// rx_pair_to with the MFMA of the slot fused in front (see rx_mfma_pair).
template <int UP, int KS, int T, int SEL, int STREAM>
__device__ __forceinline__ void rx_mfma_pair_to(floatx4& acc, const halfx8& fb, const halfx8& fa, RxRegs& r,
                                                halfx8& dst) {
  uint32_t (&o)[4] = r.o[STREAM];
  rx_mfma_pair<SEL, (KS >> 1)>(acc, fb, fa, r.cw[T][KS], r.pr[UP][T], o[SEL]);
  if constexpr (SEL == 3) dst = __builtin_bit_cast(halfx8, make_uint4(o[0], o[1], o[2], o[3]));
}

// Schedule of one step: MFMA k (0..63) multiplies B tile k >> 3 by A tile
// k & 7, and exactly one expansion pair (two VALU operations) follows each
// MFMA.  One wave per SIMD issues every instruction itself: between two
// 16x16x32 FP16 MFMAs it has room for two more instructions at no cost, and
// each further one, VALU or not, delays the next MFMA (register-only loops
// of this MFMA ran at 99% of the MFMA-only rate with two VALU operations
// after each, 77% with three, and 91% with four and none alternating).
// During step s the wave expands every fragment step s + 1 needs except B
// tile 7: the eight A tiles into the other A buffer and B tiles 0-6 in place,
// each starting two MFMAs after step s has read it for the last time; B tile
// 7 of step s itself is expanded after MFMAs 1-4 (step s - 1 read it last at
// its MFMA 63):
//   slot 0: A0 pair 0; slots 1-4: B7 (this step) pairs 0-3; 5-7: A0 pairs 1-3;
//   even k >= 8: A tile k / 8, pair (k % 8) / 2;
//   odd k >= 9: B tile (k - 9) / 8 of the next step, pair ((k - 9) % 8) / 2.
// Every fragment is complete at least two MFMAs before its first reader.
// Returns T * 4 + SEL (T 0-7 A tiles, 8-15 B tiles), plus 64 for B7 of this step.
__host__ __device__ constexpr int rx_slot(int k) {
  if (k == 0) return 0;
  if (k <= 4) return 64 + 15 * 4 + (k - 1);
  if (k <= 7) return k - 4;
  if ((k & 1) == 0) return (k >> 3) * 4 + ((k & 7) >> 1);
  return (8 + ((k - 9) >> 3)) * 4 + (((k - 9) & 7) >> 1);
}

// LDS code reads of the next unit (after MFMA K of step KS): a tile's 16 code
// bytes for all four steps, read in one piece once the tile's last expansion
// from the current unit's bytes is done (its step-3 pairs, placed in step 2,
// B7 in step 3).  Step 2: A tiles 0-5 after MFMA 8 m + 8 and B tiles 0-4
// after 8 n + 17 (their pairs end at 8 m + 7 and 8 n + 15); the wait at the
// start of step 3 covers them.  Step 3: B7 after MFMA 5, then A6, B5, A7, B6
// (whose step-2 pairs end at 54-63) after 7, 9, 11, 13; the compiler waits for
// these before their first pairs at slots 48-57.  Returns the tile, or -1.
__host__ __device__ constexpr int rx_cread(int KS, int K) {
  if (KS == 2) {
    if (K >= 8 && K <= 48 && (K & 7) == 0) return (K >> 3) - 1;
    if (K >= 17 && K <= 49 && ((K - 17) & 7) == 0) return 8 + ((K - 17) >> 3);
  }
  if (KS == 3) {
    if (K == 5) return 15;
    if (K == 7) return 6;
    if (K == 9) return 13;
    if (K == 11) return 7;
    if (K == 13) return 14;
  }
  return -1;
}

// Reads after MFMA K of step KS: code reads (rx_cread) and, in step 0, the
// scale bytes of the next unit (tile K / 2 after odd K < 32), converted in
// step 1 after the same MFMAs.  NP is the next unit's parity in its pair.
template <int NP, int KS, int K>
__device__ __forceinline__ void rx_reads(RxRegs& r, const uint8_t* unxt, const RxLane& ln) {
  if constexpr (rx_cread(KS, K) >= 0) {
    constexpr int T = rx_cread(KS, K);
    const uint4 q = *reinterpret_cast<const uint4*>(unxt + (T < 8 ? ln.ca[NP] : ln.cb[NP]) + (T & 7) * 2048);
    r.cw[T][0] = q.x;
    r.cw[T][1] = q.y;
    r.cw[T][2] = q.z;
    r.cw[T][3] = q.w;
  }
  if constexpr (KS == 0 && (K & 1) == 1 && K < 32) {
    constexpr int T = K >> 1;
    r.sraw[T] = *reinterpret_cast<const uint16_t*>(unxt + (T < 8 ? ln.sa : ln.sb) + NP * 8 + (T & 7) * 256);
  }
}

// MFMA K (0..63) of step KS of a unit of parity UP, then the work placed after it.
template <int UP, bool LOADS, int KS, int K>
__device__ __forceinline__ void rx_step(floatx4 (&acc)[8][8], RxRegs& r, const uint8_t* unxt,
                                        const RxLane& ln, const RxLd& ld) {
  constexpr int n = K >> 3, mi = K & 7;
  constexpr int e = rx_slot(K);
  // the next step: step KS + 1 of this unit, or step 0 of the next (parity UP ^ 1)
  constexpr int NKS = (KS + 1) & 3, NUP = KS == 3 ? (UP ^ 1) : UP;
  floatx4& c = acc[mi][n];
  const halfx8& fa = r.a[KS & 1][mi];
  const halfx8& fb = r.b[n];
  if constexpr (e >= 64)
    rx_mfma_pair_to<UP, KS, 15, (e & 3), 1>(c, fb, fa, r, r.b[7]);
  else if constexpr ((e >> 2) < 8)
    rx_mfma_pair_to<NUP, NKS, (e >> 2), (e & 3), 0>(c, fb, fa, r, r.a[(KS + 1) & 1][e >> 2]);
  else
    rx_mfma_pair_to<NUP, NKS, (e >> 2), (e & 3), 1>(c, fb, fa, r, r.b[(e >> 2) - 8]);
  if constexpr (LOADS && rx_ld_at(KS, K) >= 0) rx_stage_one<rx_ld_at(KS, K)>(*ld.s, ld.u, ld.raw, ld.w, ld.lane);
  rx_reads<UP ^ 1, KS, K>(r, unxt, ln);
  // step 3: the reads issued after MFMAs 5-13 have completed before the
  // first pairs that use them (slots 48-57): one wait instead of four
  if constexpr (KS == 3 && K == 40) __builtin_amdgcn_s_waitcnt(0xC07F);
  // the next unit's scale pairs (read in step 0)
  if constexpr (KS == 1 && (K & 1) == 1 && K < 32) {
    r.pr[UP ^ 1][K >> 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.sraw[K >> 1], 128.0f, false);
    asm volatile("" : "+v"(r.pr[UP ^ 1][K >> 1]));
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <int UP, bool LOADS, int KS, int K>
__device__ __forceinline__ void rx_steps(floatx4 (&acc)[8][8], RxRegs& r, const uint8_t* unxt,
                                         const RxLane& ln, const RxLd& ld) {
  if constexpr (K < 64) {
    rx_step<UP, LOADS, KS, K>(acc, r, unxt, ln, ld);
    rx_steps<UP, LOADS, KS, K + 1>(acc, r, unxt, ln, ld);
  }
}

template <int UP, bool LOADS, int KS>
__device__ __forceinline__ void rx_kstep(floatx4 (&acc)[8][8], RxRegs& r, const uint8_t* unxt,
                                         const RxLane& ln, const RxLd& ld) {
  // every LDS read issued before this step has completed (lgkmcnt(0) through
  // the builtin, so the compiler knows and places no waits for them later);
  // the reads of a step are issued at least 14 MFMAs before its end
  __builtin_amdgcn_s_waitcnt(0xC07F);
  rx_steps<UP, LOADS, KS, 0>(acc, r, unxt, ln, ld);
}

// Unit U (parity UP): make unit U + 1 visible to every wave (this wave's own
// loads of it waited for, then a barrier, which also means every wave has
// finished reading unit U - 1), then the four steps, which (LOADS: unless
// U + 3 is past the last unit) issue unit U + 3 into the buffer of unit U - 1
// on the way.  Past the last unit, the next-unit reads fetch the last unit
// again (its buffer is never refilled), which keeps the steps branch-free.
// Only odd units synchronise: an odd unit reads unit U + 1, the first unit
// of the pair issued two units before it, so it waits for all of its own
// loads and passes a barrier, after which every wave's loads of that pair
// have landed and every wave has finished reading units U - 1 and U (read
// during the units before them), whose buffer its loads then refill.  An
// even unit reads unit U + 1 from its own pair, made visible by the previous
// odd unit's barrier (the prologue's for unit 1), and issues no loads.
template <int UP, bool LOADS>
__device__ __forceinline__ void rx_unit(floatx4 (&acc)[8][8], RxRegs& r, uint8_t* smem,
                                        uint32_t smem_lds, const RxSrc& s, int U, int NU, int w,
                                        int lane, const RxLane& ln) {
  if constexpr (UP == 1) {
    wait_vmcnt<0>();
    lds_barrier();
  }
  // an odd unit issues pair (U + 3) / 2 (units U + 3, U + 4) into the buffer
  // of units U - 1, U, which every wave has finished reading (the codes and
  // scales of a unit are read during the unit before it)
  RxLd ld;
  ld.s = &s;
  ld.u = (uint32_t)((U + 3) >> 1);
  ld.raw = smem_lds + (uint32_t)((((U + 3) >> 1) & 1) * kRxUnitB);
  ld.w = w;
  ld.lane = lane;
  const uint8_t* unxt = smem + (((U + 1 < NU ? U + 1 : NU - 1) >> 1) & 1) * kRxUnitB;
  rx_kstep<UP, LOADS, 0>(acc, r, unxt, ln, ld);
  rx_kstep<UP, LOADS, 1>(acc, r, unxt, ln, ld);
  rx_kstep<UP, LOADS, 2>(acc, r, unxt, ln, ld);
  rx_kstep<UP, LOADS, 3>(acc, r, unxt, ln, ld);
}

// Expansion of the A tiles (into a[0]) and B tiles 0-6 (into b) of step 0
// of unit 0 (prologue), from cw[T][0] and pr[0]; B tile 7 follows in step 0.
template <int T>
__device__ __forceinline__ void rx_prologue_tiles(RxRegs& r) {
  if constexpr (T < 15) {
    halfx8& d = T < 8 ? r.a[0][T & 7] : r.b[T & 7];
    rx_pair_to<0, 0, T, 0, 0>(r, d);
    rx_pair_to<0, 0, T, 1, 0>(r, d);
    rx_pair_to<0, 0, T, 2, 0>(r, d);
    rx_pair_to<0, 0, T, 3, 0>(r, d);
    rx_prologue_tiles<T + 1>(r);
  }
}

template <bool SPLIT>
__global__ __launch_bounds__(kRxThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_gemm_nvfp4_rx(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                     const uint8_t* a_scales, const float* __restrict__ a_amax,
                     const uint8_t* b_codes, const uint8_t* b_scales,
                     const float* __restrict__ b_amax, uint16_t* __restrict__ c, int64_t ldc,
                     int tiles_m, int tiles_n, int vec_store, int tiles_full, int tail,
                     floatx4* __restrict__ part) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // SPLIT: block h * tail + j computes tile tiles_full + j over the K half h
  // and writes FP32 partials; otherwise block b computes tile b.
  const int half = SPLIT ? (int)blockIdx.x / tail : -1;
  const int pid = SPLIT ? tiles_full + ((int)blockIdx.x - half * tail) : (int)blockIdx.x;
  int tm, tn;
  tile_of_block(pid, tiles_m, tiles_n, tm, tn);
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = w >> 1, wn = w & 1;
  const uint32_t smem_lds = (uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t*)smem;
  RxSrc s;
  // a K half starts NU units in (64 code bytes and 8 scale bytes per unit and row)
  const int NU = SPLIT ? (int)(K / 256) : (int)(K / 128);
  const uint32_t ku = SPLIT ? (uint32_t)(half * NU) : 0u;
  s.a_codes = a_codes + ku * 64;
  s.a_scales = a_scales + ku * 8;
  s.b_codes = b_codes + ku * 64;
  s.b_scales = b_scales + ku * 8;
  s.m0 = (uint32_t)tm * 256u;
  s.n0 = (uint32_t)tn * 256u;
  s.last_m = (uint32_t)(M - 1);
  s.last_n = (uint32_t)(N - 1);
  s.code_ld = (uint32_t)(K / 2);
  s.scale_ld = (uint32_t)(K / 16);
  RxLane ln;
  {
    const int r16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int P = 0; P < 2; ++P) {
      const int chunk = ((4 * P + g) ^ rx_swz(r16)) << 4;  // rows 16 i + r16 share swz(r16)
      ln.ca[P] = (wm * 128 + r16) * kRxRowB + chunk;
      ln.cb[P] = kRxOpB + (wn * 128 + r16) * kRxRowB + chunk;
    }
    ln.sa = kRxCodeB + (wm * 128 + r16) * 16 + 2 * g;
    ln.sb = kRxOpB + kRxCodeB + (wn * 128 + r16) * 16 + 2 * g;
  }

  floatx4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int jn = 0; jn < 8; ++jn) acc[i][jn] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  // prologue: pairs 0 and 1 (units 0-3) in flight; unit 0's codes and
  // scales in registers; the A tiles and B tiles 0-6 of step 0 expanded
  RxRegs r;
  rx_stage(s, 0, smem_lds, w, lane);
  if (NU > 2) rx_stage(s, 1, smem_lds + kRxUnitB, w, lane);
  // pair 0 landed (at most pair 1's loads still outstanding)
  if (NU > 2) wait_vmcnt<kRxLoadsPerPair>();
  else wait_vmcnt<0>();
  lds_barrier();
#pragma unroll
  for (int T = 0; T < 16; ++T) {
    const uint4 q = *reinterpret_cast<const uint4*>(smem + (T < 8 ? ln.ca[0] : ln.cb[0]) + (T & 7) * 2048);
    r.cw[T][0] = q.x;
    r.cw[T][1] = q.y;
    r.cw[T][2] = q.z;
    r.cw[T][3] = q.w;
    r.pr[0][T] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(
        *reinterpret_cast<const uint16_t*>(smem + (T < 8 ? ln.sa : ln.sb) + (T & 7) * 256), 128.0f, false);
  }
  rx_prologue_tiles<0>(r);

  // odd units whose pair two ahead exists (units U + 3, U + 4) issue its
  // loads; NU is even
  int U = 0;
  for (; U + 4 < NU; U += 2) {
    rx_unit<0, false>(acc, r, smem, smem_lds, s, U, NU, w, lane, ln);
    rx_unit<1, true>(acc, r, smem, smem_lds, s, U + 1, NU, w, lane, ln);
  }
  for (; U < NU; U += 2) {
    rx_unit<0, false>(acc, r, smem, smem_lds, s, U, NU, w, lane, ln);
    rx_unit<1, false>(acc, r, smem, smem_lds, s, U + 1, NU, w, lane, ln);
  }

  // every wave is done with the unit buffers (the epilogue reuses the LDS),
  // and the last MFMAs' results have reached the accumulator registers
  lds_barrier();
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  // the accumulators count as written here, so no read of them (which the
  // compiler would otherwise hoist above the wait states, into the loop's
  // exit block) precedes the barrier and the wait states
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int jn = 0; jn < 8; ++jn) asm volatile("" : "+a"(acc[i][jn]));
  __builtin_amdgcn_sched_barrier(0);

  if constexpr (SPLIT) {
    // FP32 partial of a split tile, in accumulator order: pair (mi, ni) of
    // thread t at part[((h * tail + j) * 64 + mi * 8 + ni) * 256 + t]
    floatx4* P = part + ((size_t)(half * tail + (pid - tiles_full)) * 64) * kRxThreads + t;
#pragma unroll
    for (int mi = 0; mi < 8; ++mi)
#pragma unroll
      for (int ni = 0; ni < 8; ++ni) P[(mi * 8 + ni) * kRxThreads] = acc[mi][ni];
    return;
  }

  // epilogue: alpha * acc -> BF16 (RNE), staged per wave through LDS so that
  // global stores are 256-byte row segments.  acc[mi][ni] holds, in lane l,
  // output row 16 mi + (l & 15) and columns 16 ni + 4 (l >> 4) + e of the
  // wave's quarter.
  const float alpha = nvfp4_s_dec(*a_amax) * nvfp4_s_dec(*b_amax) * 16384.0f;
  uint8_t* E = smem + w * (128 * kRxEpiRowB);
#pragma unroll
  for (int mi = 0; mi < 8; ++mi)
#pragma unroll
    for (int ni = 0; ni < 8; ++ni) {
      const floatx4 v = acc[mi][ni];
      *reinterpret_cast<uint2*>(E + (mi * 16 + (lane & 15)) * kRxEpiRowB + (ni * 16 + (lane >> 4) * 4) * 2) =
          make_uint2(pack_bf16x2(v[0] * alpha, v[1] * alpha), pack_bf16x2(v[2] * alpha, v[3] * alpha));
    }
  __syncthreads();
  const int64_t gm0 = (int64_t)s.m0 + wm * 128, gn = (int64_t)s.n0 + wn * 128 + (lane & 15) * 8;
#pragma unroll 4
  for (int it = 0; it < 32; ++it) {
    const int row = it * 4 + (lane >> 4);
    const int64_t gm = gm0 + row;
    if (gm >= M) continue;
    const uint4 v = *reinterpret_cast<const uint4*>(E + row * kRxEpiRowB + (lane & 15) * 16);
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

// Second pass of a split last wave: C = BF16_RNE(alpha * (p0 + p1)) for the
// split tiles, p0 and p1 the partials of the two K halves (same order for
// every element, so the result is deterministic).  Block b: tile j = b / 4,
// accumulator rows mi = 2 (b % 4), 2 (b % 4) + 1 of every wave.
__global__ __launch_bounds__(kRxThreads)
void k_gemm_nvfp4_rx_join(int64_t M, int64_t N, const floatx4* __restrict__ part,
                          const float* __restrict__ a_amax, const float* __restrict__ b_amax,
                          uint16_t* __restrict__ c, int64_t ldc, int tiles_m, int tiles_n,
                          int tiles_full, int tail, int vec_store) {
  const int j = blockIdx.x >> 2, q = blockIdx.x & 3;
  int tm, tn;
  tile_of_block(tiles_full + j, tiles_m, tiles_n, tm, tn);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, wm = w >> 1, wn = w & 1;
  const float alpha = nvfp4_s_dec(*a_amax) * nvfp4_s_dec(*b_amax) * 16384.0f;
  const floatx4* P0 = part + (size_t)j * 64 * kRxThreads + t;
  const floatx4* P1 = part + (size_t)(tail + j) * 64 * kRxThreads + t;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int mi = 2 * q + h;
    const int64_t gm = (int64_t)tm * 256 + wm * 128 + mi * 16 + (lane & 15);
    if (gm >= M) continue;
#pragma unroll
    for (int ni = 0; ni < 8; ++ni) {
      const floatx4 a = P0[(mi * 8 + ni) * kRxThreads], b = P1[(mi * 8 + ni) * kRxThreads];
      const floatx4 v = a + b;
      const int64_t gn = (int64_t)tn * 256 + wn * 128 + ni * 16 + (lane >> 4) * 4;
      const uint32_t lo = pack_bf16x2(v[0] * alpha, v[1] * alpha), hi = pack_bf16x2(v[2] * alpha, v[3] * alpha);
      uint16_t* dst = c + gm * ldc + gn;
      if (vec_store && gn + 3 < N) {
        *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
      } else {
        const uint32_t wv[2] = {lo, hi};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (gn + e < N) dst[e] = (uint16_t)(wv[e >> 1] >> (16 * (e & 1)));
      }
    }
  }
}

}  // namespace

// Workspace of the split last wave for callers that cannot allocate
// (bs_gemm_noalloc): FP32 partials of at most 128 split tiles, which is what
// the split needs on 256 compute units.  Each device that loads this code
// holds its own copy until the process ends; host code uses the address
// that hipGetSymbolAddress returns for the current device, never the name.
constexpr size_t kRxScratchBytes = (size_t)128 * kRxSplitTileBytes;   // 64 MiB
static __device__ __align__(256) uint8_t scratch[kRxScratchBytes];

hipError_t gemm_nvfp4_static_scratch(void** ptr, size_t* bytes) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    // once per device, with that device current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  *bytes = kRxScratchBytes;
  return hipSuccess;
}

int gemm_nvfp4_rx_split(int64_t M, int64_t N, int64_t K, int cus) {
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  if (cus <= 0 || tiles < cus || K % 512 != 0 || K < 4096) return 0;
  const int tail = (int)(tiles % cus);
  return tail <= cus / 2 ? tail : 0;
}

bool gemm_nvfp4_rx_fits(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                        const uint8_t* bc, const uint8_t* bs) {
  const auto al = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; };
  return K > 0 && K % 256 == 0 && al(ac, 16) && al(bc, 16) && al(as, 16) && al(bs, 16) &&
         M * (K / 2) < ((int64_t)1 << 32) && N * (K / 2) < ((int64_t)1 << 32);
}

hipError_t launch_gemm_nvfp4_rx(int64_t M, int64_t N, int64_t K, const uint8_t* ac,
                                const uint8_t* as, const float* aa, const uint8_t* bc,
                                const uint8_t* bs, const float* ba, void* c, int64_t ldc,
                                int tail, void* part, hipStream_t s) {
  const int tiles_m = (int)((M + 255) / 256), tiles_n = (int)((N + 255) / 256);
  const int tiles = tiles_m * tiles_n, tiles_full = tiles - tail;
  const bool vec_store = (ldc % 8 == 0) && (reinterpret_cast<uintptr_t>(c) % 16 == 0);
  if (tail < 0 || tail > tiles || (tail > 0 && (part == nullptr || K % 512 != 0)))
    return hipErrorInvalidValue;
  if (set_lds_limit(reinterpret_cast<const void*>(&k_gemm_nvfp4_rx<false>), kRxLds) != hipSuccess ||
      set_lds_limit(reinterpret_cast<const void*>(&k_gemm_nvfp4_rx<true>), kRxLds) != hipSuccess)
    return hipErrorInvalidConfiguration;
  uint16_t* cp = static_cast<uint16_t*>(c);
  floatx4* pp = static_cast<floatx4*>(part);
  // the full waves, then the split last wave (two K halves per tile) and the
  // join of its partials
  if (tiles_full > 0)
    hipLaunchKernelGGL(k_gemm_nvfp4_rx<false>, dim3((unsigned)tiles_full), dim3(kRxThreads), kRxLds, s,
                       M, N, K, ac, as, aa, bc, bs, ba, cp, ldc, tiles_m, tiles_n, vec_store ? 1 : 0,
                       tiles_full, 1, nullptr);
  if (tail > 0) {
    hipLaunchKernelGGL(k_gemm_nvfp4_rx<true>, dim3((unsigned)(2 * tail)), dim3(kRxThreads), kRxLds, s,
                       M, N, K, ac, as, aa, bc, bs, ba, cp, ldc, tiles_m, tiles_n, vec_store ? 1 : 0,
                       tiles_full, tail, pp);
    hipLaunchKernelGGL(k_gemm_nvfp4_rx_join, dim3((unsigned)(4 * tail)), dim3(kRxThreads), 0, s, M, N, pp,
                       aa, ba, cp, ldc, tiles_m, tiles_n, tiles_full, tail, vec_store ? 1 : 0);
  }
  return hipGetLastError();
}

}  // namespace bsq
