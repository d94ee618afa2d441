// Block quantizers for gfx950: amax passes, rowwise (flat) encoder and the
// row+column (tile) encoder.
//
// NVFP4 pretraining post, "NVFP4 pretraining recipe": 1x16 E4M3 block scales
// under a per-tensor FP32 scale (ingredients 1-2), RHT on WGRAD inputs
// (ingredient 3), 16x16 weight tiles (ingredient 4), RNE / stochastic rounding
// (ingredient 5).  HN page opcode84: MXFP4 / MXFP8 with E8M0 scales per 32.
//
// Memory layout and work split (all kernels are HBM-bound streams, the
// stochastic-rounding encoders excepted: Philox makes them VALU-bound):
//  * Lanes move 16-byte chunks of 8 BF16 values (8-byte chunks in the RHT
//    amax pass) and every global access instruction of a wave covers one
//    contiguous run per row (codes and scales contiguous across lanes).
//  * Amax passes: each wave reduces grid-stride work items with the next
//    item's loads in flight; one atomic max per workgroup at the end.
//  * Rowwise: a 1x16 block is a lane pair, a 1x32 MX block a lane quad; the
//    block amax is combined with quad_perm DPP moves, no LDS.
//  * Row + column: a lane owns 8 columns x 16 (or 32) rows, so each column
//    block sits in one lane's registers (the transpose happens in registers)
//    and each row block is again a lane pair/quad.  A lane walks down several
//    row blocks so its column outputs fill whole cache lines over time.
#include "bsq_device.hpp"
#include "bsq_internal.hpp"

namespace bsq {

namespace {

constexpr int kUnroll = 4;          // chunks per lane per loop trip (flat kernels)

__device__ __forceinline__ uint32_t absbits(float v) { return f2u(v) & 0x7FFFFFFFu; }

// 8 floats from a 16-byte chunk of BF16 values (element e = half e of the chunk).
__device__ __forceinline__ void unpack8(const uint4& v, float (&y)[8]) {
  y[0] = bf16_lo(v.x); y[1] = bf16_hi(v.x);
  y[2] = bf16_lo(v.y); y[3] = bf16_hi(v.y);
  y[4] = bf16_lo(v.z); y[5] = bf16_hi(v.z);
  y[6] = bf16_lo(v.w); y[7] = bf16_hi(v.w);
}

// Element (row i, column j) of a lane's 8-column tile held as rows of uint4.
__device__ __forceinline__ float tile_elem(const uint4& row, int j) {
  const uint32_t w = (j >> 1) == 0 ? row.x : (j >> 1) == 1 ? row.y : (j >> 1) == 2 ? row.z : row.w;
  return (j & 1) ? bf16_hi(w) : bf16_lo(w);
}

// 16-point RHT of a 16-chunk split over a lane pair: this lane holds elements
// 8*odd .. 8*odd+7.  Stages h = 1, 2, 4 are in-lane, h = 8 pairs the lanes.
__device__ __forceinline__ void rht16_pair(float (&y)[8], bool odd, uint32_t signs) {
  const uint32_t sg = odd ? (signs >> 8) : signs;
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = u2f(f2u(y[e]) ^ (((sg >> e) & 1u) << 31));
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if ((e & h) == 0) {
        const float a = y[e], b = y[e + h];
        y[e] = a + b;
        y[e + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float p = dpp_xor1f(y[e]);
    y[e] = odd ? (p - y[e]) : (y[e] + p);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = y[e] * 0.25f;
}

// Encode 8 scaled values to 8 E2M1 codes packed low-nibble-first: RNE or
// stochastic rounding, both on the hardware converts.
template <bool SR>
__device__ __forceinline__ uint32_t encode8_fp4(const float (&v)[8], const R16x8& rnd) {
  return SR ? fp4x8_sr(v, rnd) : fp4x8_rne(v);
}

// Encode 8 scaled values to 8 signed E4M3 bytes (RNE, saturating at 448):
// clamp, then the hardware FP32 -> E4M3 convert (RNE on [0, 464)).
__device__ __forceinline__ uint2 encode8_fp8(const float (&v)[8]) {
  float c[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) c[e] = fmaxf(fminf(v[e], 448.0f), -448.0f);
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(c[4], c[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(c[6], c[7], hi, true);
  return make_uint2((uint32_t)lo, (uint32_t)hi);
}

// LDS table of encode factors enc[S] = s_enc / S for the 128 E4M3 codes.
__device__ __forceinline__ void fill_enc_table(float* tab, float s_enc) {
  for (int c = threadIdx.x; c < 128; c += blockDim.x) tab[c] = nvfp4_enc_of_code((uint32_t)c, s_enc);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t m) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  return m;
}

// Block-level max into one or two global accumulators.
__device__ __forceinline__ void block_max_atomic(uint32_t m, float* a0, float* a1) {
  __shared__ uint32_t red[16];
  __syncthreads();                 // a previous call's reads of red[] are done
  m = wave_max_u32(m);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int nw = (blockDim.x + 63) >> 6;
    for (int i = 1; i < nw; ++i) m = max(m, red[i]);
    if (a0) atomicMax(reinterpret_cast<unsigned int*>(a0), m);
    if (a1) atomicMax(reinterpret_cast<unsigned int*>(a1), m);
  }
}

// ---------------------------------------------------------------- small kernels

__global__ void k_zero_amax(float* a, float* b) {
  if (threadIdx.x == 0) {
    if (a) *a = 0.0f;
    if (b) *b = 0.0f;
  }
}

__global__ void k_copy_amax(const float* src, float* dst) {
  if (threadIdx.x == 0) *dst = *src;
}

// ---------------------------------------------------------------- amax passes

// Word 3 of a raw buffer resource on gfx9-family GPUs (32-bit data format,
// no swizzle): out-of-range loads return zero.
constexpr int kBufRsrcWord3 = 0x00020000;
constexpr int kAmaxRhtBlocks = 768;                   // workgroups of the RHT amax pass (3 per CU)
constexpr int kAmaxFlatBlocks = 1024;                  // workgroups of the flat amax pass (4 per CU)

typedef unsigned short ushort2v __attribute__((ext_vector_type(2)));

// Flat amax over a contiguous tensor of nchunk 16-byte chunks (8 BF16 values).
// A work item is 512 consecutive chunks (8 KiB), one per wave: lane l loads
// chunks 64 k + l (k = 0..7), so every load instruction covers 1 KiB.  Waves
// walk the items grid-stride with the next item's loads in flight.  Without
// RHT the magnitudes are compared as packed 16-bit integers; with RHT each
// aligned 16-chunk (a lane pair) is transformed first.
template <bool RHT>
__device__ __forceinline__ void amax_flat_load(const uint4* __restrict__ x, int64_t nchunk,
                                               int64_t item, int lane, uint4 (&v)[8]) {
  const int64_t c0 = item * 512;
  const int64_t left = nchunk - c0;
  const int nrec = (int)(left >= 512 ? 512 * 16 : left * 16);
  __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(x + c0), (short)0, nrec,
                                                                kBufRsrcWord3);
#pragma unroll
  for (int k = 0; k < 8; ++k)
    v[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16, k * 1024, 0));
}

template <bool RHT>
__device__ __forceinline__ void amax_flat_item(const uint4 (&v)[8], int lane, uint32_t signs,
                                               ushort2v& m16, uint32_t& m32) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (!RHT) {
      const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
      for (int d = 0; d < 4; ++d) m16 = __builtin_elementwise_max(m16, __builtin_bit_cast(ushort2v, w[d] & 0x7FFF7FFFu));
    } else {
      float y[8];
      unpack8(v[k], y);
      rht16_pair(y, lane & 1, signs);
#pragma unroll
      for (int e = 0; e < 8; ++e) m32 = max(m32, absbits(y[e]));
    }
  }
}

template <bool RHT>
__global__ __launch_bounds__(256) void k_amax_flat(const uint4* __restrict__ x, int64_t nchunk,
                                                   uint32_t signs, float* a0, float* a1) {
  const int lane = threadIdx.x & 63;
  const int64_t nitems = (nchunk + 511) / 512;
  const int64_t nw = (int64_t)gridDim.x * 4;
  int64_t it = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  ushort2v m16 = {0, 0};
  uint32_t m32 = 0;
  uint4 a[8], b[8];
  if (it < nitems) amax_flat_load<RHT>(x, nchunk, it, lane, a);
  while (it < nitems) {
    if (it + nw < nitems) amax_flat_load<RHT>(x, nchunk, it + nw, lane, b);
    amax_flat_item<RHT>(a, lane, signs, m16, m32);
    it += nw;
    if (it >= nitems) break;
    if (it + nw < nitems) amax_flat_load<RHT>(x, nchunk, it + nw, lane, a);
    amax_flat_item<RHT>(b, lane, signs, m16, m32);
    it += nw;
  }
  const uint32_t m = RHT ? m32 : max((uint32_t)m16.x, (uint32_t)m16.y) << 16;
  block_max_atomic(m, a0, a1);
}

// amax of x and of RHT(x^T) for x [R, C] (R % 16 == 0, C % 4 == 0).  A work
// item is 16 rows x 256 columns, one per wave (a lane owns 4 columns); waves
// walk the items grid-stride, the next item's 16 row loads in flight while the
// current one is reduced.
//  * x amax: BF16 magnitudes compared as packed 16-bit integers.
//  * RHT amax: the column transform along the 16 rows, with D applied to the
//    packed BF16 pairs (sign-bit flips) and the 1/4 applied to the final max
//    (exact: inputs are multiples of 2^-133, so every transformed value is,
//    and scaling by 1/4 stays in the FP32 range without rounding).
__device__ __forceinline__ void amax_rht_item(const uint2 (&v)[16], uint32_t signs, ushort2v& mr,
                                              float& mc) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    mr = __builtin_elementwise_max(mr, __builtin_bit_cast(ushort2v, v[i].x & 0x7FFF7FFFu));
    mr = __builtin_elementwise_max(mr, __builtin_bit_cast(ushort2v, v[i].y & 0x7FFF7FFFu));
  }
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    uint32_t s[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = (d == 0 ? v[i].x : v[i].y) ^ (((signs >> i) & 1u) * 0x80008000u);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      float y[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) y[i] = half ? bf16_hi(s[i]) : bf16_lo(s[i]);
#pragma unroll
      for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if ((i & h) == 0) {
            const float a = y[i], b = y[i + h];
            y[i] = a + b;
            y[i + h] = a - b;
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 16; i += 2) mc = fmaxf(mc, fmaxf(fabsf(y[i]), fabsf(y[i + 1])));
    }
  }
}

// Loads of one item through a buffer resource over its 16 rows (the item
// index is wave-uniform): row i is the scalar offset i * 2C, the lane's
// column offset the one vector offset.  Lanes past the last column get an
// offset beyond the resource and read zeros.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void amax_rht_load(const uint16_t* __restrict__ x, int64_t C, int64_t ncg,
                                              int64_t item, int lane, uint2 (&v)[16]) {
  const int64_t rb = item / ncg, cg = item - rb * ncg;
  const uint32_t rowb = (uint32_t)C * 2u;
  __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(x + rb * 16 * C), (short)0, (int)(16u * rowb), kBufRsrcWord3);
  const int64_t c0 = cg * 256 + lane * 4;
  const int voff = c0 < C ? (int)(c0 * 2) : (int)0x7FFFFFF0;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    v[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, voff, (int)(i * rowb), 0));
}

__global__ __launch_bounds__(256) void k_amax_tile_rht(const uint16_t* __restrict__ x, int64_t R,
                                                       int64_t C, uint32_t signs, float* amax_row,
                                                       float* amax_col) {
  const int lane = threadIdx.x & 63;
  const int64_t ncg = (C + 255) / 256, nitems = ncg * (R / 16);
  const int64_t nw = (int64_t)gridDim.x * 4;
  int64_t it = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  ushort2v mr = {0, 0};
  float mc = 0.0f;
  uint2 a[16], b[16];
  if (it < nitems) amax_rht_load(x, C, ncg, it, lane, a);
  while (it < nitems) {
    if (it + nw < nitems) amax_rht_load(x, C, ncg, it + nw, lane, b);
    amax_rht_item(a, signs, mr, mc);
    it += nw;
    if (it >= nitems) break;
    if (it + nw < nitems) amax_rht_load(x, C, ncg, it + nw, lane, a);
    amax_rht_item(b, signs, mr, mc);
    it += nw;
  }
  const uint32_t m = max((uint32_t)mr.x, (uint32_t)mr.y) << 16;
  block_max_atomic(m, amax_row, nullptr);
  block_max_atomic(f2u(mc * 0.25f), amax_col, nullptr);
}

// ---------------------------------------------------------------- SwiGLU producers
// The MLP of the measured Llama models feeds the down projection with
// H = silu(G) * U of the fused gate/up output Y = [G | U] [R, 2F], and its
// backward turns dH into dY = [dG | dU].  Both are produced here together with
// the per-tensor amaxes the NVFP4 quantizer of the output needs (plain, and the
// column RHT amax when the column side is transformed), so the quantizer that
// follows skips its own amax pass: one full read of the BF16 output less.
//
// A work item is 16 rows x 256 columns of H, one per wave; a lane owns 4
// columns (8-byte loads, 512 contiguous bytes per wave and row), so the 16
// values of a column chunk sit in one lane and the column RHT amax is
// amax_rht_item on the rounded BF16 outputs: the standalone pass bit for bit.
// Waves walk the items grid-stride (one atomic max per workgroup at the end).
constexpr int kSwigluBlocks = 1024;                    // 4 workgroups per CU
constexpr float kLog2e = 1.44269504088896340736f;

// ln 2 split for the argument reduction (Cody and Waite): the high part has
// 16 significant bits, so n * kLn2Hi is exact for |n| < 2^8.
constexpr float kLn2Hi = 0.693145751953125f;
constexpr float kLn2Lo = 1.42860682030941723212e-6f;

// sigma(g) and sigma(-g) = 1 - sigma(g), each without cancellation, from
// e = exp(-|g|) (never overflows).  The argument is reduced first, |g| =
// n ln 2 + r with |r| <= ln2 / 2 (n = rint(|g| log2 e), r by two FMAs), and
// e = 2^-n exp(-r): the exponential's argument then carries no rounding error
// that grows with |g|, and the relative error stays at a few FP32 ulps (v_exp
// on a small argument, v_rcp) for every gate; 2^-n is an exact exponent
// shift, rounding once where e falls below the normal range.
struct SigPair { float s, c; };
__device__ __forceinline__ SigPair sigmoid_pair(float g) {
  const float a = fabsf(g);
  const float nn = __builtin_rintf(-a * kLog2e);                 // -n
  const float t = __builtin_fmaf(nn, kLn2Lo, __builtin_fmaf(nn, kLn2Hi, a));
  // v_exp_f32 on -t log2 e in [-0.5, 0.5] (no range handling needed), then 2^-n
  const float e = __builtin_ldexpf(__builtin_amdgcn_exp2f(-t * kLog2e), (int)nn);
  const float r = __builtin_amdgcn_rcpf(1.0f + e);
  const float er = e * r;
  return g >= 0.0f ? SigPair{r, er} : SigPair{er, r};
}

__device__ __forceinline__ float swiglu1(float g, float u) { return g * sigmoid_pair(g).s * u; }

// dG and dU of one element: dU = dH * silu(g), dG = dH * U * silu'(g) with
// silu'(g) = sigma(g) * (1 + g * sigma(-g)).
__device__ __forceinline__ void swiglu_bwd1(float g, float u, float d, float& dg, float& du) {
  const SigPair p = sigmoid_pair(g);
  du = d * (g * p.s);
  dg = (d * u) * (p.s * (1.0f + g * p.c));
}

// Loads of one 16-row slab through a buffer resource (row i at scalar offset
// i * row_bytes); dead lanes pass an offset beyond the resource and read zeros.
__device__ __forceinline__ void slab_load(__amdgpu_buffer_rsrc_t rs, int voff, uint32_t row_bytes,
                                          uint2 (&v)[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i)
    v[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, voff, (int)(i * row_bytes), 0));
}

__device__ __forceinline__ void slab_store(uint16_t* p, int64_t ld, const uint2 (&v)[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) *reinterpret_cast<uint2*>(p + i * ld) = v[i];
}

__device__ __forceinline__ void slab_max(const uint2 (&v)[16], ushort2v& mr) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    mr = __builtin_elementwise_max(mr, __builtin_bit_cast(ushort2v, v[i].x & 0x7FFF7FFFu));
    mr = __builtin_elementwise_max(mr, __builtin_bit_cast(ushort2v, v[i].y & 0x7FFF7FFFu));
  }
}

// AMAX: 0 none; 1 plain amax into both outputs; 2 plain amax into amax_row and
// the column RHT amax into amax_col.
template <int AMAX>
__device__ __forceinline__ void swiglu_amax_out(ushort2v mr, float mc, float* amax_row, float* amax_col) {
  if (AMAX == 0) return;
  const uint32_t m = max((uint32_t)mr.x, (uint32_t)mr.y) << 16;
  if (AMAX == 1) {
    block_max_atomic(m, amax_row, amax_col);
  } else {
    block_max_atomic(m, amax_row, nullptr);
    block_max_atomic(f2u(mc * 0.25f), amax_col, nullptr);
  }
}

template <int AMAX>
__global__ __launch_bounds__(256) void k_swiglu_fwd(const uint16_t* __restrict__ y, int64_t R,
                                                    int64_t F, uint32_t signs, uint16_t* __restrict__ h,
                                                    float* amax_row, float* amax_col) {
  const int lane = threadIdx.x & 63;
  const int64_t ncg = (F + 255) / 256, nitems = ncg * (R / 16);
  const int64_t nw = (int64_t)gridDim.x * 4;
  const uint32_t yrow = (uint32_t)F * 4u;                 // bytes per row of Y
  ushort2v mr = {0, 0};
  float mc = 0.0f;
  for (int64_t it = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
       it < nitems; it += nw) {
    const int64_t rb = it / ncg, cg = it - rb * ncg;
    const int64_t c0 = cg * 256 + lane * 4;
    const bool live = c0 < F;
    __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(y + rb * 32 * F), (short)0, (int)(16u * yrow), kBufRsrcWord3);
    uint2 g[16], u[16], hv[16];
    slab_load(rs, live ? (int)(c0 * 2) : (int)0x7FFFFFF0, yrow, g);
    slab_load(rs, live ? (int)((F + c0) * 2) : (int)0x7FFFFFF0, yrow, u);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      hv[i].x = pack_bf16x2(swiglu1(bf16_lo(g[i].x), bf16_lo(u[i].x)), swiglu1(bf16_hi(g[i].x), bf16_hi(u[i].x)));
      hv[i].y = pack_bf16x2(swiglu1(bf16_lo(g[i].y), bf16_lo(u[i].y)), swiglu1(bf16_hi(g[i].y), bf16_hi(u[i].y)));
    }
    if (live) slab_store(h + rb * 16 * F + c0, F, hv);
    if (AMAX == 2) amax_rht_item(hv, signs, mr, mc);
    else if (AMAX == 1) slab_max(hv, mr);
  }
  swiglu_amax_out<AMAX>(mr, mc, amax_row, amax_col);
}

template <int AMAX>
__global__ __launch_bounds__(256) void k_swiglu_bwd(const uint16_t* __restrict__ y,
                                                    const uint16_t* __restrict__ dh, int64_t R,
                                                    int64_t F, uint32_t signs, uint16_t* __restrict__ dy,
                                                    float* amax_row, float* amax_col) {
  const int lane = threadIdx.x & 63;
  const int64_t ncg = (F + 255) / 256, nitems = ncg * (R / 16);
  const int64_t nw = (int64_t)gridDim.x * 4;
  const uint32_t yrow = (uint32_t)F * 4u, drow = (uint32_t)F * 2u;
  ushort2v mr = {0, 0};
  float mc = 0.0f;
  for (int64_t it = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
       it < nitems; it += nw) {
    const int64_t rb = it / ncg, cg = it - rb * ncg;
    const int64_t c0 = cg * 256 + lane * 4;
    const bool live = c0 < F;
    __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(y + rb * 32 * F), (short)0, (int)(16u * yrow), kBufRsrcWord3);
    __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(dh + rb * 16 * F), (short)0, (int)(16u * drow), kBufRsrcWord3);
    uint2 g[16], u[16], d[16], dg[16], du[16];
    slab_load(ry, live ? (int)(c0 * 2) : (int)0x7FFFFFF0, yrow, g);
    slab_load(ry, live ? (int)((F + c0) * 2) : (int)0x7FFFFFF0, yrow, u);
    slab_load(rd, live ? (int)(c0 * 2) : (int)0x7FFFFFF0, drow, d);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float a0, a1, a2, a3, b0, b1, b2, b3;
      swiglu_bwd1(bf16_lo(g[i].x), bf16_lo(u[i].x), bf16_lo(d[i].x), a0, b0);
      swiglu_bwd1(bf16_hi(g[i].x), bf16_hi(u[i].x), bf16_hi(d[i].x), a1, b1);
      swiglu_bwd1(bf16_lo(g[i].y), bf16_lo(u[i].y), bf16_lo(d[i].y), a2, b2);
      swiglu_bwd1(bf16_hi(g[i].y), bf16_hi(u[i].y), bf16_hi(d[i].y), a3, b3);
      dg[i] = make_uint2(pack_bf16x2(a0, a1), pack_bf16x2(a2, a3));
      du[i] = make_uint2(pack_bf16x2(b0, b1), pack_bf16x2(b2, b3));
    }
    if (live) {
      slab_store(dy + rb * 32 * F + c0, 2 * F, dg);
      slab_store(dy + rb * 32 * F + F + c0, 2 * F, du);
    }
    if (AMAX == 2) {
      amax_rht_item(dg, signs, mr, mc);
      amax_rht_item(du, signs, mr, mc);
    } else if (AMAX == 1) {
      slab_max(dg, mr);
      slab_max(du, mr);
    }
  }
  swiglu_amax_out<AMAX>(mr, mc, amax_row, amax_col);
}

// ---------------------------------------------------------------- master-weight update
// The optimizer step folds the BF16 weight gradient into the FP32 master
// weight: w <- w - lr * dW as an FP32 product and an FP32 difference (this
// file is built without multiply-add contraction), then writes the BF16
// working copy RNE(w) that the next step quantizes, and reduces its amax (the
// per-tensor amax of the next 16x16 weight quantization).  A lane moves one
// 8-element chunk per trip: 16 bytes of gradient, 32 of w in and out, 16 of
// the copy; grid-stride, one atomic max per workgroup.
constexpr int kUpdateBlocks = 2048;

template <bool AMAX>
__global__ __launch_bounds__(256) void k_master_update(float* __restrict__ w, const uint4* __restrict__ g,
                                                       int64_t nchunk, float lr, uint4* __restrict__ wb,
                                                       float* amax) {
  ushort2v m16 = {0, 0};
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < nchunk; c += stride) {
    const uint4 gv = g[c];
    float4* wp = reinterpret_cast<float4*>(w) + 2 * c;
    float4 a = wp[0], b = wp[1];
    a.x = a.x - lr * bf16_lo(gv.x);
    a.y = a.y - lr * bf16_hi(gv.x);
    a.z = a.z - lr * bf16_lo(gv.y);
    a.w = a.w - lr * bf16_hi(gv.y);
    b.x = b.x - lr * bf16_lo(gv.z);
    b.y = b.y - lr * bf16_hi(gv.z);
    b.z = b.z - lr * bf16_lo(gv.w);
    b.w = b.w - lr * bf16_hi(gv.w);
    wp[0] = a;
    wp[1] = b;
    const uint4 o = make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y),
                               pack_bf16x2(b.z, b.w));
    wb[c] = o;
    if (AMAX) {
      m16 = __builtin_elementwise_max(m16, __builtin_bit_cast(ushort2v, o.x & 0x7FFF7FFFu));
      m16 = __builtin_elementwise_max(m16, __builtin_bit_cast(ushort2v, o.y & 0x7FFF7FFFu));
      m16 = __builtin_elementwise_max(m16, __builtin_bit_cast(ushort2v, o.z & 0x7FFF7FFFu));
      m16 = __builtin_elementwise_max(m16, __builtin_bit_cast(ushort2v, o.w & 0x7FFF7FFFu));
    }
  }
  if (AMAX) block_max_atomic(max((uint32_t)m16.x, (uint32_t)m16.y) << 16, amax, nullptr);
}

// ---------------------------------------------------------------- rowwise encoder

template <int FMT, bool SR, bool RHT>
__global__ __launch_bounds__(256) void k_quant_flat(const uint4* __restrict__ x, int64_t nchunk,
                                                    const float* __restrict__ amax, uint32_t signs,
                                                    uint64_t seed, uint32_t offset,
                                                    uint8_t* __restrict__ codes,
                                                    uint8_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  __shared__ float enc_tab[128];
  float s_enc = 0.0f;
  if (FMT == kNVFP4) {
    s_enc = nvfp4_s_enc(*amax);
    fill_enc_table(enc_tab, s_enc);
    __syncthreads();
  }
  for (int64_t base = wave * 64 * kUnroll; base < nchunk; base += nwaves * 64 * kUnroll) {
    uint4 v[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      const int64_t q = base + k * 64 + lane;
      v[k] = q < nchunk ? x[q] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      const int64_t q = base + k * 64 + lane;
      float y[8];
      unpack8(v[k], y);
      if (RHT) rht16_pair(y, lane & 1, signs);
      uint32_t m = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) m = max(m, absbits(y[e]));
      m = max(m, dpp_xor1(m));
      if (FMT != kNVFP4) m = max(m, dpp_xor2(m));
      const float a_b = u2f(m);
      uint32_t scode;
      float mult;
      if (FMT == kNVFP4) {
        scode = nvfp4_scale_code(a_b, s_enc);
        mult = enc_tab[scode];
      } else {
        const int e = mx_exponent(a_b, FMT == kMXFP4 ? 2 : 8);
        scode = (uint32_t)(e + 127);
        mult = exp2_neg(e);
      }
      float v8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v8[e] = y[e] * mult;
      if (q < nchunk) {
        if (FMT == kMXFP8) {
          reinterpret_cast<uint2*>(codes)[q] = encode8_fp8(v8);
        } else {
          R16x8 rnd{};
          if (SR) rnd = sr_words((uint64_t)q, seed, offset, 0u);
          reinterpret_cast<uint32_t*>(codes)[q] = encode8_fp4<SR>(v8, rnd);
        }
        if (FMT == kNVFP4) {
          if ((lane & 1) == 0) scales[q >> 1] = (uint8_t)scode;
        } else {
          if ((lane & 3) == 0) scales[q >> 2] = (uint8_t)scode;
        }
      }
    }
  }
}

// ---------------------------------------------------------------- row + column encoder

// One lane owns columns [c0, c0+8) and walks `rbs` blocks of BLK rows.
//  row output : per row, this lane's 8 values; the block spans BLK/8 lanes.
//  col output : per column, the BLK values of this lane's registers.
//  TWO_D      : one 16x16 tile scale for both orientations (NVFP4 only).
template <int FMT, bool SR, bool RHT, bool TWO_D>
__global__ __launch_bounds__(64) void k_quant_tile(
    const uint16_t* __restrict__ x, int64_t R, int64_t C, int gx, int rbs, int do_row, int do_col,
    const float* __restrict__ amax_row, const float* __restrict__ amax_col, uint32_t signs,
    uint64_t seed, uint32_t offset, uint8_t* __restrict__ codes_row,
    uint8_t* __restrict__ scales_row, uint8_t* __restrict__ codes_col,
    uint8_t* __restrict__ scales_col) {
  constexpr int BLK = FMT == kNVFP4 ? 16 : 32;
  constexpr int EMAX = FMT == kMXFP4 ? 2 : 8;
  const int bx = blockIdx.x % gx, by = blockIdx.x / gx;
  const int lane = threadIdx.x;
  const int64_t c0 = ((int64_t)bx * 64 + lane) * 8;
  __shared__ float enc_row[128], enc_col[128];
  float s_enc_row = 0.0f, s_enc_col = 0.0f;
  if (FMT == kNVFP4) {
    if (do_row) s_enc_row = nvfp4_s_enc(*amax_row);
    if (do_col) s_enc_col = nvfp4_s_enc(*amax_col);
    fill_enc_table(enc_row, s_enc_row);
    fill_enc_table(enc_col, s_enc_col);
    __syncthreads();
  }
  if (c0 >= C) return;                       // whole lane groups leave together (C % BLK == 0)
  for (int k = 0; k < rbs; ++k) {
    const int64_t r0 = ((int64_t)by * rbs + k) * BLK;
    if (r0 >= R) break;
    uint4 v[BLK];
#pragma unroll
    for (int i = 0; i < BLK; ++i) v[i] = *reinterpret_cast<const uint4*>(x + (r0 + i) * C + c0);

    BlockScale tile{};
    if (TWO_D) {
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < BLK; ++i) {
        float y[8];
        unpack8(v[i], y);
#pragma unroll
        for (int e = 0; e < 8; ++e) m = max(m, absbits(y[e]));
      }
      m = max(m, dpp_xor1(m));
      tile.code = nvfp4_scale_code(u2f(m), do_row ? s_enc_row : s_enc_col);
      tile.enc = do_row ? enc_row[tile.code] : enc_col[tile.code];
    }

    if (do_row) {
#pragma unroll
      for (int i = 0; i < BLK; ++i) {
        const int64_t r = r0 + i;
        float y[8];
        unpack8(v[i], y);
        uint32_t scode;
        float mult;
        if (TWO_D) {
          scode = tile.code;
          mult = tile.enc;
        } else {
          uint32_t m = 0;
#pragma unroll
          for (int e = 0; e < 8; ++e) m = max(m, absbits(y[e]));
          m = max(m, dpp_xor1(m));
          if (FMT != kNVFP4) m = max(m, dpp_xor2(m));
          if (FMT == kNVFP4) {
            scode = nvfp4_scale_code(u2f(m), s_enc_row);
            mult = enc_row[scode];
          } else {
            const int e = mx_exponent(u2f(m), EMAX);
            scode = (uint32_t)(e + 127);
            mult = exp2_neg(e);
          }
        }
        float v8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v8[e] = y[e] * mult;
        const int64_t flat = r * C + c0;                 // element index of the chunk
        if (FMT == kMXFP8) {
          reinterpret_cast<uint2*>(codes_row)[flat >> 3] = encode8_fp8(v8);
        } else {
          R16x8 rnd{};
          if (SR) rnd = sr_words((uint64_t)(flat >> 3), seed, offset, 0u);
          reinterpret_cast<uint32_t*>(codes_row)[flat >> 3] = encode8_fp4<SR>(v8, rnd);
        }
        if ((lane & (BLK / 8 - 1)) == 0) scales_row[flat / BLK] = (uint8_t)scode;
      }
    }

    if (do_col) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t c = c0 + j;
        float y[BLK];
#pragma unroll
        for (int i = 0; i < BLK; ++i) y[i] = tile_elem(v[i], j);
        if (RHT) {
          float (&y16)[16] = *reinterpret_cast<float(*)[16]>(&y[0]);
          rht16(y16, signs);
        }
        uint32_t scode;
        float mult;
        if (TWO_D) {
          scode = tile.code;
          mult = tile.enc;
        } else {
          uint32_t m = 0;
#pragma unroll
          for (int i = 0; i < BLK; ++i) m = max(m, absbits(y[i]));
          if (FMT == kNVFP4) {
            scode = nvfp4_scale_code(u2f(m), s_enc_col);
            mult = enc_col[scode];
          } else {
            const int e = mx_exponent(u2f(m), EMAX);
            scode = (uint32_t)(e + 127);
            mult = exp2_neg(e);
          }
        }
        const int64_t flat = c * R + r0;                 // element index in the [C, R] output
#pragma unroll
        for (int h = 0; h < BLK / 8; ++h) {
          float v8[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v8[e] = y[8 * h + e] * mult;
          const int64_t grp = (flat >> 3) + h;
          if (FMT == kMXFP8) {
            reinterpret_cast<uint2*>(codes_col)[grp] = encode8_fp8(v8);
          } else {
            R16x8 rnd{};
            if (SR) rnd = sr_words((uint64_t)grp, seed, offset, 1u);
            reinterpret_cast<uint32_t*>(codes_col)[grp] = encode8_fp4<SR>(v8, rnd);
          }
        }
        scales_col[flat / BLK] = (uint8_t)scode;
      }
    }
  }
}

// ---------------------------------------------------------------- NVFP4 row + column encoder, 256 x 256 tiles
//
// One 512-thread workgroup per 256 x 256 tile (R and C multiples of 256).
// Thread t owns columns 8 * (t % 32) .. +8 of the tile and its 16-row block
// t / 32, so every 1x16 column block (and every 16x16 weight tile, with the
// neighbouring lane) sits in registers, exactly as in k_quant_tile.  What
// differs is the output path: row codes go straight out (32 lanes write one
// 128-byte row segment), while column codes and both scale arrays are staged in
// LDS and written as whole 128-byte lines (column codes) or 16-byte runs
// (scales), so no partial line is left for the L2 to merge.  Tiles are dealt
// to the XCDs in contiguous runs of the row-major tile order, so the eight
// tiles that share a row-scale line finish in one L2.
constexpr int kQtThreads = 512;
constexpr int kQtTile = 256;

__device__ __forceinline__ void qt_tile_of_block(int pid, int tiles_r, int tiles_c, int& tr, int& tc) {
  constexpr int kXcd = 8;
  const int nt = tiles_r * tiles_c;
  const int q = nt / kXcd, r = nt % kXcd;
  const int xcd = pid % kXcd, i = pid / kXcd;
  const int idx = xcd * q + (xcd < r ? xcd : r) + i;
  tr = idx / tiles_c;
  tc = idx % tiles_c;
}

// max |x| over a thread's 16 rows x 8 BF16 values, as FP32 bits: the
// magnitudes are compared as packed 16-bit integers, without unpacking.
__device__ __forceinline__ uint32_t amax16x8_bits(const uint4 (&v)[16]) {
  ushort2v m = {0, 0};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
    for (int d = 0; d < 4; ++d) m = __builtin_elementwise_max(m, __builtin_bit_cast(ushort2v, w[d] & 0x7FFF7FFFu));
  }
  return max((uint32_t)m.x, (uint32_t)m.y) << 16;
}

template <bool SR, bool RHT, bool TWO_D>
__global__ __launch_bounds__(kQtThreads) void k_qt_nvfp4(
    const uint16_t* __restrict__ x, int64_t R, int64_t C, int tiles_r, int tiles_c, int do_row,
    int do_col, const float* __restrict__ amax_row, const float* __restrict__ amax_col,
    uint32_t signs, uint64_t seed, uint32_t offset, uint8_t* __restrict__ codes_row,
    uint8_t* __restrict__ scales_row, uint8_t* __restrict__ codes_col,
    uint8_t* __restrict__ scales_col) {
  // column codes: 256 columns x 128 bytes, 8-byte unit u of column c stored at
  // unit u ^ ((c / 8) % 16), so the 16 lanes of a write phase hit distinct banks
  __shared__ __attribute__((aligned(16))) uint8_t col_codes[kQtTile * 128];
  __shared__ __attribute__((aligned(16))) uint8_t col_sc[16 * kQtTile];   // [row block][column]
  __shared__ __attribute__((aligned(16))) uint8_t row_sc[kQtTile * 16];   // [row][column block]
  __shared__ float enc_row[128], enc_col[128];
  int tr, tc;
  qt_tile_of_block(blockIdx.x, tiles_r, tiles_c, tr, tc);
  const int t = threadIdx.x, cg = t & 31, rb = t >> 5;
  const int64_t r0 = (int64_t)tr * kQtTile + rb * 16, c0 = (int64_t)tc * kQtTile + cg * 8;

  uint4 v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = *reinterpret_cast<const uint4*>(x + (r0 + i) * C + c0);

  const float s_enc_row = do_row ? nvfp4_s_enc(*amax_row) : 0.0f;
  const float s_enc_col = do_col ? nvfp4_s_enc(*amax_col) : 0.0f;
  if (t < 128) enc_row[t] = nvfp4_enc_of_code((uint32_t)t, s_enc_row);
  else if (t < 256) enc_col[t - 128] = nvfp4_enc_of_code((uint32_t)(t - 128), s_enc_col);
  __syncthreads();

  BlockScale tile{};
  if (TWO_D) {
    uint32_t m = amax16x8_bits(v);
    m = max(m, dpp_xor1(m));
    tile.code = nvfp4_scale_code(u2f(m), do_row ? s_enc_row : s_enc_col);
    tile.enc = do_row ? enc_row[tile.code] : enc_col[tile.code];
  }

  if (do_row) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float y[8];
      unpack8(v[i], y);
      uint32_t scode;
      float mult;
      if (TWO_D) {
        scode = tile.code;
        mult = tile.enc;
      } else {
        uint32_t m = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) m = max(m, absbits(y[e]));
        m = max(m, dpp_xor1(m));
        scode = nvfp4_scale_code(u2f(m), s_enc_row);
        mult = enc_row[scode];
      }
      float v8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v8[e] = y[e] * mult;
      const int64_t flat = (r0 + i) * C + c0;
      R16x8 rnd{};
      if (SR) rnd = sr_words((uint64_t)(flat >> 3), seed, offset, 0u);
      reinterpret_cast<uint32_t*>(codes_row)[flat >> 3] = encode8_fp4<SR>(v8, rnd);
      if ((cg & 1) == 0) row_sc[(rb * 16 + i) * 16 + (cg >> 1)] = (uint8_t)scode;
    }
  }

  if (do_col) {
    uint32_t sc_lo = 0, sc_hi = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float y[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) y[i] = tile_elem(v[i], j);
      uint32_t scode;
      float mult;
      if (TWO_D) {
        scode = tile.code;
        mult = tile.enc;
      } else if (RHT) {
        // The transform is taken without its 1/4.  The block amax of the
        // transformed values is then 1/4 of this one exactly (all values are
        // multiples of 2^-133), and y/4 * enc equals y * (enc/4), the same
        // single rounding, whenever enc/4 is exact (enc >= 2^-124); smaller
        // factors (amax near the top of the FP32 range) take the 1/4 on y.
        rht16_unscaled(y, signs);
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; i += 2) m = fmaxf(m, fmaxf(fabsf(y[i]), fabsf(y[i + 1])));
        scode = nvfp4_scale_code(m * 0.25f, s_enc_col);
        mult = enc_col[scode];
        if (mult < 0x1p-124f) {
#pragma unroll
          for (int i = 0; i < 16; ++i) y[i] = y[i] * 0.25f;
        } else {
          mult = mult * 0.25f;
        }
      } else {
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) m = max(m, absbits(y[i]));
        scode = nvfp4_scale_code(u2f(m), s_enc_col);
        mult = enc_col[scode];
      }
      const int64_t flat = (c0 + j) * R + r0;
      uint32_t w[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float v8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v8[e] = y[8 * h + e] * mult;
        R16x8 rnd{};
        if (SR) rnd = sr_words((uint64_t)(flat >> 3) + h, seed, offset, 1u);
        w[h] = encode8_fp4<SR>(v8, rnd);
      }
      const int cl = cg * 8 + j;
      *reinterpret_cast<uint2*>(col_codes + cl * 128 + ((rb ^ (cg & 15)) << 3)) = make_uint2(w[0], w[1]);
      if (j < 4) sc_lo |= scode << (8 * j);
      else sc_hi |= scode << (8 * (j - 4));
    }
    *reinterpret_cast<uint2*>(col_sc + rb * kQtTile + cg * 8) = make_uint2(sc_lo, sc_hi);
  }
  __syncthreads();

  if (do_col) {
    const int64_t ld = R / 2;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int q = t + kQtThreads * k;
      const int cl = q >> 3, ch = q & 7;
      const int f = (cl >> 3) & 15;
      uint4 val = *reinterpret_cast<const uint4*>(col_codes + cl * 128 + (((2 * ch) ^ (f & 14)) << 3));
      if (f & 1) val = make_uint4(val.z, val.w, val.x, val.y);
      *reinterpret_cast<uint4*>(codes_col + ((int64_t)tc * kQtTile + cl) * ld + (int64_t)tr * 128 + ch * 16) = val;
    }
    if (t < kQtTile) {
      uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int b = 0; b < 16; ++b) w[b >> 2] |= (uint32_t)col_sc[b * kQtTile + t] << (8 * (b & 3));
      *reinterpret_cast<uint4*>(scales_col + ((int64_t)tc * kQtTile + t) * (R / 16) + (int64_t)tr * 16) =
          make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
  if (do_row && t >= kQtThreads - kQtTile) {
    const int row = t - (kQtThreads - kQtTile);
    *reinterpret_cast<uint4*>(scales_row + ((int64_t)tr * kQtTile + row) * (C / 16) + (int64_t)tc * 16) =
        *reinterpret_cast<const uint4*>(row_sc + row * 16);
  }
}

// ---------------------------------------------------------------- per-tensor FP8, row + column
//
// The FP8 baseline's operands: code = E4M3(x * s_enc), s_enc = 448 / amax.
// The rule does not depend on the orientation, so the column output is the
// row codes transposed.

__device__ __forceinline__ float fp8_s_enc(float amax) {
  if (amax == 0.0f) return 1.0f;
  return fminf(448.0f / amax, kFltMax);
}

// 4 x 4 byte transpose: rows a, b, c, d (4 bytes each) -> columns 0..3.
__device__ __forceinline__ void transpose4x4(uint32_t a, uint32_t b, uint32_t c, uint32_t d,
                                             uint32_t (&o)[4]) {
  const uint32_t t0 = __builtin_amdgcn_perm(b, a, 0x05010400u);   // a0 b0 a1 b1
  const uint32_t t1 = __builtin_amdgcn_perm(b, a, 0x07030602u);   // a2 b2 a3 b3
  const uint32_t t2 = __builtin_amdgcn_perm(d, c, 0x05010400u);   // c0 d0 c1 d1
  const uint32_t t3 = __builtin_amdgcn_perm(d, c, 0x07030602u);   // c2 d2 c3 d3
  o[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);              // a0 b0 c0 d0
  o[1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);              // a1 b1 c1 d1
  o[2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
  o[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

// One 512-thread workgroup per 256 x 256 tile (R and C multiples of 256).
// Thread t owns columns 8 (t % 32) .. +8 of rows 16 (t / 32) .. +16.  Row
// codes go straight out (32 lanes write one 256-byte row segment).  Column
// codes are transposed in registers, staged in LDS (256 columns x 256 bytes,
// 16-byte unit u of column c at unit u ^ ((c / 8) % 16), so the eight lanes
// of a write phase hit distinct banks) and written as whole 256-byte
// segments of the [C, R] output.
__global__ __launch_bounds__(kQtThreads) void k_fp8_qt(const uint16_t* __restrict__ x, int64_t R,
                                                       int64_t C, int tiles_r, int tiles_c,
                                                       const float* __restrict__ amax,
                                                       uint8_t* __restrict__ codes_row,
                                                       uint8_t* __restrict__ codes_col) {
  __shared__ __attribute__((aligned(16))) uint8_t col_codes[kQtTile * kQtTile];
  int tr, tc;
  qt_tile_of_block(blockIdx.x, tiles_r, tiles_c, tr, tc);
  const int t = threadIdx.x, cg = t & 31, rb = t >> 5;
  const int64_t r0 = (int64_t)tr * kQtTile + rb * 16, c0 = (int64_t)tc * kQtTile + cg * 8;

  uint4 v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = *reinterpret_cast<const uint4*>(x + (r0 + i) * C + c0);
  const float s_enc = fp8_s_enc(*amax);

  uint2 code[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float y[8];
    unpack8(v[i], y);
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = y[e] * s_enc;
    code[i] = encode8_fp8(y);
    if (codes_row) *reinterpret_cast<uint2*>(codes_row + (r0 + i) * C + c0) = code[i];
  }
  if (!codes_col) return;

#pragma unroll
  for (int half = 0; half < 2; ++half) {           // columns 4 half .. 4 half + 3
    uint32_t col[4][4];                              // [column][row group of 4]
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint32_t o[4];
      const int i = 4 * g;
      if (half == 0) transpose4x4(code[i].x, code[i + 1].x, code[i + 2].x, code[i + 3].x, o);
      else transpose4x4(code[i].y, code[i + 1].y, code[i + 2].y, code[i + 3].y, o);
#pragma unroll
      for (int j = 0; j < 4; ++j) col[j][g] = o[j];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int cl = cg * 8 + 4 * half + j;
      *reinterpret_cast<uint4*>(col_codes + cl * kQtTile + ((rb ^ (cg & 15)) << 4)) =
          make_uint4(col[j][0], col[j][1], col[j][2], col[j][3]);
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int q = t + kQtThreads * k;
    const int cl = q >> 4, u = q & 15;
    const uint4 val = *reinterpret_cast<const uint4*>(col_codes + cl * kQtTile + ((u ^ ((cl >> 3) & 15)) << 4));
    *reinterpret_cast<uint4*>(codes_col + ((int64_t)tc * kQtTile + cl) * R + (int64_t)tr * kQtTile + u * 16) = val;
  }
}

// Any R, C multiples of 16: one 8-element row chunk per lane (grid-stride);
// column codes are stored byte by byte.
__global__ __launch_bounds__(256) void k_fp8_qt_flat(const uint4* __restrict__ x, int64_t R,
                                                     int64_t C, const float* __restrict__ amax,
                                                     uint8_t* __restrict__ codes_row,
                                                     uint8_t* __restrict__ codes_col) {
  const float s_enc = fp8_s_enc(*amax);
  const int64_t nchunk = R * C / 8;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < nchunk;
       q += (int64_t)gridDim.x * blockDim.x) {
    float y[8];
    unpack8(x[q], y);
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = y[e] * s_enc;
    const uint2 code = encode8_fp8(y);
    if (codes_row) reinterpret_cast<uint2*>(codes_row)[q] = code;
    if (codes_col) {
      const int64_t r = (q * 8) / C, c0 = (q * 8) % C;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        codes_col[(c0 + e) * R + r] = (uint8_t)((e < 4 ? code.x : code.y) >> (8 * (e & 3)));
    }
  }
}

// Row-blocks per lane: as many as keeps >= 4096 waves in flight (up to 16).
int pick_rbs(int64_t nrowblocks, int64_t waves_x) {
  int rbs = 16;
  while (rbs > 1 && ((nrowblocks + rbs - 1) / rbs) * waves_x < 4096) rbs >>= 1;
  return rbs;
}

int64_t flat_grid(int64_t nchunk) {
  const int64_t per_block = 256 * kUnroll;        // chunks per block per trip
  int64_t g = (nchunk + per_block - 1) / per_block;
  const int64_t cap = 256 * 32;                   // grid-stride beyond 32 blocks per CU
  return g < 1 ? 1 : (g > cap ? cap : g);
}

}  // namespace

// ---------------------------------------------------------------- launchers

hipError_t launch_zero_amax(float* a, float* b, hipStream_t s) {
  hipLaunchKernelGGL(k_zero_amax, dim3(1), dim3(64), 0, s, a, b);
  return hipGetLastError();
}

hipError_t launch_copy_amax(const float* src, float* dst, hipStream_t s) {
  hipLaunchKernelGGL(k_copy_amax, dim3(1), dim3(64), 0, s, src, dst);
  return hipGetLastError();
}

hipError_t launch_amax_flat(const void* x, int64_t nchunk, bool rht, uint32_t signs, float* a0,
                            float* a1, hipStream_t s) {
  const int64_t nitems = (nchunk + 511) / 512;
  int64_t g = (nitems + 3) / 4;
  g = g < 1 ? 1 : (g > kAmaxFlatBlocks ? kAmaxFlatBlocks : g);
  const dim3 grid((unsigned)g), block(256);
  const uint4* xp = static_cast<const uint4*>(x);
  if (rht)
    hipLaunchKernelGGL(k_amax_flat<true>, grid, block, 0, s, xp, nchunk, signs, a0, a1);
  else
    hipLaunchKernelGGL(k_amax_flat<false>, grid, block, 0, s, xp, nchunk, signs, a0, a1);
  return hipGetLastError();
}

hipError_t launch_amax_tile_rht(const void* x, int64_t R, int64_t C, uint32_t signs,
                                float* amax_row, float* amax_col, hipStream_t s) {
  if (C * 32 >= ((int64_t)1 << 31)) return hipErrorInvalidValue;   // 16 rows per buffer resource
  const int64_t nitems = ((C + 255) / 256) * (R / 16);
  int64_t g = (nitems + 3) / 4;
  g = g < 1 ? 1 : (g > kAmaxRhtBlocks ? kAmaxRhtBlocks : g);
  hipLaunchKernelGGL(k_amax_tile_rht, dim3((unsigned)g), dim3(256), 0, s,
                     static_cast<const uint16_t*>(x), R, C, signs, amax_row, amax_col);
  return hipGetLastError();
}

hipError_t launch_swiglu(const void* y, const void* dh, int64_t R, int64_t F, int amax_mode,
                         uint32_t signs, void* out, float* amax_row, float* amax_col, hipStream_t s) {
  if (F * 64 >= ((int64_t)1 << 31)) return hipErrorInvalidValue;   // 16 rows of Y per buffer resource
  const int64_t nitems = ((F + 255) / 256) * (R / 16);
  int64_t g = (nitems + 3) / 4;
  g = g < 1 ? 1 : (g > kSwigluBlocks ? kSwigluBlocks : g);
  const dim3 grid((unsigned)g), block(256);
  const uint16_t* yp = static_cast<const uint16_t*>(y);
  uint16_t* op = static_cast<uint16_t*>(out);
#define BSQ_SWIGLU(A)                                                                              \
  do {                                                                                             \
    if (dh)                                                                                        \
      hipLaunchKernelGGL(k_swiglu_bwd<A>, grid, block, 0, s, yp, static_cast<const uint16_t*>(dh), \
                         R, F, signs, op, amax_row, amax_col);                                     \
    else                                                                                           \
      hipLaunchKernelGGL(k_swiglu_fwd<A>, grid, block, 0, s, yp, R, F, signs, op, amax_row,        \
                         amax_col);                                                                \
  } while (0)
  if (amax_mode == 2) BSQ_SWIGLU(2);
  else if (amax_mode == 1) BSQ_SWIGLU(1);
  else BSQ_SWIGLU(0);
#undef BSQ_SWIGLU
  return hipGetLastError();
}

hipError_t launch_master_update(float* w, const void* g, int64_t n, float lr, void* wb, float* amax,
                                hipStream_t s) {
  const int64_t nchunk = n / 8;
  int64_t grid = (nchunk + 255) / 256;
  grid = grid < 1 ? 1 : (grid > kUpdateBlocks ? kUpdateBlocks : grid);
  const uint4* gp = static_cast<const uint4*>(g);
  uint4* wbp = static_cast<uint4*>(wb);
  if (amax)
    hipLaunchKernelGGL(k_master_update<true>, dim3((unsigned)grid), dim3(256), 0, s, w, gp, nchunk, lr,
                       wbp, amax);
  else
    hipLaunchKernelGGL(k_master_update<false>, dim3((unsigned)grid), dim3(256), 0, s, w, gp, nchunk, lr,
                       wbp, amax);
  return hipGetLastError();
}

hipError_t launch_quant_flat(Fmt fmt, bool sr, bool rht, const void* x, int64_t nchunk,
                             const float* amax, uint32_t signs, uint64_t seed, uint32_t offset,
                             uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const dim3 grid((unsigned)flat_grid(nchunk)), block(256);
  const uint4* xp = static_cast<const uint4*>(x);
#define BSQ_FLAT(F, S, H)                                                                  \
  hipLaunchKernelGGL((k_quant_flat<F, S, H>), grid, block, 0, s, xp, nchunk, amax, signs, \
                     seed, offset, codes, scales)
  if (fmt == kNVFP4) {
    if (sr) {
      if (rht) BSQ_FLAT(kNVFP4, true, true); else BSQ_FLAT(kNVFP4, true, false);
    } else {
      if (rht) BSQ_FLAT(kNVFP4, false, true); else BSQ_FLAT(kNVFP4, false, false);
    }
  } else if (fmt == kMXFP4) {
    if (sr) BSQ_FLAT(kMXFP4, true, false); else BSQ_FLAT(kMXFP4, false, false);
  } else {
    BSQ_FLAT(kMXFP8, false, false);
  }
#undef BSQ_FLAT
  return hipGetLastError();
}

hipError_t launch_fp8_qt(const void* x, int64_t R, int64_t C, const float* amax,
                         uint8_t* codes_row, uint8_t* codes_col, hipStream_t s) {
  const auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  if (R % kQtTile == 0 && C % kQtTile == 0 && R > 0 && C > 0 && al16(x) &&
      (!codes_row || al16(codes_row)) && (!codes_col || al16(codes_col)) &&
      (R / kQtTile) * (C / kQtTile) < (int64_t)1 << 31) {
    const int tiles_r = (int)(R / kQtTile), tiles_c = (int)(C / kQtTile);
    hipLaunchKernelGGL(k_fp8_qt, dim3((unsigned)(tiles_r * tiles_c)), dim3(kQtThreads), 0, s,
                       static_cast<const uint16_t*>(x), R, C, tiles_r, tiles_c, amax, codes_row,
                       codes_col);
    return hipGetLastError();
  }
  const int64_t nchunk = R * C / 8;
  int64_t g = (nchunk + 255) / 256;
  g = g < 1 ? 1 : (g > 256 * 32 ? 256 * 32 : g);
  hipLaunchKernelGGL(k_fp8_qt_flat, dim3((unsigned)g), dim3(256), 0, s,
                     static_cast<const uint4*>(x), R, C, amax, codes_row, codes_col);
  return hipGetLastError();
}

hipError_t launch_quant_tile(Fmt fmt, bool sr, bool rht_col, bool two_d, const void* x,
                             int64_t R, int64_t C, bool do_row, bool do_col,
                             const float* amax_row, const float* amax_col, uint32_t signs,
                             uint64_t seed, uint32_t offset, uint8_t* codes_row,
                             uint8_t* scales_row, uint8_t* codes_col, uint8_t* scales_col,
                             hipStream_t s) {
  const auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  if (fmt == kNVFP4 && R % kQtTile == 0 && C % kQtTile == 0 && R > 0 && C > 0 && al16(x) &&
      (!do_row || (al16(codes_row) && al16(scales_row))) &&
      (!do_col || (al16(codes_col) && al16(scales_col))) &&
      (R / kQtTile) * (C / kQtTile) < (int64_t)1 << 31) {
    const int tiles_r = (int)(R / kQtTile), tiles_c = (int)(C / kQtTile);
    const dim3 grid((unsigned)(tiles_r * tiles_c)), block(kQtThreads);
    const uint16_t* xp = static_cast<const uint16_t*>(x);
    const int dr = do_row ? 1 : 0, dc = do_col ? 1 : 0;
#define BSQ_QT(S, H, D)                                                                           \
  hipLaunchKernelGGL((k_qt_nvfp4<S, H, D>), grid, block, 0, s, xp, R, C, tiles_r, tiles_c, dr, dc, \
                     amax_row, amax_col, signs, seed, offset, codes_row, scales_row, codes_col,   \
                     scales_col)
    if (two_d) BSQ_QT(false, false, true);
    else if (sr) { if (rht_col) BSQ_QT(true, true, false); else BSQ_QT(true, false, false); }
    else { if (rht_col) BSQ_QT(false, true, false); else BSQ_QT(false, false, false); }
#undef BSQ_QT
    return hipGetLastError();
  }
  const int blk = fmt == kNVFP4 ? 16 : 32;
  const int64_t lanes = C / 8;
  const int gx = (int)((lanes + 63) / 64);
  const int64_t nrb = R / blk;
  const int rbs = pick_rbs(nrb, gx);
  const int64_t gy = (nrb + rbs - 1) / rbs;
  const dim3 grid((unsigned)(gx * gy)), block(64);
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const int dr = do_row ? 1 : 0, dc = do_col ? 1 : 0;
#define BSQ_TILE(F, S, H, D)                                                                  \
  hipLaunchKernelGGL((k_quant_tile<F, S, H, D>), grid, block, 0, s, xp, R, C, gx, rbs, dr, dc, \
                     amax_row, amax_col, signs, seed, offset, codes_row, scales_row, codes_col, \
                     scales_col)
  if (fmt == kNVFP4) {
    if (two_d) {
      BSQ_TILE(kNVFP4, false, false, true);
    } else if (sr) {
      if (rht_col) BSQ_TILE(kNVFP4, true, true, false); else BSQ_TILE(kNVFP4, true, false, false);
    } else {
      if (rht_col) BSQ_TILE(kNVFP4, false, true, false); else BSQ_TILE(kNVFP4, false, false, false);
    }
  } else if (fmt == kMXFP4) {
    if (sr) BSQ_TILE(kMXFP4, true, false, false); else BSQ_TILE(kMXFP4, false, false, false);
  } else {
    BSQ_TILE(kMXFP8, false, false, false);
  }
#undef BSQ_TILE
  return hipGetLastError();
}

}  // namespace bsq
