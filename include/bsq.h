/*
 * bsq.h -- block-scaled quantize + GEMM for MI355X (gfx950).  C ABI.
 *
 * What is computed (source pages):
 *  - NVFP4 pretraining post, section "NVFP4 pretraining recipe":
 *      ingredient 1  16-element micro-blocks (1x16) along the reduction dim;
 *      ingredient 2  E4M3 block scale factors under a per-tensor FP32 scale;
 *      ingredient 3  16-point Random Hadamard Transform on WGRAD inputs only;
 *      ingredient 4  16x16 2D weight scaling, so FPROP and the transposed
 *                    DGRAD see identical values;
 *      ingredient 5  round-to-nearest-even for weights/activations,
 *                    stochastic rounding for gradients;
 *    and the data-flow paragraph after Figure 1: the FPROP, DGRAD and WGRAD
 *    GEMMs consume NVFP4 operands and emit BF16.
 *  - HN page opcode84 (Triton on Blackwell quote, OCP MX spec link): MXFP8
 *    (E4M3 elements) and MXFP4 (E2M1 elements) with one E8M0 power-of-two
 *    scale per 32 elements, applied inside the matrix unit.
 *  - NVFP4 pretraining post, the paragraph after the example script (the FP8
 *    baseline run, quantization=te_fp8_delayedscaling) and section
 *    "Performance results" (Table 1, Figure 2: NVFP4 against that FP8
 *    baseline): the per-tensor FP8 format BSQ_FP8 below.
 *
 * Numerical definitions (bit-exact contract of the quantizers):
 *  - E2M1 magnitudes {0,0.5,1,1.5,2,3,4,6}, ties to the even code, saturate
 *    at 6; sign bit 0x8 kept (-0 -> 0x8).  Two codes per byte, the element
 *    with the even index in the low nibble.
 *  - E4M3 = OCP E4M3FN, subnormals kept, saturate at 448 (0x7E).
 *  - NVFP4 per-tensor scale: amax = max|x| (of the transformed values when the
 *    RHT applies); s_enc = 2688/amax (FP32; 1 if amax == 0; <= FLT_MAX);
 *    s_dec = 1/s_enc.  Block: sf = (a_b/6)*s_enc; S = E4M3(sf);
 *    enc = S ? min(s_enc/S, FLT_MAX) : 0; code = E2M1(x*enc).  FP32 IEEE
 *    RNE at every step, no fused multiply-add.
 *  - Per-tensor FP8 (BSQ_FP8): amax = max|x|; s_enc = 448/amax (FP32; 1 if
 *    amax == 0; <= FLT_MAX); s_dec = 1/s_enc; code = E4M3(x*s_enc), signed,
 *    RNE, saturating at 448.  No block scales; the column output is the same
 *    rule on x^T (the row codes transposed).  The delayed-scaling amax history
 *    of the baseline recipe spans training steps and is not modelled.
 *  - MX scale: e = floor(log2 a_b) - emax (emax 2 for E2M1, 8 for E4M3),
 *    -127 for an all-zero block, clamped to [-127,127], stored as e+127;
 *    element = E2M1/E4M3(x * 2^-e).
 *  - RHT: for each aligned 16-chunk y along the blocked dim: negate y_i where
 *    bit i of rht_signs is set, then butterflies h = 1,2,4,8
 *    (y_i, y_i+h) <- (y_i + y_i+h, y_i - y_i+h), then y *= 0.25 (FP32).
 *  - Stochastic rounding: element (r,c) of an output of shape [R',C'] in its
 *    own orientation has idx = r*C' + c; Philox4x32-10 (Salmon et al., SC'11)
 *    with key (seed lo, seed hi) and counter (lo(idx>>3), hi(idx>>3), offset,
 *    stream) gives 8 16-bit halves, the element takes half idx&7 (word
 *    (idx&7)>>1, low half first); stream 0 = rowwise, 1 = columnwise.  With
 *    lo <= |v| < hi the neighbouring E2M1 points, round up iff
 *    r16 < floor((|v|-lo)/(hi-lo) * 65536); |v| >= 6 -> 6.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers, row-major and contiguous, and
 *    must be 16-byte aligned.  `x` is BF16.  The caller allocates every
 *    buffer; the library never allocates, frees or retains device memory and
 *    keeps no state between calls.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream) and never synchronizes the host.
 *  - Argument errors are detected before anything is launched: the call
 *    returns BSQ_EINVAL / BSQ_EUNSUPPORTED and no output is touched.  A launch
 *    failure returns BSQ_EHIP.  No exception crosses the ABI.
 *  - Inputs must be finite; NaN/Inf inputs give unspecified codes but never a
 *    fault.
 *  - Sizes: rows, cols, M, N, K >= 0; a zero-size call returns BSQ_OK and
 *    launches nothing except that amax outputs are set to 0.  An element
 *    count above 2^48 (rows * cols, n, M * K, N * K or M * ldc) returns
 *    BSQ_EINVAL.
 */
#ifndef BSQ_H
#define BSQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BSQ_OK = 0,
  BSQ_EINVAL = 1,        /* null pointer, bad size, misalignment */
  BSQ_EUNSUPPORTED = 2,  /* combination the recipe does not define */
  BSQ_EHIP = 3           /* HIP launch error */
} bsq_status;

/* BSQ_FP8: per-tensor FP8, accepted by fp8_quantize_transpose (implied) and
 * bs_gemm only; the other quantizers return BSQ_EUNSUPPORTED for it. */
typedef enum { BSQ_NVFP4 = 0, BSQ_MXFP4 = 1, BSQ_MXFP8 = 2, BSQ_FP8 = 3 } bsq_format;
typedef enum { BSQ_RNE = 0, BSQ_SR = 1 } bsq_rounding;

/*
 * Rowwise NVFP4 of x[rows, cols] (BF16), blocks along cols.
 * Recipe ingredients 1, 2, 4, 5 (and 3 when rht != 0).
 *   block_rows : 1 (1x16 blocks) or 16 (16x16 tiles, rows % 16 == 0; the tile
 *                scale is written to each of its 16 rows).
 *   rnd        : BSQ_RNE or BSQ_SR (SR uses stream 0); SR with block_rows 16
 *                is BSQ_EUNSUPPORTED (it would break the transpose invariant).
 *   seed/offset: Philox key and counter word 2 for SR (ignored for RNE).
 *   rht        : nonzero = apply the 16-point RHT along cols first (amax is then
 *                taken over the transformed values); not with block_rows 16.
 *   amax_in    : NULL, or a device FP32 amax to use instead of computing it.
 *   codes      : out, uint8 [rows, cols/2], packed E2M1.
 *   scales     : out, uint8 [rows, cols/16], E4M3 block scales.
 *   amax_out   : out, device FP32 scalar: the amax used.  Required when
 *                amax_in is NULL (it is the reduction's accumulator); may be
 *                NULL otherwise.
 * Requires cols % 16 == 0.
 */
bsq_status nvfp4_quantize(const void* x, int64_t rows, int64_t cols, int block_rows,
                          bsq_rounding rnd, uint64_t seed, uint32_t offset,
                          int rht, uint16_t rht_signs, const float* amax_in,
                          uint8_t* codes, uint8_t* scales, float* amax_out,
                          void* stream);

/*
 * Rowwise MXFP4 (fmt BSQ_MXFP4, E2M1 elements) or MXFP8 (BSQ_MXFP8, E4M3
 * elements) of x[rows, cols] with one E8M0 scale per 32 elements along cols.
 * HN page opcode84 (MX formats; OCP MX spec).
 *   rnd    : BSQ_RNE, or BSQ_SR for MXFP4 only (stream 0).
 *   codes  : out, uint8 [rows, cols/2] (MXFP4) or [rows, cols] (MXFP8).
 *   scales : out, uint8 [rows, cols/32], E8M0.
 * Requires cols % 32 == 0.
 */
bsq_status mx_quantize(const void* x, int64_t rows, int64_t cols, bsq_format fmt,
                       bsq_rounding rnd, uint64_t seed, uint32_t offset,
                       uint8_t* codes, uint8_t* scales, void* stream);

/*
 * Both orientations from one read of x[rows, cols]:
 *   row = quantize(x)    -> codes_row [rows, cols/2 or cols], scales_row [rows, cols/B]
 *   col = quantize(x^T)  -> codes_col [cols, rows/2 or rows], scales_col [cols, rows/B]
 * B = 16 (NVFP4) or 32 (MX).  Recipe: ingredient 4 (the transposed DGRAD
 * operand of 2D-scaled weights), ingredient 3 (WGRAD operands are quantized
 * along tokens, with the RHT), data-flow paragraph.
 *   fmt        : BSQ_NVFP4, BSQ_MXFP4 or BSQ_MXFP8.
 *   block_rows : 1, or 16 for NVFP4 2D tiles (then row and col codes are the
 *                same values transposed and both scale arrays hold the same
 *                tile scales).
 *   rnd        : RNE or SR (SR: rowwise stream 0, columnwise stream 1); not SR
 *                with 2D tiles or MXFP8.
 *   rht_col    : nonzero = RHT along rows (the blocked dim of x^T) for the col
 *                output only; NVFP4 1x16 only; with the col output it needs
 *                cols < 2^26 (BSQ_EINVAL otherwise).
 *   amax_row / amax_col : out, device FP32 (NVFP4 only; ignored for MX).
 *                amax_row = max|x|; amax_col = max|RHT(x^T)| with rht_col,
 *                else equal to amax_row.
 * Either triple (codes_row, scales_row, amax_row) or (codes_col, scales_col,
 * amax_col) may be all-NULL to skip that orientation (not both).
 * Requires rows % 16 == 0 and cols % 16 == 0 (NVFP4) or rows % 32 == 0 and
 * cols % 32 == 0 (MX).
 */
bsq_status quantize_transpose(const void* x, int64_t rows, int64_t cols, bsq_format fmt,
                              int block_rows, bsq_rounding rnd, uint64_t seed, uint32_t offset,
                              int rht_col, uint16_t rht_signs,
                              uint8_t* codes_row, uint8_t* scales_row, float* amax_row,
                              uint8_t* codes_col, uint8_t* scales_col, float* amax_col,
                              void* stream);

/*
 * NVFP4 row and column outputs of x[rows, cols] under per-tensor amaxes the
 * caller already holds, typically from the producer of x (swiglu_amax,
 * swiglu_backward_amax below): the encode pass of quantize_transpose without
 * its amax pass.  Recipe ingredients 1-5 as for quantize_transpose with
 * fmt = BSQ_NVFP4; given the amaxes quantize_transpose would compute, the
 * codes and scales are the same bytes.
 *   block_rows, rnd, seed, offset, rht_col, rht_signs : as quantize_transpose.
 *   amax_row : in, device FP32 max|x|; required with the row outputs.
 *   amax_col : in, device FP32 amax of the col side (max|RHT(x^T)| with
 *              rht_col, else max|x|); required with the col outputs.  With
 *              block_rows 16 and both orientations it must be the same
 *              pointer as amax_row (one amax encodes both sides of a 16x16
 *              tile); BSQ_EINVAL otherwise.
 *   codes_row, scales_row / codes_col, scales_col : out, as quantize_transpose;
 *              either pair may be NULL to skip that orientation (not both).
 * Requires rows % 16 == 0 and cols % 16 == 0.
 */
bsq_status quantize_transpose_amax(const void* x, int64_t rows, int64_t cols, int block_rows,
                                   bsq_rounding rnd, uint64_t seed, uint32_t offset, int rht_col,
                                   uint16_t rht_signs, const float* amax_row, const float* amax_col,
                                   uint8_t* codes_row, uint8_t* scales_row, uint8_t* codes_col,
                                   uint8_t* scales_col, void* stream);

/*
 * SwiGLU forward of the MLP whose GEMMs the NVFP4 post measures (section
 * "Performance results": Llama 3 8B and Llama 3.1 405B, whose MLP is the
 * gate/up GEMM, SwiGLU, then the down GEMM), producing the BF16 input of the
 * down projection together with the amaxes its NVFP4 quantizer needs (the
 * data-flow paragraph after Figure 1: activations enter the next GEMM in
 * NVFP4).  The pages give no SwiGLU formula; the reading used:
 *   y_gu : in, BF16 [rows, 2f] = [G | U] (gate = first f columns).
 *   h    : out, BF16 [rows, f], h = BF16_RNE(silu(G) * U), silu(g) =
 *          g / (1 + exp(-g)); computed in FP32 (v_exp / v_rcp), so an element
 *          may differ from the exactly rounded value by one BF16 ulp.
 *   amax_row : out, device FP32 max|h| (or NULL).
 *   amax_col : out, device FP32: with rht_col, max|RHT(h^T)| (16-row chunks,
 *              rht_signs, the quantize_transpose rule); else max|h| (or NULL).
 *              Both amaxes equal what quantize_transpose computes on h.
 * With both amax pointers NULL only h is written.  h must not overlap y_gu.
 * Requires rows % 16 == 0, f % 16 == 0 and f < 2^25.
 */
bsq_status swiglu_amax(const void* y_gu, int64_t rows, int64_t f, int rht_col, uint16_t rht_signs,
                       void* h, float* amax_row, float* amax_col, void* stream);

/*
 * SwiGLU backward (the chain rule of h = silu(G) * U) producing the BF16
 * gradient of the gate/up GEMM output with the amaxes of its NVFP4 quantizer
 * (rowwise SR for DGRAD, columnwise SR + RHT for WGRAD: recipe ingredients 3
 * and 5).
 *   y_gu   : in, BF16 [rows, 2f] = [G | U], the forward's input.
 *   d_h    : in, BF16 [rows, f], gradient of h.
 *   d_y_gu : out, BF16 [rows, 2f] = [dG | dU], dU = BF16_RNE(dH * silu(G)),
 *            dG = BF16_RNE(dH * U * silu'(G)), silu'(g) = sigma(g) *
 *            (1 + g * (1 - sigma(g))); FP32 arithmetic, one BF16 ulp as for
 *            swiglu_amax.
 *   amax_row, amax_col : out, as for swiglu_amax, over d_y_gu.
 * d_y_gu must not overlap y_gu or d_h.  Requires rows % 16 == 0, f % 16 == 0
 * and f < 2^25.
 */
bsq_status swiglu_backward_amax(const void* y_gu, const void* d_h, int64_t rows, int64_t f,
                                int rht_col, uint16_t rht_signs, void* d_y_gu, float* amax_row,
                                float* amax_col, void* stream);

/*
 * FP32 master-weight update of the optimizer step: the data-flow paragraph
 * after Figure 1 of the NVFP4 post folds the BF16 GEMM outputs (here the
 * WGRAD output dW) into an FP32 master weight; the pages name no optimizer,
 * so the plain fold is used.  For each of the n elements:
 *   w32[i]    <- FP32(w32[i] - FP32(lr * grad[i]))   (two RNE roundings, no FMA)
 *   w_bf16[i] <- BF16_RNE(w32[i])                     (the copy the next step quantizes)
 *   amax      <- max |w_bf16|                         (device FP32, or NULL)
 * The amax is the per-tensor amax of the next 16x16 weight quantization
 * (quantize_transpose_amax with block_rows 16, as amax_row and amax_col).
 *   w32    : in/out, FP32 [n].       grad : in, BF16 [n].
 *   w_bf16 : out, BF16 [n].  The three arrays must not overlap.
 * Requires n % 8 == 0.
 */
bsq_status master_weight_update(float* w32, const void* grad, int64_t n, float lr, void* w_bf16,
                                float* amax, void* stream);

/*
 * Per-tensor FP8 (E4M3) of x[rows, cols] (BF16) in both orientations from
 * one amax pass and one encode pass: the FP8 baseline's operands for FPROP
 * (rowwise), DGRAD (W columnwise) and WGRAD (dY and X columnwise).
 *   codes_row : out, uint8 [rows, cols], E4M3 codes of x (or NULL).
 *   codes_col : out, uint8 [cols, rows], E4M3 codes of x^T, i.e. codes_row
 *               transposed (or NULL; not both NULL).
 *   amax      : out, device FP32 scalar max|x| (the reduction's accumulator;
 *               required).  The GEMM derives s_dec from it.
 * Requires rows % 16 == 0 and cols % 16 == 0.
 */
bsq_status fp8_quantize_transpose(const void* x, int64_t rows, int64_t cols, uint8_t* codes_row,
                                  uint8_t* codes_col, float* amax, void* stream);

/*
 * C[M, N] (BF16, row-major, row stride ldc >= N elements) =
 *     alpha * sum_k deq(A)[m, k] * deq(B)[n, k]
 * with A [M, K] and B [N, K] both K-major (quantized along K), FP32
 * accumulation and one BF16 round-to-nearest-even at the end.  Data-flow
 * paragraph: FPROP (A = X rowwise, B = W rowwise 2D), DGRAD (A = dY rowwise,
 * B = W columnwise 2D), WGRAD (A = dY columnwise, B = X columnwise, K = tokens).
 *   NVFP4: codes [M, K/2] + E4M3 scales [M, K/16] per operand and a device
 *          FP32 amax per operand; alpha = s_dec(a_amax) * s_dec(b_amax).
 *          Requires K % 16 == 0.
 *   MXFP4: codes [M, K/2], MXFP8: codes [M, K]; E8M0 scales [M, K/32];
 *          a_amax and b_amax are ignored (may be NULL); alpha = 1.
 *          Requires K % 32 == 0.
 *   FP8:   per-tensor E4M3 codes [M, K] (fp8_quantize_transpose); a_scales
 *          and b_scales are ignored (may be NULL); device FP32 a_amax and
 *          b_amax required; alpha = s_dec(a_amax) * s_dec(b_amax) with
 *          s_dec = 1/(448/amax).  Requires K % 32 == 0.
 * M and N may be any value >= 0.  C must not alias any input.
 * Workspace (NVFP4 only): when the 256 x 256 output tiles fill at least one
 * wave of the device's compute units and leave a last wave of at most half
 * of them (K % 512 == 0, K >= 4096), each tile of that last wave is computed
 * as two FP32 partial sums over the two halves of K, added in a second
 * kernel (the same order for every element: repeated calls give identical
 * bits; the sum differs from a one-pass accumulation only in FP32 rounding).
 * Their 512 KiB per tile come from the stream-ordered allocator
 * (hipMallocAsync / hipFreeAsync on `stream`); BSQ_EHIP if that fails.
 */
bsq_status bs_gemm(bsq_format fmt, int64_t M, int64_t N, int64_t K,
                   const uint8_t* a_codes, const uint8_t* a_scales, const float* a_amax,
                   const uint8_t* b_codes, const uint8_t* b_scales, const float* b_amax,
                   void* c, int64_t ldc, void* stream);

/*
 * bs_gemm for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, checks and results (bit for bit) as bs_gemm; the NVFP4
 * split-last-wave workspace is the library's static per-device array of
 * 64 MiB (held by each device the library runs on until the process ends)
 * instead of the stream-ordered allocator, and no call allocates.  The
 * first call on a device looks up that array's address (make it outside
 * graph capture).  Returns BSQ_EUNSUPPORTED if the split would need more
 * than 64 MiB (more than 256 compute units).  Calls that overlap on one
 * device (other streams, other host threads) share the array and race.
 */
bsq_status bs_gemm_noalloc(bsq_format fmt, int64_t M, int64_t N, int64_t K,
                           const uint8_t* a_codes, const uint8_t* a_scales, const float* a_amax,
                           const uint8_t* b_codes, const uint8_t* b_scales, const float* b_amax,
                           void* c, int64_t ldc, void* stream);

/*
 * FP16 expansion of an NVFP4 operand (recipe ingredients 1-2: E2M1 codes
 * under E4M3 block scales), without its per-tensor scale:
 *   out[r, k] = v * S * 2^-7   (FP16, exact: v * S has at most 6 significant
 *                               bits and lies in [2^-10, 2688])
 * with v the E2M1 value of element (r, k) and S its block's E4M3 scale.
 *   codes  : in, uint8 [rows, cols/2] (8-byte aligned); scales : in, uint8 [rows, cols/16].
 *   out    : out, FP16 [rows, cols].
 * Requires cols % 16 == 0.  This is the B operand of bs_gemm_nvfp4_bx.
 */
bsq_status nvfp4_expand(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                        void* out, void* stream);

/*
 * The NVFP4 GEMM of bs_gemm (data-flow paragraph after Figure 1: FPROP,
 * DGRAD, WGRAD consume NVFP4 operands, emit BF16) with B handed over as its
 * FP16 expansion (nvfp4_expand of B's codes and scales): the kernel expands
 * only A.  The result is bit-identical to bs_gemm(BSQ_NVFP4, ...) on the
 * same operands whenever bs_gemm does not split its last wave over K (see
 * bs_gemm's workspace note).  For operands used by several GEMMs or much smaller than
 * the other operand (weights, the smaller WGRAD input), expanding once and
 * streaming FP16 costs less than expanding inside every output tile.
 *   a_codes [M, K/2], a_scales [M, K/16], a_amax : the NVFP4 A operand.
 *   b_x    : FP16 [N, K], nvfp4_expand of B;  b_amax : B's per-tensor amax.
 *   c      : BF16 [M, N], row stride ldc; alpha = s_dec(a_amax) * s_dec(b_amax).
 * BSQ_EUNSUPPORTED unless K % 128 == 0, K > 0, a_codes and b_x are 16-byte
 * aligned, a_scales 4-byte aligned, M * K / 2 < 2^32 and N * K * 2 < 2^32
 * (bs_gemm covers every other shape).
 */
bsq_status bs_gemm_nvfp4_bx(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                            const uint8_t* a_scales, const float* a_amax, const void* b_x,
                            const float* b_amax, void* c, int64_t ldc, void* stream);

/* Static, human-readable name of a status code; host-side, thread-safe. */
const char* bsq_status_string(bsq_status status);

#ifdef __cplusplus
}
#endif

#endif /* BSQ_H */
