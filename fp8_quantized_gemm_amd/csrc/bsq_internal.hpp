// Internal launch interface between the C-ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsq {

enum Fmt { kNVFP4 = 0, kMXFP4 = 1, kMXFP8 = 2, kFP8 = 3 };   // kFP8: per-tensor E4M3

// One-byte (E4M3) elements: MXFP8 and per-tensor FP8.
constexpr bool fp8_elems(int f) { return f == kMXFP8 || f == kFP8; }

// Raises the dynamic-LDS limit of kernel `fn` to `bytes` on the current
// device, once per (device, kernel): later calls return the first call's
// result.  Thread-safe (several host threads may launch at once).
hipError_t set_lds_limit(const void* fn, int bytes);

// Sets *a = 0 and *b = 0 (either may be null).
hipError_t launch_zero_amax(float* a, float* b, hipStream_t s);
// *dst = *src.
hipError_t launch_copy_amax(const float* src, float* dst, hipStream_t s);

// amax over a contiguous BF16 tensor of nchunk 8-element chunks; with rht the
// amax is over the 16-point RHT of each aligned 16-chunk.  Atomically maxes
// into a0 and (if non-null) a1, which must have been zeroed.
hipError_t launch_amax_flat(const void* x, int64_t nchunk, bool rht, uint32_t signs,
                            float* a0, float* a1, hipStream_t s);

// amax of x (into amax_row, may be null) and of the RHT of x^T along rows
// (into amax_col) for x [R, C].
hipError_t launch_amax_tile_rht(const void* x, int64_t R, int64_t C, uint32_t signs,
                                float* amax_row, float* amax_col, hipStream_t s);

// SwiGLU of Y = [G | U] [R, 2F] (R % 16 == 0, F % 4 == 0): with dh null, the
// forward H = silu(G) * U into out [R, F]; else the backward [dG | dU] of dh
// [R, F] into out [R, 2F].  amax_mode 0: no amax; 1: max |out| into both amax
// outputs (either may be null); 2: max |out| into amax_row and the column RHT
// amax (16-row chunks) into amax_col.  Amax outputs must have been zeroed.
hipError_t launch_swiglu(const void* y, const void* dh, int64_t R, int64_t F, int amax_mode,
                         uint32_t signs, void* out, float* amax_row, float* amax_col, hipStream_t s);

// FP32 master-weight update of n elements (n % 8 == 0): w <- w - lr * g
// (BF16 g), wb = BF16 RNE of the new w, and max |wb| into amax (zeroed
// before; may be null).
hipError_t launch_master_update(float* w, const void* g, int64_t n, float lr, void* wb, float* amax,
                                hipStream_t s);

// Rowwise quantization over a contiguous tensor of nchunk 8-element chunks
// (NVFP4 1x16 or MX 1x32 blocks; rows are implied since cols % block == 0).
hipError_t launch_quant_flat(Fmt fmt, bool sr, bool rht, const void* x, int64_t nchunk,
                             const float* amax, uint32_t signs, uint64_t seed, uint32_t offset,
                             uint8_t* codes, uint8_t* scales, hipStream_t s);

// Row and/or column quantization of x [R, C] from one read.
hipError_t launch_quant_tile(Fmt fmt, bool sr, bool rht_col, bool two_d, const void* x,
                             int64_t R, int64_t C, bool do_row, bool do_col,
                             const float* amax_row, const float* amax_col, uint32_t signs,
                             uint64_t seed, uint32_t offset, uint8_t* codes_row,
                             uint8_t* scales_row, uint8_t* codes_col, uint8_t* scales_col,
                             hipStream_t s);

// Per-tensor FP8 codes of x [R, C] (codes_row [R, C]) and of x^T (codes_col
// [C, R]), either may be null, under the already reduced *amax.
hipError_t launch_fp8_qt(const void* x, int64_t R, int64_t C, const float* amax,
                         uint8_t* codes_row, uint8_t* codes_col, hipStream_t s);

// Number of compute units of the current device (cached per device).
int device_cus();

// NVFP4 GEMM (exact FP16 dequant + FP16 MFMA).  scratch: null = workspace of
// the split last wave (see gemm_nvfp4_rx_split) from the stream-ordered
// allocator; otherwise a device buffer of scratch_bytes used for it
// (hipErrorInvalidValue when too small).
hipError_t launch_gemm_nvfp4(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                             const float* aa, const uint8_t* bc, const uint8_t* bs,
                             const float* ba, void* c, int64_t ldc, void* scratch,
                             size_t scratch_bytes, hipStream_t s);
// The library's static workspace for the NVFP4 GEMM on the current device
// (address looked up once per device) and its size.
hipError_t gemm_nvfp4_static_scratch(void** ptr, size_t* bytes);
// Workspace bytes the NVFP4 GEMM of these operands needs on the current device.
size_t gemm_nvfp4_scratch_bytes(int64_t M, int64_t N, int64_t K, const uint8_t* ac,
                                const uint8_t* as, const uint8_t* bc, const uint8_t* bs);

// The register-expansion NVFP4 GEMM (four waves, codes expanded in registers):
// whether it takes these operands (K % 256 == 0, codes 16-byte and scales
// 4-byte aligned, each operand below 4 GiB), and its launch.
bool gemm_nvfp4_rx_fits(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                        const uint8_t* bc, const uint8_t* bs);
// Split last wave: when the tiles fill at least one wave of `cus` workgroups
// and leave a last wave of at most cus / 2 tiles (K % 512 == 0, K >= 4096),
// the number of those tiles; each runs as two workgroups over the two K
// halves, which write FP32 partials (kRxSplitTileBytes per tile) that a
// second kernel adds, scales and rounds.  0 = no split.
int gemm_nvfp4_rx_split(int64_t M, int64_t N, int64_t K, int cus);
constexpr size_t kRxSplitTileBytes = (size_t)2 * 256 * 256 * 4;
// tail: gemm_nvfp4_rx_split's count (or 0); part: tail * kRxSplitTileBytes
// bytes of device memory when tail > 0.
hipError_t launch_gemm_nvfp4_rx(int64_t M, int64_t N, int64_t K, const uint8_t* ac,
                                const uint8_t* as, const float* aa, const uint8_t* bc,
                                const uint8_t* bs, const float* ba, void* c, int64_t ldc,
                                int tail, void* part, hipStream_t s);

// NVFP4 GEMM with B pre-expanded to FP16 (bx [N, K] = v * S * 2^-7, from
// launch_nvfp4_expand).  hipErrorNotSupported unless K % 128 == 0, the
// operands are 16-byte aligned (scales 4) and M * K / 2, N * K * 2 < 2^32.
hipError_t launch_gemm_nvfp4_bx(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                                const float* aa, const void* bx, const float* ba, void* c,
                                int64_t ldc, hipStream_t s);
// FP16 expansion out [R, K] of NVFP4 codes [R, K/2] and scales [R, K/16].
hipError_t launch_nvfp4_expand(const uint8_t* codes, const uint8_t* scales, int64_t R, int64_t K,
                               void* out, hipStream_t s);

// The four-wave MX / per-tensor FP8 GEMM (FMT kMXFP4, kMXFP8, kFP8): whether it
// takes these operands (K % 512 == 0, codes and scales 16-byte aligned, 32-bit
// offsets suffice), and its launch.
template <int FMT>
bool gemm_mx_rx_fits(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                     const uint8_t* bc, const uint8_t* bs);
template <int FMT>
hipError_t launch_gemm_mx_rx(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                             const float* aa, const uint8_t* bc, const uint8_t* bs, const float* ba,
                             void* c, int64_t ldc, hipStream_t s);

// C[M, N] = alpha * A . B^T, block-scaled operands, BF16 out.  scratch as
// for launch_gemm_nvfp4 (only NVFP4 uses it).
hipError_t launch_gemm(Fmt fmt, int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                       const uint8_t* a_scales, const float* a_amax, const uint8_t* b_codes,
                       const uint8_t* b_scales, const float* b_amax, void* c, int64_t ldc,
                       void* scratch, size_t scratch_bytes, hipStream_t s);

}  // namespace bsq
