// C-ABI entry points of libbsq: argument validation and kernel dispatch.
// The contract of every function is documented in include/bsq.h.
#include "bsq.h"

#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <utility>

#include "bsq_internal.hpp"

namespace bsq {

hipError_t set_lds_limit(const void* fn, int bytes) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, hipError_t> done;   // (device, kernel) -> result
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(dev, fn);
  const auto it = done.find(key);
  if (it != done.end()) return it->second;
  const hipError_t r = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  done.emplace(key, r);
  return r;
}

int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static int cus[kMaxDevices] = {};   // device -> compute units (0: not looked up yet)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (cus[dev] == 0 &&
      hipDeviceGetAttribute(&cus[dev], hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus[dev] = 0;
  return cus[dev];
}

}  // namespace bsq

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned16_or_null(const void* p) { return p == nullptr || aligned16(p); }

// Device pointers handed to us must at least be 4-byte aligned for scalars.
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

bsq_status hip_status(hipError_t e) { return e == hipSuccess ? BSQ_OK : BSQ_EHIP; }

// a * b would exceed 2^48 (no device holds that many elements; the bound also
// keeps every byte offset the kernels form far inside int64).  a, b >= 0.
bool too_many(int64_t a, int64_t b) { return a > 0 && b > (((int64_t)1 << 48) / a); }

// [a, a + na) and [b, b + nb) share a byte.
bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + (uintptr_t)nb && pb < pa + (uintptr_t)na;
}

// Checks and dispatch of bs_gemm (static_scratch false: the NVFP4 split
// workspace from the stream-ordered allocator) and bs_gemm_noalloc (true:
// the library's static per-device workspace, nothing allocated).
bsq_status gemm_common(bsq_format fmt, int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                       const uint8_t* a_scales, const float* a_amax, const uint8_t* b_codes,
                       const uint8_t* b_scales, const float* b_amax, void* c, int64_t ldc,
                       void* stream, bool static_scratch) {
  if (fmt != BSQ_NVFP4 && fmt != BSQ_MXFP4 && fmt != BSQ_MXFP8 && fmt != BSQ_FP8) return BSQ_EINVAL;
  const bool per_tensor = fmt == BSQ_NVFP4 || fmt == BSQ_FP8;   // alpha from the two amaxes
  if (M < 0 || N < 0 || K < 0) return BSQ_EINVAL;
  if (K % (fmt == BSQ_NVFP4 ? 16 : 32) != 0) return BSQ_EINVAL;
  if (ldc < N || ldc < 0) return BSQ_EINVAL;
  if (too_many(M, K) || too_many(N, K) || too_many(M, ldc)) return BSQ_EINVAL;
  if (M > (int64_t)256 * 0x7FFFFF || N > (int64_t)256 * 0x7FFFFF) return BSQ_EINVAL;
  if (M == 0 || N == 0) return BSQ_OK;
  if (!c || ((reinterpret_cast<uintptr_t>(c) & 1u) != 0)) return BSQ_EINVAL;
  if (K > 0) {
    if (!a_codes || !b_codes) return BSQ_EINVAL;
    if (fmt != BSQ_FP8 && (!a_scales || !b_scales)) return BSQ_EINVAL;
  }
  if (per_tensor && (!a_amax || !b_amax)) return BSQ_EINVAL;
  const bsq::Fmt f = fmt == BSQ_NVFP4 ? bsq::kNVFP4
                     : fmt == BSQ_MXFP4 ? bsq::kMXFP4
                     : fmt == BSQ_MXFP8 ? bsq::kMXFP8 : bsq::kFP8;
  void* scratch = nullptr;
  size_t scratch_bytes = 0;
  if (static_scratch && fmt == BSQ_NVFP4) {
    if (bsq::gemm_nvfp4_static_scratch(&scratch, &scratch_bytes) != hipSuccess) return BSQ_EHIP;
    if (bsq::gemm_nvfp4_scratch_bytes(M, N, K, a_codes, a_scales, b_codes, b_scales) > scratch_bytes)
      return BSQ_EUNSUPPORTED;
  }
  return hip_status(bsq::launch_gemm(f, M, N, K, a_codes, a_scales, a_amax, b_codes, b_scales,
                                     b_amax, c, ldc, scratch, scratch_bytes,
                                     static_cast<hipStream_t>(stream)));
}

// Shared checks and dispatch of the SwiGLU forward (dh null) and backward.
bsq_status swiglu_common(const void* y, const void* dh, int64_t rows, int64_t f, int rht_col,
                         uint16_t signs, void* out, float* amax_row, float* amax_col, void* stream) {
  if (rows < 0 || f < 0 || rows % 16 != 0 || f % 16 != 0) return BSQ_EINVAL;
  if (too_many(rows, 2 * f)) return BSQ_EINVAL;
  if (!aligned4(amax_row) || !aligned4(amax_col)) return BSQ_EINVAL;
  if (f >= ((int64_t)1 << 25)) return BSQ_EINVAL;    // 16 rows of y per buffer resource
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool amax = amax_row || amax_col;
  if (rows * f == 0) return amax ? hip_status(bsq::launch_zero_amax(amax_row, amax_col, s)) : BSQ_OK;
  const bool bwd = dh != nullptr;
  if (!y || !out || !aligned16(y) || !aligned16(out) || !aligned16_or_null(dh)) return BSQ_EINVAL;
  const int64_t ybytes = rows * f * 4, obytes = rows * f * (bwd ? 4 : 2);
  if (overlap(out, obytes, y, ybytes) || (bwd && overlap(out, obytes, dh, rows * f * 2)))
    return BSQ_EINVAL;
  if (amax) {
    const hipError_t e = bsq::launch_zero_amax(amax_row, amax_col, s);
    if (e != hipSuccess) return BSQ_EHIP;
  }
  return hip_status(bsq::launch_swiglu(y, dh, rows, f, amax ? (rht_col ? 2 : 1) : 0, signs, out,
                                       amax_row, amax_col, s));
}

}  // namespace

extern "C" {

const char* bsq_status_string(bsq_status status) {
  switch (status) {
    case BSQ_OK: return "BSQ_OK";
    case BSQ_EINVAL: return "BSQ_EINVAL: invalid argument (null pointer, size or alignment)";
    case BSQ_EUNSUPPORTED: return "BSQ_EUNSUPPORTED: combination not defined by the recipe";
    case BSQ_EHIP: return "BSQ_EHIP: HIP launch error";
    default: return "BSQ_UNKNOWN";
  }
}

bsq_status nvfp4_quantize(const void* x, int64_t rows, int64_t cols, int block_rows,
                          bsq_rounding rnd, uint64_t seed, uint32_t offset, int rht,
                          uint16_t rht_signs, const float* amax_in, uint8_t* codes,
                          uint8_t* scales, float* amax_out, void* stream) {
  if (rows < 0 || cols < 0 || cols % 16 != 0 || too_many(rows, cols)) return BSQ_EINVAL;
  if (block_rows != 1 && block_rows != 16) return BSQ_EINVAL;
  if (rnd != BSQ_RNE && rnd != BSQ_SR) return BSQ_EINVAL;
  if (block_rows == 16 && rows % 16 != 0) return BSQ_EINVAL;
  if (amax_in == nullptr && amax_out == nullptr) return BSQ_EINVAL;
  if (!aligned4(amax_in) || !aligned4(amax_out)) return BSQ_EINVAL;
  if (block_rows == 16 && (rnd == BSQ_SR || rht)) return BSQ_EUNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t n = rows * cols;
  if (n == 0) {
    if (amax_out) return hip_status(bsq::launch_zero_amax(amax_out, nullptr, s));
    return BSQ_OK;
  }
  if (!x || !codes || !scales) return BSQ_EINVAL;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return BSQ_EINVAL;

  const float* amax = amax_in;
  hipError_t e;
  if (amax_in == nullptr) {
    e = bsq::launch_zero_amax(amax_out, nullptr, s);
    if (e != hipSuccess) return BSQ_EHIP;
    e = bsq::launch_amax_flat(x, n / 8, rht != 0, rht_signs, amax_out, nullptr, s);
    if (e != hipSuccess) return BSQ_EHIP;
    amax = amax_out;
  } else if (amax_out != nullptr && amax_out != amax_in) {
    e = bsq::launch_copy_amax(amax_in, amax_out, s);
    if (e != hipSuccess) return BSQ_EHIP;
  }
  if (block_rows == 1)
    e = bsq::launch_quant_flat(bsq::kNVFP4, rnd == BSQ_SR, rht != 0, x, n / 8, amax, rht_signs,
                               seed, offset, codes, scales, s);
  else
    e = bsq::launch_quant_tile(bsq::kNVFP4, false, false, true, x, rows, cols, true, false, amax,
                               amax, 0, seed, offset, codes, scales, nullptr, nullptr, s);
  return hip_status(e);
}

bsq_status mx_quantize(const void* x, int64_t rows, int64_t cols, bsq_format fmt,
                       bsq_rounding rnd, uint64_t seed, uint32_t offset, uint8_t* codes,
                       uint8_t* scales, void* stream) {
  if (rows < 0 || cols < 0 || cols % 32 != 0 || too_many(rows, cols)) return BSQ_EINVAL;
  if (fmt != BSQ_MXFP4 && fmt != BSQ_MXFP8)
    return fmt == BSQ_NVFP4 || fmt == BSQ_FP8 ? BSQ_EUNSUPPORTED : BSQ_EINVAL;
  if (rnd != BSQ_RNE && rnd != BSQ_SR) return BSQ_EINVAL;
  if (fmt == BSQ_MXFP8 && rnd == BSQ_SR) return BSQ_EUNSUPPORTED;
  const int64_t n = rows * cols;
  if (n == 0) return BSQ_OK;
  if (!x || !codes || !scales) return BSQ_EINVAL;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return BSQ_EINVAL;
  return hip_status(bsq::launch_quant_flat(fmt == BSQ_MXFP4 ? bsq::kMXFP4 : bsq::kMXFP8,
                                           rnd == BSQ_SR, false, x, n / 8, nullptr, 0, seed,
                                           offset, codes, scales,
                                           static_cast<hipStream_t>(stream)));
}

bsq_status quantize_transpose(const void* x, int64_t rows, int64_t cols, bsq_format fmt,
                              int block_rows, bsq_rounding rnd, uint64_t seed, uint32_t offset,
                              int rht_col, uint16_t rht_signs, uint8_t* codes_row,
                              uint8_t* scales_row, float* amax_row, uint8_t* codes_col,
                              uint8_t* scales_col, float* amax_col, void* stream) {
  if (fmt == BSQ_FP8) return BSQ_EUNSUPPORTED;      // fp8_quantize_transpose
  if (fmt != BSQ_NVFP4 && fmt != BSQ_MXFP4 && fmt != BSQ_MXFP8) return BSQ_EINVAL;
  const bool nv = fmt == BSQ_NVFP4;
  const int blk = nv ? 16 : 32;
  if (rows < 0 || cols < 0 || rows % blk != 0 || cols % blk != 0) return BSQ_EINVAL;
  if (too_many(rows, cols)) return BSQ_EINVAL;
  if (block_rows != 1 && block_rows != 16) return BSQ_EINVAL;
  if (rnd != BSQ_RNE && rnd != BSQ_SR) return BSQ_EINVAL;
  const bool do_row = codes_row || scales_row || (nv && amax_row);
  const bool do_col = codes_col || scales_col || (nv && amax_col);
  if (!do_row && !do_col) return BSQ_EINVAL;
  if (!nv && (block_rows == 16 || rht_col)) return BSQ_EUNSUPPORTED;
  if (fmt == BSQ_MXFP8 && rnd == BSQ_SR) return BSQ_EUNSUPPORTED;
  if (block_rows == 16 && (rnd == BSQ_SR || rht_col)) return BSQ_EUNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (rows * cols == 0) {                      // empty tensor: only the amax outputs are defined
    if (nv && (!aligned4(amax_row) || !aligned4(amax_col))) return BSQ_EINVAL;
    if (nv) return hip_status(bsq::launch_zero_amax(amax_row, amax_col, s));
    return BSQ_OK;
  }
  if (do_row && (!codes_row || !scales_row || (nv && !amax_row))) return BSQ_EINVAL;
  if (do_col && (!codes_col || !scales_col || (nv && !amax_col))) return BSQ_EINVAL;
  if (!aligned16_or_null(codes_row) || !aligned16_or_null(scales_row) ||
      !aligned16_or_null(codes_col) || !aligned16_or_null(scales_col))
    return BSQ_EINVAL;
  if (nv && (!aligned4(amax_row) || !aligned4(amax_col))) return BSQ_EINVAL;
  float* ar = do_row ? amax_row : nullptr;
  float* ac = do_col ? amax_col : nullptr;
  if (!x || !aligned16(x)) return BSQ_EINVAL;
  // the column RHT amax pass addresses 16 rows (32 * cols bytes) per buffer resource
  if (nv && rht_col && do_col && cols >= ((int64_t)1 << 26)) return BSQ_EINVAL;

  hipError_t e;
  if (nv) {
    e = bsq::launch_zero_amax(ar, ac, s);
    if (e != hipSuccess) return BSQ_EHIP;
    if (rht_col && do_col)
      e = bsq::launch_amax_tile_rht(x, rows, cols, rht_signs, ar, ac, s);
    else
      e = bsq::launch_amax_flat(x, rows * cols / 8, false, 0, ar ? ar : ac, ar ? ac : nullptr, s);
    if (e != hipSuccess) return BSQ_EHIP;
  }
  const bsq::Fmt f = nv ? bsq::kNVFP4 : (fmt == BSQ_MXFP4 ? bsq::kMXFP4 : bsq::kMXFP8);
  e = bsq::launch_quant_tile(f, rnd == BSQ_SR, rht_col != 0 && do_col, block_rows == 16, x, rows,
                             cols, do_row, do_col, ar, ac, rht_signs, seed, offset, codes_row,
                             scales_row, codes_col, scales_col, s);
  return hip_status(e);
}

bsq_status fp8_quantize_transpose(const void* x, int64_t rows, int64_t cols, uint8_t* codes_row,
                                  uint8_t* codes_col, float* amax, void* stream) {
  if (rows < 0 || cols < 0 || rows % 16 != 0 || cols % 16 != 0) return BSQ_EINVAL;
  if (too_many(rows, cols)) return BSQ_EINVAL;
  if (!amax || !aligned4(amax)) return BSQ_EINVAL;
  if (!codes_row && !codes_col) return BSQ_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (rows * cols == 0) return hip_status(bsq::launch_zero_amax(amax, nullptr, s));
  if (!x || !aligned16(x) || !aligned16_or_null(codes_row) || !aligned16_or_null(codes_col))
    return BSQ_EINVAL;
  hipError_t e = bsq::launch_zero_amax(amax, nullptr, s);
  if (e != hipSuccess) return BSQ_EHIP;
  e = bsq::launch_amax_flat(x, rows * cols / 8, false, 0, amax, nullptr, s);
  if (e != hipSuccess) return BSQ_EHIP;
  return hip_status(bsq::launch_fp8_qt(x, rows, cols, amax, codes_row, codes_col, s));
}

bsq_status quantize_transpose_amax(const void* x, int64_t rows, int64_t cols, int block_rows,
                                   bsq_rounding rnd, uint64_t seed, uint32_t offset, int rht_col,
                                   uint16_t rht_signs, const float* amax_row, const float* amax_col,
                                   uint8_t* codes_row, uint8_t* scales_row, uint8_t* codes_col,
                                   uint8_t* scales_col, void* stream) {
  if (rows < 0 || cols < 0 || rows % 16 != 0 || cols % 16 != 0) return BSQ_EINVAL;
  if (too_many(rows, cols)) return BSQ_EINVAL;
  if (block_rows != 1 && block_rows != 16) return BSQ_EINVAL;
  if (rnd != BSQ_RNE && rnd != BSQ_SR) return BSQ_EINVAL;
  const bool do_row = codes_row || scales_row;
  const bool do_col = codes_col || scales_col;
  if (!do_row && !do_col) return BSQ_EINVAL;
  if (block_rows == 16 && (rnd == BSQ_SR || rht_col)) return BSQ_EUNSUPPORTED;
  // 16x16 tiles encode both orientations under one amax (the codes of x^T
  // are the codes of x transposed), so the caller must pass that one amax
  // for both sides
  if (block_rows == 16 && do_row && do_col && amax_row != amax_col) return BSQ_EINVAL;
  if (rows * cols == 0) return BSQ_OK;
  if (do_row && (!codes_row || !scales_row || !amax_row)) return BSQ_EINVAL;
  if (do_col && (!codes_col || !scales_col || !amax_col)) return BSQ_EINVAL;
  if (!aligned16_or_null(codes_row) || !aligned16_or_null(scales_row) ||
      !aligned16_or_null(codes_col) || !aligned16_or_null(scales_col))
    return BSQ_EINVAL;
  if (!aligned4(amax_row) || !aligned4(amax_col)) return BSQ_EINVAL;
  if (!x || !aligned16(x)) return BSQ_EINVAL;
  return hip_status(bsq::launch_quant_tile(
      bsq::kNVFP4, rnd == BSQ_SR, rht_col != 0 && do_col, block_rows == 16, x, rows, cols, do_row,
      do_col, do_row ? amax_row : nullptr, do_col ? amax_col : nullptr, rht_signs, seed, offset,
      codes_row, scales_row, codes_col, scales_col, static_cast<hipStream_t>(stream)));
}

bsq_status swiglu_amax(const void* y_gu, int64_t rows, int64_t f, int rht_col, uint16_t rht_signs,
                       void* h, float* amax_row, float* amax_col, void* stream) {
  return swiglu_common(y_gu, nullptr, rows, f, rht_col, rht_signs, h, amax_row, amax_col, stream);
}

bsq_status swiglu_backward_amax(const void* y_gu, const void* d_h, int64_t rows, int64_t f,
                                int rht_col, uint16_t rht_signs, void* d_y_gu, float* amax_row,
                                float* amax_col, void* stream) {
  if (rows * f != 0 && !d_h) return BSQ_EINVAL;
  return swiglu_common(y_gu, d_h, rows, f, rht_col, rht_signs, d_y_gu, amax_row, amax_col, stream);
}

bsq_status master_weight_update(float* w32, const void* grad, int64_t n, float lr, void* w_bf16,
                                float* amax, void* stream) {
  if (n < 0 || n % 8 != 0 || too_many(1, n) || !aligned4(amax)) return BSQ_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (n == 0) return amax ? hip_status(bsq::launch_zero_amax(amax, nullptr, s)) : BSQ_OK;
  if (!w32 || !grad || !w_bf16 || !aligned16(w32) || !aligned16(grad) || !aligned16(w_bf16))
    return BSQ_EINVAL;
  if (overlap(w32, n * 4, grad, n * 2) || overlap(w32, n * 4, w_bf16, n * 2) ||
      overlap(grad, n * 2, w_bf16, n * 2))
    return BSQ_EINVAL;
  if (amax) {
    const hipError_t e = bsq::launch_zero_amax(amax, nullptr, s);
    if (e != hipSuccess) return BSQ_EHIP;
  }
  return hip_status(bsq::launch_master_update(w32, grad, n, lr, w_bf16, amax, s));
}

bsq_status nvfp4_expand(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                        void* out, void* stream) {
  if (rows < 0 || cols < 0 || cols % 16 != 0 || too_many(rows, cols)) return BSQ_EINVAL;
  if (rows * cols == 0) return BSQ_OK;
  if (!codes || !scales || !out || !aligned16(out) || (reinterpret_cast<uintptr_t>(codes) & 7u) != 0)
    return BSQ_EINVAL;
  return hip_status(bsq::launch_nvfp4_expand(codes, scales, rows, cols, out,
                                             static_cast<hipStream_t>(stream)));
}

bsq_status bs_gemm_nvfp4_bx(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                            const uint8_t* a_scales, const float* a_amax, const void* b_x,
                            const float* b_amax, void* c, int64_t ldc, void* stream) {
  if (M < 0 || N < 0 || K < 0 || ldc < N) return BSQ_EINVAL;
  if (too_many(M, K) || too_many(N, K) || too_many(M, ldc)) return BSQ_EINVAL;
  if (M > (int64_t)256 * 0x7FFFFF || N > (int64_t)256 * 0x7FFFFF) return BSQ_EINVAL;
  if (M == 0 || N == 0) return BSQ_OK;
  if (!a_codes || !a_scales || !b_x || !a_amax || !b_amax || !c) return BSQ_EINVAL;
  if ((reinterpret_cast<uintptr_t>(c) & 1u) != 0 || !aligned4(a_amax) || !aligned4(b_amax))
    return BSQ_EINVAL;
  if (K == 0 || K % 128 != 0 || !aligned16(a_codes) || !aligned4(a_scales) || !aligned16(b_x) ||
      M * (K / 2) >= ((int64_t)1 << 32) || N * K * 2 >= ((int64_t)1 << 32))
    return BSQ_EUNSUPPORTED;
  return hip_status(bsq::launch_gemm_nvfp4_bx(M, N, K, a_codes, a_scales, a_amax, b_x, b_amax, c,
                                              ldc, static_cast<hipStream_t>(stream)));
}

bsq_status bs_gemm(bsq_format fmt, int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                   const uint8_t* a_scales, const float* a_amax, const uint8_t* b_codes,
                   const uint8_t* b_scales, const float* b_amax, void* c, int64_t ldc,
                   void* stream) {
  return gemm_common(fmt, M, N, K, a_codes, a_scales, a_amax, b_codes, b_scales, b_amax, c, ldc,
                     stream, false);
}

bsq_status bs_gemm_noalloc(bsq_format fmt, int64_t M, int64_t N, int64_t K,
                           const uint8_t* a_codes, const uint8_t* a_scales, const float* a_amax,
                           const uint8_t* b_codes, const uint8_t* b_scales, const float* b_amax,
                           void* c, int64_t ldc, void* stream) {
  return gemm_common(fmt, M, N, K, a_codes, a_scales, a_amax, b_codes, b_scales, b_amax, c, ldc,
                     stream, true);
}

}  // extern "C"
