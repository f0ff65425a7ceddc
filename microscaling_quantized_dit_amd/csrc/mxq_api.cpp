// C-ABI host layer of libmxq: argument validation, device check, launches.
// Every entry point validates all arguments on the host before touching the HIP
// runtime, so invalid calls return without any launch or device query.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/mxq.h"
#include "mxq_internal.h"

namespace {

thread_local char g_last_error[512] = "";

mxq_status fail(mxq_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

mxq_status ok() {
  g_last_error[0] = '\0';
  return MXQ_SUCCESS;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Per-device result of the architecture check: 0 unknown, 1 gfx950, 2 other.
std::atomic<int> g_arch[64];

mxq_status check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(MXQ_ERROR_UNSUPPORTED_DEVICE, "no current HIP device");
  if (dev < 0 || dev >= 64) return fail(MXQ_ERROR_UNSUPPORTED_DEVICE, "device index %d out of range", dev);
  int st = g_arch[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
      return fail(MXQ_ERROR_UNSUPPORTED_DEVICE, "cannot query device %d", dev);
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch[dev].store(st, std::memory_order_relaxed);
    if (st == 2) return fail(MXQ_ERROR_UNSUPPORTED_DEVICE, "device %d is %s, gfx950 required", dev, prop.gcnArchName);
  }
  if (st != 1) return fail(MXQ_ERROR_UNSUPPORTED_DEVICE, "device %d is not gfx950", dev);
  return MXQ_SUCCESS;
}

mxq_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MXQ_ERROR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

constexpr int64_t kMax32 = (int64_t)1 << 31;

// Validates a quantizer's scale layout for a [rows, cols] tensor: the tiled order
// groups rows by 64 and K by 128 values.
mxq_status check_scale_layout(mxq_scale_layout layout, int64_t rows, int64_t cols) {
  if (layout != MXQ_SCALES_ROW_MAJOR && layout != MXQ_SCALES_TILED)
    return fail(MXQ_ERROR_INVALID_VALUE, "bad scale layout %d", (int)layout);
  if (layout == MXQ_SCALES_TILED && (rows % 64 != 0 || cols % 128 != 0))
    return fail(MXQ_ERROR_UNSUPPORTED_SHAPE, "tiled scales need rows %% 64 == 0 and cols %% 128 == 0 (got %lld, %lld)",
                (long long)rows, (long long)cols);
  // one workgroup per 64 x 128 values, numbered with 31 bits (with room to spare)
  if (layout == MXQ_SCALES_TILED && rows > ((int64_t)1 << 43) / cols)
    return fail(MXQ_ERROR_UNSUPPORTED_SHAPE, "tensor too large for tiled scales");
  return MXQ_SUCCESS;
}

std::atomic<int> g_cus[64];

}  // namespace

namespace mxq {
int device_compute_units() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = g_cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    g_cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}
ScaleTiling scale_tiling(int64_t cols) { return ScaleTiling{cols / 8, (int)(cols / 128)}; }
}  // namespace mxq

extern "C" {

mxq_status mxq_quantize_mxfp8(const void* x, int64_t rows, int64_t cols, mxq_fp8_kind kind, void* q,
                              void* scales, mxq_scale_layout scale_layout, void* stream) {
  if (!x || !q || !scales) return fail(MXQ_ERROR_INVALID_VALUE, "null pointer argument");
  if (rows <= 0 || cols <= 0) return fail(MXQ_ERROR_INVALID_VALUE, "rows and cols must be positive");
  if (kind != MXQ_FP8_E4M3 && kind != MXQ_FP8_E5M2) return fail(MXQ_ERROR_INVALID_VALUE, "bad fp8 kind %d", (int)kind);
  if (cols % 32 != 0) return fail(MXQ_ERROR_UNSUPPORTED_SHAPE, "cols (%lld) must be a multiple of 32", (long long)cols);
  if (rows > INT64_MAX / cols) return fail(MXQ_ERROR_UNSUPPORTED_SHAPE, "rows * cols overflows");
  mxq_status l = check_scale_layout(scale_layout, rows, cols);
  if (l != MXQ_SUCCESS) return l;
  if (!aligned16(x) || !aligned16(q) || !aligned16(scales))
    return fail(MXQ_ERROR_MISALIGNED, "x, q and scales must be 16-byte aligned");
  mxq_status d = check_device();
  if (d != MXQ_SUCCESS) return d;
  const mxq::ScaleTiling tiling = mxq::scale_tiling(scale_layout == MXQ_SCALES_TILED ? cols : 0);
  return launched(mxq::launch_quantize_mxfp8(x, rows * cols, (int)kind, q, scales, tiling, (hipStream_t)stream),
                  "mxq_quantize_mxfp8 launch");
}

size_t mxq_quantize_nvfp4_workspace_size(int64_t rows, int64_t cols) {
  if (rows <= 0 || cols <= 0 || cols % 16 != 0 || rows > INT64_MAX / cols) return 0;
  return (size_t)mxq::nvfp4_amax_partials(rows * cols) * sizeof(uint32_t);
}

mxq_status mxq_quantize_nvfp4(const void* x, int64_t rows, int64_t cols, const float* global_scale_in, void* q,
                              void* scales, mxq_scale_layout scale_layout, float* global_scale_out, void* workspace,
                              size_t ws_bytes, void* stream) {
  if (!x || !q || !scales || !global_scale_out) return fail(MXQ_ERROR_INVALID_VALUE, "null pointer argument");
  if (rows <= 0 || cols <= 0) return fail(MXQ_ERROR_INVALID_VALUE, "rows and cols must be positive");
  if (cols % 16 != 0) return fail(MXQ_ERROR_UNSUPPORTED_SHAPE, "cols (%lld) must be a multiple of 16", (long long)cols);
  if (rows > INT64_MAX / cols) return fail(MXQ_ERROR_UNSUPPORTED_SHAPE, "rows * cols overflows");
  mxq_status l = check_scale_layout(scale_layout, rows, cols);
  if (l != MXQ_SUCCESS) return l;
  if (!aligned16(x) || !aligned16(q) || !aligned16(scales))
    return fail(MXQ_ERROR_MISALIGNED, "x, q and scales must be 16-byte aligned");
  if (((uintptr_t)global_scale_out & 3u) || ((uintptr_t)global_scale_in & 3u))
    return fail(MXQ_ERROR_MISALIGNED, "global scale pointers must be 4-byte aligned");
  if (!global_scale_in) {
    const size_t need = mxq_quantize_nvfp4_workspace_size(rows, cols);
    if (!workspace || ws_bytes < need)
      return fail(MXQ_ERROR_WORKSPACE, "dynamic mode needs a %zu-byte workspace (got %zu)", need,
                  workspace ? ws_bytes : (size_t)0);
    if ((uintptr_t)workspace & 3u) return fail(MXQ_ERROR_MISALIGNED, "workspace must be 4-byte aligned");
  }
  mxq_status d = check_device();
  if (d != MXQ_SUCCESS) return d;
  const mxq::ScaleTiling tiling = mxq::scale_tiling(scale_layout == MXQ_SCALES_TILED ? cols : 0);
  return launched(mxq::launch_quantize_nvfp4(x, rows * cols, global_scale_in, q, scales, global_scale_out,
                                             (uint32_t*)workspace, tiling, (hipStream_t)stream),
                  "mxq_quantize_nvfp4 launch");
}

mxq_status mxq_quantize_nvfp4_noalloc(const void* x, int64_t rows, int64_t cols, const float* global_scale_in,
                                      void* q, void* scales, mxq_scale_layout scale_layout,
                                      float* global_scale_out, void* stream) {
  if (!x || !q || !scales || !global_scale_out) return fail(MXQ_ERROR_INVALID_VALUE, "null pointer argument");
  if (rows <= 0 || cols <= 0) return fail(MXQ_ERROR_INVALID_VALUE, "rows and cols must be positive");
  if (cols % 16 != 0) return fail(MXQ_ERROR_UNSUPPORTED_SHAPE, "cols (%lld) must be a multiple of 16", (long long)cols);
  if (rows > INT64_MAX / cols) return fail(MXQ_ERROR_UNSUPPORTED_SHAPE, "rows * cols overflows");
  mxq_status l = check_scale_layout(scale_layout, rows, cols);
  if (l != MXQ_SUCCESS) return l;
  if (!aligned16(x) || !aligned16(q) || !aligned16(scales))
    return fail(MXQ_ERROR_MISALIGNED, "x, q and scales must be 16-byte aligned");
  if (((uintptr_t)global_scale_out & 3u) || ((uintptr_t)global_scale_in & 3u))
    return fail(MXQ_ERROR_MISALIGNED, "global scale pointers must be 4-byte aligned");
  mxq_status d = check_device();
  if (d != MXQ_SUCCESS) return d;
  uint32_t* partials = nullptr;
  if (!global_scale_in) {
    int words = 0;
    hipError_t e = mxq::amax_scratch(&partials, &words);
    if (e != hipSuccess) return fail(MXQ_ERROR_LAUNCH, "scratch address lookup: %s", hipGetErrorString(e));
    const int need = mxq::nvfp4_amax_partials(rows * cols);
    if (need > words)
      return fail(MXQ_ERROR_WORKSPACE, "tensor needs %d partial maxima, the scratch holds %d", need, words);
  }
  const mxq::ScaleTiling tiling = mxq::scale_tiling(scale_layout == MXQ_SCALES_TILED ? cols : 0);
  return launched(mxq::launch_quantize_nvfp4(x, rows * cols, global_scale_in, q, scales, global_scale_out, partials,
                                             tiling, (hipStream_t)stream),
                  "mxq_quantize_nvfp4_noalloc launch");
}

mxq_status mxq_nvfp4_calibrate(const void* x, int64_t rows, int64_t cols, float* running_scale, void* workspace,
                               size_t ws_bytes, void* stream) {
  if (!x || !running_scale) return fail(MXQ_ERROR_INVALID_VALUE, "null pointer argument");
  if (rows <= 0 || cols <= 0) return fail(MXQ_ERROR_INVALID_VALUE, "rows and cols must be positive");
  if (cols % 16 != 0) return fail(MXQ_ERROR_UNSUPPORTED_SHAPE, "cols (%lld) must be a multiple of 16", (long long)cols);
  if (rows > INT64_MAX / cols) return fail(MXQ_ERROR_UNSUPPORTED_SHAPE, "rows * cols overflows");
  if (!aligned16(x)) return fail(MXQ_ERROR_MISALIGNED, "x must be 16-byte aligned");
  if ((uintptr_t)running_scale & 3u) return fail(MXQ_ERROR_MISALIGNED, "running_scale must be 4-byte aligned");
  const size_t need = mxq_quantize_nvfp4_workspace_size(rows, cols);
  if (!workspace || ws_bytes < need)
    return fail(MXQ_ERROR_WORKSPACE, "calibration needs a %zu-byte workspace (got %zu)", need,
                workspace ? ws_bytes : (size_t)0);
  if ((uintptr_t)workspace & 3u) return fail(MXQ_ERROR_MISALIGNED, "workspace must be 4-byte aligned");
  mxq_status d = check_device();
  if (d != MXQ_SUCCESS) return d;
  return launched(mxq::launch_nvfp4_calibrate(x, rows * cols, running_scale, (uint32_t*)workspace,
                                              (hipStream_t)stream),
                  "mxq_nvfp4_calibrate launch");
}

mxq_status mxq_quantize_fp8_weight(const void* w, int64_t rows, int64_t cols, const float* scale_in, void* q,
                                   float* scale_out, void* workspace, size_t ws_bytes, void* stream) {
  if (!w || !q || !scale_out) return fail(MXQ_ERROR_INVALID_VALUE, "null pointer argument");
  if (rows <= 0 || cols <= 0) return fail(MXQ_ERROR_INVALID_VALUE, "rows and cols must be positive");
  if (cols % 16 != 0) return fail(MXQ_ERROR_UNSUPPORTED_SHAPE, "cols (%lld) must be a multiple of 16", (long long)cols);
  if (rows > INT64_MAX / cols) return fail(MXQ_ERROR_UNSUPPORTED_SHAPE, "rows * cols overflows");
  if (!aligned16(w) || !aligned16(q)) return fail(MXQ_ERROR_MISALIGNED, "w and q must be 16-byte aligned");
  if (((uintptr_t)scale_out & 3u) || ((uintptr_t)scale_in & 3u))
    return fail(MXQ_ERROR_MISALIGNED, "scale pointers must be 4-byte aligned");
  if (!scale_in) {
    const size_t need = mxq_quantize_nvfp4_workspace_size(rows, cols);
    if (!workspace || ws_bytes < need)
      return fail(MXQ_ERROR_WORKSPACE, "dynamic mode needs a %zu-byte workspace (got %zu)", need,
                  workspace ? ws_bytes : (size_t)0);
    if ((uintptr_t)workspace & 3u) return fail(MXQ_ERROR_MISALIGNED, "workspace must be 4-byte aligned");
  }
  mxq_status d = check_device();
  if (d != MXQ_SUCCESS) return d;
  return launched(mxq::launch_quantize_fp8_tensor(w, rows * cols, scale_in, q, scale_out, (uint32_t*)workspace,
                                                  (hipStream_t)stream),
                  "mxq_quantize_fp8_weight launch");
}

static mxq_status check_attention_shape(int64_t heads, int64_t L, int64_t d) {
  if (heads <= 0 || L <= 0) return fail(MXQ_ERROR_INVALID_VALUE, "heads and L must be positive");
  if (d != 128) return fail(MXQ_ERROR_UNSUPPORTED_SHAPE, "head dimension %lld (only 128)", (long long)d);
  if (L % 128 != 0) return fail(MXQ_ERROR_UNSUPPORTED_SHAPE, "L (%lld) must be a multiple of 128", (long long)L);
  if (L >= kMax32 / 128) return fail(MXQ_ERROR_UNSUPPORTED_SHAPE, "L * 128 must be < 2^31");
  if (heads > INT32_MAX / 2 || heads > INT64_MAX / (L * 128)) return fail(MXQ_ERROR_UNSUPPORTED_SHAPE, "too many heads");
  return MXQ_SUCCESS;
}

mxq_status mxq_quantize_fp8_v(const void* v, int64_t heads, int64_t L, int64_t d, const float* scale_in, void* vt,
                              float* scale_out, void* workspace, size_t ws_bytes, void* stream) {
  if (!v || !vt || !scale_out) return fail(MXQ_ERROR_INVALID_VALUE, "null pointer argument");
  mxq_status s = check_attention_shape(heads, L, d);
  if (s != MXQ_SUCCESS) return s;
  if (!aligned16(v) || !aligned16(vt)) return fail(MXQ_ERROR_MISALIGNED, "v and vt must be 16-byte aligned");
  if (((uintptr_t)scale_out & 3u) || ((uintptr_t)scale_in & 3u))
    return fail(MXQ_ERROR_MISALIGNED, "scale pointers must be 4-byte aligned");
  if (!scale_in) {
    const size_t need = mxq_quantize_nvfp4_workspace_size(heads * L, d);
    if (!workspace || ws_bytes < need)
      return fail(MXQ_ERROR_WORKSPACE, "dynamic mode needs a %zu-byte workspace (got %zu)", need,
                  workspace ? ws_bytes : (size_t)0);
    if ((uintptr_t)workspace & 3u) return fail(MXQ_ERROR_MISALIGNED, "workspace must be 4-byte aligned");
  }
  mxq_status dv = check_device();
  if (dv != MXQ_SUCCESS) return dv;
  return launched(mxq::launch_quantize_fp8_vt(v, heads, L, scale_in, vt, scale_out, (uint32_t*)workspace,
                                              (hipStream_t)stream),
                  "mxq_quantize_fp8_v launch");
}

mxq_status mxq_attention_fp8(const void* q, const float* q_scale, const void* k, const float* k_scale, const void* vt,
                             const float* v_scale, int64_t heads, int64_t L, int64_t d, void* o, void* stream) {
  if (!q || !q_scale || !k || !k_scale || !vt || !v_scale || !o)
    return fail(MXQ_ERROR_INVALID_VALUE, "null pointer argument");
  mxq_status s = check_attention_shape(heads, L, d);
  if (s != MXQ_SUCCESS) return s;
  if (!aligned16(q) || !aligned16(k) || !aligned16(vt) || !aligned16(o))
    return fail(MXQ_ERROR_MISALIGNED, "q, k, vt and o must be 16-byte aligned");
  if (((uintptr_t)q_scale & 3u) || ((uintptr_t)k_scale & 3u) || ((uintptr_t)v_scale & 3u))
    return fail(MXQ_ERROR_MISALIGNED, "scale pointers must be 4-byte aligned");
  mxq_status dv = check_device();
  if (dv != MXQ_SUCCESS) return dv;
  return launched(mxq::launch_attention_fp8(q, q_scale, k, k_scale, vt, v_scale, heads, L, o, (hipStream_t)stream),
                  "mxq_attention_fp8 launch");
}

static mxq_status check_gemm_common(int64_t M, int64_t N, int64_t K, const void* bias, mxq_epilogue epi, void* c,
                                    int64_t a_row_bytes_num, int64_t a_row_bytes_den) {
  if (!c) return fail(MXQ_ERROR_INVALID_VALUE, "null output pointer");
  if (M <= 0 || N <= 0 || K <= 0) return fail(MXQ_ERROR_INVALID_VALUE, "M, N, K must be positive");
  if (epi != MXQ_EPI_NONE && epi != MXQ_EPI_BIAS && epi != MXQ_EPI_BIAS_GELU_TANH)
    return fail(MXQ_ERROR_INVALID_VALUE, "bad epilogue %d", (int)epi);
  if (epi != MXQ_EPI_NONE && !bias) return fail(MXQ_ERROR_INVALID_VALUE, "epilogue needs a bias");
  if (M % 128 || N % 128 || K % 128)
    return fail(MXQ_ERROR_UNSUPPORTED_SHAPE, "M, N, K (%lld, %lld, %lld) must be multiples of 128", (long long)M,
                (long long)N, (long long)K);
  // operands are addressed with 32-bit byte offsets
  const int64_t kb = K * a_row_bytes_num / a_row_bytes_den;
  if (M >= kMax32 / kb || N >= kMax32 / kb)
    return fail(MXQ_ERROR_UNSUPPORTED_SHAPE, "operands must each be < 2 GiB");
  if (!aligned16(c) || (bias && !aligned16(bias)))
    return fail(MXQ_ERROR_MISALIGNED, "c and bias must be 16-byte aligned");
  return MXQ_SUCCESS;
}

mxq_status mxq_gemm_bf16_fp8w(const void* a, const void* w_q, const float* w_scale, int64_t M, int64_t N, int64_t K,
                              const void* bias, mxq_epilogue epi, void* c, void* stream) {
  if (!a || !w_q || !w_scale) return fail(MXQ_ERROR_INVALID_VALUE, "null pointer argument");
  mxq_status s = check_gemm_common(M, N, K, bias, epi, c, 2, 1);
  if (s != MXQ_SUCCESS) return s;
  if (!aligned16(a) || !aligned16(w_q)) return fail(MXQ_ERROR_MISALIGNED, "operands must be 16-byte aligned");
  if ((uintptr_t)w_scale & 3u) return fail(MXQ_ERROR_MISALIGNED, "w_scale must be 4-byte aligned");
  mxq_status d = check_device();
  if (d != MXQ_SUCCESS) return d;
  return launched(mxq::launch_gemm_w8(a, w_q, w_scale, M, N, K, bias, (int)epi, c, (hipStream_t)stream),
                  "mxq_gemm_bf16_fp8w launch");
}

mxq_status mxq_gemm_mxfp8(const void* a_q, const void* a_scales, mxq_fp8_kind a_kind, const void* w_q,
                          const void* w_scales, mxq_fp8_kind w_kind, mxq_scale_layout scale_layout, int64_t M,
                          int64_t N, int64_t K, const void* bias, mxq_epilogue epi, void* c, void* stream) {
  if (!a_q || !a_scales || !w_q || !w_scales) return fail(MXQ_ERROR_INVALID_VALUE, "null pointer argument");
  if ((a_kind != MXQ_FP8_E4M3 && a_kind != MXQ_FP8_E5M2) || (w_kind != MXQ_FP8_E4M3 && w_kind != MXQ_FP8_E5M2))
    return fail(MXQ_ERROR_INVALID_VALUE, "bad fp8 kind");
  if (scale_layout != MXQ_SCALES_ROW_MAJOR && scale_layout != MXQ_SCALES_TILED)
    return fail(MXQ_ERROR_INVALID_VALUE, "bad scale layout %d", (int)scale_layout);
  mxq_status s = check_gemm_common(M, N, K, bias, epi, c, 1, 1);
  if (s != MXQ_SUCCESS) return s;
  if (!aligned16(a_q) || !aligned16(a_scales) || !aligned16(w_q) || !aligned16(w_scales))
    return fail(MXQ_ERROR_MISALIGNED, "operands must be 16-byte aligned");
  mxq_status d = check_device();
  if (d != MXQ_SUCCESS) return d;
  return launched(mxq::launch_gemm_mxfp8(a_q, a_scales, (int)a_kind, w_q, w_scales, (int)w_kind, M, N, K, bias,
                                         (int)epi, c, scale_layout == MXQ_SCALES_TILED, (hipStream_t)stream),
                  "mxq_gemm_mxfp8 launch");
}

mxq_status mxq_gemm_mxfp8_fused(const void* a, mxq_fp8_kind kind, const void* w_q, const void* w_scales,
                                mxq_scale_layout scale_layout, int64_t M, int64_t N, int64_t K, const void* bias,
                                mxq_epilogue epi, void* c, void* stream) {
  if (!a || !w_q || !w_scales) return fail(MXQ_ERROR_INVALID_VALUE, "null pointer argument");
  if (kind != MXQ_FP8_E4M3 && kind != MXQ_FP8_E5M2) return fail(MXQ_ERROR_INVALID_VALUE, "bad fp8 kind");
  if (scale_layout != MXQ_SCALES_ROW_MAJOR && scale_layout != MXQ_SCALES_TILED)
    return fail(MXQ_ERROR_INVALID_VALUE, "bad scale layout %d", (int)scale_layout);
  mxq_status s = check_gemm_common(M, N, K, bias, epi, c, 2, 1);
  if (s != MXQ_SUCCESS) return s;
  if (!aligned16(a) || !aligned16(w_q) || !aligned16(w_scales))
    return fail(MXQ_ERROR_MISALIGNED, "operands must be 16-byte aligned");
  mxq_status d = check_device();
  if (d != MXQ_SUCCESS) return d;
  return launched(mxq::launch_gemm_mxfp8_fused(a, (int)kind, w_q, w_scales, M, N, K, bias, (int)epi, c,
                                               scale_layout == MXQ_SCALES_TILED, (hipStream_t)stream),
                  "mxq_gemm_mxfp8_fused launch");
}

size_t mxq_gemm_nvfp4_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || M % 128 || N % 128 || K % 128) return 0;
  if (M >= kMax32 || N >= kMax32 || K >= kMax32) return 0;
  return mxq::gemm_nvfp4_workspace_bytes(M, N, K);
}

mxq_status mxq_gemm_nvfp4(const void* a_q, const void* a_scales, const float* a_global, const void* w_q,
                          const void* w_scales, const float* w_global, mxq_scale_layout scale_layout, int64_t M,
                          int64_t N, int64_t K, const void* bias, mxq_epilogue epi, void* c, void* workspace,
                          size_t ws_bytes, void* stream) {
  if (!a_q || !a_scales || !a_global || !w_q || !w_scales || !w_global)
    return fail(MXQ_ERROR_INVALID_VALUE, "null pointer argument");
  if (scale_layout != MXQ_SCALES_ROW_MAJOR && scale_layout != MXQ_SCALES_TILED)
    return fail(MXQ_ERROR_INVALID_VALUE, "bad scale layout %d", (int)scale_layout);
  mxq_status s = check_gemm_common(M, N, K, bias, epi, c, 1, 2);
  if (s != MXQ_SUCCESS) return s;
  if (!aligned16(a_q) || !aligned16(a_scales) || !aligned16(w_q) || !aligned16(w_scales))
    return fail(MXQ_ERROR_MISALIGNED, "operands must be 16-byte aligned");
  if (((uintptr_t)a_global & 3u) || ((uintptr_t)w_global & 3u))
    return fail(MXQ_ERROR_MISALIGNED, "global scale pointers must be 4-byte aligned");
  if (workspace) {
    if (!aligned16(workspace)) return fail(MXQ_ERROR_MISALIGNED, "workspace must be 16-byte aligned");
    const size_t need = mxq::gemm_nvfp4_workspace_bytes(M, N, K);
    if (ws_bytes < need)
      return fail(MXQ_ERROR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, need);
  }
  mxq_status d = check_device();
  if (d != MXQ_SUCCESS) return d;
  return launched(mxq::launch_gemm_nvfp4(a_q, a_scales, a_global, w_q, w_scales, w_global, M, N, K, bias, (int)epi,
                                         c, scale_layout == MXQ_SCALES_TILED, workspace, (hipStream_t)stream),
                  "mxq_gemm_nvfp4 launch");
}

const char* mxq_status_string(mxq_status s) {
  switch (s) {
    case MXQ_SUCCESS: return "success";
    case MXQ_ERROR_INVALID_VALUE: return "invalid value";
    case MXQ_ERROR_UNSUPPORTED_SHAPE: return "unsupported shape";
    case MXQ_ERROR_MISALIGNED: return "misaligned pointer";
    case MXQ_ERROR_WORKSPACE: return "workspace missing or too small";
    case MXQ_ERROR_UNSUPPORTED_DEVICE: return "unsupported device";
    case MXQ_ERROR_LAUNCH: return "launch failed";
  }
  return "unknown status";
}

const char* mxq_last_error(void) { return g_last_error; }

}  // extern "C"
