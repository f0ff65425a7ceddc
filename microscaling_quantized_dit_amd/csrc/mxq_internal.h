// Internal declarations shared by the gfx950 kernels and the C-ABI host layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

// Compute units of the current device (cached per device; 256 on MI355X).
int device_compute_units();

// Host-side launchers (each returns the hipError_t of its launch).
hipError_t launch_quantize_mxfp8(const void* x, int64_t n_elems, int kind, void* q, void* scales,
                                 hipStream_t stream);

// Workgroups (= partial maxima) the NVFP4 amax pass uses for n_elems.
int nvfp4_amax_partials(int64_t n_elems);
hipError_t launch_quantize_nvfp4(const void* x, int64_t n_elems, const float* global_in, void* q,
                                 void* scales, float* global_out, uint32_t* partials,
                                 hipStream_t stream);

// running = max(running, RN_fp32(amax(x) / 2688)); partials as for the quantizer.
hipError_t launch_nvfp4_calibrate(const void* x, int64_t n_elems, float* running, uint32_t* partials,
                                  hipStream_t stream);

hipError_t launch_gemm_mxfp8(const void* a_q, const void* a_s, int a_kind, const void* w_q,
                             const void* w_s, int w_kind, int64_t M, int64_t N, int64_t K,
                             const void* bias, int epi, void* c, hipStream_t stream);

hipError_t launch_gemm_nvfp4(const void* a_q, const void* a_s, const float* a_g, const void* w_q,
                             const void* w_s, const float* w_g, int64_t M, int64_t N, int64_t K,
                             const void* bias, int epi, void* c, hipStream_t stream);

}  // namespace mxq

#if defined(__HIP_DEVICE_COMPILE__) || defined(__HIPCC__)
namespace mxq {
namespace dev {

// bf16 bit pattern (low/high half of a dword) widened exactly to fp32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Max of the 15-bit magnitudes of the eight bf16 values in a uint4, as a
// packed pair (the caller folds the halves).  Integer order of bf16 magnitude
// bits is the order of the magnitudes for finite values.
__device__ __forceinline__ uint32_t mag_max_pk(uint4 v) {
  typedef unsigned short us2 __attribute__((ext_vector_type(2)));
  const uint32_t m = 0x7FFF7FFFu;
  us2 a = __builtin_bit_cast(us2, v.x & m), b = __builtin_bit_cast(us2, v.y & m);
  us2 c = __builtin_bit_cast(us2, v.z & m), d = __builtin_bit_cast(us2, v.w & m);
  us2 ab = __builtin_elementwise_max(a, b), cd = __builtin_elementwise_max(c, d);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(ab, cd));
}

__device__ __forceinline__ uint32_t fold_halves_max(uint32_t pk) {
  uint32_t lo = pk & 0xFFFFu, hi = pk >> 16;
  return lo > hi ? lo : hi;
}

// Two fp32 -> two bf16 (nearest, ties to even) packed low|high: v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
  v2bf r = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, r);
}

// GELU, tanh form: 0.5 y (1 + tanh(u)), u = sqrt(2/pi) (y + 0.044715 y^3).
// Since 1 + tanh(u) = 2 / (1 + e^(-2u)), this is y / (1 + 2^(-2u log2 e)): one
// hardware exp2 and one reciprocal, each within about 1 ulp, with no cancellation
// for large negative y (the quotient tends to -0) or overflow for large positive
// y (the exponential tends to 0).
__device__ __forceinline__ float gelu_tanh(float y) {
  const float k0 = 0.7978845608028654f;             // sqrt(2/pi)
  const float k1 = 0.044715f;
  const float m2log2e = -2.0f * 1.4426950408889634f; // -2 log2(e)
  const float u = k0 * (y + k1 * y * y * y);
  return y * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(m2log2e * u));
}

// Remap a linear workgroup id so that ids placed round-robin on the 8 XCDs
// become contiguous ranges per XCD (neighbouring tiles share one L2).
__device__ __forceinline__ int xcd_remap(int wg, int n_wg) {
  const int n_xcd = 8;
  int per = n_wg / n_xcd;
  if (wg >= per * n_xcd) return wg;
  return (wg % n_xcd) * per + wg / n_xcd;
}

}  // namespace dev
}  // namespace mxq
#endif
