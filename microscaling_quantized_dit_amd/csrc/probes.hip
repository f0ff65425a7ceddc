// Measurement probes for gfx950 (libmxq_probes.so, used by bench.py and the tests;
// not part of the quantized-linear library):
//   * back-to-back matrix-core loops on register data -- the scaled fp8
//     v_mfma_scale_f32_32x32x64_f8f6f4 the MXFP8 GEMM and the attention run on, and
//     the fp16 v_mfma_f32_32x32x16_f16 the NVFP4 GEMM runs on -- with the shader
//     clock read at both ends (s_memtime against the constant-rate s_memrealtime),
//     for the machine's attainable MFMA rate and clock under load;
//   * a streaming copy (16-byte loads and stores) for the attainable HBM rate;
//   * single-instruction matrix-core probes on given operands, for the
//     accumulation behaviour the tests' error bounds rest on.
// Every kernel reads and writes only the buffers it is given, within the sizes
// the launchers state.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace mxq {
hipError_t launch_gemm_mxfp8_a_twice(const void* a_q, const void* a_s, const void* w_q, const void* w_s, int64_t M,
                                     int64_t N, int64_t K, void* c, hipStream_t stream);
// Compute units of the current device (the GEMM launcher's persistent grid).
int device_compute_units() {
  static std::atomic<int> cached{0};
  int n = cached.load(std::memory_order_relaxed);
  if (n == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                 hipSuccess || n <= 0)
      n = 256;
    cached.store(n, std::memory_order_relaxed);
  }
  return n;
}
}  // namespace mxq

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t mix(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7FEB352Du;
  x ^= x >> 15;
  x *= 0x846CA68Bu;
  x ^= x >> 16;
  return x;
}

// Operand bytes from a hash of the lane and register index; for fp8 the
// exponent field stays below the NaN pattern (0x7F / 0xFF never occur), signs random.
__device__ __forceinline__ v8i random_fp8_operand(uint32_t seed) {
  v8i a;
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = (int)(mix(seed * 8u + i) & 0xEFEFEFEFu);
  return a;
}

// Clock samples of one lane per workgroup: [0] s_memtime at start, [1] at end,
// [2] s_memrealtime at start, [3] at end.
__device__ __forceinline__ void sample_clocks(uint64_t* clocks, int slot) {
  if (threadIdx.x == 0) {
    clocks[4 * blockIdx.x + slot] = clock64();
    clocks[4 * blockIdx.x + 2 + slot] = wall_clock64();
  }
}

// fp8 loop: 4 independent 32x32 accumulators per wave, `iters` rounds of 8 MFMAs.
__global__ __launch_bounds__(256) void k_loop_fp8(int iters, float* sink, uint64_t* clocks) {
  const uint32_t id = blockIdx.x * blockDim.x + threadIdx.x;
  v8i a0 = random_fp8_operand(id), a1 = random_fp8_operand(id + 0x9E3779B9u);
  v8i b0 = random_fp8_operand(id + 0x7F4A7C15u), b1 = random_fp8_operand(id + 0x94D049BBu);
  v16f c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) c[j][v] = 0.0f;
  __syncthreads();
  sample_clocks(clocks, 0);
  for (int it = 0; it < iters; ++it) {   // four independent MFMAs between dependent ones
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, b0, c[j], 0, 0, 0, 127, 0, 127);
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, b1, c[j], 0, 0, 0, 127, 0, 127);
  }
  __syncthreads();
  sample_clocks(clocks, 1);
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += c[j][v];
  sink[id] = s;
}

// fp16 loop: the same structure on v_mfma_f32_32x32x16_f16 (8 MFMAs per round).
__global__ __launch_bounds__(256) void k_loop_f16(int iters, float* sink, uint64_t* clocks) {
  const uint32_t id = blockIdx.x * blockDim.x + threadIdx.x;
  v8h a0, a1, b0, b1;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a0[i] = (_Float16)((float)(mix(id * 32u + i) & 0xFFFF) * (1.0f / 65536.0f) - 0.5f);
    a1[i] = (_Float16)((float)(mix(id * 32u + 8 + i) & 0xFFFF) * (1.0f / 65536.0f) - 0.5f);
    b0[i] = (_Float16)((float)(mix(id * 32u + 16 + i) & 0xFFFF) * (1.0f / 65536.0f) - 0.5f);
    b1[i] = (_Float16)((float)(mix(id * 32u + 24 + i) & 0xFFFF) * (1.0f / 65536.0f) - 0.5f);
  }
  v16f c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) c[j][v] = 0.0f;
  __syncthreads();
  sample_clocks(clocks, 0);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b0, c[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b1, c[j], 0, 0, 0);
  }
  __syncthreads();
  sample_clocks(clocks, 1);
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += c[j][v];
  sink[id] = s;
}

// Streaming copy of n16 16-byte chunks: each workgroup moves consecutive slabs of
// 4 x 256 chunks (four 16-byte loads in flight per thread, then four stores),
// nontemporal both ways; the remainder chunk by chunk.
__global__ __launch_bounds__(256) void k_copy(const uint4* __restrict__ src, uint4* __restrict__ dst, int64_t n16) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const int64_t slab = 4 * 256;
  const int64_t n_slabs = n16 / slab;
  for (int64_t b = blockIdx.x; b < n_slabs; b += gridDim.x) {
    const int64_t base = b * slab + threadIdx.x;
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load((const u32x4*)(src + base + 256 * u));
#pragma unroll
    for (int u = 0; u < 4; ++u) __builtin_nontemporal_store(v[u], (u32x4*)(dst + base + 256 * u));
  }
  for (int64_t i = n_slabs * slab + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * blockDim.x)
    __builtin_nontemporal_store(__builtin_nontemporal_load((const u32x4*)(src + i)), (u32x4*)(dst + i));
}

// One fp8 MFMA on given operands (one wave).  a, b: 32 rows x 64 E4M3 bytes; c_in,
// out: 32 x 32 fp32 row-major, out = A B^T + C.  Operand layout of the instruction:
// lane l holds row l % 32 and bytes [16g, 16g+16), [32+16g, 32+16g+16) of it (g = l / 32),
// which are K positions [16g, 16g+16) and [32+16g, 32+16g+16); result
// D[8(v/4) + 4g + v%4][l % 32] in element v.
__global__ __launch_bounds__(64) void k_once_fp8(const uint8_t* a, const uint8_t* b, const float* c_in,
                                                 float* out) {
  const int l = threadIdx.x, r = l & 31, g = l >> 5;
  const uint4* pa = (const uint4*)(a + r * 64);
  const uint4* pb = (const uint4*)(b + r * 64);
  const uint4 a0 = pa[g], a1 = pa[2 + g], b0 = pb[g], b1 = pb[2 + g];
  const v8i A = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
  const v8i B = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
  v16f C;
#pragma unroll
  for (int v = 0; v < 16; ++v) C[v] = c_in[(8 * (v / 4) + 4 * g + v % 4) * 32 + r];
  const v16f D = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, C, 0, 0, 0, 127, 0, 127);
#pragma unroll
  for (int v = 0; v < 16; ++v) out[(8 * (v / 4) + 4 * g + v % 4) * 32 + r] = D[v];
}

// One 16-bit MFMA (kind 0: fp16, 1: bf16).  a, b: 32 rows x 16 values (2 bytes
// each); lane l holds row l % 32, K [8g, 8g + 8); c_in, out as above.
__global__ __launch_bounds__(64) void k_once_16(const uint16_t* a, const uint16_t* b, const float* c_in,
                                                float* out, int kind) {
  const int l = threadIdx.x, r = l & 31, g = l >> 5;
  const uint4 ua = *(const uint4*)(a + r * 16 + 8 * g), ub = *(const uint4*)(b + r * 16 + 8 * g);
  v16f C;
#pragma unroll
  for (int v = 0; v < 16; ++v) C[v] = c_in[(8 * (v / 4) + 4 * g + v % 4) * 32 + r];
  v16f D;
  if (kind == 0)
    D = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, ua), __builtin_bit_cast(v8h, ub), C, 0, 0, 0);
  else
    D = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, ua), __builtin_bit_cast(v8bf, ub), C, 0, 0,
                                                0);
#pragma unroll
  for (int v = 0; v < 16; ++v) out[(8 * (v / 4) + 4 * g + v % 4) * 32 + r] = D[v];
}

}  // namespace

// The hardware base-2 exponential (v_exp_f32, what the attention kernel's
// probabilities go through) on n given arguments.
__global__ __launch_bounds__(256) void k_exp2(const float* x, float* y, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) y[i] = __builtin_amdgcn_exp2f(x[i]);
}

extern "C" {

// MFMA loops: `blocks` workgroups of 256 threads, `iters` rounds of 8 MFMAs per
// wave.  sink: blocks * 256 floats; clocks: blocks * 4 uint64.  kind 0: fp8
// (32x32x64, 131072 flops each), 1: fp16 (32x32x16, 32768 flops each).
int probe_mfma_loop(int kind, int blocks, int iters, float* sink, uint64_t* clocks, void* stream) {
  if (kind == 0)
    hipLaunchKernelGGL(k_loop_fp8, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, sink, clocks);
  else
    hipLaunchKernelGGL(k_loop_f16, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, sink, clocks);
  return (int)hipGetLastError();
}

// Copy n_bytes (a multiple of 16) from src to dst.
int probe_copy(const void* src, void* dst, int64_t n_bytes, int blocks, void* stream) {
  hipLaunchKernelGGL(k_copy, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const uint4*)src, (uint4*)dst,
                     n_bytes / 16);
  return (int)hipGetLastError();
}

// Single matrix-core instructions on given operands (see the kernels above).
int probe_mfma_once_fp8(const void* a, const void* b, const float* c_in, float* out, void* stream) {
  hipLaunchKernelGGL(k_once_fp8, dim3(1), dim3(64), 0, (hipStream_t)stream, (const uint8_t*)a, (const uint8_t*)b,
                     c_in, out);
  return (int)hipGetLastError();
}

int probe_mfma_once_16(const void* a, const void* b, const float* c_in, float* out, int kind, void* stream) {
  hipLaunchKernelGGL(k_once_16, dim3(1), dim3(64), 0, (hipStream_t)stream, (const uint16_t*)a, (const uint16_t*)b,
                     c_in, out, kind);
  return (int)hipGetLastError();
}

// The MXFP8 GEMM (E4M3, tiled scales, no epilogue) with each A stage DMA'd twice:
// the lower bound of a GEMM that reads bf16 activations to quantize them itself.
// Operands validated by the caller: M, N, K multiples of 128, operands < 2 GiB.
int probe_gemm_mxfp8_a_twice(const void* a_q, const void* a_s, const void* w_q, const void* w_s, int64_t M,
                             int64_t N, int64_t K, void* c, void* stream) {
  return (int)mxq::launch_gemm_mxfp8_a_twice(a_q, a_s, w_q, w_s, M, N, K, c, (hipStream_t)stream);
}

// Rate of the constant clock s_memrealtime counts (Hz).
int64_t probe_wall_clock_hz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
  return (int64_t)khz * 1000;
}

// y[i] = v_exp_f32(x[i]) for i < n (device fp32 arrays).
int probe_exp2(const float* x, float* y, int n, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_exp2, dim3((n + 255) / 256), dim3(256), 0, (hipStream_t)stream, x, y, n);
  return (int)hipGetLastError();
}

}  // extern "C"
