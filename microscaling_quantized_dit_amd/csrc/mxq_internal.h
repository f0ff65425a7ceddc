// Internal declarations shared by the gfx950 kernels and the C-ABI host layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

// Compute units of the current device (cached per device; 256 on MI355X).
int device_compute_units();

// Block scales in the GEMM-tiled order: the scales of a [rows, cols] tensor stored
// as [rows / 64][cols / 128][64 rows][P bytes], P = scales per 128 values (4 for
// MXFP8, 8 for NVFP4); rows % 64 == 0, cols % 128 == 0, rows * cols < 2^43.
// The quantizers take nst = 0 for row-major scales.
struct ScaleTiling {
  int64_t cpr;  // 16-byte chunks (8 values) per row
  int nst;      // 128-value steps per row; 0 = row-major scales
};
ScaleTiling scale_tiling(int64_t cols);   // cols 0 -> row-major

// Host-side launchers (each returns the hipError_t of its launch).
hipError_t launch_quantize_mxfp8(const void* x, int64_t n_elems, int kind, void* q, void* scales,
                                 ScaleTiling tiling, hipStream_t stream);

// Workgroups (= partial maxima) the NVFP4 amax pass uses for n_elems.
int nvfp4_amax_partials(int64_t n_elems);

// Device address (for the current device) and size in words of the library's
// own partial-maxima scratch, a file-scope device array used by the entry point
// that allocates nothing.  Looked up once per device with hipGetSymbolAddress.
hipError_t amax_scratch(uint32_t** ptr, int* words);
hipError_t launch_quantize_nvfp4(const void* x, int64_t n_elems, const float* global_in, void* q,
                                 void* scales, float* global_out, uint32_t* partials,
                                 ScaleTiling tiling, hipStream_t stream);

// running = max(running, RN_fp32(amax(x) / 2688)); partials as for the quantizer.
hipError_t launch_nvfp4_calibrate(const void* x, int64_t n_elems, float* running, uint32_t* partials,
                                  hipStream_t stream);

// Per-tensor E4M3 weights: scale_in NULL = RN_fp32(amax / 448) via the partials.
hipError_t launch_quantize_fp8_tensor(const void* x, int64_t n_elems, const float* scale_in, void* q,
                                     float* scale_out, uint32_t* partials, hipStream_t stream);

// Work division of a persistent GEMM launch over its 256 x 256 output tiles (ids in
// the order of dev::tile_origin).  Tiles [0, dp_tiles) are computed whole, the same
// number by every workgroup.  Each remaining tile is cut along K into `parts`
// equal ranges; workgroup u < (n_tiles - dp_tiles) * parts computes range u % parts
// of tile dp_tiles + u / parts into partial[u] (256 x 256 fp32, row-major), and
// launch_gemm_fixup sums the parts and applies the epilogue.  parts == 0: no split.
struct GemmSplit {
  int dp_tiles;
  int parts;
  float* partial;
};

// Split for `tiles` tiles of `nk` K-stages on `cus` persistent workgroups: the
// remaining tiles cut into the most parts that still fit in one round, each part
// an even number (>= 2) of stages; parts = 0 when there is no partial last round
// or no such cut.  Bytes of partial tiles it needs.
GemmSplit plan_gemm_split(int tiles, int cus, int nk);
size_t gemm_split_bytes(const GemmSplit& sp, int tiles);

// Sums the K parts of the split tiles and writes epi(alpha * sum) to C (bf16),
// alpha = (*alpha_a) * (*alpha_b) with a null pointer read as 1.
hipError_t launch_gemm_fixup(const GemmSplit& sp, int64_t M, int64_t N, const float* alpha_a, const float* alpha_b,
                             const void* bias, int epi, void* c, hipStream_t stream);

// V of the FP8 attention: [heads * L, 128] bf16 -> codes in the attention's V
// layout (see k_quant_fp8_vt); partials as for the quantizers (scale_in NULL).
hipError_t launch_quantize_fp8_vt(const void* v, int64_t heads, int64_t L, const float* scale_in, void* vt,
                                  float* scale_out, uint32_t* partials, hipStream_t stream);

// FP8 attention: q, k codes [heads * L, 128], vt in the V layout, per-tensor
// decode scales, o bf16 [heads * L, 128]; L a multiple of 128.
hipError_t launch_attention_fp8(const void* q, const float* q_scale, const void* k, const float* k_scale,
                                const void* vt, const float* v_scale, int64_t heads, int64_t L, void* o,
                                hipStream_t stream);

hipError_t launch_gemm_w8(const void* a, const void* w_q, const float* w_scale, int64_t M, int64_t N, int64_t K,
                          const void* bias, int epi, void* c, hipStream_t stream);

// scales_tiled: both operands' scales in the tiled order above (else row-major)
hipError_t launch_gemm_mxfp8(const void* a_q, const void* a_s, int a_kind, const void* w_q,
                             const void* w_s, int w_kind, int64_t M, int64_t N, int64_t K,
                             const void* bias, int epi, void* c, bool scales_tiled, hipStream_t stream);

// a: bf16 [M, K]; kind: A's code format and W's; scales_tiled: W's scale order
hipError_t launch_gemm_mxfp8_fused(const void* a, int kind, const void* w_q, const void* w_s, int64_t M, int64_t N,
                                   int64_t K, const void* bias, int epi, void* c, bool scales_tiled,
                                   hipStream_t stream);

// workspace: NULL (no split) or at least gemm_nvfp4_workspace_bytes(M, N, K) bytes
size_t gemm_nvfp4_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_nvfp4(const void* a_q, const void* a_s, const float* a_g, const void* w_q,
                             const void* w_s, const float* w_g, int64_t M, int64_t N, int64_t K,
                             const void* bias, int epi, void* c, bool scales_tiled, void* workspace,
                             hipStream_t stream);

}  // namespace mxq

#if defined(__HIP_DEVICE_COMPILE__) || defined(__HIPCC__)
namespace mxq {
namespace dev {

// bf16 bit pattern (low/high half of a dword) widened exactly to fp32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Streaming load for data touched once (global_load with the nt bit set).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4_t*)p));
}

// Work split of the quantizers when they write tiled scales: workgroup b takes the
// 16 U rows from row 16 U (b / nst) on, columns [128 st, 128 st + 128) with
// st = b % nst, and thread t the 16-byte chunk t % 16 of that step in rows
// t / 16 + 16 u, u < U (16 U divides 64).  A wave's 64 lanes then cover four
// consecutive rows of one step: their scales are one contiguous run of the tiled
// order.  chunk(u) is the row-major chunk index, scale(u) + lane's block in the
// run the byte offset of the scale of row t / 16 + 16 u (P scales per row and step).
template <int U, int P>
struct TiledSlab {
  int64_t chunk0 = 0;  // chunk of the thread's first row
  int64_t scale0 = 0;  // scale run offset of the thread's first row
  int64_t cpr = 0;
  __device__ __forceinline__ TiledSlab() = default;   // row-major scales: unused
  __device__ __forceinline__ TiledSlab(int b, int t, const mxq::ScaleTiling& tl) : cpr(tl.cpr) {
    const int g = b / tl.nst, st = b - g * tl.nst;
    const int64_t row = (int64_t)g * (16 * U) + (t >> 4);
    chunk0 = row * tl.cpr + (int64_t)st * 16 + (t & 15);
    scale0 = ((row >> 6) * tl.nst + st) * (64 * P) + (row & 63) * P + (t & 15) / (16 / P);
  }
  __device__ __forceinline__ int64_t chunk(int u) const { return chunk0 + (int64_t)(16 * u) * cpr; }
  __device__ __forceinline__ int64_t scale(int u) const { return scale0 + 16 * u * P; }
};

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

// MXFP8 element formats: E4M3 ("fn", largest finite 448 = 1.75 * 2^8) and E5M2
// (largest finite 57344 = 1.75 * 2^15), with the hardware's round-to-nearest-even
// pair conversion into the low (HI = false) or high half of a dword.
template <int KIND>
struct Fp8Traits;
template <>
struct Fp8Traits<0> {
  static constexpr int emax = 8;
  static constexpr float maxval = 448.0f;
  template <bool HI>
  static __device__ __forceinline__ int cvt(float a, float b, int old) {
    return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
  }
};
template <>
struct Fp8Traits<1> {
  static constexpr int emax = 15;
  static constexpr float maxval = 57344.0f;
  template <bool HI>
  static __device__ __forceinline__ int cvt(float a, float b, int old) {
    return __builtin_amdgcn_cvt_pk_bf8_f32(a, b, old, HI);
  }
};

// MX block exponent E = floor(log2 amax) - emax, clamped to [-127, 127] (-127 for
// an all-zero block), from the block's largest bf16 magnitude bits.  For a normal
// amax floor(log2 amax) is its exponent field - 127; a subnormal (or zero) amax
// has floor(log2) <= -127 and every emax is positive, so the clamp gives -127
// whatever its mantissa: the exponent field alone decides.
template <int KIND>
__device__ __forceinline__ int mx_block_exponent(uint32_t amax_bits) {
  const int e = (int)(amax_bits >> 7) - 127 - Fp8Traits<KIND>::emax;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Four bf16 values (two dwords) times inv = 2^-E -> four fp8 codes.  x * 2^-E is
// exact in fp32; the hardware conversion rounds to nearest even but turns
// magnitudes at or above the saturation midpoint into NaN, so values are clamped
// to the largest finite one first (which never changes an RNE result below the
// clamp and yields the saturated code above it).
template <int KIND>
__device__ __forceinline__ int mx_encode4(uint32_t w0, uint32_t w1, float inv) {
  using T = Fp8Traits<KIND>;
  const float hi = T::maxval, lo = -T::maxval;
  float f0 = __builtin_amdgcn_fmed3f(bf16_lo(w0) * inv, lo, hi);
  float f1 = __builtin_amdgcn_fmed3f(bf16_hi(w0) * inv, lo, hi);
  float f2 = __builtin_amdgcn_fmed3f(bf16_lo(w1) * inv, lo, hi);
  float f3 = __builtin_amdgcn_fmed3f(bf16_hi(w1) * inv, lo, hi);
  int r = T::template cvt<false>(f0, f1, 0);
  return T::template cvt<true>(f2, f3, r);
}

// Two fp32 -> two bf16 (nearest, ties to even) packed low|high: v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
  v2bf r = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, r);
}

// GELU, tanh form: 0.5 y (1 + tanh(u)), u = sqrt(2/pi) (y + 0.044715 y^3).
// Since 1 + tanh(u) = 2 / (1 + e^(-2u)), this is y / (1 + 2^x) with
// x = -2 log2(e) u = y (c0 + c1 y^2), the constants folded (c0 = -2 log2(e)
// sqrt(2/pi), c1 = 0.044715 c0): one hardware exp2 and one reciprocal, each within
// about 1 ulp, five other operations, no cancellation for large negative y (the
// quotient tends to -0) and no overflow for large positive y (2^x tends to 0).
__device__ __forceinline__ float gelu_tanh(float y) {
  constexpr double kC0 = -2.0 * 1.4426950408889634 * 0.7978845608028654;
  const float c0 = (float)kC0;
  const float c1 = (float)(kC0 * 0.044715);
  const float x = y * __builtin_fmaf(y * y, c1, c0);
  return y * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x));
}

// s_waitcnt immediate for vmcnt = vm (0..63) and lgkmcnt = lgkm (0..15), expcnt
// left open.  vmcnt counts vector loads (LDS DMA included) and stores alike, and
// loads and stores may retire out of order with respect to each other.
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8); }
constexpr int kWaitLgkm = waitcnt_imm(63, 0);   // LDS reads only
constexpr int kWaitAll = waitcnt_imm(0, 0);     // vector memory and LDS reads
constexpr int kWaitVm = waitcnt_imm(0, 15);     // vector memory only

// Workgroup barrier without the memory fences of __syncthreads(): those make the
// compiler wait for every vector memory operation in flight, epilogue stores
// included.  The caller's s_waitcnt retires the LDS writes (DMA or ds_write) that
// the barrier publishes; the signal fences keep the compiler from moving LDS
// accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

typedef float v16f_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr;

// Bytes of LDS one wave needs to stage its output for epilogue_block<.., W, ..>.
constexpr int epilogue_lds_bytes(int W) { return 32 * (2 * W + 16); }

// The tile's bias for one wave's 128 columns [n, n + 128) -> bias_w in LDS (one
// 1 KiB DMA, of which the first 256 bytes are used; reads past the end of the bias
// return zeros).  Retired by the next vmcnt(0); the wave's own epilogue reads it.
__device__ __forceinline__ void load_bias(__amdgpu_buffer_rsrc_t rb, uint8_t* bias_w, int n, int lane) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr)bias_w, 16, lane * 16, n * 2, 0, 0);
}

// Epilogue of one wave's 128 x 128 block of a 32x32-MFMA GEMM, whose lane l holds
// in acc[i][j][v] the result for row 32j + l % 32 and column
// 32i + 8(v / 4) + 4(l / 32) + v % 4 of the block:
//   C[m_base + row][n_base + col] = bf16(epi(alpha * acc + bias[col]))
// (alpha applied when SCALE).  The block goes out 32 rows and W (128 or 64)
// columns at a time through `stage` (epilogue_lds_bytes(W) of this wave's LDS):
// each lane writes its values there, then reads 16 bytes of a row back, so that
// every global store covers whole row segments of 2W bytes instead of 32 rows of
// 16 bytes.  A wave's LDS accesses complete in order, so no barrier is needed.
template <int EPI, int W, bool SCALE>
__device__ __forceinline__ void epilogue_block(const v16f_t (&acc)[4][4], float alpha, const uint8_t* bias_w,
                                               uint8_t* stage, uint16_t* c, int N, int m_base, int n_base,
                                               int lane) {
  constexpr int kRow = 2 * W + 16;            // staged row bytes (+16 against bank conflicts)
  constexpr int kLanesPerRow = 2 * W / 16;    // 16-byte chunks per staged row
  constexpr int kRowsPerStore = 64 / kLanesPerRow;
  const int r = lane & 31, g = lane >> 5;
  const int srow = lane / kLanesPerRow, chunk = lane % kLanesPerRow;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int h = 0; h < 128 / W; ++h) {
#pragma unroll
      for (int ii = 0; ii < W / 32; ++ii) {
        const int i = h * (W / 32) + ii;
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const int col = 32 * i + 8 * qd + 4 * g;
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = SCALE ? alpha * acc[i][j][4 * qd + e] : acc[i][j][4 * qd + e];
          if (EPI >= 1) {
            const uint2 b = *(const uint2*)(bias_w + 2 * col);
            y[0] += bf16_lo(b.x);
            y[1] += bf16_hi(b.x);
            y[2] += bf16_lo(b.y);
            y[3] += bf16_hi(b.y);
          }
          if (EPI == 2) {
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = gelu_tanh(y[e]);
          }
          uint2 o;
          o.x = pack_bf16x2(y[0], y[1]);
          o.y = pack_bf16x2(y[2], y[3]);
          *(uint2*)(stage + r * kRow + 2 * (col - h * W)) = o;
        }
      }
      uint16_t* cb = c + (size_t)(m_base + 32 * j) * N + n_base + h * W + 8 * chunk;
#pragma unroll
      for (int q = 0; q < 32 / kRowsPerStore; ++q) {
        const int row = kRowsPerStore * q + srow;
        const uint4 v = *(const uint4*)(stage + row * kRow + 16 * chunk);
        *(uint4*)(cb + (size_t)row * N) = v;
      }
    }
  }
}

// Remap a linear workgroup id so that ids placed round-robin on the 8 XCDs
// become contiguous ranges per XCD (neighbouring tiles share one L2).
__device__ __forceinline__ int xcd_remap(int wg, int n_wg) {
  const int n_xcd = 8;
  int per = n_wg / n_xcd;
  if (wg >= per * n_xcd) return wg;
  return (wg % n_xcd) * per + wg / n_xcd;
}

// Origin of output tile v of a GEMM with tiles_m x tiles_n tiles of 256 x 256:
// ids spread round-robin over the XCDs become contiguous ranges per XCD, and a
// range walks groups of four M-tiles column by column, so that neighbouring
// workgroups share A and W panels in their L2.  A bijection on [0, tiles).
__device__ __forceinline__ void tile_origin(int v, int tiles_m, int tiles_n, int& m0, int& n0) {
  const int group_m = 4;
  const int wg = xcd_remap(v, tiles_m * tiles_n);
  const int per_group = group_m * tiles_n;
  const int first_m = (wg / per_group) * group_m;
  const int gsize = min(tiles_m - first_m, group_m);
  m0 = (first_m + (wg % per_group) % gsize) * 256;
  n0 = ((wg % per_group) / gsize) * 256;
}

// fp32 partial tile of a split unit: the wave's 128 x 128 block of acc (layout as
// for epilogue_block) into partial (256 x 256 fp32, row-major) at its place
// (wm, wn).  Staged like epilogue_block, 32 rows x 64 columns at a time through
// the same epilogue_lds_bytes(128) of LDS, so every store covers 256-byte rows.
__device__ __forceinline__ void store_partial(const v16f_t (&acc)[4][4], float* partial, uint8_t* stage, int wm,
                                              int wn, int lane) {
  constexpr int kRow = 4 * 64 + 16;
  const int r = lane & 31, g = lane >> 5;
  const int srow = lane >> 4, chunk = lane & 15;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const int i = 2 * h + ii;
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const int col = 32 * ii + 8 * qd + 4 * g;   // within the 64-column half
          *(float4*)(stage + r * kRow + 4 * col) =
              float4{acc[i][j][4 * qd], acc[i][j][4 * qd + 1], acc[i][j][4 * qd + 2], acc[i][j][4 * qd + 3]};
        }
      }
      float* dst = partial + (wm * 128 + 32 * j) * 256 + wn * 128 + 64 * h + 4 * chunk;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int row = 4 * q + srow;
        *(float4*)(dst + row * 256) = *(const float4*)(stage + row * kRow + 16 * chunk);
      }
    }
  }
}

}  // namespace dev
}  // namespace mxq
#endif
