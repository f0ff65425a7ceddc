// MXFP8 quantizer for gfx950: bf16 -> E4M3/E5M2 codes + one E8M0 scale per 32
// values along a row.
//
// Definition (page "NVIDIA量化推理：5步极速优化显存+成功率翻倍", section
// "MXFP8和NVFP4技术背景解析": MXFP8 = OCP 8-bit microscaling, blocks of 32 sharing
// one scale; page "FP8量化技术提升SD3.5…", step 2: q = round(x / scale)):
//   E = floor(log2 amax_block) - emax (8 for E4M3, 15 for E5M2), clamped to
//   [-127, 127], -127 for an all-zero block; scale byte E + 127;
//   q = RNE_sat(x / 2^E), sign bit copied from x.
//
// HBM-bound, one pass.  The tensor is treated as a flat stream (cols % 32 == 0,
// so blocks never straddle rows and the scale of element e is scales[e / 32]),
// read with streaming (nt) loads, each input byte being touched once.  The codes
// go out with ordinary stores: the GEMM reads them next, and codes left in the
// caches spare its first touch of HBM (the quantizer and the GEMM after a cache
// flush ran 0.5-6% faster together than with streaming stores).
// Scales go out row-major or in the GEMM-tiled order (mxq_internal.h); for the
// latter a workgroup takes 64 rows x 128 values, four rows per wave, so that
// each wave's scale bytes form one contiguous run.
// Each lane takes 8 consecutive values (one 16-byte load), four neighbouring
// lanes form a 32-block and find its amax with two cross-lane max steps.
// x / 2^E is exact in fp32 (2^-E is a normal fp32 for every reachable E), and
// the hardware fp8 conversion rounds to nearest even; it turns magnitudes at or
// above the saturation midpoint into NaN, so inputs are clamped to the largest
// finite value first (clamping an exactly scaled value never changes an RNE
// result below the clamp and yields the saturated code above it).
#include "mxq_internal.h"

namespace mxq {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 2;  // 16-byte chunks per lane, kept in flight together
constexpr int kUnrollTiled = 4;   // with tiled scales: 64 rows x 128 values per workgroup

// TILED: scales in the GEMM-tiled order, with the work split of dev::TiledSlab
// (every chunk in range); else the tensor is a flat stream of chunks.
template <int KIND, bool TILED>
__global__ __launch_bounds__(kThreads) void k_quant_mxfp8(const uint4* __restrict__ x, int64_t n_chunks,
                                                          uint2* __restrict__ q, uint8_t* __restrict__ s,
                                                          ScaleTiling tiling) {
  constexpr int U = TILED ? kUnrollTiled : kUnroll;
  const int t = threadIdx.x;
  const int64_t base = (int64_t)blockIdx.x * (kThreads * U);
  const auto ts = TILED ? dev::TiledSlab<U, 4>((int)blockIdx.x, t, tiling) : dev::TiledSlab<U, 4>();
  auto chunk = [&](int u) { return TILED ? ts.chunk(u) : base + u * kThreads + t; };
  uint4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t c = chunk(u);
    v[u] = TILED || c < n_chunks ? dev::load_nt(x + c) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t c = chunk(u);
    // Lanes 4j..4j+3 hold chunks 4j'..4j'+3 of one 32-block (n_chunks % 4 == 0,
    // so a group is entirely in or entirely out of range); their maxima meet
    // through two DPP swaps within the quad, [1,0,3,2] then [2,3,0,1].
    uint32_t m = dev::fold_halves_max(dev::mag_max_pk(v[u]));
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, false));
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xF, 0xF, false));
    const int E = dev::mx_block_exponent<KIND>(m);
    const float inv = __uint_as_float((uint32_t)(127 - E) << 23);  // 2^-E, normal
    uint2 out;
    out.x = (uint32_t)dev::mx_encode4<KIND>(v[u].x, v[u].y, inv);
    out.y = (uint32_t)dev::mx_encode4<KIND>(v[u].z, v[u].w, inv);
    if (TILED || c < n_chunks) {
      q[c] = out;
      if ((t & 3) == 0) s[TILED ? ts.scale(u) : c >> 2] = (uint8_t)(E + 127);
    }
  }
}

}  // namespace

hipError_t launch_quantize_mxfp8(const void* x, int64_t n_elems, int kind, void* q, void* scales,
                                 ScaleTiling tiling, hipStream_t stream) {
  const int64_t n_chunks = n_elems / 8;
  const int64_t per_wg = (int64_t)kThreads * (tiling.nst ? kUnrollTiled : kUnroll);
  const int64_t grid = (n_chunks + per_wg - 1) / per_wg;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 g((unsigned)grid), b(kThreads);
  auto X = (const uint4*)x;
  auto Q = (uint2*)q;
  auto S = (uint8_t*)scales;
  if (tiling.nst) {
    if (kind == 0) hipLaunchKernelGGL((k_quant_mxfp8<0, true>), g, b, 0, stream, X, n_chunks, Q, S, tiling);
    else hipLaunchKernelGGL((k_quant_mxfp8<1, true>), g, b, 0, stream, X, n_chunks, Q, S, tiling);
  } else {
    if (kind == 0) hipLaunchKernelGGL((k_quant_mxfp8<0, false>), g, b, 0, stream, X, n_chunks, Q, S, tiling);
    else hipLaunchKernelGGL((k_quant_mxfp8<1, false>), g, b, 0, stream, X, n_chunks, Q, S, tiling);
  }
  return hipGetLastError();
}

}  // namespace mxq
