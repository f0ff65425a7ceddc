// Split-K completion of the tiles a persistent GEMM launch leaves for its last,
// partial round.
//
// A launch with T output tiles on P persistent workgroups runs ceil(T / P) rounds;
// when T % P is small, the last round keeps most compute units idle.  Instead,
// the first T - T % P tiles are computed whole (the same number per workgroup) and
// each remaining tile is cut along K into `parts` ranges, one workgroup per range,
// so the last round takes 1 / parts of a tile's time.  Each range's fp32 sum goes
// to a partial tile; this kernel adds a tile's parts in order and applies the
// GEMM's epilogue (alpha, bias, GELU-tanh, one rounding to bf16).  The order of
// the fp32 additions differs from the unsplit accumulation, which is within the
// GEMMs' tolerance like any other accumulation order.
#include "mxq_internal.h"

namespace mxq {

GemmSplit plan_gemm_split(int tiles, int cus, int nk) {
  GemmSplit sp{tiles, 0, nullptr};
  if (tiles <= cus) return sp;
  const int tail = tiles % cus;
  if (tail == 0) return sp;
  for (int s = 2; tail * s <= cus; ++s)
    if (nk % s == 0 && (nk / s) % 2 == 0) sp.parts = s;
  if (sp.parts) sp.dp_tiles = tiles - tail;
  return sp;
}

size_t gemm_split_bytes(const GemmSplit& sp, int tiles) {
  if (!sp.parts) return 0;
  return (size_t)(tiles - sp.dp_tiles) * sp.parts * 256 * 256 * sizeof(float);
}

namespace {

// One workgroup per 8-row band of a split tile; thread -> one row, 8 columns.
template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_fixup(const float* __restrict__ partial, int parts, int dp_tiles,
                                                    int tiles_m, int tiles_n, const float* __restrict__ alpha_a,
                                                    const float* __restrict__ alpha_b,
                                                    const uint16_t* __restrict__ bias, uint16_t* __restrict__ c,
                                                    int M, int N) {
  const int t = blockIdx.x / 32, band = blockIdx.x % 32;
  const int row = band * 8 + (int)threadIdx.x / 32, col = ((int)threadIdx.x % 32) * 8;
  int m0, n0;
  dev::tile_origin(dp_tiles + t, tiles_m, tiles_n, m0, n0);
  const int m = m0 + row, n = n0 + col;
  if (m >= M || n >= N) return;   // N is a multiple of 128: eight columns are all in or all out
  float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int p = 0; p < parts; ++p) {
    const float* src = partial + ((size_t)(t * parts + p) * 256 + row) * 256 + col;
    const float4 lo = *(const float4*)src, hi = *(const float4*)(src + 4);
    y[0] += lo.x;
    y[1] += lo.y;
    y[2] += lo.z;
    y[3] += lo.w;
    y[4] += hi.x;
    y[5] += hi.y;
    y[6] += hi.z;
    y[7] += hi.w;
  }
  const float alpha = (alpha_a ? *alpha_a : 1.0f) * (alpha_b ? *alpha_b : 1.0f);
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] *= alpha;
  if (EPI >= 1) {
    const uint4 b = *(const uint4*)(bias + n);
    const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      y[2 * e] += dev::bf16_lo(bw[e]);
      y[2 * e + 1] += dev::bf16_hi(bw[e]);
    }
  }
  if (EPI == 2) {
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = dev::gelu_tanh(y[e]);
  }
  uint4 o;
  o.x = dev::pack_bf16x2(y[0], y[1]);
  o.y = dev::pack_bf16x2(y[2], y[3]);
  o.z = dev::pack_bf16x2(y[4], y[5]);
  o.w = dev::pack_bf16x2(y[6], y[7]);
  *(uint4*)(c + (size_t)m * N + n) = o;
}

}  // namespace

hipError_t launch_gemm_fixup(const GemmSplit& sp, int64_t M, int64_t N, const float* alpha_a, const float* alpha_b,
                             const void* bias, int epi, void* c, hipStream_t stream) {
  if (!sp.parts) return hipSuccess;
  const int tiles_m = (int)((M + 255) / 256), tiles_n = (int)((N + 255) / 256);
  const int split_tiles = tiles_m * tiles_n - sp.dp_tiles;
  dim3 grid(split_tiles * 32), block(256);
  auto B = (const uint16_t*)bias;
  auto C = (uint16_t*)c;
  const int m = (int)M, n = (int)N;
  if (epi == 0)
    hipLaunchKernelGGL(k_gemm_fixup<0>, grid, block, 0, stream, sp.partial, sp.parts, sp.dp_tiles, tiles_m, tiles_n,
                       alpha_a, alpha_b, B, C, m, n);
  else if (epi == 1)
    hipLaunchKernelGGL(k_gemm_fixup<1>, grid, block, 0, stream, sp.partial, sp.parts, sp.dp_tiles, tiles_m, tiles_n,
                       alpha_a, alpha_b, B, C, m, n);
  else
    hipLaunchKernelGGL(k_gemm_fixup<2>, grid, block, 0, stream, sp.partial, sp.parts, sp.dp_tiles, tiles_m, tiles_n,
                       alpha_a, alpha_b, B, C, m, n);
  return hipGetLastError();
}

}  // namespace mxq
