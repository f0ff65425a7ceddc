// Weight-only FP8 GEMM for gfx950:  C[M,N] = epi(s_w A[M,K] . W[N,K]^T), bf16 out,
// A in bf16, W in E4M3 with one fp32 per-tensor decode scale s_w.
//
// Definition (page "麦橘超然性能实战分析：float8量化如何提升GPU利用率", section 3.2:
// the DiT weights are kept as float8_e4m3fn while activations stay bf16, and
// converted back for the product; page "FP8量化技术提升SD3.5在低带宽环境下的响应速度",
// step 2: q = round(w / scale), dequantized as q * scale):
//   C[m,n] = epi( s_w sum_k a[m,k] val(q[n,k]) )
// with fp32 accumulation and one round-to-nearest-even to bf16.
//
// Scheme.  Every E4M3 value (4 significant bits, magnitudes 2^-9 .. 448) is exact
// in bf16, so W is converted in registers (v_cvt_scalef32_pk_bf16_fp8, scale 1)
// and multiplied with the bf16 activations by v_mfma_f32_32x32x16_bf16: exact
// products, fp32 accumulation.  s_w is applied once, in the epilogue.
//
// Operand layout (measured on gfx950): lane l holds row l % 32 and K [8g, 8g+8) of
// the 16-K step (g = l / 32); result D[8(v/4) + 4g + v%4][l % 32].  W is the first
// operand, A the second (each lane stores 4 consecutive n).  Inside each 32-K
// group lane group g takes the 16 consecutive values [16g, 16g+16) -- one 16-byte
// LDS read of W codes, two of A -- and K-step j their values [8j, 8j+8); both
// operands use this K order.
//
// Tiling as the block-scaled kernels: 256 x 256 output tiles, 4 waves of 128 x 128,
// both operands copied global -> LDS by buffer_load ... lds into two stage buffers
// of 64 K (A rows of 128 bytes, W rows of 64 bytes, XOR-swizzled), one 32-K group
// per half stage around the mid-stage barrier; persistent over tiles.
#include <type_traits>

#include "mxq_internal.h"

namespace mxq {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kThreads = 256;
constexpr int kTile = 256;
constexpr int kBK = 64;                        // K values per stage
constexpr int kRowA = kBK * 2;                 // 128 bytes of bf16 per A row and stage
constexpr int kRowW = kBK;                     // 64 bytes of E4M3 per W row and stage
constexpr int kOpA = kTile * kRowA;            // 32 KiB
constexpr int kOpW = kTile * kRowW;            // 16 KiB
constexpr int kStage = kOpW + kOpA;            // W then A
constexpr int kGroupM = 4;
constexpr int kCStage = dev::epilogue_lds_bytes(128);   // epilogue staging per wave

// Swizzles: 128-byte A rows keep 16-byte chunk c at c ^ ((row >> 1) & 7), 64-byte W
// rows at c ^ ((row >> 2) & 3); the 16 rows of a quarter-wave read then land on
// 16 distinct bank groups.
__device__ __forceinline__ int swz_a(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int swz_w(int row) { return (row >> 2) & 3; }

// Eight E4M3 codes (two dwords) -> eight bf16 values, exactly.
__device__ __forceinline__ v8bf dequant8(uint32_t lo, uint32_t hi) {
  v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return v8bf{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

template <int EPI>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_w8(
    const uint16_t* __restrict__ a, const uint8_t* __restrict__ wq, const float* __restrict__ wscale,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ c, int M, int N, int K) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[kStage];
  // per wave: the bias of its 128 columns (the first 256 B of one 1 KiB DMA), and
  // its output rows on their way to global memory
  __shared__ __attribute__((aligned(16))) uint8_t bias_lds[4 * 1024];
  __shared__ __attribute__((aligned(16))) uint8_t c_lds[4 * kCStage];

  const int tiles_m = (M + kTile - 1) / kTile, tiles_n = (N + kTile - 1) / kTile;
  const int n_tiles = tiles_m * tiles_n;
  const int nk = K / kBK;
  const int my_tiles = (n_tiles - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  auto origin = [&](int ti, int& m0, int& n0) {
    const int v = blockIdx.x + ti * gridDim.x;
    const int wg_id = dev::xcd_remap(v, n_tiles);
    const int per_group = kGroupM * tiles_n;
    const int first_m = (wg_id / per_group) * kGroupM;
    const int gsize = min(tiles_m - first_m, kGroupM);
    m0 = (first_m + (wg_id % per_group) % gsize) * kTile;
    n0 = ((wg_id % per_group) / gsize) * kTile;
  };

  const int t = threadIdx.x;
  int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wn = wave & 1, wm = wave >> 1;
  int r = lane & 31, g = lane >> 5;
  const int KA = K * 2;                 // bytes per A row

  // 32-bit offsets: operands are < 2 GiB (checked by the host)
  const auto ra = __builtin_amdgcn_make_buffer_rsrc((void*)a, (short)0, M * KA, 0x00020000);
  const auto rw = __builtin_amdgcn_make_buffer_rsrc((void*)wq, (short)0, N * K, 0x00020000);
  const auto rb = __builtin_amdgcn_make_buffer_rsrc((void*)bias, (short)0, EPI >= 1 ? N * 2 : 0, 0x00020000);

  // Global -> LDS, 1 KiB per wave and load.  A: 8 rows of 128 B per load, lane i ->
  // row i / 8, physical chunk i % 8; rows 8j + i/8 have swizzle ((i/8) >> 1) + 4 (j & 1),
  // hence two lane offsets.  W: 16 rows of 64 B per load, lane i -> row i / 4,
  // physical chunk i % 4; rows 16j + i/4 have swizzle (i >> 4) & 3 for every j.
  int voa0, voa1, vow;
  // Every load stays inside its operand: a wave's 64 rows lie wholly inside or past
  // M (N); rows past the end, and stages after the last tile, read rows [0, 64).
  // Part p (0..3) of a stage: W rows 16p.. of this wave's 64, A rows 16p.. (two loads).
  auto dma_part = [&](int p, uint8_t* buf, int m0, int n0, int k0, bool valid) {
    const int rw0 = n0 + wave * 64, ra0 = m0 + wave * 64;
    const bool vw = valid && rw0 < N, va = valid && ra0 < M;
    const int off_w = vw ? rw0 * K + k0 : 0, off_a = va ? ra0 * KA + k0 * 2 : 0;
    uint8_t* bw = buf + wave * 64 * kRowW;
    uint8_t* ba = buf + kOpW + wave * 64 * kRowA;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_ptr_t)(bw + p * 16 * kRowW), 16, vow, off_w + p * 16 * K, 0,
                                             0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(ba + (2 * p) * 8 * kRowA), 16, voa0,
                                             off_a + (2 * p) * 8 * KA, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(ba + (2 * p + 1) * 8 * kRowA), 16, voa1,
                                             off_a + (2 * p + 1) * 8 * KA, 0, 0);
  };
  auto dma_stage = [&](uint8_t* buf, int m0, int n0, int k0, bool valid) {
#pragma unroll
    for (int p = 0; p < 4; ++p) dma_part(p, buf, m0, n0, k0, valid);
  };

  int xw, xa, wrow, arow2;                   // rows wn*128 + 32i + r share xw, xa
  // The lane-derived offsets are recomputed at the top of every tile from the lane
  // id (mbcnt, in a volatile asm block so that it is not hoisted): otherwise they
  // stay live across the epilogue, get spilled there, and their reloads queue
  // behind its stores.
  auto lane_setup = [&](bool opaque) {
    if (opaque) asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
    r = lane & 31;
    g = lane >> 5;
    const int arow = lane >> 3, achunk = lane & 7;
    const int acx = achunk ^ (arow >> 1);
    voa0 = arow * KA + acx * 16;
    voa1 = arow * KA + (acx ^ 4) * 16;
    vow = (lane >> 2) * K + (((lane & 3) ^ ((lane >> 4) & 3)) << 4);
    xw = swz_w(r);
    xa = swz_a(r);
    wrow = wn * 128 + r;
    arow2 = wm * 128 + r;
  };
  lane_setup(false);
  uint4 cw0[4], cw1[4];                      // W codes of the stage's 32-K groups 0 and 1
  uint4 a0[4][2], a1[4][2];                  // A (bf16) of groups 0 and 1: two K-steps each
  v8bf dw[2][4];                             // dequantized W, double-buffered by K-step

  // group G's W codes (chunk 2G + g) and A values (chunks 4G + 2g, 4G + 2g + 1)
  auto read_group = [&](uint4 (&cw)[4], uint4 (&av)[4][2], const uint8_t* buf, int G) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      cw[i] = *(const uint4*)(buf + (wrow + 32 * i) * kRowW + (((2 * G + g) ^ xw) << 4));
      const uint8_t* pa = buf + kOpW + (arow2 + 32 * i) * kRowA;
      av[i][0] = *(const uint4*)(pa + (((4 * G + 2 * g) ^ xa) << 4));
      av[i][1] = *(const uint4*)(pa + (((4 * G + 2 * g + 1) ^ xa) << 4));
    }
  };
  auto dequant = [&](auto B_, auto J_, const uint4 (&cw)[4]) {
    constexpr int B = decltype(B_)::value, J = decltype(J_)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i) dw[B][i] = J == 0 ? dequant8(cw[i].x, cw[i].y) : dequant8(cw[i].z, cw[i].w);
  };
  auto mfma_step = [&](v16f (&acc)[4][4], auto B_, auto J_, const uint4 (&av)[4][2]) {
    constexpr int B = decltype(B_)::value, J = decltype(J_)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dw[B][i], __builtin_bit_cast(v8bf, av[j][J]),
                                                            acc[i][j], 0, 0, 0);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  // 16 MFMAs, each followed by one of the next step's conversions (and, for the
  // first `reads` MFMAs, one LDS read; when `vmem`, the six DMA loads issued just
  // before, spread over the step)
  auto interleave = [&](int reads, bool vmem) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);  // VALU
      if (i < reads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (vmem && (i % 3 == 1) && i < 17) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  const float alpha = *wscale;
  auto epilogue = [&](const v16f (&acc)[4][4], int m0, int n0) {
    // M and N are multiples of 128: a wave's 128 x 128 block is wholly in or out
    if (m0 + wm * 128 >= M || n0 + wn * 128 >= N) return;
    dev::epilogue_block<EPI, 128, true>(acc, alpha, bias_lds + wave * 1024, c_lds + wave * kCStage, c, N,
                                        m0 + wm * 128, n0 + wn * 128, lane);
  };

  // One stage (cur holds it, nxt the next one):
  //   A: group 0's two K-steps || LDS reads of group 1; the last step converts
  //      group 1's first step
  //   B: wait for the next stage's DMA and this wave's reads, barrier (a tile's
  //      first stage finds the next stage's DMA retired before the previous tile's
  //      epilogue and waits for its reads only, leaving the epilogue's stores in
  //      flight)
  //   C: group 1's K-steps || LDS reads of the next stage's group 0, DMA of the
  //      stage after next into cur (in four parts); the last step converts the
  //      next stage's first step.
  // On entry dw[0] holds group 0's first step.
  auto stage = [&](auto first_, v16f (&acc)[4][4], uint8_t* cur, uint8_t* nxt, int dm0, int dn0, int dk0,
                   bool dvalid) {
    // ---- A
    read_group(cw1, a1, cur, 1);
    mfma_step(acc, I0(), I0(), a0);
    dequant(I1(), I1(), cw0);
    interleave(6, false);
    mfma_step(acc, I1(), I1(), a0);
    dequant(I0(), I0(), cw1);
    interleave(6, false);
    // ---- B
    if constexpr (decltype(first_)::value) __builtin_amdgcn_s_waitcnt(dev::kWaitLgkm);
    else __builtin_amdgcn_s_waitcnt(dev::kWaitAll);
    dev::lds_barrier();
    // ---- C
    read_group(cw0, a0, nxt, 0);
    dma_part(0, cur, dm0, dn0, dk0, dvalid);
    dma_part(1, cur, dm0, dn0, dk0, dvalid);
    mfma_step(acc, I0(), I0(), a1);
    dequant(I1(), I1(), cw1);
    interleave(12, true);
    dma_part(2, cur, dm0, dn0, dk0, dvalid);
    dma_part(3, cur, dm0, dn0, dk0, dvalid);
    mfma_step(acc, I1(), I1(), a1);
    dequant(I0(), I0(), cw0);
    interleave(0, true);
  };

  int m0 = 0, n0 = 0, m0n = 0, n0n = 0;
  origin(0, m0, n0);
  if (my_tiles > 1) origin(1, m0n, n0n);

  // Prologue: the first two stages in flight; wait; stage 0's group 0 and first step.
  {
    const bool nx1 = nk < 2;
    dma_stage(lds0, m0, n0, 0, true);
    dma_stage(lds1, nx1 ? m0n : m0, nx1 ? n0n : n0, nx1 ? 0 : kBK, !nx1 || my_tiles > 1);
  }
  __builtin_amdgcn_s_waitcnt(dev::kWaitVm);
  dev::lds_barrier();
  read_group(cw0, a0, lds0, 0);
  dequant(I0(), I0(), cw0);

  // Global stage s uses buffer s & 1; with an even number of stages per tile every
  // tile starts in buffer 0 (the launcher gives each workgroup one tile otherwise).
  using First = std::integral_constant<bool, true>;
  using Later = std::integral_constant<bool, false>;
  for (int ti = 0; ti < my_tiles; ++ti) {
    lane_setup(true);
    const bool has_next = ti + 1 < my_tiles;
    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    auto one = [&](auto first_, uint8_t* b0, uint8_t* b1, int kt) {
      const int kk = kt + 2;
      const bool nx = kk >= nk;
      stage(first_, acc, b0, b1, nx ? m0n : m0, nx ? n0n : n0, (nx ? kk - nk : kk) * kBK, !nx || has_next);
    };
    one(First(), lds0, lds1, 0);
    // the tile's bias, read by this wave's epilogue from LDS, so that no global load
    // there queues behind the epilogue's own stores (issued after the first stage:
    // its reads then need not wait for it)
    if constexpr (EPI >= 1) dev::load_bias(rb, bias_lds + wave * 1024, n0 + wn * 128, lane);
    int kt = 1;
    for (; kt + 1 < nk; kt += 2) {
      one(Later(), lds1, lds0, kt);
      one(Later(), lds0, lds1, kt + 1);
    }
    if (kt < nk) one(Later(), lds1, lds0, kt);
    // Retire the next tile's first two stages of DMA now: the stores below share
    // the counter, and the next tile's first stage then waits for none of them.
    __builtin_amdgcn_s_waitcnt(dev::kWaitVm);
    epilogue(acc, m0, n0);
    m0 = m0n;
    n0 = n0n;
    if (ti + 2 < my_tiles) origin(ti + 2, m0n, n0n);
  }
  __builtin_amdgcn_s_waitcnt(dev::kWaitVm);   // no DMA outlives the workgroup
}

}  // namespace

// Shapes reaching here are validated: M, N, K positive multiples of 128, epi 0..2.
hipError_t launch_gemm_w8(const void* a, const void* w_q, const float* w_scale, int64_t M, int64_t N, int64_t K,
                          const void* bias, int epi, void* c, hipStream_t stream) {
  const int m = (int)M, n = (int)N, k = (int)K;
  const int tiles = ((m + kTile - 1) / kTile) * ((n + kTile - 1) / kTile);
  // persistent (one workgroup per CU) when a tile has an even number of K stages
  // (always: K is a multiple of 128), unless there are fewer tiles than CUs
  const int cus = device_compute_units();
  const int grid_n = ((k / kBK) % 2 != 0 || tiles < cus) ? tiles : cus;
  dim3 grid(grid_n), block(kThreads);
  auto A = (const uint16_t*)a;
  auto W = (const uint8_t*)w_q;
  auto B = (const uint16_t*)bias;
  auto C = (uint16_t*)c;
  if (epi == 0) hipLaunchKernelGGL(k_gemm_w8<0>, grid, block, 0, stream, A, W, w_scale, B, C, m, n, k);
  else if (epi == 1) hipLaunchKernelGGL(k_gemm_w8<1>, grid, block, 0, stream, A, W, w_scale, B, C, m, n, k);
  else hipLaunchKernelGGL(k_gemm_w8<2>, grid, block, 0, stream, A, W, w_scale, B, C, m, n, k);
  return hipGetLastError();
}

}  // namespace mxq
