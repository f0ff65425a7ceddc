// MXFP8 GEMM with the activation quantizer in its prologue, for gfx950:
//   C[M,N] = epi( Q(A)[M,K] . W[N,K]^T ),  A bf16, W MXFP8 codes + E8M0 scales,
// where Q is the MXFP8 activation quantizer of quant_mxfp8.hip (per row, blocks
// of 32 along K: E = floor(log2 amax) - emax, codes RNE_sat(x / 2^E)).
//
// Definition (page "NVIDIA Blackwell平台FP4量化技术解析与图像生成优化", section
// 3.1: at run time a bf16 activation is quantized dynamically and fed, with its
// scales, to the low-precision GEMM; page "NVIDIA量化推理：5步极速优化显存+成功率
// 翻倍", MXFP8 paragraph: blocks of 32 sharing one E8M0 scale).  The result is the
// one of mxq_quantize_mxfp8 followed by mxq_gemm_mxfp8, bit for bit: the same
// quantization helpers (mxq_internal.h), the same products in the same matrix-core
// instruction, accumulated in the same K order, and the same epilogue.  What is
// saved is the activation codes' trip through memory and the separate launch.
//
// Structure: the tiling, persistence, XCD-aware tile order, swizzles and epilogue
// of gemm_mxfp8.hip, with 64-K stages (a bf16 A stage is twice the bytes of an
// fp8 one and the LDS must hold two of them).  Per stage s, with the stage's W
// and quantized-A fragments already in registers:
//   a) wait for stage s+1's DMA (W codes and scale dwords, A bf16), barrier;
//   b) DMA stage s+2 into the buffers stage s used;
//   c) the MFMAs of stage s, interleaved with the quantization of stage s+1: each
//      lane encodes one row's 64 values (two blocks) from the bf16 buffer into the
//      fp8 buffer and its two scale bytes into the row's scale dword;
//   d) barrier; read stage s+1's fragments and scale dwords.
// A tile's first stage waits for LDS only (its DMA was retired before the previous
// tile's epilogue, whose stores drain meanwhile); its second waits for everything,
// since loads and those stores may retire out of order.
#include <type_traits>

#include "mxq_internal.h"

namespace mxq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kThreads = 256;
constexpr int kTile = 256;
constexpr int kBK = 64;                       // K values per stage
constexpr int kRowA = 2 * kBK;                // bf16 A row: 128 bytes
constexpr int kRowQ = kBK;                    // fp8 row (W, quantized A): 64 bytes
constexpr int kGroupM = 8;
constexpr int kCStage = dev::epilogue_lds_bytes(64);

// XOR swizzles of the 16-byte chunks of a row: eight chunks of a 128-byte row by
// (row / 2), four of a 64-byte row by (row / 4); the 16 rows a quarter-wave touches
// then cover all 64 banks.
__device__ __forceinline__ int swz128(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int swz64(int row) { return (row >> 2) & 3; }

// Four bf16 values (two dwords) -> four codes of x / 2^E, scale = 2^E: the
// hardware's scaled conversion (v_cvt_scalef32_pk_fp8_bf16 / _bf8_bf16), which
// divides by the scale exactly and rounds to nearest even -- the quantizer's
// codes (mxq_internal.h mx_encode4) for every finite input below the saturation
// midpoint (measured: every finite bf16 pattern under scales 2^-127 .. 2^127).
// Above it the conversion gives NaN (E4M3: 0x7F) or infinity (E5M2: 0x7C) where
// the quantizer clamps first; those codes are replaced by the largest finite one
// (0x7E, 0x7B), sign kept: adding 1 (E4M3) or 4 (E5M2) to a code's magnitude
// carries into bit 7 exactly for them.  Every magnitude reaching here is below
// 2^(emax+1) x 2^E, where no other code can come out.
template <int KIND>
__device__ __forceinline__ uint32_t enc4_hw(uint32_t w0, uint32_t w1, float scale) {
  typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
  typedef short v2s __attribute__((ext_vector_type(2)));
  v2s r = {0, 0};
  if constexpr (KIND == 0) {
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(v2bf, w0), scale, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(v2bf, w1), scale, true);
  } else {
    r = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(r, __builtin_bit_cast(v2bf, w0), scale, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(r, __builtin_bit_cast(v2bf, w1), scale, true);
  }
  const uint32_t c = __builtin_bit_cast(uint32_t, r);
  const uint32_t carry = KIND == 0 ? 0x01010101u : 0x04040404u;
  return c - ((((c & 0x7F7F7F7Fu) + carry) & 0x80808080u) >> 7);
}

// Fragment of the 32x32x64 operand for this lane from a 64-byte fp8 row: the
// 16-byte chunks g and g + 2 (K [16g, 16g+16) and [32+16g, 48+16g)).
__device__ __forceinline__ v8i frag(const uint8_t* buf, int R, int g) {
  const uint8_t* p = buf + R * kRowQ;
  const int x = swz64(R);
  uint4 lo = *(const uint4*)(p + ((g ^ x) << 4));
  uint4 hi = *(const uint4*)(p + (((2 + g) ^ x) << 4));
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

template <int KIND, int EPI, bool TILED>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_mxfp8_fused(
    const uint16_t* __restrict__ a, const uint8_t* __restrict__ wq, const uint8_t* __restrict__ ws,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ c, int M, int N, int K) {
  __shared__ __attribute__((aligned(1024))) uint8_t abf0[kTile * kRowA];   // A stage, bf16
  __shared__ __attribute__((aligned(1024))) uint8_t abf1[kTile * kRowA];
  __shared__ __attribute__((aligned(1024))) uint8_t w0[kTile * kRowQ];     // W stage, fp8
  __shared__ __attribute__((aligned(1024))) uint8_t w1[kTile * kRowQ];
  __shared__ __attribute__((aligned(1024))) uint8_t q0[kTile * kRowQ];     // A stage, quantized
  __shared__ __attribute__((aligned(1024))) uint8_t q1[kTile * kRowQ];
  __shared__ __attribute__((aligned(16))) uint32_t ws0[kTile], ws1[kTile];  // W scale dword per row
  __shared__ __attribute__((aligned(16))) uint32_t as0[kTile], as1[kTile];  // A scale bytes per row
  __shared__ __attribute__((aligned(16))) uint8_t bias_lds[4 * 1024];
  __shared__ __attribute__((aligned(16))) uint8_t c_lds[4 * kCStage];

  const int tiles_m = (M + kTile - 1) / kTile, tiles_n = (N + kTile - 1) / kTile;
  const int n_tiles = tiles_m * tiles_n;
  const int nk = K / kBK;   // stages per tile, even
  const int my_tiles = (n_tiles - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  auto origin = [&](int ti, int& m0, int& n0) {
    const int v = blockIdx.x + ti * gridDim.x;
    const int wg = dev::xcd_remap(v, n_tiles);
    const int per_group = kGroupM * tiles_n;
    const int first_m = (wg / per_group) * kGroupM;
    const int gsize = min(tiles_m - first_m, kGroupM);
    m0 = (first_m + (wg % per_group) % gsize) * kTile;
    n0 = ((wg % per_group) / gsize) * kTile;
  };

  const int t = threadIdx.x;
  int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wn = wave & 1, wm = wave >> 1;
  int r = lane & 31, g = lane >> 5;
  const int KB = K / 32;       // W scale bytes per row
  const int NST = K / 128;     // 128-K steps per row (TILED: scale runs per 64-row block)

  // 32-bit offsets: operands are < 2 GiB (checked by the host)
  const auto ra = __builtin_amdgcn_make_buffer_rsrc((void*)a, (short)0, M * K * 2, 0x00020000);
  const auto rw = __builtin_amdgcn_make_buffer_rsrc((void*)wq, (short)0, N * K, 0x00020000);
  const auto rsw = __builtin_amdgcn_make_buffer_rsrc((void*)ws, (short)0, N * KB, 0x00020000);
  const auto rb = __builtin_amdgcn_make_buffer_rsrc((void*)bias, (short)0, EPI >= 1 ? N * 2 : 0, 0x00020000);

  // Global -> LDS (buffer_load ... lds, 1 KiB per wave and load; wave w fills rows
  // [64w, 64w + 64)).  A bf16: 8 rows of 128 B per load, lane i -> row i / 8 and the
  // global chunk that lands at physical chunk i % 8 (swz128 of rows 8j + i/8 is
  // ((i/8) >> 1) + 4 (j & 1): two lane offsets).  W fp8: 16 rows of 64 B per load,
  // lane i -> row i / 4 (swz64 = (i >> 4) & 3 whatever the load).  W scale dwords:
  // one per row, lane i -> row 64w + i: the dword of the stage's 128-K step.
  // Every load stays inside its operand: rows past M (N), and stages after the last
  // tile, read rows [0, 64); their products only reach outputs never stored.
  int va0, va1, vw, vsc;
  auto dma_stage = [&](uint8_t* abuf, uint8_t* wbuf, uint32_t* wsbuf, int m0, int n0, int k0, bool valid) {
    const int ra0 = m0 + wave * 64, rw0 = n0 + wave * 64;
    const bool okA = valid && ra0 < M, okW = valid && rw0 < N;
    const int off_a = okA ? (ra0 * K + k0) * 2 : 0, off_w = okW ? rw0 * K + k0 : 0;
    const int st = k0 / 128;
    const int off_s = okW ? (TILED ? ((rw0 >> 6) * NST + st) * 256 : rw0 * KB + 4 * st) : 0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(abuf + (wave * 64 + 8 * j) * kRowA), 16,
                                               (j & 1) ? va1 : va0, off_a + 8 * j * K * 2, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_ptr_t)(wbuf + (wave * 64 + 16 * j) * kRowQ), 16, vw,
                                               off_w + 16 * j * K, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsw, (lds_ptr_t)(wsbuf + wave * 64), 4, vsc, off_s, 0, 0);
  };

  auto lane_setup = [&](bool opaque) {
    if (opaque) asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
    r = lane & 31;
    g = lane >> 5;
    const int arow = lane >> 3, achunk = lane & 7;
    const int cx = achunk ^ (arow >> 1);
    va0 = arow * K * 2 + cx * 16;
    va1 = arow * K * 2 + (cx ^ 4) * 16;
    vw = (lane >> 2) * K + (((lane & 3) ^ ((lane >> 4) & 3)) << 4);
    vsc = TILED ? lane * 4 : lane * KB;
  };
  lane_setup(false);

  // Quantization of one A stage: lane l of wave w encodes row 64w + l (both 32-blocks
  // of the stage) from abuf into qbuf, and its scale bytes into the row's dword.
  auto quantize = [&](const uint8_t* abuf, uint8_t* qbuf, uint32_t* asbuf) {
    const int row = wave * 64 + lane;
    const uint8_t* src = abuf + row * kRowA;
    const int xs = swz128(row), xq = swz64(row);
    uint32_t e2 = 0;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = *(const uint4*)(src + (((4 * blk + u) ^ xs) << 4));
      // the block's largest magnitude: each chunk's packed pair folded, then the four
      const uint32_t m = max(max(dev::fold_halves_max(dev::mag_max_pk(v[0])), dev::fold_halves_max(dev::mag_max_pk(v[1]))),
                             max(dev::fold_halves_max(dev::mag_max_pk(v[2])), dev::fold_halves_max(dev::mag_max_pk(v[3]))));
      const int E = dev::mx_block_exponent<KIND>(m);
      // 2^E as an fp32 (2^-127 is the subnormal 0x00400000)
      const float scale = __uint_as_float(E > -127 ? (uint32_t)(E + 127) << 23 : 0x00400000u);
      e2 |= (uint32_t)(E + 127) << (8 * blk);
#pragma unroll
      for (int h = 0; h < 2; ++h) {   // 16 values -> one 16-byte chunk of codes
        uint4 o;
        o.x = enc4_hw<KIND>(v[2 * h].x, v[2 * h].y, scale);
        o.y = enc4_hw<KIND>(v[2 * h].z, v[2 * h].w, scale);
        o.z = enc4_hw<KIND>(v[2 * h + 1].x, v[2 * h + 1].y, scale);
        o.w = enc4_hw<KIND>(v[2 * h + 1].z, v[2 * h + 1].w, scale);
        *(uint4*)(qbuf + row * kRowQ + (((2 * blk + h) ^ xq) << 4)) = o;
      }
    }
    asbuf[row] = e2;
  };

  v8i fw[4], fa[4];
  uint32_t scw[4], sca[4];
  auto read_frags = [&](const uint8_t* wbuf, const uint8_t* qbuf, const uint32_t* wsbuf, const uint32_t* asbuf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fw[i] = frag(wbuf, wn * 128 + 32 * i + r, g);
      fa[i] = frag(qbuf, wm * 128 + 32 * i + r, g);
      scw[i] = wsbuf[wn * 128 + 32 * i + r] >> (8 * g);
      sca[i] = asbuf[wm * 128 + 32 * i + r] >> (8 * g);
    }
  };

  auto epilogue = [&](const v16f (&acc)[4][4], int m0, int n0) {
    if (m0 + wm * 128 >= M || n0 + wn * 128 >= N) return;
    dev::epilogue_block<EPI, 64, false>(acc, 1.0f, bias_lds + wave * 1024, c_lds + wave * kCStage, c, N,
                                        m0 + wm * 128, n0 + wn * 128, lane);
  };

  // One stage: buffers (b*) of this stage hold its data, (n*) the next stage's.
  // HALF: the stage's 64-K half of its 128-K step (the W scale byte pair).
  auto stage = [&](auto kind_, auto half_, v16f (&acc)[4][4], uint8_t* ab, uint8_t* wb, uint32_t* wsb,
                   uint8_t* an, uint8_t* wn_, uint8_t* qn, uint32_t* wsn, uint32_t* asn, int dm0, int dn0, int dk0,
                   bool dvalid) {
    constexpr int kind = decltype(kind_)::value, HALF = decltype(half_)::value;
    // a) stage s+1's DMA has landed (a tile's first stage: retired before the epilogue)
    if constexpr (kind == 0) __builtin_amdgcn_s_waitcnt(dev::kWaitLgkm);
    else __builtin_amdgcn_s_waitcnt(dev::kWaitAll);
    dev::lds_barrier();
    // b) stage s+2 into this stage's buffers (its A was quantized, its W read)
    dma_stage(ab, wb, wsb, dm0, dn0, dk0, dvalid);
    __builtin_amdgcn_sched_barrier(0);
    // c) MFMAs of stage s || quantization of stage s+1
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fw[i], fa[j], acc[i][j], KIND, KIND, 2 * HALF,
                                                                   (int)scw[i], 0, (int)sca[j]);
    quantize(an, qn, asn);
    // the quantization's LDS reads first, then each MFMA followed by a share of its
    // VALU work, its LDS writes last
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 14, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x200, 5, 0);
    __builtin_amdgcn_sched_barrier(0);
    // d) stage s+1's quantized A visible; its fragments
    __builtin_amdgcn_s_waitcnt(dev::kWaitLgkm);
    dev::lds_barrier();
    read_frags(wn_, qn, wsn, asn);
    __builtin_amdgcn_sched_barrier(0);
  };

  int m0 = 0, n0 = 0, m0n = 0, n0n = 0;
  origin(0, m0, n0);
  if (my_tiles > 1) origin(1, m0n, n0n);

  // Prologue: stages 0 and 1 in flight; stage 0 quantized; its fragments.
  dma_stage(abf0, w0, ws0, m0, n0, 0, true);
  dma_stage(abf1, w1, ws1, m0, n0, kBK, true);
  __builtin_amdgcn_s_waitcnt(dev::kWaitAll);
  dev::lds_barrier();
  quantize(abf0, q0, as0);
  __builtin_amdgcn_s_waitcnt(dev::kWaitLgkm);
  dev::lds_barrier();
  read_frags(w0, q0, ws0, as0);

  // Stage s of a tile uses buffers s & 1 (nk is even); its DMA target, stage s + 2,
  // may be the next tile's.
  using First = std::integral_constant<int, 0>;
  using Later = std::integral_constant<int, 1>;
  using H0 = std::integral_constant<int, 0>;
  using H1 = std::integral_constant<int, 1>;
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
    auto one = [&](auto kind_, auto half_, bool odd, int kt) {
      const int kk = kt + 2;
      const bool nx = kk >= nk;
      const int dm0 = nx ? m0n : m0, dn0 = nx ? n0n : n0, dk0 = (nx ? kk - nk : kk) * kBK;
      const bool dv = !nx | has_next;
      if (odd)
        stage(kind_, half_, acc, abf1, w1, ws1, abf0, w0, q0, ws0, as0, dm0, dn0, dk0, dv);
      else
        stage(kind_, half_, acc, abf0, w0, ws0, abf1, w1, q1, ws1, as1, dm0, dn0, dk0, dv);
    };
    one(First(), H0(), false, 0);
    if constexpr (EPI >= 1) dev::load_bias(rb, bias_lds + wave * 1024, n0 + wn * 128, lane);
    one(Later(), H1(), true, 1);
    for (int kt = 2; kt < nk; kt += 2) {
      one(Later(), H0(), false, kt);
      one(Later(), H1(), true, kt + 1);
    }
    // the next tile's stage-1 DMA retired before the stores (they share the counter)
    __builtin_amdgcn_s_waitcnt(dev::kWaitVm);
    epilogue(acc, m0, n0);
    m0 = m0n;
    n0 = n0n;
    if (ti + 2 < my_tiles) origin(ti + 2, m0n, n0n);
  }
  __builtin_amdgcn_s_waitcnt(dev::kWaitVm);   // no DMA outlives the workgroup
}

}  // namespace

// Shapes reaching here are validated: M, N, K positive multiples of 128, kind 0/1,
// epi 0..2.  Persistent (one workgroup per CU) when there are more tiles than CUs.
hipError_t launch_gemm_mxfp8_fused(const void* a, int kind, const void* w_q, const void* w_s, int64_t M, int64_t N,
                                   int64_t K, const void* bias, int epi, void* c, bool scales_tiled,
                                   hipStream_t stream) {
  const int m = (int)M, n = (int)N, k = (int)K;
  const int tiles = ((m + kTile - 1) / kTile) * ((n + kTile - 1) / kTile);
  const int cus = device_compute_units();
  dim3 grid(tiles < cus ? tiles : cus), block(kThreads);
  auto A = (const uint16_t*)a;
  auto W = (const uint8_t*)w_q;
  auto Ws = (const uint8_t*)w_s;
  auto B = (const uint16_t*)bias;
  auto C = (uint16_t*)c;
#define MXQ_FUSED(KD, E, T) \
  hipLaunchKernelGGL((k_gemm_mxfp8_fused<KD, E, T>), grid, block, 0, stream, A, W, Ws, B, C, m, n, k)
#define MXQ_FUSED_EPI(KD, T)          \
  if (epi == 0) MXQ_FUSED(KD, 0, T);  \
  else if (epi == 1) MXQ_FUSED(KD, 1, T); \
  else MXQ_FUSED(KD, 2, T);
  if (scales_tiled) {
    if (kind == 0) { MXQ_FUSED_EPI(0, true) } else { MXQ_FUSED_EPI(1, true) }
  } else {
    if (kind == 0) { MXQ_FUSED_EPI(0, false) } else { MXQ_FUSED_EPI(1, false) }
  }
#undef MXQ_FUSED_EPI
#undef MXQ_FUSED
  return hipGetLastError();
}

}  // namespace mxq
