// NVFP4 block-scaled GEMM for gfx950:  C[M,N] = epi(s_ga s_gw A[M,K] . W[N,K]^T), bf16 out.
//
// Definition (page "NVIDIA量化推理：5步极速优化显存+成功率翻倍", NVFP4 paragraph:
// E2M1 elements, one FP8 scale per 16 values; page "NVIDIA Blackwell平台FP4量化
// 技术解析与图像生成优化", section 3.1: FP32 global scale, FP8 block scales):
//   C[m,n] = epi( s_ga s_gw sum_k val(a[m,k]) val(Sa[m,k/16]) val(w[n,k]) val(Sw[n,k/16]) )
// with fp32 accumulation and one round-to-nearest-even to bf16.
//
// Scheme.  gfx950's scaled MFMA applies one power-of-two (E8M0) scale per 32
// K-values, while NVFP4 carries a scale with 3 mantissa bits per 16 values, so
// the block scale cannot ride inside the matrix core.  Instead every element is
// dequantized in registers, exactly, to fp16:  e2m1 (2 significant bits) x E4M3
// scale (4 significant bits) has at most 6 significant bits and lies in
// [2^-10, 2688], inside fp16's normal range, so val(q) * val(S) is exact in fp16
// and the fp16 MFMA (v_mfma_f32_32x32x16_f16) multiplies exact dequantized values
// with fp32 accumulation.  The global scales are applied once, in the epilogue.
// Dequantization costs one VALU op per element per wave (fp4 -> fp16 pair
// conversion, then a packed fp16 multiply) and runs under the MFMAs of the
// previous K-step.
//
// fp16 operand layout (measured on gfx950): lane l holds row l % 32, K
// [8g, 8g+8) of the 16-K step (g = l / 32); result D[8(v/4) + 4g + v%4][l % 32].
// W is the first operand, A the second (each lane stores 4 consecutive n).
// The K order inside an MFMA is free as long as both operands use the same one:
// in a 64-K group lane group g reads the 32 consecutive values [32g, 32g+32) (one
// 16-byte LDS read) and K-step j takes its values [8j, 8j+8).  Those 8 values sit
// in NVFP4 block 2g + j/2 of the group, so each lane's step has a single scale.
//
// Tiling as the MXFP8 kernel: 256 x 256 output tiles, 4 waves of 128 x 128,
// codes and block scales copied global -> LDS by buffer_load ... lds into two
// stage buffers of 128 K (64-byte rows, XOR-swizzled), one 64-K group per half
// stage with the mid-stage barrier between them; persistent over tiles.
//
// Scale layout.  The texture unit's work for a load goes by the rows (cache
// lines) it touches, and a stage needs only 8 scale bytes of each of 64 rows per
// wave and operand.  In the tiled order of mxq_internal.h ([R/64][K/128][64][8 B],
// which the quantizer can write directly), the GEMM (TILED) fetches a stage's
// scales for its 64 rows as one contiguous 1 KiB load per wave and operand (with
// the next stage's along).  Row-major scales are rewritten into that order by
// k_tile_scales when a workspace is given, and read in place, 16 bytes per row,
// when not.
#include <type_traits>

#include "mxq_internal.h"

namespace mxq {
namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kThreads = 256;
constexpr int kTile = 256;
constexpr int kBK = 128;                       // K values per stage
constexpr int kRowB = kBK / 2;                 // 64 code bytes per row and stage
constexpr int kOperand = kTile * kRowB;        // 16 KiB
constexpr int kStage = 2 * kOperand;           // W then A
constexpr int kCStage = dev::epilogue_lds_bytes(128);

// Swizzle of the four 16-byte chunks of a 64-byte LDS row: the 16 rows read by a
// quarter-wave land on 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

// This lane's 16 code bytes of 64-K group G in row R (logical chunk 2G + g).
__device__ __forceinline__ uint4 codes(const uint8_t* tile, int R, int x, int G, int g) {
  return *(const uint4*)(tile + R * kRowB + (((2 * G + g) ^ x) << 4));
}

// 8 packed E2M1 values (element 2e in the low nibble of byte e) times the fp16
// scale s -> v8h, exactly.
__device__ __forceinline__ v8h dequant8(uint32_t d, _Float16 s) {
  v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 0);
  v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 1);
  v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 2);
  v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 3);
  const v2h ss = {s, s};
  p0 *= ss;
  p1 *= ss;
  p2 *= ss;
  p3 *= ss;
  return v8h{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// The two E4M3 block scales in the low 16 bits of w -> fp16 pair (exact).
__device__ __forceinline__ v2h scale_pair(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
}

template <int J>
__device__ __forceinline__ uint32_t word(const uint4& v) {
  return J == 0 ? v.x : J == 1 ? v.y : J == 2 ? v.z : v.w;
}

// PART = false: tiles [0, sp.dp_tiles) whole, round-robin over the workgroups.
// PART = true: one K range of a split tile per workgroup, its fp32 sum into
// sp.partial (the fixup kernel completes the tile).
// TILED: as_ and ws are the scales rewritten by k_tile_scales.
template <int EPI, bool PART, bool TILED>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_nvfp4(
    const uint8_t* __restrict__ aq, const uint8_t* __restrict__ as_, const float* __restrict__ ag,
    const uint8_t* __restrict__ wq, const uint8_t* __restrict__ ws, const float* __restrict__ wg,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ c, int M, int N, int K, GemmSplit sp) {
  // two stage buffers as distinct objects: codes, and 16 scale bytes per row (in
  // place: [W rows, A rows][row][4 dwords], the stage's d0, d1, then the next
  // stage's; TILED: [W, A][wave][next stage?][64 rows][2 dwords])
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[kStage];
  __shared__ __attribute__((aligned(16))) uint32_t sc0[8 * kTile];
  __shared__ __attribute__((aligned(16))) uint32_t sc1[8 * kTile];
  // per wave: the bias of its 128 columns (the first 256 B of one 1 KiB DMA)
  __shared__ __attribute__((aligned(16))) uint8_t bias_lds[4 * 1024];
  // per wave: output rows on their way to global memory
  __shared__ __attribute__((aligned(16))) uint8_t c_lds[4 * kCStage];

  const int tiles_m = (M + kTile - 1) / kTile, tiles_n = (N + kTile - 1) / kTile;
  const int nk = K / kBK;
  // This workgroup's tiles: whole tiles blockIdx + i * gridDim below dp_tiles, or
  // (PART) one K range of a split tile.  Every tile has an even number >= 2 of
  // stages when the launch is persistent.
  const int my_tiles = PART ? 1 : (sp.dp_tiles - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  struct Tile {
    int m0, n0, kb, nkt;   // origin, first K stage, stages
  };
  auto tile_info = [&](int ti, Tile& T) {
    int v;
    if constexpr (PART) {
      v = sp.dp_tiles + (int)blockIdx.x / sp.parts;
      T.nkt = nk / sp.parts;
      T.kb = ((int)blockIdx.x % sp.parts) * T.nkt;
    } else {
      v = blockIdx.x + ti * gridDim.x;
      T.kb = 0;
      T.nkt = nk;
    }
    dev::tile_origin(v, tiles_m, tiles_n, T.m0, T.n0);
  };

  const int t = threadIdx.x;
  int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wn = wave & 1, wm = wave >> 1;
  int r = lane & 31, g = lane >> 5;
  const int KP = K / 2, KS = K / 16;    // bytes per row: codes, scales

  // 32-bit offsets: operands are < 2 GiB (checked by the host)
  const auto rw = __builtin_amdgcn_make_buffer_rsrc((void*)wq, (short)0, N * KP, 0x00020000);
  const auto ra = __builtin_amdgcn_make_buffer_rsrc((void*)aq, (short)0, M * KP, 0x00020000);
  const auto rsw = __builtin_amdgcn_make_buffer_rsrc((void*)ws, (short)0, N * KS, 0x00020000);
  const auto rsa = __builtin_amdgcn_make_buffer_rsrc((void*)as_, (short)0, M * KS, 0x00020000);
  const int NST = K / kBK;          // stages per row (TILED scale blocks per 64-row block)
  const auto rb = __builtin_amdgcn_make_buffer_rsrc((void*)bias, (short)0, EPI >= 1 ? N * 2 : 0, 0x00020000);

  // Global -> LDS: one buffer_load ... lds moves 1 KiB per wave = 16 rows of 64 B
  // (lane i -> row i / 4, physical chunk i % 4, i.e. global chunk (i % 4) ^ swz).
  // Rows 16j + i/4 have swz = (i >> 4) & 3 whatever j, so one lane offset serves
  // all four loads of a wave's 64 rows.  Scales: lane i -> row 64w + i, 16 bytes
  // from the stage's first block on (the stage's 8 bytes and the next stage's,
  // which are not used: one 16-byte load per row costs the texture unit half of
  // what two 4-byte loads do).  TILED: lane i -> bytes [16i, 16i + 16) of the
  // stage's 512-byte run and the next one.  At the last stage the load reaches 8
  // (row-major) or 512 (TILED) bytes past the end of the operand; the buffer
  // resource's bound returns zeros there, and those bytes are never used.
  int voff = (lane >> 2) * KP + (((lane & 3) ^ ((lane >> 4) & 3)) << 4);
  int vsc = TILED ? lane * 16 : lane * KS;
  // Every code load stays inside its operand: a wave's 64 rows lie wholly inside
  // or past M (N); rows past the end, and stages after the last tile, read rows
  // [0, 64).  (A scale load can reach past the end, see above.)
  // Part p (0..3) of a stage's DMA: code rows 16p..16p+15 of this wave's 64 for W
  // and A, and in parts 0 and 1 the W and the A scale load.  The parts
  // are issued a quarter of a phase apart so that the four waves' loads reach the
  // texture unit spread out rather than in one burst.
  auto dma_part = [&](int p, uint8_t* buf, uint32_t* sc, int m0, int n0, int k0, bool valid) {
    const int rw0 = n0 + wave * 64, ra0 = m0 + wave * 64;
    const bool vw = valid && rw0 < N, va = valid && ra0 < M;
    const int off_w = vw ? rw0 * KP + k0 / 2 : 0, off_a = va ? ra0 * KP + k0 / 2 : 0;
    const int st = k0 / kBK;
    const int off_sw = vw ? (TILED ? ((rw0 >> 6) * NST + st) * 512 : rw0 * KS + k0 / 16) : 0;
    const int off_sa = va ? (TILED ? ((ra0 >> 6) * NST + st) * 512 : ra0 * KS + k0 / 16) : 0;
    uint8_t* base = buf + wave * 64 * kRowB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_ptr_t)(base + p * 16 * kRowB), 16, voff,
                                             off_w + p * 16 * KP, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(base + kOperand + p * 16 * kRowB), 16, voff,
                                             off_a + p * 16 * KP, 0, 0);
    // both layouts: 1 KiB per wave and operand at dword 256 * (4 op + w)
    if (p == 0)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsw, (lds_ptr_t)(sc + 256 * wave), 16, vsc, off_sw, 0, 0);
    else if (p == 1)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_ptr_t)(sc + 256 * (4 + wave)), 16, vsc, off_sa, 0, 0);
  };
  auto dma_stage = [&](uint8_t* buf, uint32_t* sc, int m0, int n0, int k0, bool valid) {
#pragma unroll
    for (int p = 0; p < 4; ++p) dma_part(p, buf, sc, m0, n0, k0, valid);
  };

  int x = swz(r);                   // rows wn*128 + 32i + r all share swz(r)
  int wrow = wn * 128 + r, arow = wm * 128 + r;
  // The lane-derived offsets are recomputed at the top of every tile from the lane
  // id (mbcnt, in a volatile asm block so that it is not hoisted): otherwise they
  // stay live across the epilogue, get spilled there, and their reloads queue
  // behind its stores.
  auto lane_setup = [&]() {
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
    r = lane & 31;
    g = lane >> 5;
    voff = (lane >> 2) * KP + (((lane & 3) ^ ((lane >> 4) & 3)) << 4);
    vsc = TILED ? lane * 16 : lane * KS;
    x = swz(r);
    wrow = wn * 128 + r;
    arow = wm * 128 + r;
  };
  uint4 c0w[4], c0a[4], c1w[4], c1a[4];     // codes of the stage's 64-K groups 0 and 1
  v2h s0w[4], s0a[4], s1w[4], s1a[4];       // their scales: {steps 0-1, steps 2-3}
  v8h dw[2][4], da[2][4];                   // dequantized operands, double-buffered by K-step

  // Scale dwords of group G of a stage, converted to fp16 pairs.  Group 0's are
  // read while the previous stage's group 1 runs, group 1's while the stage's own
  // group 0 runs: each when its registers are free.  Lane group g uses blocks
  // 2g, 2g + 1 of each group: the g-th 16-bit half.
  uint32_t dsw[4], dsa[4];                  // scale dwords on their way from LDS
  auto read_scales = [&](const uint32_t* sc, int G) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (TILED) {   // row R: dword 256 * (4 op + R / 64) + 2 (R % 64) + G
        dsw[i] = sc[256 * (2 * wn + (i >> 1)) + 2 * (32 * (i & 1) + r) + G];
        dsa[i] = sc[256 * (4 + 2 * wm + (i >> 1)) + 2 * (32 * (i & 1) + r) + G];
      } else {
        dsw[i] = sc[4 * (wrow + 32 * i) + G];
        dsa[i] = sc[4 * (kTile + arow + 32 * i) + G];
      }
    }
  };
  auto convert_scales = [&](v2h (&sw)[4], v2h (&sa)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sw[i] = scale_pair(dsw[i] >> (16 * g));
      sa[i] = scale_pair(dsa[i] >> (16 * g));
    }
  };
  auto read_codes = [&](uint4 (&cw)[4], uint4 (&ca)[4], const uint8_t* buf, int G) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      cw[i] = codes(buf, wrow + 32 * i, x, G, g);
      ca[i] = codes(buf + kOperand, arow + 32 * i, x, G, g);
    }
  };
  // dequantize K-step J of a group into buffer B
  auto dequant = [&](auto B_, auto J_, const uint4 (&cw)[4], const uint4 (&ca)[4], const v2h (&sw)[4],
                     const v2h (&sa)[4]) {
    constexpr int B = decltype(B_)::value, J = decltype(J_)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dw[B][i] = dequant8(word<J>(cw[i]), sw[i][J >> 1]);
      da[B][i] = dequant8(word<J>(ca[i]), sa[i][J >> 1]);
    }
  };
  auto mfma_step = [&](v16f (&acc)[4][4], auto B_) {
    constexpr int B = decltype(B_)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(dw[B][i], da[B][j], acc[i][j], 0, 0, 0);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  // 16 MFMAs, each followed by 4 of the next step's dequantization ops
  // (and, for the first `reads` MFMAs, one LDS read; for MFMAs 0, 5 and 10 when
  // `vmem`, one DMA load)
  auto interleave = [&](int reads, bool vmem) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
      if (i < reads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (vmem && i % 5 == 0 && i < 15) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  const float alpha = (*ag) * (*wg);
  auto epilogue = [&](const v16f (&acc)[4][4], int m0, int n0) {
    // M and N are multiples of 128: a wave's 128 x 128 block is wholly in or out
    if (m0 + wm * 128 >= M || n0 + wn * 128 >= N) return;
    // a fresh lane id (opaque to the compiler): nothing lane-derived stays live
    // across the K loop for the epilogue's sake
    int el;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(el));
    dev::epilogue_block<EPI, 128, true>(acc, alpha, bias_lds + wave * 1024, c_lds + wave * kCStage, c, N,
                                        m0 + wm * 128, n0 + wn * 128, el);
  };

  // One stage (cur holds it, nxt the next one):
  //   A: group 0's four K-steps on MFMA || LDS reads of group 1's codes; the last
  //      step dequantizes group 1's first step
  //   B: wait for the next stage's DMA and this wave's reads, barrier (a tile's
  //      first stage finds the next stage's DMA retired before the previous tile's
  //      epilogue and waits for its reads only, leaving the epilogue's stores in
  //      flight)
  //   C: group 1's K-steps || LDS reads of the next stage's scales and group-0 codes,
  //      DMA of the stage after next into cur; the last step dequantizes the next
  //      stage's first step.
  // On entry dw/da[0] hold group 0's first step, dequantized.
  auto stage = [&](auto first_, v16f (&acc)[4][4], uint8_t* cur, uint8_t* nxt, uint32_t* scur, uint32_t* snxt,
                   int dm0, int dn0, int dk0, bool dvalid) {
    // ---- A  (group 1's scale dwords are read one K-step before they are converted,
    // so that no wait for LDS reads stalls the MFMAs)
    read_codes(c1w, c1a, cur, 1);
    mfma_step(acc, I0());
    dequant(I1(), I1(), c0w, c0a, s0w, s0a);
    interleave(16, false);
    mfma_step(acc, I1());
    dequant(I0(), I2(), c0w, c0a, s0w, s0a);
    interleave(0, false);
    read_scales(scur, 1);
    mfma_step(acc, I0());
    dequant(I1(), I3(), c0w, c0a, s0w, s0a);
    interleave(8, false);
    convert_scales(s1w, s1a);
    mfma_step(acc, I1());
    dequant(I0(), I0(), c1w, c1a, s1w, s1a);
    interleave(0, false);
    // ---- B
    if constexpr (decltype(first_)::value) __builtin_amdgcn_s_waitcnt(dev::kWaitLgkm);
    else __builtin_amdgcn_s_waitcnt(dev::kWaitAll);
    dev::lds_barrier();
    // ---- C
    read_scales(snxt, 0);
    read_codes(c0w, c0a, nxt, 0);
    dma_part(0, cur, scur, dm0, dn0, dk0, dvalid);
    mfma_step(acc, I0());
    dequant(I1(), I1(), c1w, c1a, s1w, s1a);
    interleave(16, true);
    dma_part(1, cur, scur, dm0, dn0, dk0, dvalid);
    mfma_step(acc, I1());
    dequant(I0(), I2(), c1w, c1a, s1w, s1a);
    interleave(8, true);
    dma_part(2, cur, scur, dm0, dn0, dk0, dvalid);
    mfma_step(acc, I0());
    dequant(I1(), I3(), c1w, c1a, s1w, s1a);
    interleave(0, true);
    convert_scales(s0w, s0a);
    dma_part(3, cur, scur, dm0, dn0, dk0, dvalid);
    mfma_step(acc, I1());
    dequant(I0(), I0(), c0w, c0a, s0w, s0a);
    interleave(0, true);
  };

  Tile cu{0, 0, 0, 2}, nx{0, 0, 0, 2};
  tile_info(0, cu);
  if (my_tiles > 1) tile_info(1, nx);

  // Prologue: the first two stages in flight; wait; stage 0's scales, codes and first step.
  {
    const bool nx1 = cu.nkt < 2;
    dma_stage(lds0, sc0, cu.m0, cu.n0, cu.kb * kBK, true);
    dma_stage(lds1, sc1, nx1 ? nx.m0 : cu.m0, nx1 ? nx.n0 : cu.n0, (nx1 ? nx.kb : cu.kb + 1) * kBK,
              !nx1 || my_tiles > 1);
  }
  __builtin_amdgcn_s_waitcnt(dev::kWaitVm);
  dev::lds_barrier();
  read_scales(sc0, 0);
  read_codes(c0w, c0a, lds0, 0);
  convert_scales(s0w, s0a);
  dequant(I0(), I0(), c0w, c0a, s0w, s0a);

  // Global stage s uses buffer s & 1; with an even number of stages per tile every
  // tile starts in buffer 0 (the launcher gives each workgroup one tile otherwise,
  // and cuts split tiles into even ranges).
  using First = std::integral_constant<bool, true>;
  using Later = std::integral_constant<bool, false>;
  for (int ti = 0; ti < my_tiles; ++ti) {
    lane_setup();
    const bool has_next = ti + 1 < my_tiles;
    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    // DMA of stage kt + 2: this tile's, or the next tile's first two
    auto one = [&](auto first_, uint8_t* b0, uint8_t* b1, uint32_t* t0, uint32_t* t1, int kt) {
      const int kk = kt + 2;
      const bool in_next = kk >= cu.nkt;
      stage(first_, acc, b0, b1, t0, t1, in_next ? nx.m0 : cu.m0, in_next ? nx.n0 : cu.n0,
            (in_next ? nx.kb + kk - cu.nkt : cu.kb + kk) * kBK, !in_next || has_next);
    };
    one(First(), lds0, lds1, sc0, sc1, 0);
    if constexpr (EPI >= 1) {
      // the tile's bias, read by this wave's epilogue from LDS, so that no global
      // load there queues behind the epilogue's own stores; any later vmcnt(0)
      // retires it, and this wave's previous epilogue has finished with the slot
      if constexpr (!PART) dev::load_bias(rb, bias_lds + wave * 1024, cu.n0 + wn * 128, lane);
    }
    int kt = 1;
    for (; kt + 1 < cu.nkt; kt += 2) {
      one(Later(), lds1, lds0, sc1, sc0, kt);
      one(Later(), lds0, lds1, sc0, sc1, kt + 1);
    }
    if (kt < cu.nkt) one(Later(), lds1, lds0, sc1, sc0, kt);
    // Retire the next tile's first two stages of DMA now: the stores below share
    // the counter, and the next tile's first stage then waits for none of them.
    __builtin_amdgcn_s_waitcnt(dev::kWaitVm);
    if constexpr (PART)
      dev::store_partial(acc, sp.partial + (size_t)blockIdx.x * kTile * kTile, c_lds + wave * kCStage, wm, wn, lane);
    else
      epilogue(acc, cu.m0, cu.n0);
    cu = nx;
    if (ti + 2 < my_tiles) tile_info(ti + 2, nx);
  }
  __builtin_amdgcn_s_waitcnt(dev::kWaitVm);   // no DMA outlives the workgroup
}

// Scales [R, K/16] row-major -> [R/64][K/128][64 rows][8 B]: a stage's 8 bytes of
// 64 consecutive rows become 512 contiguous bytes.  One launch for both operands:
// workgroup (x, y) takes 16 stages of 64-row block y, of A's rows for y < ra64 and
// of W's after them.  The rows' segments go through LDS so that both the reads
// (along a row) and the writes (along a stage block) are contiguous.  V16: rows
// start 16-byte aligned (K a multiple of 256), so the reads are 16 bytes wide.
template <bool V16>
__global__ __launch_bounds__(256) void k_tile_scales(const uint8_t* __restrict__ a_src, uint8_t* __restrict__ a_dst,
                                                     int ra64, const uint8_t* __restrict__ w_src,
                                                     uint8_t* __restrict__ w_dst, int KS, int nst) {
  __shared__ __attribute__((aligned(16))) uint8_t seg[64 * 128];   // [row][16 stages][8 B]
  const int t = threadIdx.x;
  const bool is_a = (int)blockIdx.y < ra64;
  const int rb = is_a ? (int)blockIdx.y : (int)blockIdx.y - ra64;
  const uint8_t* src = is_a ? a_src : w_src;
  uint8_t* dst = is_a ? a_dst : w_dst;
  const int st0 = blockIdx.x * 16, ns = min(16, nst - st0);
  {  // thread t: row t / 4, stages 4 (t % 4) .. +3 of the group (32 bytes)
    const int row = t >> 2, st = 4 * (t & 3);
    const uint8_t* p = src + (size_t)(rb * 64 + row) * KS + (size_t)(st0 + st) * 8;
    uint8_t* q = seg + row * 128 + st * 8;
    if (V16) {
      if (st < ns) *(uint4*)q = *(const uint4*)p;                       // stages st, st + 1
      if (st + 2 < ns) *(uint4*)(q + 16) = *(const uint4*)(p + 16);     // (nst is even here)
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (st + u < ns) *(uint2*)(q + 8 * u) = *(const uint2*)(p + 8 * u);
    }
  }
  __syncthreads();
  {  // thread t: stage t / 16, rows 4 (t % 16) .. +3: 32 contiguous bytes of its block
    const int st = t >> 4, r0 = 4 * (t & 15);
    if (st < ns) {
      uint2 v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = *(const uint2*)(seg + (r0 + q) * 128 + st * 8);
      uint4* o = (uint4*)(dst + ((size_t)rb * nst + st0 + st) * 512 + r0 * 8);
      o[0] = make_uint4(v[0].x, v[0].y, v[1].x, v[1].y);
      o[1] = make_uint4(v[2].x, v[2].y, v[3].x, v[3].y);
    }
  }
}

}  // namespace

static GemmSplit nvfp4_split(int64_t M, int64_t N, int64_t K) {
  const int tiles = (int)(((M + kTile - 1) / kTile) * ((N + kTile - 1) / kTile));
  const int nk = (int)(K / kBK);
  if (nk % 2 != 0) return GemmSplit{tiles, 0, nullptr};   // not persistent
  return plan_gemm_split(tiles, device_compute_units(), nk);
}

static size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

// Workspace: the split's partial tiles (if any), then A's and W's scales in the
// layout k_tile_scales writes.
size_t gemm_nvfp4_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const size_t split = gemm_split_bytes(nvfp4_split(M, N, K), (int)(((M + kTile - 1) / kTile) * ((N + kTile - 1) / kTile)));
  return round256(split) + round256((size_t)M * (K / 16)) + round256((size_t)N * (K / 16));
}

// Shapes reaching here are validated: M, N, K positive multiples of 128, epi 0..2;
// workspace is NULL or holds gemm_nvfp4_workspace_bytes(M, N, K).
hipError_t launch_gemm_nvfp4(const void* a_q, const void* a_s, const float* a_g, const void* w_q, const void* w_s,
                             const float* w_g, int64_t M, int64_t N, int64_t K, const void* bias, int epi, void* c,
                             bool scales_tiled, void* workspace, hipStream_t stream) {
  const int m = (int)M, n = (int)N, k = (int)K;
  const int tiles = ((m + kTile - 1) / kTile) * ((n + kTile - 1) / kTile);
  // persistent (one workgroup per CU) when a tile has an even number of K stages;
  // otherwise one workgroup per tile.  With a workspace, the tiles of a partial
  // last round are split along K: a second launch computes the K ranges, the
  // fixup kernel completes them (gemm_fixup.hip).
  const int cus = device_compute_units();
  const bool persistent = (k / kBK) % 2 == 0 && tiles >= cus;
  GemmSplit sp{tiles, 0, nullptr};
  if (persistent && workspace) {
    sp = nvfp4_split(M, N, K);
    sp.partial = (float*)workspace;
  }
  auto A = (const uint8_t*)a_q;
  auto As = (const uint8_t*)a_s;
  auto W = (const uint8_t*)w_q;
  auto Ws = (const uint8_t*)w_s;
  // Row-major scales with a workspace: both operands' scales into the GEMM's
  // layout first.  Scales that come tiled are read in place.
  const bool tiled = scales_tiled || workspace != nullptr;
  if (tiled && !scales_tiled) {
    const int KS = k / 16, nst = k / kBK;
    uint8_t* at = (uint8_t*)workspace + round256(gemm_split_bytes(nvfp4_split(M, N, K), tiles));
    uint8_t* wt = at + round256((size_t)M * KS);
    const dim3 tg((nst + 15) / 16, m / 64 + n / 64);
    if (KS % 16 == 0)
      hipLaunchKernelGGL(k_tile_scales<true>, tg, dim3(256), 0, stream, As, at, m / 64, Ws, wt, KS, nst);
    else
      hipLaunchKernelGGL(k_tile_scales<false>, tg, dim3(256), 0, stream, As, at, m / 64, Ws, wt, KS, nst);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    As = at;
    Ws = wt;
  }
  auto B = (const uint16_t*)bias;
  auto C = (uint16_t*)c;
  dim3 block(kThreads);
  dim3 grid(persistent ? cus : tiles);
#define MXQ_NV_LAUNCH(E, P, T, G)                                                                               \
  hipLaunchKernelGGL((k_gemm_nvfp4<E, P, T>), G, block, 0, stream, A, As, a_g, W, Ws, w_g, B, C, m, n, k, sp)
  if (tiled) {
    if (epi == 0) MXQ_NV_LAUNCH(0, false, true, grid);
    else if (epi == 1) MXQ_NV_LAUNCH(1, false, true, grid);
    else MXQ_NV_LAUNCH(2, false, true, grid);
  } else {
    if (epi == 0) MXQ_NV_LAUNCH(0, false, false, grid);
    else if (epi == 1) MXQ_NV_LAUNCH(1, false, false, grid);
    else MXQ_NV_LAUNCH(2, false, false, grid);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !sp.parts) return e;
  dim3 grid_p((tiles - sp.dp_tiles) * sp.parts);
  MXQ_NV_LAUNCH(0, true, true, grid_p);   // a split implies a workspace
#undef MXQ_NV_LAUNCH
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_gemm_fixup(sp, M, N, a_g, w_g, bias, epi, c, stream);
}

}  // namespace mxq
