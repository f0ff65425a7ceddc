// MXFP8 block-scaled GEMM for gfx950:  C[M,N] = epi(A[M,K] . W[N,K]^T), bf16 out.
//
// Definition (page "Modelos de Difusão": every nn.Linear of the transformer runs
// quantized; page "NVIDIA量化推理：5步极速优化显存+成功率翻倍", MXFP8 paragraph):
//   C[m,n] = epi( sum_k val(a[m,k]) 2^(sa[m,k/32]-127) val(w[n,k]) 2^(sw[n,k/32]-127) )
// with fp32 accumulation and one round-to-nearest-even to bf16.
//
// The contraction runs on v_mfma_scale_f32_32x32x64_f8f6f4, which multiplies fp8
// operands and applies one E8M0 scale per 32 K-values per row inside the matrix
// core -- exactly the MX block structure, so codes and scale bytes are consumed
// as stored, with no dequantization.
//
// Operand layout of that instruction (measured on gfx950): lane l holds row
// l % 32 and lane group g = l / 32; its 32 bytes are K [16g, 16g+16) followed by
// K [32+16g, 32+16g+16) of the 64-K step, and its scale byte covers K [32g, 32g+32).
// The 32x32 fp32 result sits as D[8(v/4) + 4g + v%4][l % 32] in element v.
// W is fed as the first operand and A as the second, so each lane ends up with
// four consecutive output columns n of one output row m: 8-byte bf16 stores.
//
// Tiling: 256 (n) x 256 (m) per workgroup, 4 waves in 2 x 2, 128 x 128 per wave
// (4 x 4 MFMA tiles), K step 128 bytes, two LDS stages (rows padded to 144 B so
// the 32 rows read by one instruction spread over all banks), next stage loaded
// into registers while the current one is multiplied.  Workgroup ids are
// remapped so that tiles sharing operands land on one XCD (one L2), in groups of
// four M-tiles.
#include "mxq_internal.h"

namespace mxq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kThreads = 256;
constexpr int kTile = 256;        // rows of W (n) and of A (m) per workgroup
constexpr int kBK = 128;          // K bytes per stage = one LDS row
constexpr int kOperand = kTile * kBK;          // 32 KiB
constexpr int kStage = 2 * kOperand;           // W then A
constexpr int kGroupM = 4;

// XOR swizzle of the eight 16-byte chunks of an LDS row: row R keeps logical
// chunk c at physical chunk c ^ swz(R).  The 16 rows read by one quarter-wave
// (ds_read_b128 is served 16 lanes at a time) then cover all 64 banks.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// Fragment of the 32x32x64 operand for this lane: row R of the stage, the two
// 16-byte chunks c and c + 2 of 64-K half S (lane group g picks c = 4S + g).
__device__ __forceinline__ v8i frag(const uint8_t* tile, int R, int x, int S, int g) {
  const uint8_t* p = tile + R * kBK;
  uint4 lo = *(const uint4*)(p + (((4 * S + g) ^ x) << 4));
  uint4 hi = *(const uint4*)(p + (((4 * S + 2 + g) ^ x) << 4));
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

template <int AK, int WK, int EPI>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_mxfp8(
    const uint8_t* __restrict__ aq, const uint8_t* __restrict__ as_, const uint8_t* __restrict__ wq,
    const uint8_t* __restrict__ ws, const uint16_t* __restrict__ bias, uint16_t* __restrict__ c, int M, int N,
    int K) {
  // Two stage buffers (codes, then the stage's scale dwords) as distinct objects:
  // alias analysis can then tell the DMA into one from the reads of the other.
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[kStage];
  __shared__ __attribute__((aligned(16))) uint32_t sc0[2 * kTile];
  __shared__ __attribute__((aligned(16))) uint32_t sc1[2 * kTile];

  const int tiles_m = (M + kTile - 1) / kTile, tiles_n = (N + kTile - 1) / kTile;
  const int wg = dev::xcd_remap(blockIdx.x, gridDim.x);
  const int per_group = kGroupM * tiles_n;
  const int first_m = (wg / per_group) * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int tm = first_m + (wg % per_group) % gsize;
  const int tn = (wg % per_group) / gsize;
  const int m0 = tm * kTile, n0 = tn * kTile;

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // wave-uniform (an SGPR)
  const int wn = wave & 1, wm = wave >> 1;
  const int r = lane & 31, g = lane >> 5;
  const int KB = K / 32;            // scale bytes per row

  // Buffer resources: 32-bit offsets (operands are < 2 GiB, checked by the host),
  // reads past the end return 0 (rows past M or N are never stored).
  const auto rw = __builtin_amdgcn_make_buffer_rsrc((void*)wq, (short)0, N * K, 0x00020000);
  const auto ra = __builtin_amdgcn_make_buffer_rsrc((void*)aq, (short)0, M * K, 0x00020000);
  const auto rsw = __builtin_amdgcn_make_buffer_rsrc((void*)ws, (short)0, N * KB, 0x00020000);
  const auto rsa = __builtin_amdgcn_make_buffer_rsrc((void*)as_, (short)0, M * KB, 0x00020000);

  // Global -> LDS without registers: each buffer_load ... lds moves 1 KiB per wave
  // (lane i -> LDS bytes [16i, 16i+16) after M0) = 8 rows of 128 B.  Wave w fills
  // rows [64w, 64w+64) of each operand in 8 loads; lane i takes row (i / 8) of the
  // load and the global chunk that lands at physical chunk i % 8.  Rows 8j + i/8
  // have swz = ((i/8) >> 1) + 4 (j & 1), hence two lane offsets.  The stage's scale
  // dwords (4 MX blocks of every row) follow with one 4-byte-per-lane load per
  // operand: lane i of wave w -> row 64w + i.
  const int lrow = lane >> 3, lchunk = lane & 7;
  const int cx = lchunk ^ (lrow >> 1);
  const int voff0 = lrow * K + cx * 16, voff1 = lrow * K + (cx ^ 4) * 16;
  const int vsc = lane * KB;
  auto dma_stage = [&](uint8_t* buf, uint32_t* sc, int k0) {
    uint8_t* base = buf + wave * 64 * kBK;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int vo = (j & 1) ? voff1 : voff0;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_ptr_t)(base + j * 8 * kBK), 16, vo,
                                               (n0 + wave * 64 + 8 * j) * K + k0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(base + kOperand + j * 8 * kBK), 16, vo,
                                               (m0 + wave * 64 + 8 * j) * K + k0, 0, 0);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsw, (lds_ptr_t)(sc + wave * 64), 4, vsc,
                                             (n0 + wave * 64) * KB + k0 / 32, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_ptr_t)(sc + kTile + wave * 64), 4, vsc,
                                             (m0 + wave * 64) * KB + k0 / 32, 0, 0);
  };

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int nk = K / kBK;
  const int x = swz(r);             // rows wn*128 + 32i + r all share swz(r)
  const int wrow = wn * 128 + r, arow = wm * 128 + r;
  v8i f0w[4], f0a[4], f1w[4], f1a[4];   // fragments of the first / second 64-K half
  uint32_t scw[4], sca[4], nscw[4], nsca[4];
  // scale dwords of this lane's rows, shifted so byte 0 / byte 2 hold its block
  auto read_scales = [&](const uint32_t* sc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      nscw[i] = sc[wrow + 32 * i];
      nsca[i] = sc[kTile + arow + 32 * i];
    }
  };

  // Prologue: stages 0 and 1 in flight; wait; stage 0's scales and first-half fragments.
  dma_stage(lds0, sc0, 0);
  dma_stage(lds1, sc1, kBK);        // nk == 1: reads past K, never used
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  read_scales(sc0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f0w[i] = frag(lds0, wrow + 32 * i, x, 0, g);
    f0a[i] = frag(lds0 + kOperand, arow + 32 * i, x, 0, g);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) { scw[i] = nscw[i] >> (8 * g); sca[i] = nsca[i] >> (8 * g); }

  // Steady state, per stage k (buffer cur = k even ? lds0 : lds1):
  //   A: MFMAs of half 0 (registers) || LDS reads of half 1 of stage k
  //   B: wait for stage k+1's DMA and this wave's reads, barrier (cur is now free in
  //      every wave, stage k+1 visible in nxt)
  //   C: MFMAs of half 1 || LDS reads of half 0 and the scales of stage k+1; DMA of
  //      stage k+2 into cur.
  // Stages past the last are fetched from past K (next row, or zeros past the buffer
  // end) and never used.
  auto stage = [&](uint8_t* cur, uint8_t* nxt, uint32_t* scur, uint32_t* snxt, int kt) {
    // ---- A
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f1w[i] = frag(cur, wrow + 32 * i, x, 1, g);
      f1a[i] = frag(cur + kOperand, arow + 32 * i, x, 1, g);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f0w[i], f0a[j], acc[i][j], WK, AK, 0,
                                                                   (int)scw[i], 0, (int)sca[j]);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    }
    __builtin_amdgcn_sched_barrier(0);
    // ---- B
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __syncthreads();
    // ---- C
    read_scales(snxt);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f0w[i] = frag(nxt, wrow + 32 * i, x, 0, g);
      f0a[i] = frag(nxt + kOperand, arow + 32 * i, x, 0, g);
    }
    dma_stage(cur, scur, (kt + 2) * kBK);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f1w[i], f1a[j], acc[i][j], WK, AK, 2,
                                                                   (int)scw[i], 2, (int)sca[j]);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);    // scale reads
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
      if (i < 9) __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);   // 2 LDS-DMA loads
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) { scw[i] = nscw[i] >> (8 * g); sca[i] = nsca[i] >> (8 * g); }
  };
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    stage(lds0, lds1, sc0, sc1, kt);
    stage(lds1, lds0, sc1, sc0, kt + 1);
  }
  if (kt < nk) stage(lds0, lds1, sc0, sc1, kt);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no DMA outlives the workgroup

  // ---- epilogue: epi(acc) -> bf16, four consecutive n per store
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + wm * 128 + 32 * j + r;
    if (m >= M) continue;
    uint16_t* crow = c + (size_t)m * N;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (n0 + wn * 128 + 32 * i >= N) continue;        // N % 128 == 0: whole 32-column tiles
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int n = n0 + wn * 128 + 32 * i + 8 * qd + 4 * g;
        float y[4] = {acc[i][j][4 * qd], acc[i][j][4 * qd + 1], acc[i][j][4 * qd + 2], acc[i][j][4 * qd + 3]};
        if (EPI >= 1) {
          uint2 b = *(const uint2*)(bias + n);
          y[0] += dev::bf16_lo(b.x);
          y[1] += dev::bf16_hi(b.x);
          y[2] += dev::bf16_lo(b.y);
          y[3] += dev::bf16_hi(b.y);
        }
        if (EPI == 2) {
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = dev::gelu_tanh(y[e]);
        }
        uint2 o;
        o.x = dev::pack_bf16x2(y[0], y[1]);
        o.y = dev::pack_bf16x2(y[2], y[3]);
        *(uint2*)(crow + n) = o;
      }
    }
  }
}

template <int AK, int WK>
hipError_t launch_kinds(const void* a_q, const void* a_s, const void* w_q, const void* w_s, int M, int N, int K,
                        const void* bias, int epi, void* c, hipStream_t stream) {
  const int tiles = ((M + kTile - 1) / kTile) * ((N + kTile - 1) / kTile);
  dim3 grid(tiles), block(kThreads);
  auto A = (const uint8_t*)a_q;
  auto As = (const uint8_t*)a_s;
  auto W = (const uint8_t*)w_q;
  auto Ws = (const uint8_t*)w_s;
  auto B = (const uint16_t*)bias;
  auto C = (uint16_t*)c;
  if (epi == 0) hipLaunchKernelGGL((k_gemm_mxfp8<AK, WK, 0>), grid, block, 0, stream, A, As, W, Ws, B, C, M, N, K);
  else if (epi == 1) hipLaunchKernelGGL((k_gemm_mxfp8<AK, WK, 1>), grid, block, 0, stream, A, As, W, Ws, B, C, M, N, K);
  else hipLaunchKernelGGL((k_gemm_mxfp8<AK, WK, 2>), grid, block, 0, stream, A, As, W, Ws, B, C, M, N, K);
  return hipGetLastError();
}

}  // namespace

// Shapes reaching here are validated: M, N, K positive multiples of 128, kinds 0/1, epi 0..2.
// Partial 256-tiles (M or N = 128 mod 256) load clamped rows and skip their stores.
hipError_t launch_gemm_mxfp8(const void* a_q, const void* a_s, int a_kind, const void* w_q, const void* w_s,
                             int w_kind, int64_t M, int64_t N, int64_t K, const void* bias, int epi, void* c,
                             hipStream_t stream) {
  const int m = (int)M, n = (int)N, k = (int)K;
  if (a_kind == 0 && w_kind == 0) return launch_kinds<0, 0>(a_q, a_s, w_q, w_s, m, n, k, bias, epi, c, stream);
  if (a_kind == 1 && w_kind == 1) return launch_kinds<1, 1>(a_q, a_s, w_q, w_s, m, n, k, bias, epi, c, stream);
  if (a_kind == 0 && w_kind == 1) return launch_kinds<0, 1>(a_q, a_s, w_q, w_s, m, n, k, bias, epi, c, stream);
  return launch_kinds<1, 0>(a_q, a_s, w_q, w_s, m, n, k, bias, epi, c, stream);
}

}  // namespace mxq
