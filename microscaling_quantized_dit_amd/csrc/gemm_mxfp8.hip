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

constexpr int kThreads = 256;
constexpr int kTile = 256;        // rows of W (n) and of A (m) per workgroup
constexpr int kBK = 128;          // K bytes per stage
constexpr int kRow = kBK + 16;    // padded LDS row (bytes)
constexpr int kStage = 2 * kTile * kRow;
constexpr int kGroupM = 4;

// One 64-K step of the wave's 128 x 128 tile: 4 W fragments, 4 A fragments,
// 16 scaled MFMAs.  S selects the 64-K half of the 128-byte stage; the scale
// dwords were pre-shifted so that byte 2S holds this lane's block.
template <int AK, int WK, int S>
__device__ __forceinline__ void substep(v16f (&acc)[4][4], const uint8_t* wl, const uint8_t* al, int g,
                                        const uint32_t (&scw)[4], const uint32_t (&sca)[4]) {
  v8i wf[4], af[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint8_t* p = wl + 32 * i * kRow;
    uint4 lo = *(const uint4*)(p + (4 * S + g) * 16), hi = *(const uint4*)(p + (4 * S + 2 + g) * 16);
    wf[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    const uint8_t* q = al + 32 * i * kRow;
    uint4 lo2 = *(const uint4*)(q + (4 * S + g) * 16), hi2 = *(const uint4*)(q + (4 * S + 2 + g) * 16);
    af[i] = v8i{(int)lo2.x, (int)lo2.y, (int)lo2.z, (int)lo2.w, (int)hi2.x, (int)hi2.y, (int)hi2.z, (int)hi2.w};
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf[i], af[j], acc[i][j], WK, AK, 2 * S,
                                                                 (int)scw[i], 2 * S, (int)sca[j]);
}

template <int AK, int WK, int EPI>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_mxfp8(
    const uint8_t* __restrict__ aq, const uint8_t* __restrict__ as_, const uint8_t* __restrict__ wq,
    const uint8_t* __restrict__ ws, const uint16_t* __restrict__ bias, uint16_t* __restrict__ c, int M, int N,
    int K) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStage];

  const int tiles_m = (M + kTile - 1) / kTile, tiles_n = (N + kTile - 1) / kTile;
  const int wg = dev::xcd_remap(blockIdx.x, gridDim.x);
  const int per_group = kGroupM * tiles_n;
  const int first_m = (wg / per_group) * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int tm = first_m + (wg % per_group) % gsize;
  const int tn = (wg % per_group) / gsize;
  const int m0 = tm * kTile, n0 = tn * kTile;

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int r = lane & 31, g = lane >> 5;
  const int KB = K / 32;            // scale bytes per row

  // Buffer resources: 32-bit offsets (operands are < 2 GiB, checked by the host),
  // reads past the end return 0 (rows past M or N are never stored).
  const auto rw = __builtin_amdgcn_make_buffer_rsrc((void*)wq, (short)0, N * K, 0x00020000);
  const auto ra = __builtin_amdgcn_make_buffer_rsrc((void*)aq, (short)0, M * K, 0x00020000);
  const auto rsw = __builtin_amdgcn_make_buffer_rsrc((void*)ws, (short)0, N * KB, 0x00020000);
  const auto rsa = __builtin_amdgcn_make_buffer_rsrc((void*)as_, (short)0, M * KB, 0x00020000);
  // staging: thread t copies 16-byte chunk (t & 7) of rows (t >> 3) + 32 i, i = 0..7
  const int voff = (t >> 3) * K + (t & 7) * 16;
  const int loff = (t >> 3) * kRow + (t & 7) * 16;
  const int vsw = (wn * 128 + r) * KB, vsa = (wm * 128 + r) * KB;

  uint4 stw[8], sta[8];
  uint32_t scw[4], sca[4], nscw[4], nsca[4];
  auto load_stage = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      stw[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, voff, (n0 + 32 * i) * K + k0, 0));
      sta[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ra, voff, (m0 + 32 * i) * K + k0, 0));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      nscw[i] = __builtin_amdgcn_raw_buffer_load_b32(rsw, vsw, (n0 + 32 * i) * KB + k0 / 32, 0);
      nsca[i] = __builtin_amdgcn_raw_buffer_load_b32(rsa, vsa, (m0 + 32 * i) * KB + k0 / 32, 0);
    }
  };
  auto store_stage = [&](int st) {
    uint8_t* base = lds + st * kStage + loff;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      *(uint4*)(base + 32 * i * kRow) = stw[i];
      *(uint4*)(base + kTile * kRow + 32 * i * kRow) = sta[i];
    }
  };

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int nk = K / kBK;
  load_stage(0);
  store_stage(0);
#pragma unroll
  for (int i = 0; i < 4; ++i) { scw[i] = nscw[i] >> (8 * g); sca[i] = nsca[i] >> (8 * g); }
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) load_stage((kt + 1) * kBK);
    const uint8_t* wl = lds + st * kStage + (wn * 128 + r) * kRow;
    const uint8_t* al = lds + st * kStage + kTile * kRow + (wm * 128 + r) * kRow;
    substep<AK, WK, 0>(acc, wl, al, g, scw, sca);
    substep<AK, WK, 1>(acc, wl, al, g, scw, sca);
    if (kt + 1 < nk) {
      store_stage(st ^ 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) { scw[i] = nscw[i] >> (8 * g); sca[i] = nsca[i] >> (8 * g); }
    }
    __syncthreads();
  }

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
        o.x = dev::f32_to_bf16_rne(y[0]) | (dev::f32_to_bf16_rne(y[1]) << 16);
        o.y = dev::f32_to_bf16_rne(y[2]) | (dev::f32_to_bf16_rne(y[3]) << 16);
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
