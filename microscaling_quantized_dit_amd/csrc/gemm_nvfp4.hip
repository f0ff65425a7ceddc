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
// One 16-K MFMA step is exactly one NVFP4 block, so every lane's 8 values of a
// step share one scale.  Dequantization costs one VALU op per element
// (fp4 -> fp16 pair conversion, then a packed fp16 multiply), hidden under MFMA.
//
// fp16 operand layout (measured on gfx950): lane l holds row l % 32, K
// [8g, 8g+8) of the 16-K step (g = l / 32); result D[8(v/4) + 4g + v%4][l % 32].
// W is the first operand, A the second (each lane stores 4 consecutive n).
//
// Tiling as the MXFP8 kernel: 256 x 256 per workgroup, 4 waves of 128 x 128,
// 128 K (64 bytes) per LDS stage, two stages.  In LDS each row's 16 dwords are
// regrouped so that one lane finds all 8 of its K-steps in 32 contiguous bytes
// (two 16-byte reads), rows padded to 80 bytes against bank conflicts.
#include "mxq_internal.h"

namespace mxq {
namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kTile = 256;
constexpr int kBK = 128;              // K elements per stage (64 bytes per row)
constexpr int kRow = 64 + 16;         // padded LDS row (bytes)
constexpr int kStage = 2 * kTile * kRow;
constexpr int kGroupM = 4;

// 8 packed E2M1 values (one dword, element 2j in the low nibble of byte j) times
// the fp16 scale s -> v8h, exactly.
__device__ __forceinline__ v8h dequant8(uint32_t d, _Float16 s) {
  v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 0);
  v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 1);
  v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 2);
  v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 3);
  v2h ss = {s, s};
  p0 *= ss;
  p1 *= ss;
  p2 *= ss;
  p3 *= ss;
  return v8h{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// The 8 E4M3 block scales of one row for this stage (a uint2) -> 8 fp16 values.
__device__ __forceinline__ void scales8(uint2 b, _Float16 (&s)[8]) {
  v2h a0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b.x, 1.0f, false);
  v2h a1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b.x, 1.0f, true);
  v2h a2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b.y, 1.0f, false);
  v2h a3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b.y, 1.0f, true);
  s[0] = a0[0]; s[1] = a0[1]; s[2] = a1[0]; s[3] = a1[1];
  s[4] = a2[0]; s[5] = a2[1]; s[6] = a3[0]; s[7] = a3[1];
}

template <int EPI>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_nvfp4(
    const uint8_t* __restrict__ aq, const uint8_t* __restrict__ as_, const float* __restrict__ ag,
    const uint8_t* __restrict__ wq, const uint8_t* __restrict__ ws, const float* __restrict__ wg,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ c, int M, int N, int K) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStage];

  const int tiles_m = (M + kTile - 1) / kTile, tiles_n = (N + kTile - 1) / kTile;
  const int wg_id = dev::xcd_remap(blockIdx.x, gridDim.x);
  const int per_group = kGroupM * tiles_n;
  const int first_m = (wg_id / per_group) * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int tm = first_m + (wg_id % per_group) % gsize;
  const int tn = (wg_id % per_group) / gsize;
  const int m0 = tm * kTile, n0 = tn * kTile;

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int r = lane & 31, g = lane >> 5;
  const int KP = K / 2, KS = K / 16;   // bytes per row: codes, scales

  const auto rw = __builtin_amdgcn_make_buffer_rsrc((void*)wq, (short)0, N * KP, 0x00020000);
  const auto ra = __builtin_amdgcn_make_buffer_rsrc((void*)aq, (short)0, M * KP, 0x00020000);
  const auto rsw = __builtin_amdgcn_make_buffer_rsrc((void*)ws, (short)0, N * KS, 0x00020000);
  const auto rsa = __builtin_amdgcn_make_buffer_rsrc((void*)as_, (short)0, M * KS, 0x00020000);
  // staging: thread t copies 16-byte chunk (t & 3) of rows (t >> 2) + 64 i, i = 0..3
  const int cc = t & 3;
  const int voff = (t >> 2) * KP + cc * 16;
  // LDS regrouping: row dword o = 2*step + half goes to slot 8*half + step; chunk cc
  // holds dwords 4cc..4cc+3 = (step 2cc, half 0/1), (step 2cc+1, half 0/1).
  const int loff = (t >> 2) * kRow + 8 * cc;
  const int vsw = (wn * 128 + r) * KS, vsa = (wm * 128 + r) * KS;

  uint4 stw[4], sta[4];
  uint2 nscw[4], nsca[4];
  auto load_stage = [&](int k0) {   // k0 in elements
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      stw[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, voff, (n0 + 64 * i) * KP + k0 / 2, 0));
      sta[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ra, voff, (m0 + 64 * i) * KP + k0 / 2, 0));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      nscw[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rsw, vsw, (n0 + 32 * i) * KS + k0 / 16, 0));
      nsca[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rsa, vsa, (m0 + 32 * i) * KS + k0 / 16, 0));
    }
  };
  auto store_stage = [&](int st) {
    uint8_t* base = lds + st * kStage + loff;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint8_t* pw = base + 64 * i * kRow;
      *(uint2*)(pw) = make_uint2(stw[i].x, stw[i].z);
      *(uint2*)(pw + 32) = make_uint2(stw[i].y, stw[i].w);
      uint8_t* pa = base + kTile * kRow + 64 * i * kRow;
      *(uint2*)(pa) = make_uint2(sta[i].x, sta[i].z);
      *(uint2*)(pa + 32) = make_uint2(sta[i].y, sta[i].w);
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
  uint2 scw[4], sca[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { scw[i] = nscw[i]; sca[i] = nsca[i]; }
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) load_stage((kt + 1) * kBK);
    const uint8_t* wl = lds + st * kStage + (wn * 128 + r) * kRow + 32 * g;
    const uint8_t* al = lds + st * kStage + kTile * kRow + (wm * 128 + r) * kRow + 32 * g;
    uint4 wd[4][2], ad[4][2];
    _Float16 sw[4][8], sa[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      wd[i][0] = *(const uint4*)(wl + 32 * i * kRow);
      wd[i][1] = *(const uint4*)(wl + 32 * i * kRow + 16);
      ad[i][0] = *(const uint4*)(al + 32 * i * kRow);
      ad[i][1] = *(const uint4*)(al + 32 * i * kRow + 16);
      scales8(scw[i], sw[i]);
      scales8(sca[i], sa[i]);
    }
#pragma unroll
    for (int step = 0; step < 8; ++step) {
      v8h wf[4], af[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4& x = wd[i][step >> 2];
        const uint4& y = ad[i][step >> 2];
        const int e = step & 3;
        wf[i] = dequant8(e == 0 ? x.x : e == 1 ? x.y : e == 2 ? x.z : x.w, sw[i][step]);
        af[i] = dequant8(e == 0 ? y.x : e == 1 ? y.y : e == 2 ? y.z : y.w, sa[i][step]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wf[i], af[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      store_stage(st ^ 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) { scw[i] = nscw[i]; sca[i] = nsca[i]; }
    }
    __syncthreads();
  }

  // ---- epilogue: epi(alpha * acc) -> bf16
  const float alpha = (*ag) * (*wg);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + wm * 128 + 32 * j + r;
    if (m >= M) continue;
    uint16_t* crow = c + (size_t)m * N;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (n0 + wn * 128 + 32 * i >= N) continue;
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int n = n0 + wn * 128 + 32 * i + 8 * qd + 4 * g;
        float y[4] = {alpha * acc[i][j][4 * qd], alpha * acc[i][j][4 * qd + 1], alpha * acc[i][j][4 * qd + 2],
                      alpha * acc[i][j][4 * qd + 3]};
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

}  // namespace

hipError_t launch_gemm_nvfp4(const void* a_q, const void* a_s, const float* a_g, const void* w_q, const void* w_s,
                             const float* w_g, int64_t M, int64_t N, int64_t K, const void* bias, int epi, void* c,
                             hipStream_t stream) {
  const int m = (int)M, n = (int)N, k = (int)K;
  const int tiles = ((m + kTile - 1) / kTile) * ((n + kTile - 1) / kTile);
  dim3 grid(tiles), block(kThreads);
  auto A = (const uint8_t*)a_q;
  auto As = (const uint8_t*)a_s;
  auto W = (const uint8_t*)w_q;
  auto Ws = (const uint8_t*)w_s;
  auto B = (const uint16_t*)bias;
  auto C = (uint16_t*)c;
  if (epi == 0) hipLaunchKernelGGL(k_gemm_nvfp4<0>, grid, block, 0, stream, A, As, a_g, W, Ws, w_g, B, C, m, n, k);
  else if (epi == 1) hipLaunchKernelGGL(k_gemm_nvfp4<1>, grid, block, 0, stream, A, As, a_g, W, Ws, w_g, B, C, m, n, k);
  else hipLaunchKernelGGL(k_gemm_nvfp4<2>, grid, block, 0, stream, A, As, a_g, W, Ws, w_g, B, C, m, n, k);
  return hipGetLastError();
}

}  // namespace mxq
