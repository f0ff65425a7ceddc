// NVFP4 quantizer for gfx950: bf16 -> packed E2M1 codes, one E4M3 scale per 16
// values along a row, and an fp32 per-tensor decode scale.
//
// Definition (page "NVIDIA量化推理：5步极速优化显存+成功率翻倍", NVFP4 paragraph:
// E2M1 in blocks of 16 with FP8 scales; step 2: dynamic per-tensor scale;
// page "NVIDIA Blackwell平台FP4量化技术解析与图像生成优化", section 3.1: the runtime
// quantizer outputs FP4 data, FP8 block scales and an FP32 global scale):
//   s_g = RN_fp32(amax_tensor / 2688)   (1 for an all-zero tensor; or given)
//   S_b = RN_E4M3_sat(amax_block / (6 s_g))
//   q   = RN_E2M1_sat(x / (S_b s_g))    (magnitude 0 when S_b = 0), sign copied.
//
// Dynamic mode is two passes: k_amax_partials writes one maximum per workgroup
// (no zero-initialised state, no atomics), k_quant_nvfp4 folds those and encodes.
// Both passes read with streaming (nt) loads.  (Ordinary loads in the amax pass,
// leaving the tail of the tensor in the last-level cache for the encode pass,
// measured faster in isolation but 6% slower at 113 MB and 16% at 566 MB right
// after an NVFP4 GEMM.)  The encode pass still takes the slabs last to first, and
// stores the codes with ordinary stores, since the GEMM reads them next.  Block scales go out row-major or in the GEMM-tiled
// order (mxq_internal.h); for the latter a workgroup takes 64 rows x 128 values,
// four rows per wave, so that each wave's scale bytes form one contiguous run.
//
// Exact rounding at HBM speed.  Both quotients above are inexact in fp32, so
// each is evaluated twice, with the divisor's reciprocal nudged down and up by
// 2^-19 (far more than the <= ~2^-21.5 total relative error of the fp32
// reciprocal and products).  The two results bracket the exact quotient; if
// the hardware round-to-nearest conversion gives the same code for both ends,
// no rounding midpoint lies between them and that code is the exact answer.
// Otherwise (an exact tie or a near tie, or a reciprocal outside the fp32
// normal range) the decision is redone with exact fp64 comparisons: every
// threshold (midpoint x S_b x s_g, or midpoint x 6 x s_g) has at most
// 5 + 4 + 24 significant bits and is exact in fp64.  The fallback is inlined
// behind a branch that is almost never taken: as a called function it would give
// every wave a private stack, which alone cost 40% of the kernel's speed.
#include <atomic>

#include "mxq_internal.h"

namespace mxq {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr int kAmaxThreads = 1024;
constexpr int kMaxPartials = 256;

__device__ __forceinline__ uint32_t max_pk_u16(uint32_t a, uint32_t b) {
  typedef unsigned short us2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(us2, a),
                                                                __builtin_bit_cast(us2, b)));
}

__device__ __forceinline__ uint32_t wave_max(uint32_t m) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
  return m;
}

// Maximum of n (1 <= n <= 256) partial maxima in two steps, with no LDS and no
// barrier.  partial_loads: each lane loads four of them (indices clamped to n - 1,
// so every load is unconditional and in bounds).  fold_wave: their maximum, then
// the lanes of each row of 16 meet through DPP (pair swap, quad swap, half-row and
// row mirrors) and the four row maxima are read out of lanes 0, 16, 32 and 48, so
// the result is the same in every lane.  Every lane of the wave must be active.
__device__ __forceinline__ uint4 partial_loads(const uint32_t* __restrict__ p, int n) {
  const int l = threadIdx.x & 63;
  const uint32_t last = (uint32_t)(n - 1);
  return make_uint4(p[min((uint32_t)l, last)], p[min((uint32_t)l + 64u, last)], p[min((uint32_t)l + 128u, last)],
                    p[min((uint32_t)l + 192u, last)]);
}

__device__ __forceinline__ uint32_t fold_wave(uint4 pl) {
  uint32_t m = max(max(pl.x, pl.y), max(pl.z, pl.w));
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, false));    // [1,0,3,2]
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xF, 0xF, false));    // [2,3,0,1]
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x141, 0xF, 0xF, false));   // row_half_mirror
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x140, 0xF, 0xF, false));   // row_mirror
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)m, 0), b = (uint32_t)__builtin_amdgcn_readlane((int)m, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)m, 32), d = (uint32_t)__builtin_amdgcn_readlane((int)m, 48);
  return max(max(a, b), max(c, d));
}

// Pass 1: per-workgroup maximum of |x| (as 15-bit bf16 magnitude bits).
__global__ __launch_bounds__(kAmaxThreads) void k_amax_partials(const uint4* __restrict__ x, int64_t n_chunks,
                                                                uint32_t* __restrict__ partials) {
  __shared__ uint32_t red[kAmaxThreads / 64];
  uint32_t pk = 0;
  const int64_t stride = (int64_t)gridDim.x * kAmaxThreads;
  int64_t c = (int64_t)blockIdx.x * kAmaxThreads + threadIdx.x;
  for (; c + 3 * stride < n_chunks; c += 4 * stride) {
    const uint4 a = dev::load_nt(x + c), b = dev::load_nt(x + c + stride);
    const uint4 d = dev::load_nt(x + c + 2 * stride), e = dev::load_nt(x + c + 3 * stride);
    pk = max_pk_u16(pk, max_pk_u16(max_pk_u16(dev::mag_max_pk(a), dev::mag_max_pk(b)),
                                   max_pk_u16(dev::mag_max_pk(d), dev::mag_max_pk(e))));
  }
  for (; c < n_chunks; c += stride) pk = max_pk_u16(pk, dev::mag_max_pk(dev::load_nt(x + c)));
  uint32_t m = wave_max(dev::fold_halves_max(pk));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int i = 0; i < kAmaxThreads / 64; ++i) r = max(r, red[i]);
    partials[blockIdx.x] = r;
  }
}

// E4M3 value of a magnitude code 0..126: subnormal m * 2^-9, normal (8+m) 2^(e-10).
__device__ __forceinline__ double e4m3_value(int c) {
  int e = c >> 3, m = c & 7;
  return e == 0 ? (double)m * 0x1p-9 : ldexp((double)(8 + m), e - 10);
}

// Exact S_b code: the E4M3 code nearest to amax / (6 s_g), ties to the even code,
// saturating at 448 (code 126).  Binary search on exact fp64 comparisons.
__device__ __forceinline__ int exact_block_scale(double amax, double six_sg) {
  if (amax >= 448.0 * six_sg) return 126;
  int lo = 0, hi = 126;                  // invariant: val(lo) * d <= amax < val(hi) * d
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (e4m3_value(mid) * six_sg <= amax) lo = mid; else hi = mid;
  }
  double t = 0.5 * (e4m3_value(lo) + e4m3_value(hi)) * six_sg;
  if (amax < t) return lo;
  if (amax > t) return hi;
  return (lo & 1) ? hi : lo;
}

// Exact E2M1 magnitude code of |x| / D (D = S_b s_g exact in fp64): count the
// rounding midpoints passed; at a tie the even code wins, so the midpoints
// between (0, 0.5), (1, 1.5), (2, 3), (4, 6) need a strict '>' and the others '>='.
__device__ __forceinline__ uint32_t exact_e2m1(double ax, double D) {
  uint32_t c = 0;
  c += ax > 0.25 * D;
  c += ax >= 0.75 * D;
  c += ax > 1.25 * D;
  c += ax >= 1.75 * D;
  c += ax > 2.5 * D;
  c += ax >= 3.5 * D;
  c += ax > 5.0 * D;
  return c;
}

// Exact codes of the eight values of a chunk for divisor S s_g (S > 0).
__device__ __forceinline__ uint32_t exact_chunk(uint4 v, float S, float sg) {
  const double Dd = (double)S * (double)sg;                 // exact (4 x 24 bits)
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t codes = 0;
  for (int e = 0; e < 8; ++e) {
    uint32_t bits = (w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
    double ax = (double)__uint_as_float((bits & 0x7FFFu) << 16);
    uint32_t nib = exact_e2m1(ax, Dd) | ((bits >> 12) & 0x8u);
    codes |= nib << (4 * e);
  }
  return codes;
}

// Is a > mid * k * sg, exactly?  (mk = mid * k exact in fp32, a within a factor
// of two of mk * sg.)  mk * sg = p + e exactly (two-product by FMA, no underflow
// for the magnitudes that reach here); a - p is exact (Sterbenz); so the sign of
// a - mk * sg is that of (a - p) - e, decided by comparing a - p with e.  At an
// exact tie the code with an even last bit wins.
__device__ __forceinline__ bool round_up_at(float a, float mk, float sg, bool upper_even) {
  const float p = mk * sg;
  const float e = __builtin_fmaf(mk, sg, -p);
  const float d = a - p;
  return d > e || (d == e && upper_even);
}

// E2M1 magnitude code 0..7 -> value {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
__device__ __forceinline__ float e2m1_mag(uint32_t c) {
  return c < 2 ? 0.5f * (float)c : __builtin_ldexpf(1.0f + 0.5f * (float)(c & 1), (int)(c >> 1) - 1);
}

// Near-tie resolution for a chunk whose two bracketing encodings lo, hi differ:
// where a value's two codes differ, exactly one rounding midpoint (between the
// adjacent magnitudes) lies between the brackets; compare against it exactly.
__device__ __forceinline__ uint32_t resolve_chunk(uint4 v, uint32_t lo, uint32_t hi, float S, float sg) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t out = lo;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t nl = (lo >> (4 * e)) & 7u, nh = (hi >> (4 * e)) & 7u;
    if (nl != nh) {
      const float ax = __uint_as_float(((w[e >> 1] >> (16 * (e & 1))) & 0x7FFFu) << 16);
      const float mk = (e2m1_mag(nl) + e2m1_mag(nh)) * (0.5f * S);   // <= 7 significant bits
      const uint32_t c = round_up_at(ax, mk, sg, (nh & 1u) == 0) ? nh : nl;
      out = (out & ~(7u << (4 * e))) | (c << (4 * e));
    }
  }
  return out;
}

// Eight bf16 values (one uint4) -> eight E2M1 codes (a dword, element 2j in the low
// nibble of byte j), using reciprocal r of the divisor (0 encodes +-0).
__device__ __forceinline__ uint32_t encode8(uint4 v, float r) {
  uint32_t out = 0;
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, dev::bf16_lo(v.x) * r, dev::bf16_hi(v.x) * r, 1.0f, 0);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, dev::bf16_lo(v.y) * r, dev::bf16_hi(v.y) * r, 1.0f, 1);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, dev::bf16_lo(v.z) * r, dev::bf16_hi(v.z) * r, 1.0f, 2);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, dev::bf16_lo(v.w) * r, dev::bf16_hi(v.w) * r, 1.0f, 3);
  return out;
}

// TILED: scales in the GEMM-tiled order, with the work split of dev::TiledSlab
// (64 rows x 128 values per workgroup, every chunk in range); else the tensor is
// a flat stream of chunks.
template <bool TILED>
__global__ __launch_bounds__(kThreads) void k_quant_nvfp4(const uint4* __restrict__ x, int64_t n_chunks,
                                                          const float* __restrict__ global_in,
                                                          const uint32_t* __restrict__ partials, int n_partials,
                                                          uint32_t* __restrict__ q, uint8_t* __restrict__ s,
                                                          float* __restrict__ global_out, int reverse,
                                                          ScaleTiling tiling) {
  const int t = threadIdx.x;
  // with `reverse` workgroups take the slabs last to first: right after the amax
  // pass, what it read last is the likeliest to be left in a cache
  const int64_t slab = reverse ? (int64_t)gridDim.x - 1 - blockIdx.x : (int64_t)blockIdx.x;
  const int64_t base = slab * (kThreads * kUnroll);
  const auto ts = TILED ? dev::TiledSlab<kUnroll, 8>((int)slab, t, tiling) : dev::TiledSlab<kUnroll, 8>();
  auto chunk = [&](int u) { return TILED ? ts.chunk(u) : base + u * kThreads + t; };
  // dynamic mode: this lane's share of the partial maxima, loaded before the tensor
  // so that the fold below need not wait for the tensor's loads
  const uint4 pl = global_in ? make_uint4(0, 0, 0, 0) : partial_loads(partials, n_partials);
  uint4 v[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t c = chunk(u);
    v[u] = TILED || c < n_chunks ? dev::load_nt(x + c) : make_uint4(0, 0, 0, 0);
  }

  // ---- the global decode scale s_g (every wave folds the partials itself)
  float sg;
  if (global_in) {
    sg = *global_in;
  } else {
    const uint32_t amax = fold_wave(pl);
    // IEEE (correctly rounded) fp32 division: RN_fp32(amax / 2688).
    sg = amax == 0 ? 1.0f : __uint_as_float(amax << 16) / 2688.0f;
  }
  if (slab == 0 && t == 0) *global_out = sg;

  // ---- per-kernel constants: bracketing reciprocals of 6 s_g.  fl(6 s_g) is within
  // 2^-24 of 6 s_g and the hardware reciprocal within one ulp, so r6 is within
  // ~2^-22.4 of 1/(6 s_g), far inside the 2^-19 nudges.  Outside fp32's normal
  // range (including a zero, negative, infinite or NaN static s_g) the fp64 search
  // decides.
  const float r6 = __builtin_amdgcn_rcpf(6.0f * sg);
  const float r6_lo = r6 * (1.0f - 0x1p-19f);
  const float r6_hi = r6 * (1.0f + 0x1p-19f);
  const bool fast6 = r6 < 0x1p126f && r6 > 0x1p-126f;

  // The chunks go through each phase in groups of kGroup, so that the fast path is
  // straight-line code and the exact fallbacks are entered once per phase and
  // group, only when some lane needs them (groups of two keep the kernel within
  // the registers of eight waves per SIMD).
  constexpr int kGroup = 2;
#pragma unroll
  for (int g0 = 0; g0 < kUnroll; g0 += kGroup) {
    // ---- block maxima: lanes 2j, 2j+1 hold the two halves of one 16-block
    // (n_chunks is even); their maxima meet through a DPP swap within lane pairs
    float amax_b[kGroup];
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      const uint32_t m = dev::fold_halves_max(dev::mag_max_pk(v[g0 + i]));
      const uint32_t other = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
      amax_b[i] = __uint_as_float(max(m, other) << 16);
    }

    // ---- S_b = RN_E4M3(amax_b / (6 s_g)), from the two bracketing quotients
    int sb[kGroup], sb_hi[kGroup];
    bool exact_sb = !fast6;
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      const float ql = __builtin_amdgcn_fmed3f(amax_b[i] * r6_lo, 0.0f, 448.0f);
      const float qh = __builtin_amdgcn_fmed3f(amax_b[i] * r6_hi, 0.0f, 448.0f);
      const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(ql, qh, 0, false);
      sb[i] = pk & 0xFF;
      sb_hi[i] = (pk >> 8) & 0xFF;
      exact_sb |= sb[i] != sb_hi[i];
    }
    if (__builtin_expect(exact_sb, 0)) {
#pragma unroll
      for (int i = 0; i < kGroup; ++i) {
        const int cl = sb[i], ch = sb_hi[i];
        if (!fast6) {
          sb[i] = exact_block_scale((double)amax_b[i], 6.0 * (double)sg);   // 6 s_g exact in fp64
        } else if (cl != ch) {
          // one midpoint between the adjacent codes cl < ch: compare exactly
          const float mk = (__builtin_amdgcn_cvt_f32_fp8(cl, 0) + __builtin_amdgcn_cvt_f32_fp8(ch, 0)) * 3.0f;
          sb[i] = round_up_at(amax_b[i], mk, sg, (ch & 1) == 0) ? ch : cl;
        }
      }
    }

    // ---- codes: x / (S s_g), bracketed.  S = 0 gives r = 0 and signed zeros.
    uint32_t codes[kGroup], codes_hi[kGroup];
    float S[kGroup];
    bool exact_c = false;
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      S[i] = __builtin_amdgcn_cvt_f32_fp8(sb[i], 0);        // E4M3 -> fp32, exact
      const float D = S[i] * sg;
      const float r = S[i] == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(D);   // <= 1 ulp
      codes[i] = encode8(v[g0 + i], r * (1.0f - 0x1p-19f));
      codes_hi[i] = encode8(v[g0 + i], r * (1.0f + 0x1p-19f));
      // the fp64 path serves a tiny divisor (reciprocal or two-product out of
      // range) or a saturated block scale (only a static s_g can then push
      // quotients far past 6); otherwise a midpoint between the brackets is
      // settled exactly in fp32
      exact_c |= S[i] != 0.0f && (codes[i] != codes_hi[i] || !(D >= 0x1p-100f) || sb[i] == 126);
    }
    if (__builtin_expect(exact_c, 0)) {
#pragma unroll
      for (int i = 0; i < kGroup; ++i) {
        if (S[i] == 0.0f) continue;
        const float D = S[i] * sg;
        if (!(D >= 0x1p-100f) || sb[i] == 126) codes[i] = exact_chunk(v[g0 + i], S[i], sg);
        else if (codes[i] != codes_hi[i]) codes[i] = resolve_chunk(v[g0 + i], codes[i], codes_hi[i], S[i], sg);
      }
    }

#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      const int u = g0 + i;
      const int64_t c = chunk(u);
      if (TILED || c < n_chunks) {
        q[c] = codes[i];
        if ((t & 1) == 0) s[TILED ? ts.scale(u) : c >> 1] = (uint8_t)sb[i];
      }
    }
  }
}

// Per-tensor E4M3 encoding, shared by the weight quantizer and the attention's V
// quantizer (page "麦橘超然性能实战分析：float8量化如何提升GPU利用率", section 3.2:
// DiT weights held as float8_e4m3fn; page "FP8量化技术提升SD3.5在低带宽环境下的响应速度",
// step 2: q = round(w / scale)):
//   s = RN_fp32(amax / 448) (1 for an all-zero tensor; or given), q = RN_E4M3_sat(w / s).
// The quotient is bracketed like the NVFP4 codes; a near tie is settled by
// round_up_at against the midpoint of the two candidate codes; an extreme s takes
// the fp64 search.
struct E4M3Encoder {
  float sw, r_lo, r_hi;
  bool fast;
};

// The decode scale: given, or RN_fp32(amax / 448) from the amax pass's partial
// maxima (every thread of the workgroup calls this; red holds 4 words of LDS).
__device__ __forceinline__ E4M3Encoder e4m3_encoder(const float* scale_in, const uint32_t* partials, int n_partials,
                                                    uint32_t* red) {
  E4M3Encoder enc;
  const int t = threadIdx.x;
  if (scale_in) {
    enc.sw = *scale_in;
  } else {
    uint32_t m = t < n_partials ? partials[t] : 0u;
    m = wave_max(m);
    if ((t & 63) == 0) red[t >> 6] = m;
    __syncthreads();
    const uint32_t amax = max(max(red[0], red[1]), max(red[2], red[3]));
    enc.sw = amax == 0 ? 1.0f : __uint_as_float(amax << 16) / 448.0f;   // IEEE division
  }
  const double rd = 1.0 / (double)enc.sw;
  enc.r_lo = (float)(rd * (1.0 - 0x1p-19));
  enc.r_hi = (float)(rd * (1.0 + 0x1p-19));
  // fp32 brackets and the two-product test need sw and 1/sw well inside fp32's range
  enc.fast = rd < 0x1p126 && rd > 0x1p-126 && enc.sw >= 0x1p-100f;
  return enc;
}

// Four values (exact fp32 of bf16 inputs) -> four E4M3 codes, byte e = xs[e].
__device__ __forceinline__ uint32_t encode_e4m3x4(const E4M3Encoder& enc, const float (&xs)[4]) {
  int lo = 0, hi = 0;
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(xs[0] * enc.r_lo, -448.0f, 448.0f),
                                       __builtin_amdgcn_fmed3f(xs[1] * enc.r_lo, -448.0f, 448.0f), lo, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(xs[2] * enc.r_lo, -448.0f, 448.0f),
                                       __builtin_amdgcn_fmed3f(xs[3] * enc.r_lo, -448.0f, 448.0f), lo, true);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(xs[0] * enc.r_hi, -448.0f, 448.0f),
                                       __builtin_amdgcn_fmed3f(xs[1] * enc.r_hi, -448.0f, 448.0f), hi, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(xs[2] * enc.r_hi, -448.0f, 448.0f),
                                       __builtin_amdgcn_fmed3f(xs[3] * enc.r_hi, -448.0f, 448.0f), hi, true);
  uint32_t codes = (uint32_t)lo;
  if (__builtin_expect(!enc.fast, 0)) {
    codes = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t mag = (uint32_t)exact_block_scale((double)fabsf(xs[e]), (double)enc.sw);
      codes |= (mag | (__float_as_uint(xs[e]) >> 31 << 7)) << (8 * e);
    }
  } else if (__builtin_expect(codes != (uint32_t)hi, 0)) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t cl = (codes >> (8 * e)) & 0x7Fu, ch = ((uint32_t)hi >> (8 * e)) & 0x7Fu;
      if (cl != ch) {
        const float mk = (__builtin_amdgcn_cvt_f32_fp8((int)cl, 0) + __builtin_amdgcn_cvt_f32_fp8((int)ch, 0)) * 0.5f;
        const uint32_t mag = round_up_at(fabsf(xs[e]), mk, enc.sw, (ch & 1) == 0) ? ch : cl;
        codes = (codes & ~(0x7Fu << (8 * e))) | (mag << (8 * e));
      }
    }
  }
  return codes;
}

// Per-tensor FP8 weights: eight values per lane (one uint4 of bf16 -> one uint2 of codes).
__global__ __launch_bounds__(kThreads) void k_quant_fp8_tensor(const uint4* __restrict__ x, int64_t n_chunks,
                                                               const float* __restrict__ scale_in,
                                                               const uint32_t* __restrict__ partials,
                                                               int n_partials, uint2* __restrict__ q,
                                                               float* __restrict__ scale_out) {
  __shared__ uint32_t red[kThreads / 64];
  const int t = threadIdx.x;
  const int64_t base = (int64_t)blockIdx.x * (kThreads * kUnroll);
  uint4 v[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t c = base + u * kThreads + t;
    v[u] = c < n_chunks ? x[c] : make_uint4(0, 0, 0, 0);
  }
  const E4M3Encoder enc = e4m3_encoder(scale_in, partials, n_partials, red);
  if (blockIdx.x == 0 && t == 0) *scale_out = enc.sw;
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t c = base + u * kThreads + t;
    const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
    uint32_t out[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float xs[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) xs[e] = (e & 1) ? dev::bf16_hi(w[2 * h + (e >> 1)]) : dev::bf16_lo(w[2 * h + (e >> 1)]);
      out[h] = encode_e4m3x4(enc, xs);
    }
    if (c < n_chunks) q[c] = make_uint2(out[0], out[1]);
  }
}

// V of the FP8 attention: [heads * L, 128] bf16 -> per-tensor E4M3 codes in the
// attention kernel's V layout, [heads][128][L] (V transposed, so that a row holds
// one output column over the keys), with the columns of every 64-key block
// permuted: column 32g + s holds key 32 (s / 16) + 8 ((s % 16) / 4) + 4g + s % 4.
// That is the key whose probability lane group g of the score MFMA holds in its
// register slot s, so the P.V operands pair up byte for byte.  One workgroup per
// 64-key block of a head: the bf16 block through LDS, then 32 codes per thread.
__global__ __launch_bounds__(kThreads) void k_quant_fp8_vt(const uint16_t* __restrict__ v, int L,
                                                           const float* __restrict__ scale_in,
                                                           const uint32_t* __restrict__ partials, int n_partials,
                                                           uint8_t* __restrict__ vt, float* __restrict__ scale_out) {
  constexpr int kRow = 136;                       // bf16 per staged key row (128 + 8 of padding)
  __shared__ __attribute__((aligned(16))) uint16_t tile[64 * kRow];
  __shared__ uint32_t red[kThreads / 64];
  const int t = threadIdx.x, kb = blockIdx.x, head = blockIdx.y;
  const uint16_t* src = v + ((size_t)head * L + kb * 64 + t / 4) * 128 + (t % 4) * 32;
#pragma unroll
  for (int u = 0; u < 4; ++u) *(uint4*)(tile + (t / 4) * kRow + (t % 4) * 32 + 8 * u) = ((const uint4*)src)[u];
  const E4M3Encoder enc = e4m3_encoder(scale_in, partials, n_partials, red);
  if (kb == 0 && head == 0 && t == 0) *scale_out = enc.sw;
  __syncthreads();
  const int e = t >> 1, g = t & 1;
  uint32_t out[8];
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    float xs[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int sl = 4 * w + u;
      const int key = 32 * (sl / 16) + 8 * ((sl % 16) / 4) + 4 * g + sl % 4;
      xs[u] = __uint_as_float((uint32_t)tile[key * kRow + e] << 16);
    }
    out[w] = encode_e4m3x4(enc, xs);
  }
  uint4* dst = (uint4*)(vt + ((size_t)head * 128 + e) * L + kb * 64 + 32 * g);
  dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
  dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
}

// Calibration fold: running = max(running, RN_fp32(amax / 2688)) over the partial
// maxima of one calibration tensor (an all-zero tensor contributes 0).  One
// workgroup; the caller orders calls on one stream.
__global__ __launch_bounds__(kThreads) void k_calib_fold(const uint32_t* __restrict__ partials, int n_partials,
                                                         float* __restrict__ running) {
  __shared__ uint32_t red[kThreads / 64];
  const int t = threadIdx.x;
  uint32_t m = t < n_partials ? partials[t] : 0u;
  m = wave_max(m);
  if ((t & 63) == 0) red[t >> 6] = m;
  __syncthreads();
  if (t == 0) {
    const uint32_t amax = max(max(red[0], red[1]), max(red[2], red[3]));
    const float sg = amax == 0 ? 0.0f : __uint_as_float(amax << 16) / 2688.0f;   // IEEE division
    *running = fmaxf(*running, sg);
  }
}

}  // namespace

// The amax pass over n_chunks 16-byte chunks into n_partials partial maxima.
static hipError_t amax_pass(const void* x, int64_t n_chunks, uint32_t* partials, int n_partials,
                            hipStream_t stream) {
  hipLaunchKernelGGL(k_amax_partials, dim3(n_partials), dim3(kAmaxThreads), 0, stream, (const uint4*)x, n_chunks,
                     partials);
  return hipGetLastError();
}

hipError_t launch_quantize_fp8_tensor(const void* x, int64_t n_elems, const float* scale_in, void* q,
                                     float* scale_out, uint32_t* partials, hipStream_t stream) {
  const int64_t n_chunks = n_elems / 8;
  int n_partials = 0;
  if (!scale_in) {
    n_partials = nvfp4_amax_partials(n_elems);
    hipError_t e = amax_pass(x, n_chunks, partials, n_partials, stream);
    if (e != hipSuccess) return e;
  }
  const int64_t per_wg = (int64_t)kThreads * kUnroll;
  const int64_t grid = (n_chunks + per_wg - 1) / per_wg;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_quant_fp8_tensor, dim3((unsigned)grid), dim3(kThreads), 0, stream, (const uint4*)x, n_chunks,
                     scale_in, partials, n_partials, (uint2*)q, scale_out);
  return hipGetLastError();
}

hipError_t launch_quantize_fp8_vt(const void* v, int64_t heads, int64_t L, const float* scale_in, void* vt,
                                  float* scale_out, uint32_t* partials, hipStream_t stream) {
  const int64_t n_elems = heads * L * 128;
  int n_partials = 0;
  if (!scale_in) {
    n_partials = nvfp4_amax_partials(n_elems);
    hipError_t e = amax_pass(v, n_elems / 8, partials, n_partials, stream);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_quant_fp8_vt, dim3((unsigned)(L / 64), (unsigned)heads), dim3(kThreads), 0, stream,
                     (const uint16_t*)v, (int)L, scale_in, partials, n_partials, (uint8_t*)vt, scale_out);
  return hipGetLastError();
}

hipError_t launch_nvfp4_calibrate(const void* x, int64_t n_elems, float* running, uint32_t* partials,
                                  hipStream_t stream) {
  const int64_t n_chunks = n_elems / 8;
  const int n_partials = nvfp4_amax_partials(n_elems);
  hipError_t e = amax_pass(x, n_chunks, partials, n_partials, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_calib_fold, dim3(1), dim3(kThreads), 0, stream, partials, n_partials, running);
  return hipGetLastError();
}

// Scratch for callers that cannot allocate (mxq_quantize_nvfp4_noalloc): the
// partial maxima of the amax pass in a file-scope device array, one copy per GPU
// at its own address.  The amax pass never uses more than kMaxPartials
// workgroups, so 1 KiB covers a tensor of any size.  Each workgroup of the pass
// writes its own slot before the encode pass reads it, so nothing needs clearing;
// calls that overlap on one GPU share the array and race.
static __device__ __align__(256) uint32_t scratch[kMaxPartials];

hipError_t amax_scratch(uint32_t** ptr, int* words) {
  constexpr int kMaxDevices = 64;
  static std::atomic<uintptr_t> addr[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  uintptr_t a = addr[dev].load(std::memory_order_acquire);
  if (a == 0) {
    // The host-side name `scratch` is not a device address: look it up once per
    // device, with that device current, and use only the address it returns.
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    a = (uintptr_t)p;
    addr[dev].store(a, std::memory_order_release);
  }
  *ptr = (uint32_t*)a;
  *words = kMaxPartials;
  return hipSuccess;
}

int nvfp4_amax_partials(int64_t n_elems) {
  const int64_t n_chunks = n_elems / 8;
  int64_t p = (n_chunks + (int64_t)kAmaxThreads * 4 - 1) / ((int64_t)kAmaxThreads * 4);
  if (p < 1) p = 1;
  if (p > kMaxPartials) p = kMaxPartials;
  return (int)p;
}

hipError_t launch_quantize_nvfp4(const void* x, int64_t n_elems, const float* global_in, void* q,
                                 void* scales, float* global_out, uint32_t* partials,
                                 ScaleTiling tiling, hipStream_t stream) {
  const int64_t n_chunks = n_elems / 8;
  int n_partials = 0;
  if (!global_in) {
    n_partials = nvfp4_amax_partials(n_elems);
    hipError_t e = amax_pass(x, n_chunks, partials, n_partials, stream);
    if (e != hipSuccess) return e;
  }
  const int64_t per_wg = (int64_t)kThreads * kUnroll;   // = 64 rows x 128 values when tiled
  const int64_t grid = (n_chunks + per_wg - 1) / per_wg;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
#define MXQ_NV_QUANT(T)                                                                                     \
  hipLaunchKernelGGL((k_quant_nvfp4<T>), dim3((unsigned)grid), dim3(kThreads), 0, stream, (const uint4*)x,   \
                     n_chunks, global_in, partials, n_partials, (uint32_t*)q, (uint8_t*)scales, global_out, \
                     global_in ? 0 : 1, tiling)
  if (tiling.nst) MXQ_NV_QUANT(true);
  else MXQ_NV_QUANT(false);
#undef MXQ_NV_QUANT
  return hipGetLastError();
}

}  // namespace mxq
