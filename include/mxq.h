/*
 * mxq.h -- C ABI of the microscaling-quantized linear layer for AMD MI355X (gfx950).
 *
 * Two parts of a quantized diffusion-transformer Linear:
 *   1. dynamic microscaling quantizers for bf16 tensors (MXFP8, NVFP4);
 *   2. block-scaled GEMMs that consume those codes and scales and return bf16,
 *      optionally with a fused bias or bias + GELU (tanh form).
 *
 * Sources (pages, by title and section):
 *   [P1] "NVIDIA量化推理：5步极速优化显存+成功率翻倍", section "MXFP8和NVFP4技术背景解析":
 *        blocks of 16 or 32 values share a high-precision scale; MXFP8 (OCP) has
 *        E4M3 and E5M2 elements; NVFP4 is E2M1 in blocks of 16 with FP8 scales.
 *        Step 2: dynamic activation + weight quantization with a dynamic
 *        per-tensor scale.
 *   [P2] "NVIDIA Blackwell平台FP4量化技术解析与图像生成优化", section 3.1: the runtime
 *        quantizer turns bf16 into [FP4 data, FP8 block scales, FP32 global
 *        scale]; weights are quantized offline the same way.  Section 5.2:
 *        quantization blocks aligned to multiples of 128.
 *   [P3] "Modelos de Difusão": every torch.nn.Linear of the transformer is
 *        quantized (nn.Linear orientation: C = A W^T).
 *   [P4] "麦橘超然性能实战分析：float8量化如何提升GPU利用率", section 2.2: E4M3 is
 *        1+4+3 bits, E5M2 1+5+2 bits.
 *   [P5] "FP8量化技术提升SD3.5在低带宽环境下的响应速度", step 2: q = round(x/scale).
 *
 * Number formats and rounding (the pages name the formats; where they are
 * silent these readings are taken):
 *   - every stored quantity is ONE round-to-nearest-even of its exact value,
 *     saturating to the largest finite magnitude (E4M3 448, E5M2 57344, E2M1 6);
 *   - the sign bit of every element code is the sign bit of the input;
 *   - MXFP8: per 32 consecutive values of a row, E = floor(log2 amax) - emax
 *     (emax = 8 for E4M3, 15 for E5M2), clamped to [-127, 127], E = -127 for an
 *     all-zero block; the E8M0 scale byte is E + 127; q = RNE_sat(x / 2^E);
 *   - NVFP4: s_g = RN_fp32(amax_tensor / 2688) (2688 = 6 * 448; 1 if the tensor
 *     is all zero) is the fp32 DECODE global scale; per 16 consecutive values
 *     S_b = RN_E4M3_sat(amax_block / (6 s_g)) (may be 0); q = RN_E2M1_sat(x / (S_b s_g)),
 *     magnitude 0 when S_b = 0; dequantized value = val(q) * val(S_b) * s_g.
 *
 * Layouts (row-major, no padding; block scales also in a tiled order, below):
 *   x        bf16  [rows, cols]            cols contiguous (K for a GEMM operand)
 *   MXFP8 q  u8    [rows, cols]            E4M3 or E5M2 codes
 *   MXFP8 s  u8    [rows, cols / 32]       E8M0 scale bytes
 *   NVFP4 q  u8    [rows, cols / 2]        byte j holds element 2j in its low nibble
 *   NVFP4 s  u8    [rows, cols / 16]       E4M3 scale codes
 *   GEMM     C[M, N] = A[M, K] * W[N, K]^T, C bf16 [M, N]
 *
 * Conventions:
 *   - All tensor pointers are DEVICE pointers on the current HIP device, owned
 *     by the caller; the library never allocates or frees (its one piece of
 *     device memory is the 1 KiB static scratch of mxq_quantize_nvfp4_noalloc).
 *     Base pointers must be 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = default stream).  Every call is
 *     asynchronous on that stream and never synchronizes; outputs are valid
 *     after the caller synchronizes the stream.
 *   - Arguments are validated before any launch; an invalid call returns a
 *     status and launches nothing.  mxq_last_error() gives the detail.
 *   - Inputs must be finite (NaN/Inf inputs give unspecified codes).
 *   - No exceptions cross the ABI; no global mutable state besides a per-thread
 *     error string, per-device caches (architecture, compute units, the scratch
 *     address) and that scratch.
 *   - Requires a gfx950 device (MXFP8/NVFP4 scaled MFMA); other devices get
 *     MXQ_ERROR_UNSUPPORTED_DEVICE.
 */
#ifndef MXQ_H_
#define MXQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MXQ_SUCCESS = 0,
  MXQ_ERROR_INVALID_VALUE = 1,     /* null pointer, non-positive size, bad enum */
  MXQ_ERROR_UNSUPPORTED_SHAPE = 2, /* size not a multiple of the block / tile rule */
  MXQ_ERROR_MISALIGNED = 3,        /* a base pointer is not 16-byte aligned */
  MXQ_ERROR_WORKSPACE = 4,         /* workspace missing or smaller than required */
  MXQ_ERROR_UNSUPPORTED_DEVICE = 5,/* current device is not gfx950 */
  MXQ_ERROR_LAUNCH = 6             /* the HIP runtime refused a launch */
} mxq_status;

typedef enum { MXQ_FP8_E4M3 = 0, MXQ_FP8_E5M2 = 1 } mxq_fp8_kind;

typedef enum {
  MXQ_EPI_NONE = 0,          /* y = acc */
  MXQ_EPI_BIAS = 1,          /* y = acc + bias[n] */
  MXQ_EPI_BIAS_GELU_TANH = 2 /* y = GELU_tanh(acc + bias[n]) */
} mxq_epilogue;

/*
 * Byte order of a block-scale array [rows, cols / B] (B = 32 for MXFP8, 16 for
 * NVFP4); the size is rows * cols / B bytes in both.  This is a storage choice of
 * this library, not a format of the pages.
 *   MXQ_SCALES_ROW_MAJOR : scale (r, j) at byte r * (cols / B) + j.
 *   MXQ_SCALES_TILED     : rows in blocks of 64, K in steps of 128 values; with
 *                          P = 128 / B scales per row and step (4 MXFP8, 8 NVFP4)
 *                          scale (r, j) at byte
 *                            ((r / 64) * (cols / 128) + j / P) * 64 P + (r % 64) P + j % P,
 *                          i.e. one contiguous run of 64 P bytes per (row block,
 *                          K step): the GEMMs fetch a K step's scales for 64 rows
 *                          with one contiguous load.  Needs rows % 64 == 0 and
 *                          cols % 128 == 0.
 * Quantizers write either order; the GEMMs read both operands' scales in the one
 * order they are given.  Codes are row-major in both.
 */
typedef enum { MXQ_SCALES_ROW_MAJOR = 0, MXQ_SCALES_TILED = 1 } mxq_scale_layout;

/*
 * MXFP8 quantizer [P1 "MXFP8和NVFP4技术背景解析"; P5 step 2].
 *   x      : bf16 [rows, cols], device, read only.
 *   rows   : > 0.   cols: > 0 and a multiple of 32 (else MXQ_ERROR_UNSUPPORTED_SHAPE).
 *   kind   : element format, E4M3 or E5M2.
 *   q      : u8 [rows, cols], device, written.
 *   scales : u8 [rows, cols/32] E8M0, device, written in the order scale_layout
 *            names (MXQ_SCALES_TILED: rows % 64 == 0 and cols % 128 == 0, else
 *            MXQ_ERROR_UNSUPPORTED_SHAPE).
 * One pass over x; codes and scales are bit-exact to the definition above.
 */
mxq_status mxq_quantize_mxfp8(const void* x, int64_t rows, int64_t cols, mxq_fp8_kind kind,
                              void* q, void* scales, mxq_scale_layout scale_layout, void* stream);

/* Bytes of device workspace mxq_quantize_nvfp4 needs (dynamic mode) for this
 * shape; 0 for invalid shapes.  The workspace holds per-workgroup partial
 * maxima; it needs no initialization and its contents are scratch. */
size_t mxq_quantize_nvfp4_workspace_size(int64_t rows, int64_t cols);

/*
 * NVFP4 quantizer [P1 "MXFP8和NVFP4技术背景解析", step 2 dynamic per-tensor scale;
 * P2 section 3.1: outputs FP4 data, FP8 scales, FP32 global scale].
 *   x                : bf16 [rows, cols], device.
 *   rows, cols       : > 0, cols a multiple of 16.
 *   global_scale_in  : device fp32 decode scale to use (static mode, must be
 *                      positive and finite), or NULL for the dynamic scale
 *                      s_g = RN_fp32(amax(x) / 2688) taken over the whole tensor.
 *   q                : u8 [rows, cols/2] packed E2M1, device, written.
 *   scales           : u8 [rows, cols/16] E4M3, device, written in the order
 *                      scale_layout names (tiled: rows % 64 == 0, cols % 128 == 0).
 *   global_scale_out : device fp32, written with the s_g used (both modes).
 *   workspace        : device scratch of mxq_quantize_nvfp4_workspace_size bytes
 *                      (dynamic mode; may be NULL in static mode).
 * Dynamic mode makes two passes over x (tensor amax, then encode).  Calls that
 * share a workspace must be ordered on one stream.
 */
mxq_status mxq_quantize_nvfp4(const void* x, int64_t rows, int64_t cols,
                              const float* global_scale_in, void* q, void* scales,
                              mxq_scale_layout scale_layout, float* global_scale_out,
                              void* workspace, size_t ws_bytes, void* stream);

/*
 * NVFP4 quantizer that allocates nothing and takes no workspace -- for callers
 * that cannot allocate device memory or pass a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 *   Arguments, layouts, results and errors: as mxq_quantize_nvfp4 without
 *   workspace and ws_bytes; the results are bit-identical to it.
 *   Dynamic mode keeps the amax pass's partial maxima in the library's own
 *   device scratch: a file-scope array of 256 words (1 KiB) per GPU, held until
 *   the process ends.  The amax pass never uses more than 256 workgroups, so any
 *   tensor size fits; a shape that would need more returns MXQ_ERROR_WORKSPACE.
 *   The scratch needs no clearing (every slot read is written first by the same
 *   call).  All calls on one GPU share it: calls that overlap in time on one GPU
 *   (on different streams, or from several host threads without ordering) race
 *   and may produce a wrong global scale; order them on one stream.
 *   The scratch address is looked up once per device on the first call made
 *   with that device current (hipGetSymbolAddress); a failed lookup returns
 *   MXQ_ERROR_LAUNCH.  No call allocates or frees memory.
 */
mxq_status mxq_quantize_nvfp4_noalloc(const void* x, int64_t rows, int64_t cols,
                                      const float* global_scale_in, void* q, void* scales,
                                      mxq_scale_layout scale_layout, float* global_scale_out,
                                      void* stream);

/*
 * Static-scale calibration for NVFP4 activations [P5 step 1 "校准": run a small
 * batch through the model and record each layer's maximum, from which the scale
 * that avoids truncation is set; P1 step 2 names the per-tensor scale].
 *   x             : bf16 [rows, cols], device: one calibration tensor.
 *   rows, cols    : > 0, cols a multiple of 16.
 *   running_scale : device fp32, read and written:
 *                   running_scale = max(running_scale, RN_fp32(amax(x) / 2688)),
 *                   where an all-zero x contributes 0.  Set it to 0 before the
 *                   first calibration tensor.  After the last one it is
 *                   RN_fp32(max amax / 2688), the decode scale the dynamic mode
 *                   would choose for the largest calibration tensor, and can be
 *                   passed as global_scale_in of mxq_quantize_nvfp4 (one pass per
 *                   call instead of two) as long as it is positive.  Values
 *                   beyond the calibrated range then saturate to +-6 x S_b.
 *   workspace     : as for mxq_quantize_nvfp4 (same size query).
 * Calls that share running_scale or the workspace must be ordered on one stream.
 */
mxq_status mxq_nvfp4_calibrate(const void* x, int64_t rows, int64_t cols, float* running_scale,
                               void* workspace, size_t ws_bytes, void* stream);

/*
 * Weight-only FP8: per-tensor E4M3 weights [P4 section 3.2: the DiT weights are
 * held as float8_e4m3fn while activations stay bf16; P5 step 2: q = round(w/scale),
 * dequantized as q * scale].
 *   w         : bf16 [rows, cols], device (a weight, N x K).
 *   rows, cols: > 0, cols a multiple of 16.
 *   scale_in  : device fp32 decode scale to use (positive, finite), or NULL for
 *               s = RN_fp32(amax(w) / 448) (1 for an all-zero tensor).
 *   q         : u8 [rows, cols] E4M3 codes, device, written: RN_E4M3_sat(w / s),
 *               sign copied.
 *   scale_out : device fp32, written with the s used.
 *   workspace : NULL mode only; size and rules as for mxq_quantize_nvfp4.
 */
mxq_status mxq_quantize_fp8_weight(const void* w, int64_t rows, int64_t cols, const float* scale_in,
                                   void* q, float* scale_out, void* workspace, size_t ws_bytes,
                                   void* stream);

/*
 * V operand of the FP8 attention [P2 section 2.1: multi-head attention in FP8;
 * per-tensor E4M3 as for mxq_quantize_fp8_weight].
 *   v         : bf16 [heads * L, d], device; head h is rows h*L .. h*L + L - 1.
 *   heads, L, d: heads > 0, d == 128, L a positive multiple of 128, L * 128 < 2^31.
 *   scale_in, scale_out, workspace: as mxq_quantize_fp8_weight with rows = heads * L,
 *               cols = d (the scale covers the whole tensor).
 *   vt        : u8 [heads, 128, L], device, written: the E4M3 codes of V transposed,
 *               with the columns of every 64-key block b permuted:
 *               vt[h][c][64 b + 32 g + s] = code(v[h L + 64 b + 32 (s / 16)
 *                                                   + 8 ((s % 16) / 4) + 4 g + s % 4][c])
 *               for g in {0, 1}, s in [0, 32) -- the order in which
 *               mxq_attention_fp8 holds the probabilities of a block.
 */
mxq_status mxq_quantize_fp8_v(const void* v, int64_t heads, int64_t L, int64_t d, const float* scale_in,
                              void* vt, float* scale_out, void* workspace, size_t ws_bytes, void* stream);

/*
 * FP8 multi-head attention [P2 section 2.1: in the mixed-precision configuration,
 * multi-head attention runs in FP8], per head, non-causal:
 *   S_ij = (s_q s_k / sqrt(d)) sum_c val(q[i,c]) val(k[j,c])
 *   m_i = max_j S_ij over every key of the row, P_ij = exp(S_ij - m_i),
 *   l_i = sum_j P_ij (unquantized),
 *   o[i,:] = bf16( s_v sum_j val(RN_E4M3(256 P_ij)) val(v[j,:]) / (256 l_i) )
 * i.e. the probabilities enter the second product as E4M3 codes of 256 P,
 * quantized against the row's own maximum (no blocking of the keys is part of
 * the result).  Both products on FP8 matrix cores with fp32 accumulation (exact
 * products); the kernel makes two passes over the keys (the maximum, then P and
 * the product).
 *   q, k      : u8 [heads * L, d] E4M3 codes (mxq_quantize_fp8_weight with
 *               rows = heads * L), device; q_scale, k_scale their device fp32 scales.
 *   vt, v_scale: V in the layout of mxq_quantize_fp8_v, and its scale.
 *   heads, L, d: as mxq_quantize_fp8_v.
 *   o         : bf16 [heads * L, d], device, written.
 * Errors: invalid value (null pointer, heads or L not positive), unsupported shape
 * (d != 128, L not a multiple of 128, L * 128 >= 2^31), misalignment (q, k, vt,
 * o not 16-byte, scales not 4-byte aligned), device, launch failure.
 */
mxq_status mxq_attention_fp8(const void* q, const float* q_scale, const void* k, const float* k_scale,
                             const void* vt, const float* v_scale, int64_t heads, int64_t L, int64_t d,
                             void* o, void* stream);

/*
 * Weight-only FP8 GEMM [P4 sections 3.2 and 4: FP8 weights converted back for a
 * bf16 product ("fake quantization", P5), at a small time cost].
 *   C[m, n] = epi( s_w sum_k a[m,k] val(w_q[n,k]) (+ bias[n]) ), fp32 accumulation,
 *   one RNE to bf16.  The E4M3 values are exact in bf16, so the products are exact.
 *   a      : bf16 [M, K] row-major, device.
 *   w_q    : u8 [N, K] E4M3 (from mxq_quantize_fp8_weight), device.
 *   w_scale: device fp32 s_w.
 *   M, N, K, bias, epi, c, errors: as mxq_gemm_mxfp8 (a counts 2 bytes per
 *   element towards the 2 GiB operand limit).
 */
mxq_status mxq_gemm_bf16_fp8w(const void* a, const void* w_q, const float* w_scale, int64_t M,
                              int64_t N, int64_t K, const void* bias, mxq_epilogue epi, void* c,
                              void* stream);

/*
 * MXFP8 block-scaled GEMM [P3: every nn.Linear runs quantized; P2 §5.2: 128 alignment].
 *   C[m, n] = epi( sum_k val(a_q[m,k]) 2^(a_s[m,k/32]-127) val(w_q[n,k]) 2^(w_s[n,k/32]-127)
 *                  (+ bias[n]) ), fp32 accumulation, one RNE to bf16.
 *   a_q, a_scales : A codes u8 [M, K] and E8M0 [M, K/32] (from mxq_quantize_mxfp8).
 *   w_q, w_scales : W codes u8 [N, K] and E8M0 [N, K/32].
 *   a_kind, w_kind: element formats of A and W (E4M3 / E5M2, may differ).
 *   scale_layout  : order of both a_scales and w_scales; the tiled order saves
 *                   the GEMM scattered scale loads.
 *   M, N, K       : > 0, multiples of 128 (else MXQ_ERROR_UNSUPPORTED_SHAPE).
 *   bias          : bf16 [N] device (required unless epi == MXQ_EPI_NONE).
 *   c             : bf16 [M, N] device, written.
 */
mxq_status mxq_gemm_mxfp8(const void* a_q, const void* a_scales, mxq_fp8_kind a_kind,
                          const void* w_q, const void* w_scales, mxq_fp8_kind w_kind,
                          mxq_scale_layout scale_layout,
                          int64_t M, int64_t N, int64_t K, const void* bias, mxq_epilogue epi,
                          void* c, void* stream);

/*
 * MXFP8 GEMM with the activation quantizer fused into its prologue [P2 section 3.1:
 * at run time the bf16 activation is quantized dynamically and handed with its
 * scales to the low-precision GEMM; P1 MXFP8 paragraph].
 *   C = epi( Q(a) . W^T ), Q the MXFP8 activation quantizer of mxq_quantize_mxfp8
 *   in format kind.  The result is bit-identical to mxq_quantize_mxfp8(a, kind)
 *   followed by mxq_gemm_mxfp8 with a_kind = w_kind = kind: the codes and scales
 *   are the same, and so are the products, their accumulation order and the
 *   epilogue.  A's codes never reach memory.
 *   a          : bf16 [M, K] row-major, device.
 *   kind       : element format of A's codes and of W (one format for both).
 *   w_q, w_scales, scale_layout: W codes u8 [N, K] and E8M0 scales [N, K/32] in
 *                scale_layout (from mxq_quantize_mxfp8).
 *   M, N, K, bias, epi, c, errors: as mxq_gemm_mxfp8 (a counts 2 bytes per
 *   element towards the 2 GiB operand limit).
 */
mxq_status mxq_gemm_mxfp8_fused(const void* a, mxq_fp8_kind kind, const void* w_q, const void* w_scales,
                                mxq_scale_layout scale_layout, int64_t M, int64_t N, int64_t K,
                                const void* bias, mxq_epilogue epi, void* c, void* stream);

/*
 * Bytes of device workspace mxq_gemm_nvfp4 can use for this shape on the current
 * device (0 for an invalid shape).  With it, row-major block scales of both
 * operands are first rewritten into the tiled order (MXQ_SCALES_TILED; scales
 * given tiled are read in place and that part goes unused), and the output
 * tiles that would otherwise run in a partial last round on the compute units
 * are cut along K into ranges computed side by side, whose fp32 partial sums are
 * added by a second kernel before the epilogue.  Its contents are scratch.
 */
size_t mxq_gemm_nvfp4_workspace_size(int64_t M, int64_t N, int64_t K);

/*
 * NVFP4 block-scaled GEMM [P1 NVFP4 paragraph; P2 §3.1].
 *   C[m, n] = epi( s_ga s_gw sum_k val(a_q) val(a_s[m,k/16]) val(w_q) val(w_s[n,k/16])
 *                  (+ bias[n]) ), fp32 accumulation, one RNE to bf16.
 *   a_q, a_scales, a_global : packed E2M1 [M, K/2], E4M3 [M, K/16], device fp32 s_ga.
 *   w_q, w_scales, w_global : packed E2M1 [N, K/2], E4M3 [N, K/16], device fp32 s_gw.
 *   scale_layout            : order of both a_scales and w_scales.
 *   M, N, K, bias, epi, c   : as mxq_gemm_mxfp8.
 *   workspace, ws_bytes     : NULL (scales read in place, no split), or device
 *                             scratch of at least mxq_gemm_nvfp4_workspace_size(M, N, K)
 *                             bytes, 16-byte aligned (else MXQ_ERROR_WORKSPACE /
 *                             MXQ_ERROR_MISALIGNED); calls sharing one must be
 *                             ordered on one stream.
 *   The fp32 additions of a split tile's parts come in a different order than an
 *   unsplit accumulation; results agree within the GEMM tolerance, not bit for bit.
 */
mxq_status mxq_gemm_nvfp4(const void* a_q, const void* a_scales, const float* a_global,
                          const void* w_q, const void* w_scales, const float* w_global,
                          mxq_scale_layout scale_layout,
                          int64_t M, int64_t N, int64_t K, const void* bias, mxq_epilogue epi,
                          void* c, void* workspace, size_t ws_bytes, void* stream);

/* Static text for a status code. */
const char* mxq_status_string(mxq_status s);

/* Detail of the last non-success status returned on this thread ("" if none). */
const char* mxq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MXQ_H_ */
