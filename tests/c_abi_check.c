/* A plain C99 client of include/mxq.h: every call below is rejected by the
 * library's host-side validation (or is a size query), so no GPU is needed.
 * Prints one result per line for tests/test_c_abi.py. */
#include <stdint.h>
#include <stdio.h>

#include "mxq.h"

int main(void) {
  void* fake = (void*)(uintptr_t)0x10000; /* aligned, never dereferenced */
  const float* gs = (const float*)(uintptr_t)0x20000;
  printf("%d\n", (int)mxq_quantize_mxfp8(NULL, 4, 64, MXQ_FP8_E4M3, fake, fake, MXQ_SCALES_ROW_MAJOR, NULL));
  printf("%d\n", (int)mxq_quantize_mxfp8(fake, 4, 48, MXQ_FP8_E4M3, fake, fake, MXQ_SCALES_ROW_MAJOR, NULL));
  printf("%d\n", (int)mxq_quantize_mxfp8(fake, 4, 128, MXQ_FP8_E5M2, fake, fake, MXQ_SCALES_TILED, NULL));
  printf("%d\n", (int)mxq_quantize_nvfp4(fake, 4, 24, NULL, fake, fake, MXQ_SCALES_ROW_MAJOR, (float*)fake, fake,
                                         64, NULL));
  printf("%d\n", (int)mxq_gemm_mxfp8(fake, fake, MXQ_FP8_E4M3, fake, fake, MXQ_FP8_E5M2, MXQ_SCALES_TILED, 128, 256,
                                     192, NULL, MXQ_EPI_NONE, fake, NULL));
  printf("%d\n", (int)mxq_gemm_nvfp4(fake, fake, gs, fake, fake, gs, MXQ_SCALES_ROW_MAJOR, 128, 256, 256, NULL,
                                     MXQ_EPI_BIAS, fake, NULL, 0, NULL));
  printf("%d\n", (int)mxq_gemm_mxfp8_fused(fake, MXQ_FP8_E5M2, fake, fake, MXQ_SCALES_TILED, 128, 256, 192, NULL,
                                           MXQ_EPI_NONE, fake, NULL));
  printf("%zu\n", mxq_gemm_nvfp4_workspace_size(128, 384, 128));
  printf("%zu\n", mxq_quantize_nvfp4_workspace_size(128, 24));
  printf("%s\n", mxq_status_string(MXQ_ERROR_MISALIGNED));
  printf("%d\n", mxq_last_error()[0] != '\0');
  return 0;
}
