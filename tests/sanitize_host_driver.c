/* sanitize_host_driver.c -- TEST INFRASTRUCTURE: drives the host-side
 * argument validation of libfp8blk (every check that runs before a launch)
 * in a build whose host code carries AddressSanitizer and
 * UndefinedBehaviorSanitizer.  Nothing here launches a kernel or needs a
 * GPU: every call either only computes (split sizes, validation) or is
 * rejected before any HIP call.  Run by tests/test_sanitized_host.py. */
#include <stdio.h>
#include <stdint.h>
#include "fp8blk.h"
int main(void) {
  int bad = 0;
  if (fp8b_abi_version() != 4) bad++;
  for (int s = -1; s < 8; ++s) if (!fp8b_status_string(s)) bad++;
  int64_t shapes[][3] = {{64,24576,4096},{1,3000,4099},{37,2304,301},{0,0,0},{-1,5,5},{65,4096,512},{64,1 << 20,128}};
  for (int i = 0; i < 7; ++i) (void)fp8_gemm_dgrad_split_bytes(shapes[i][0], shapes[i][1], shapes[i][2]);
  void* P = (void*)0x100000;
  for (int op = -1; op < 7; ++op)
    for (int64_t n = -1; n < 300; n += 97)
      (void)fp8b_validate_gemm(op, P, 256, P, 2, P, 256, P, 2, P, 1, 512, 0, n, 300, 200);
  if (fp8_quantize_act_1x128(NULL, 1, 4, 256, 256, P, 256, P, 2, NULL) != 1) bad++;
  if (fp8_gemm_fprop(P, 128, P, 1, P, 128, P, 1, P, 1, 8, 8, 8, 100, NULL) == 0) bad++;
  if (fp8_gemm_dgrad_split_noalloc(P, 4096, P, 32, P, 4096, P, 4, NULL, 0, 512, 64, 4096, 512, NULL) != 1) bad++;
  if (fp8_dequant_gemm_wgrad(P, 128, P, 256, P, 2, 0, 16, 128, 256, P, 1, 256, 0, P, 8, NULL) != 2) bad++;
  if (fp8b_mfma_peak(5, 1, 1, 0, P, NULL, NULL) != 1) bad++;
  if (fp8b_bf16_round(P, -1, P, NULL) != 2) bad++;
  if (fp8b_bf16_round(NULL, 8, P, NULL) != 1) bad++;
  if (fp8b_bf16_round(NULL, 0, NULL, NULL) != 0) bad++;
  for (int64_t d = -1; d < 40; d += 13)
    for (int part = -1; part < 3; ++part) (void)fp8_decode_pack_bytes(d, 300, part);
  if (fp8_pack_decode_weight(P, 384, P, 13, 17, 300, P, P, NULL) != 3) bad++;
  if (fp8_pack_decode_weight(P, 384, NULL, 0, 17, 300, NULL, NULL, NULL) != 1) bad++;
  if (fp8_gemm_fprop_decode(P, 384, P, 3, P, P, 3, P, 1, 24, 65, 17, 300, NULL) != 4) bad++;
  if (fp8_mx_gemm_fprop_decode(P, 384, P, 13, P, P, P, 1, 24, 64, 17, 300, NULL) != 3) bad++;
  int32_t offs[3] = {0, 1, 2};
  (void)offs;
  printf("host validation sanitizer run: %s\n", bad ? "FAILED" : "ok");
  return bad;
}
