/* A plain C99 caller of the library's host-side entry points: include/moe.h
 * must compile as C, and the exported names must link and behave as the
 * header states, without a GPU (no call here launches anything). */
#include <stdio.h>
#include <string.h>

#include "moe.h"

static int fails = 0;

static void check(int cond, const char* what) {
  if (!cond) {
    printf("FAIL: %s\n", what);
    ++fails;
  }
}

int main(void) {
  moe_desc d;
  memset(&d, 0, sizeof d);
  d.T = 256;
  d.H = 7168;
  d.E = 48;
  d.n_shared = 0;
  d.I = 640;
  d.act_dtype = MOE_BF16;
  d.w_dtype = MOE_BF16;
  d.block_m = 0;
  d.w_layout = MOE_LAYOUT_FRAG16;
  const size_t ws = moe_workspace_size(&d, 3);
  check(ws > 0, "workspace size of a valid layer");
  check(ws % 256 == 0, "workspace size is a multiple of 256 bytes");

  moe_desc bad = d;
  bad.T = 0;
  check(moe_workspace_size(&bad, 3) == 0, "workspace size of an invalid layer is 0");
  check(moe_workspace_size(&d, 0) == 0, "workspace size for topk 0 is 0");
  check(moe_workspace_size(NULL, 3) == 0, "workspace size of a null descriptor is 0");

  check(moe_forward(NULL, NULL, NULL, NULL, NULL, NULL, 3, NULL, NULL, 0, NULL) ==
            MOE_ERR_INVALID_ARG,
        "moe_forward rejects a null descriptor");
  check(moe_forward(&d, NULL, NULL, NULL, NULL, NULL, 3, NULL, NULL, ws, NULL) ==
            MOE_ERR_INVALID_ARG,
        "moe_forward rejects null buffers");
  check(moe_forward_signaled(&d, NULL, NULL, NULL, NULL, NULL, 3, NULL, NULL, ws, NULL, NULL,
                             NULL) == MOE_ERR_INVALID_ARG,
        "moe_forward_signaled rejects null buffers");
  check(moe_block_signal_count(&d) == (size_t)48 * 4, "completion counter count");
  check(moe_block_signal_count(NULL) == 0, "counter count of a null descriptor is 0");
  check(moe_set_signal_wait_us(-1) == MOE_ERR_INVALID_ARG, "bad wait bound");
  check(moe_set_signal_wait_us(10000) == MOE_OK, "default wait bound");
  check(moe_set_path_thresholds(-1, -1) == MOE_ERR_INVALID_ARG, "bad path thresholds");
  check(moe_set_fp8_mfma(2) == MOE_ERR_INVALID_ARG, "bad fp8 MFMA switch");

  const int codes[] = {MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE,
                       MOE_ERR_HIP};
  for (size_t i = 0; i < sizeof codes / sizeof codes[0]; ++i) {
    const char* s = moe_status_str(codes[i]);
    check(s != NULL && s[0] != '\0', "status string");
  }
  const int n = moe_num_stages();
  check(n > 0, "stage count");
  for (int i = 0; i < n; ++i) check(moe_stage_name(i) != NULL, "stage name");

  printf(fails ? "abi smoke: %d failures\n" : "abi smoke: ok\n", fails);
  return fails ? 1 : 0;
}
