/* A plain C client of libcsa: includes csa.h, links libcsa.so, and calls the
 * host-side parts of the boundary -- version, status strings, row sizes,
 * workspace sizes, and argument checks that every entry point makes before
 * anything is enqueued.  No GPU is needed (no call here reaches a launch).
 * Prints "c abi ok" and returns 0 when every check holds. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "csa.h"

static int failures = 0;

static void expect(int cond, const char* what) {
  if (!cond) {
    printf("FAILED: %s (last error: %s)\n", what, csa_last_error());
    ++failures;
  }
}

int main(void) {
  void* p = (void*)(uintptr_t)0x1000;          /* non-null host address: checks run before use */
  expect(csa_abi_version() == CSA_ABI_VERSION, "version");
  expect(strcmp(csa_status_string(CSA_ERR_WORKSPACE), "CSA_ERR_WORKSPACE") == 0, "status string");
  expect(csa_row_bytes(CSA_SPLIT, 512, 64) == 576, "split row bytes");
  expect(csa_row_bytes(CSA_MXFP4, 128, 0) == 68, "mxfp4 row bytes");
  expect(csa_score_topk_workspace_bytes(16) == 16u * 16640u, "fused top-k workspace bytes");
  expect(csa_topk_workspace_bytes(16, 16384, 512) == 0, "no top-k workspace for short rows");
  expect(csa_topk_workspace_bytes(16, 262144, 512) > 0, "a top-k workspace for long rows");

  expect(csa_compress(p, CSA_F32, p, 1, 8, 512, 0, 1, p, p, p, 1, NULL, 1e-6f, 64, 1e4f, p, CSA_SPLIT, NULL) ==
             CSA_ERR_INVALID_ARG, "compress: m = 0");
  expect(strstr(csa_last_error(), "csa_compress") != NULL, "compress: error names the call");
  expect(indexer_score(p, (const float*)p, -1, 64, 128, p, CSA_FP8, (const int64_t*)p, (const int64_t*)p, 4,
                       (float*)p, 1024, NULL) == CSA_ERR_INVALID_ARG, "indexer: nq < 0");
  expect(topk_select((const float*)p, 16384, 16, NULL, 0, (int32_t*)p, NULL, NULL, 0, NULL) ==
             CSA_ERR_INVALID_ARG, "top-k: k = 0");
  expect(topk_select((const float*)p, 262144, 16, NULL, 512, (int32_t*)p, NULL, NULL, 0, NULL) == CSA_ERR_WORKSPACE,
         "top-k: long rows without a workspace");
  expect(hybrid_attn_decode(NULL, CSA_BF16, 16, 64, 512, (const int64_t*)p, NULL, 1e-6f, 64, 1e4f, p, CSA_SPLIT,
                            (const int64_t*)p, 4, (const int32_t*)p, 512, p, CSA_BF16, 128, (const int32_t*)p,
                            (const float*)p, 0.044f, p, CSA_BF16, CSA_VARIANT_AUTO, NULL) == CSA_ERR_INVALID_ARG,
         "attention: null q");
  expect(csa_compress_score_topk(NULL, 0, p, (const float*)p, 16, 64, 128, p, CSA_FP8, (const int64_t*)p,
                                 (const int64_t*)p, 4, (float*)p, 16384, 512, (int32_t*)p, NULL, 0, NULL) ==
             CSA_ERR_WORKSPACE, "fused top-k: no workspace");
  expect(csa_select_and_pad(p, 0, 8, 576, (const int64_t*)p, p, NULL) == CSA_ERR_INVALID_ARG,
         "select-and-pad: no shards");
  if (failures == 0) printf("c abi ok\n");
  return failures == 0 ? 0 : 1;
}
