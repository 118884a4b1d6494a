/* Plain C use of the ABI on a host without a GPU: compiles against
 * include/cpdec.h with a C compiler, links libcpdec.so, and exercises the
 * argument checks (every call below fails validation before any HIP call). */
#include <stdio.h>
#include <string.h>

#include "cpdec.h"

#define EXPECT(cond)                                      \
  do {                                                    \
    if (!(cond)) {                                        \
      fprintf(stderr, "failed: %s (line %d)\n", #cond, __LINE__); \
      return 1;                                           \
    }                                                     \
  } while (0)

int main(void) {
  cpdec_attn_desc d;
  memset(&d, 0, sizeof d);
  d.batch = 2; d.num_q_heads = 8; d.num_kv_heads = 2; d.head_dim = 128; d.num_shards = 4;
  d.kv_capacity = 1024; d.kv_stride_token = 128; d.kv_stride_head = 1024 * 128;
  d.kv_stride_batch = 2 * 1024 * 128; d.qkv_dtype = CPDEC_BF16; d.opart_dtype = CPDEC_F32;
  d.chunk_tokens = 0;
  int32_t chunk = 0, nchunks = 0, waves = 0;
  EXPECT(cpdec_attn_plan(&d, &chunk, &nchunks, &waves) == CPDEC_OK);
  EXPECT(chunk > 0 && nchunks >= 1 && chunk * nchunks >= 1024 && waves >= 1);
  EXPECT(cpdec_attn_plan(NULL, &chunk, NULL, NULL) == CPDEC_ERR_INVALID_ARG);
  size_t ws = cpdec_attn_workspace_bytes(&d);
  EXPECT((nchunks > 1) == (ws > 0));
  d.head_dim = 96;
  EXPECT(cpdec_attn_plan(&d, NULL, NULL, NULL) == CPDEC_ERR_UNSUPPORTED);
  EXPECT(cpdec_attn_partial(&d, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) ==
         CPDEC_ERR_UNSUPPORTED);
  d.head_dim = 128;
  EXPECT(cpdec_attn_partial(&d, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) ==
         CPDEC_ERR_INVALID_ARG);
  EXPECT(cpdec_lse_merge(NULL, NULL, 4, 10, 128, CPDEC_BF16, CPDEC_BF16, NULL, NULL, NULL) ==
         CPDEC_ERR_INVALID_ARG);
  EXPECT(cpdec_workspace_clear(NULL, 0, NULL) == CPDEC_OK);
  EXPECT(strcmp(cpdec_status_string(CPDEC_ERR_WORKSPACE), "CPDEC_ERR_WORKSPACE") == 0);
  EXPECT(strstr(cpdec_version(), "gfx950") != NULL);
  printf("abi_smoke ok: chunk=%d chunks=%d waves=%d workspace=%zu\n", chunk, nchunks, waves, ws);
  return 0;
}
