/* A plain C99 program against include/kata.h: checks that the header is C, that the
 * library links from C, and that the host-side entry points (version, status strings,
 * workspace sizes, argument validation) answer without a GPU. */
#include <stdio.h>
#include <string.h>

#include "kata.h"

static int fails = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++fails;                                                        \
    }                                                                 \
  } while (0)

int main(void) {
  kata_forward_desc d;
  size_t bytes = 0;
  memset(&d, 0, sizeof d);
  d.B = 1; d.H = 16; d.T = 131072; d.d = 64; d.dv = 64; d.p = 16; d.chunk = 64;
  d.in_dtype = KATA_BF16; d.out_dtype = KATA_BF16; d.scan = KATA_SCAN_ASSOC; d.scan_leaf = 0;

  CHECK(kata_abi_version() == KATA_ABI_VERSION);
  CHECK(strlen(kata_status_string(KATA_ERR_UNSUPPORTED)) > 0);
  CHECK(kata_forward_workspace_bytes(&d, &bytes) == KATA_OK && bytes > 0);
  CHECK(kata_forward_decay_workspace_bytes(&d, &bytes) == KATA_OK && bytes > 0);
  CHECK(kata_backward_workspace_bytes(&d, &bytes) == KATA_OK && bytes > 0);
  CHECK(kata_forward_factors_workspace_bytes(&d, 2, KATA_FACTORS_CONCAT, &bytes) == KATA_OK && bytes > 0);
  CHECK(kata_forward_factors_workspace_bytes(&d, 2, KATA_FACTORS_SUM, &bytes) == KATA_OK && bytes > 0);
  CHECK(kata_forward_delta_chunked_workspace_bytes(&d, &bytes) == KATA_OK && bytes > 0);
  {
    int64_t segs = 0, seg_chunks = 0;
    CHECK(kata_forward_delta_chunked_plan(&d, &segs, &seg_chunks) == KATA_OK && segs >= 1 && seg_chunks >= 1);
    CHECK(kata_forward_delta_chunked_plan(&d, NULL, NULL) == KATA_OK);
  }
  CHECK(kata_forward_workspace_bytes(NULL, &bytes) == KATA_ERR_NULL);
  CHECK(kata_forward_workspace_bytes(&d, NULL) == KATA_ERR_NULL);
  d.p = 8;
  CHECK(kata_forward_workspace_bytes(&d, &bytes) == KATA_ERR_UNSUPPORTED);
  d.p = 16; d.T = -1;
  CHECK(kata_forward_workspace_bytes(&d, &bytes) == KATA_ERR_SHAPE);
  /* empty work is a no-op before any device call */
  d.T = 100; d.B = 0;
  CHECK(kata_forward(&d, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == KATA_OK);
  CHECK(kata_decode_step(0, 16, 64, 64, 16, KATA_BF16, KATA_F32, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                         NULL) == KATA_OK);
  CHECK(kata_decode_step_delta(0, 16, 64, 64, 16, KATA_BF16, KATA_F32, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                               NULL) == KATA_OK);
  /* the packed symmetric state: no-ops on empty input, argument errors before any device call */
  CHECK(KATA_PACKED_ROWS == 136);
  CHECK(kata_state_pack(0, 64, NULL, NULL, NULL, NULL, NULL) == KATA_OK);
  CHECK(kata_state_unpack(4, 32, NULL, NULL, NULL, NULL, NULL) == KATA_ERR_UNSUPPORTED);
  CHECK(kata_decode_step_packed(0, 16, 64, 64, 16, KATA_BF16, KATA_F32, NULL, NULL, NULL, NULL, NULL, NULL,
                                NULL, NULL) == KATA_OK);
  CHECK(kata_decode_step_decay_packed(4, 16, 64, 64, 8, KATA_BF16, KATA_F32, NULL, NULL, NULL, NULL, NULL, NULL,
                                      NULL, NULL, NULL) == KATA_ERR_UNSUPPORTED);
  CHECK(kata_decode_step_delta_packed(-1, 16, 64, 64, 16, KATA_BF16, KATA_F32, NULL, NULL, NULL, NULL, NULL,
                                      NULL, NULL, NULL) == KATA_ERR_SHAPE);
  CHECK(kata_decode_step_factors_packed(4, 16, 64, 64, 16, 4, KATA_FACTORS_SUM, KATA_BF16, KATA_F32, NULL, NULL,
                                        NULL, NULL, NULL, NULL, NULL, NULL) == KATA_ERR_UNSUPPORTED);
  if (fails == 0) printf("kata.h from C: ok\n");
  return fails == 0 ? 0 : 1;
}
