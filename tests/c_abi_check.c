/* The C ABI from C: include/spot.h compiled as strict C11 and linked against
 * the built library.  Checks the descriptor layout the header gives a C
 * compiler, and calls the entry points that run on the host only (version,
 * status strings, workspace sizes, argument validation), so it needs no GPU.
 * Prints one "key value" line per result for the test that runs it. */
#include <stddef.h>
#include <stdio.h>
#include <string.h>

#include "spot.h"

_Static_assert(sizeof(spot_desc) == 80, "descriptor size");
_Static_assert(offsetof(spot_desc, q_len) == 24, "q_len offset");
_Static_assert(offsetof(spot_desc, block) == 40, "block offset");
_Static_assert(offsetof(spot_desc, top_p) == 60, "top_p offset");
_Static_assert(offsetof(spot_desc, d_idx) == 76, "d_idx offset");

static spot_desc decode_desc(void) {
  spot_desc d;
  memset(&d, 0, sizeof d);
  d.version = SPOT_ABI_VERSION;
  d.dtype = SPOT_BF16;
  d.batch = 16;
  d.hq = 32;
  d.hkv = 8;
  d.d = 128;
  d.q_len = 1;
  d.kv_len = 131072;
  d.block = 16;
  d.n_sink = 1;
  d.n_recent = 1;
  d.top_p = 0.9f;
  d.score_kind = SPOT_SCORE_RELU_INDEXER;
  d.h_idx = 4;
  d.d_idx = 64;
  return d;
}

int main(void) {
  printf("version %d\n", spot_version());
  printf("status_invalid %s\n", spot_status_string(SPOT_ERR_INVALID));

  size_t bytes = 0;
  int st = spot_workspace_size(NULL, SPOT_OP_DECODE, &bytes);
  printf("null_desc_status %d\n", st);
  printf("null_desc_error_set %d\n", spot_last_error()[0] != '\0');

  spot_desc d = decode_desc();
  st = spot_workspace_size(&d, SPOT_OP_DECODE, &bytes);
  printf("decode_workspace_status %d\n", st);
  printf("decode_workspace_bytes %zu\n", bytes);
  st = spot_workspace_size(&d, SPOT_OP_SELECT_TOPP, &bytes);
  printf("select_workspace_bytes %zu\n", bytes);

  /* required pointers missing: rejected on the host before any launch */
  st = spot_select_topp(&d, NULL, NULL, NULL, NULL, 0, NULL);
  printf("select_null_status %d\n", st);

  /* a descriptor from another ABI version */
  d.version = SPOT_ABI_VERSION + 1;
  st = spot_workspace_size(&d, SPOT_OP_DECODE, &bytes);
  printf("bad_version_status %d\n", st);

  /* a head dimension no kernel is built for */
  d = decode_desc();
  d.d = 96;
  st = spot_workspace_size(&d, SPOT_OP_DECODE, &bytes);
  printf("bad_head_dim_status %d\n", st);
  return 0;
}
