/* Calls the host-only entry points of libfp4kv.so from plain C: size queries and argument
 * validation need no GPU.  Prints one line per check and exits non-zero on a mismatch. */
#include <stdio.h>
#include <string.h>
#include "fp4kv.h"

static int fails = 0;
static void check(int ok, const char *what) {
  printf("%s %s\n", ok ? "ok  " : "FAIL", what);
  if (!ok) fails++;
}

int main(void) {
  fp4kv_cache c;
  memset(&c, 0, sizeof c);
  c.format = FP4KV_NVFP4;
  c.attn = FP4KV_GQA;
  c.num_pages = 8;
  c.page_size = 64;
  c.num_kv_heads = 2;
  c.head_dim = 128;
  c.rope_dim = 0;
  c.max_seqs = 4;
  size_t b[6];
  check(fp4kv_cache_layout(&c, b) == FP4KV_OK, "layout of a valid GQA cache");
  check(b[0] == (size_t)8 * 2 * 64 * 64 && b[1] == (size_t)8 * 2 * 64 * 8, "key code and scale bytes");
  check(b[2] == (size_t)8 * 2 * 128 * 32 && b[3] == (size_t)8 * 2 * 128 * 4, "value code and scale bytes");
  check(fp4_decode_workspace_bytes(&c, 3, 8, 1000) > 0, "workspace bytes");
  c.page_size = 24;
  check(fp4kv_cache_layout(&c, b) == FP4KV_ERR_INVALID_ARG, "page size 24 rejected");
  c.page_size = 64;
  /* buffers left NULL: rejected on the host before anything is launched */
  check(fp4_decode_attention(&c, NULL, FP4KV_F32, 1, 4, NULL, 4, NULL, 0.1f, NULL, NULL, 0, NULL, NULL) ==
            FP4KV_ERR_INVALID_ARG, "decode with NULL buffers rejected");
  check(strcmp(fp4kv_status_string(FP4KV_ERR_WORKSPACE), "workspace too small") == 0, "status string");
  return fails ? 1 : 0;
}
