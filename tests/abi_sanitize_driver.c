/*
 * Calls the C ABI's host-side checks (configuration validation, sizes,
 * argument validation of every entry point) with good and bad arguments, for
 * a build of the library's host code under AddressSanitizer and
 * UndefinedBehaviorSanitizer.  Every call here is rejected or answered on the
 * host before anything reaches the GPU, so it runs without one.  Prints
 * "abi sanitize ok" when every status is the expected one.
 */
#include <stdio.h>
#include <string.h>

#include "hga.h"

#define FAKE ((void*)0x1000) /* never dereferenced: the calls fail validation first */
#define EXPECT(call, want)                                                              \
  do {                                                                                  \
    hga_status s_ = (call);                                                             \
    if (s_ != (want)) {                                                                 \
      printf("line %d: %s returned %d (%s), want %d\n", __LINE__, #call, (int)s_,     \
             hga_status_string(s_), (int)(want));                                       \
      return 1;                                                                         \
    }                                                                                   \
  } while (0)

static hga_config base(void) {
  hga_config c;
  memset(&c, 0, sizeof c);
  c.head_dim = 128;
  c.n_q_heads = 32;
  c.n_kv_heads = 4;
  c.chunk_size = 64;
  c.groups_per_chunk = 4;
  c.n_sink_chunks = 1;
  c.n_local_chunks = 4;
  c.topk_chunks = 52;
  c.topk_groups = 104;
  c.rope_theta = 1e6;
  c.hf_wavelength = 64.0;
  c.qkv_dtype = HGA_BF16;
  return c;
}

int main(void) {
  hga_config c = base();
  EXPECT(hga_validate(&c), HGA_OK);
  EXPECT(hga_validate(NULL), HGA_ERR_INVALID_ARGUMENT);
  hga_config b = c; b.head_dim = 96;
  EXPECT(hga_validate(&b), HGA_ERR_UNSUPPORTED);
  b = c; b.n_q_heads = 30;
  EXPECT(hga_validate(&b), HGA_ERR_INVALID_ARGUMENT);
  b = c; b.rope_theta = 0.5;
  EXPECT(hga_validate(&b), HGA_ERR_INVALID_ARGUMENT);
  b = c; b.pool_dtype = 2;
  EXPECT(hga_validate(&b), HGA_ERR_INVALID_ARGUMENT);
  b = c; b.pool_dtype = 1; b.qkv_dtype = HGA_F32;
  EXPECT(hga_validate(&b), HGA_ERR_UNSUPPORTED);
  b = c; b.route_pool = 2;
  EXPECT(hga_validate(&b), HGA_ERR_INVALID_ARGUMENT);
  for (int v = 0; v < 32; ++v) {  /* every switch combination validates and sizes */
    b = c;
    b.rep_position = v & 1;
    b.route_per_head = (v >> 1) & 1;
    b.rope_style = (v >> 2) & 1;
    b.pool_dtype = (v >> 3) & 1;
    b.route_pool = (v >> 4) & 1;
    EXPECT(hga_validate(&b), HGA_OK);
    size_t n = 0;
    EXPECT(hga_workspace_bytes(&b, 8, 65536, 1, &n), HGA_OK);
    if (n == 0) return 2;
    EXPECT(hga_workspace_bytes(&b, 8, 65536, 64, &n), HGA_OK);
  }
  int32_t ms = 0;
  EXPECT(hga_max_selected(&c, 1, &ms), HGA_OK);
  if (ms != 128) return 3;
  EXPECT(hga_max_selected(&c, 65, &ms), HGA_ERR_INVALID_ARGUMENT);
  size_t ws = 0;
  EXPECT(hga_workspace_bytes(&c, 0, 65536, 1, &ws), HGA_ERR_INVALID_ARGUMENT);
  EXPECT(hga_workspace_bytes(&c, 8, 65536, 1, NULL), HGA_ERR_INVALID_ARGUMENT);
  EXPECT(hga_prompt_workspace_bytes(&c, 1, 100, 2, &ws), HGA_ERR_INVALID_ARGUMENT);
  EXPECT(hga_warm_workspace_bytes(&c, 4, 0, &ws), HGA_ERR_INVALID_ARGUMENT);
  EXPECT(hga_workspace_reset(NULL, 16, NULL), HGA_ERR_INVALID_ARGUMENT);
  /* append / summaries */
  EXPECT(hga_build_summaries(&c, 8, FAKE, FAKE, 0, 0, FAKE, FAKE, 64, NULL, NULL, 1, NULL),
         HGA_ERR_INVALID_ARGUMENT);
  EXPECT(hga_build_summaries(&c, 8, FAKE, FAKE, 60, 10, FAKE, FAKE, 64, NULL, NULL, 1, NULL),
         HGA_ERR_OUT_OF_RANGE);
  EXPECT(hga_build_summaries(&c, 8, FAKE, FAKE, 0, 64, FAKE, FAKE, 72, NULL, NULL, 1, NULL),
         HGA_ERR_INVALID_ARGUMENT);
  EXPECT(hga_build_summaries(&c, 8, FAKE, NULL, 0, 128, NULL, NULL, 0, FAKE, FAKE, 1, NULL),
         HGA_ERR_OUT_OF_RANGE);
  EXPECT(hga_build_summaries(&c, 8, FAKE, NULL, 0, 64, NULL, NULL, 0, NULL, NULL, 1, NULL), HGA_OK);
  /* routing */
  EXPECT(hga_route(&c, 8, FAKE, 1, FAKE, FAKE, FAKE, 1024, FAKE, FAKE, 127, NULL, FAKE, 1u << 30,
                   NULL), HGA_ERR_OUT_OF_RANGE);
  EXPECT(hga_route(&c, 8, FAKE, 1, FAKE, FAKE, FAKE, 1024, FAKE, FAKE, 128, NULL, FAKE, 64, NULL),
         HGA_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(hga_route(&c, 8, FAKE, 0, FAKE, FAKE, FAKE, 1024, FAKE, FAKE, 128, NULL, FAKE, 1u << 30,
                   NULL), HGA_ERR_INVALID_ARGUMENT);
  EXPECT(hga_route(&c, 8, FAKE, 1, FAKE, FAKE, FAKE, 1 << 20, FAKE, FAKE, 128, NULL, FAKE,
                   (size_t)1 << 40, NULL), HGA_ERR_UNSUPPORTED);
  /* gather */
  EXPECT(hga_gather(&c, 8, FAKE, FAKE, 65536, 0, FAKE, FAKE, 128, NULL, HGA_PART_ROUTED, FAKE,
                    FAKE, NULL), HGA_ERR_INVALID_ARGUMENT);
  EXPECT(hga_gather(&c, 8, FAKE, FAKE, 65530, 0, FAKE, FAKE, 128, NULL, HGA_PART_ALL, FAKE, FAKE,
                    NULL), HGA_ERR_INVALID_ARGUMENT);
  /* attention */
  EXPECT(hga_attend(&c, 8, FAKE, 1, FAKE, FAKE, FAKE, 5, 65536, FAKE, FAKE, 128, 0, FAKE, NULL,
                    FAKE, 1u << 30, NULL), HGA_ERR_INVALID_ARGUMENT);
  EXPECT(hga_attend(&c, 8, FAKE, 1, FAKE, FAKE, FAKE, 0, 65536, FAKE, FAKE, 300, 0, FAKE, NULL,
                    FAKE, 1u << 30, NULL), HGA_ERR_UNSUPPORTED);
  EXPECT(hga_attend(&c, 8, FAKE, 1, FAKE, FAKE, FAKE, 0, 65536, FAKE, FAKE, 128, 0, FAKE, NULL,
                    FAKE, 64, NULL), HGA_ERR_WORKSPACE_TOO_SMALL);
  b = c; b.head_dim = 64;
  EXPECT(hga_attend(&b, 8, FAKE, 32, FAKE, FAKE, FAKE, 0, 65536, FAKE, FAKE, 128, 0, FAKE, NULL,
                    FAKE, 1u << 30, NULL), HGA_ERR_UNSUPPORTED);
  /* fused steps */
  EXPECT(hga_decode_step(&c, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 65536, FAKE, FAKE, FAKE, 1024,
                         FAKE, FAKE, 100, FAKE, NULL, FAKE, 1u << 30, NULL), HGA_ERR_OUT_OF_RANGE);
  EXPECT(hga_prefill_step(&c, 8, FAKE, 65, FAKE, FAKE, FAKE, FAKE, FAKE, 65536, FAKE, FAKE, FAKE,
                          1024, FAKE, FAKE, 128, FAKE, NULL, FAKE, 1u << 30, NULL),
         HGA_ERR_INVALID_ARGUMENT);
  b = c; b.pool_dtype = 1; b.qkv_dtype = HGA_F32;  /* the FP8 pool takes bf16 inputs */
  EXPECT(hga_prefill_step(&b, 8, FAKE, 16, FAKE, FAKE, FAKE, FAKE, FAKE, 65536, FAKE, FAKE, FAKE,
                          1024, FAKE, FAKE, 128, FAKE, NULL, FAKE, 1u << 30, NULL),
         HGA_ERR_UNSUPPORTED);
  /* whole-prompt prefill */
  EXPECT(hga_prefill_prompt(&c, 1, 100, FAKE, FAKE, FAKE, FAKE, FAKE, 128, FAKE, FAKE, 2, FAKE,
                            FAKE, 128, FAKE, NULL, HGA_PROMPT_ALL, FAKE, 1u << 30, NULL),
         HGA_ERR_INVALID_ARGUMENT);
  EXPECT(hga_prefill_prompt(&c, 1, 256, FAKE, FAKE, FAKE, FAKE, FAKE, 128, FAKE, FAKE, 4, FAKE,
                            FAKE, 128, FAKE, NULL, HGA_PROMPT_ALL, FAKE, 1u << 30, NULL),
         HGA_ERR_OUT_OF_RANGE);
  EXPECT(hga_prefill_prompt(&c, 1, 256, FAKE, FAKE, FAKE, FAKE, FAKE, 256, FAKE, FAKE, 4, FAKE,
                            FAKE, 128, FAKE, NULL, 8, FAKE, 1u << 30, NULL),
         HGA_ERR_INVALID_ARGUMENT);
  /* host tier: two streams need two distinct events */
  EXPECT(hga_attend_tiered(&c, 4, FAKE, 1, FAKE, FAKE, FAKE, 65536, FAKE, FAKE, 65536, FAKE, FAKE,
                           128, FAKE, FAKE, FAKE, NULL, FAKE, (size_t)1 << 30, NULL, FAKE, FAKE,
                           FAKE), HGA_ERR_INVALID_ARGUMENT);
  EXPECT(hga_attend_tiered(&c, 4, FAKE, 1, FAKE, FAKE, FAKE, 65536, NULL, FAKE, 65536, FAKE, FAKE,
                           128, FAKE, FAKE, FAKE, NULL, FAKE, (size_t)1 << 30, NULL, NULL, NULL,
                           NULL), HGA_ERR_INVALID_ARGUMENT);
  /* warm tier */
  EXPECT(hga_warm_gather(&c, 4, FAKE, FAKE, 65536, FAKE, FAKE, 128, FAKE, FAKE, FAKE, FAKE, FAKE,
                         50, 1, FAKE, FAKE, NULL, FAKE, (size_t)1 << 30, NULL),
         HGA_ERR_OUT_OF_RANGE);
  EXPECT(hga_warm_gather(&c, 4, FAKE, FAKE, 65536, FAKE, FAKE, 128, FAKE, FAKE, FAKE, FAKE, FAKE,
                         208, 0, FAKE, FAKE, NULL, FAKE, (size_t)1 << 30, NULL),
         HGA_ERR_INVALID_ARGUMENT);
  /* merge */
  EXPECT(hga_merge_partials(&c, 8, 1, NULL, FAKE, FAKE, FAKE, FAKE, NULL, NULL),
         HGA_ERR_INVALID_ARGUMENT);
  for (int s = 0; s <= 6; ++s) (void)strlen(hga_status_string((hga_status)s));
  if (hga_version() < 1) return 4;
  printf("abi sanitize ok\n");
  return 0;
}
