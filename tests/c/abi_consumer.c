/* A plain C99 consumer of the library's C ABI: includes include/cp_attn.h,
 * links libcpattn.so and checks, without a GPU, what the header promises for
 * sizes and host-side validation. Every attention call below fails validation
 * before anything is enqueued, so the fake device addresses are never touched.
 * Exit status 0 when every check holds; the first failing check is printed. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "cp_attn.h"

#define FAKE ((void*)(uintptr_t)0x10000)
#define FAKE_AT(off) ((void*)(uintptr_t)(0x10000 + (off)))

static int failures = 0;

#define CHECK(cond)                                                     \
  do {                                                                  \
    if (!(cond)) {                                                      \
      fprintf(stderr, "check failed at line %d: %s (last error: %s)\n", \
              __LINE__, #cond, cp_last_error());                        \
      ++failures;                                                       \
    }                                                                   \
  } while (0)

int main(void) {
  CHECK(cp_abi_version() == CP_ATTN_ABI_VERSION);

  /* sizes */
  CHECK(cp_ring_attention_workspace_size(1, 24, 2304, 128, 0) == 0);
  CHECK(cp_ring_attention_workspace_size(1, 24, 2304, 128, CP_RING_SEPARATE_MERGE) >=
        (size_t)2304 * 24 * 128 * 4 + (size_t)24 * 2304 * 4);
  CHECK(cp_attn_packed_v_bytes(1, 24, 128, 2304) == (size_t)24 * 36 * 64 * 128 * 2);
  CHECK(cp_attn_packed_v_bytes(1, 24, 80, 2304) == 0);
  CHECK(cp_attn_bwd_workspace_size(1, 2, 8, 128) > 0);
  CHECK(cp_attn_fwd_waves(1, 24, 128, 2304, 0) == 8);
  CHECK(cp_attn_fwd_waves(1, 24, 64, 2304, 0) == 4);
  CHECK(cp_attn_fwd_waves(1, 24, 128, 2304, CP_FWD_FOUR_WAVES) == 4);

  /* block attention: unsupported head dim, bad scale, unknown flag, packed f32 */
  const int64_t* contiguous = NULL;
  CHECK(cp_attn_block_fwd(FAKE, contiguous, FAKE, FAKE, contiguous, CP_BF16, 1, 2, 96, 8, 8, 0.1f, 0,
                          (float*)FAKE, contiguous, (float*)FAKE, NULL) == CP_ERR_UNSUPPORTED);
  CHECK(strstr(cp_last_error(), "head dim") != NULL);
  CHECK(cp_attn_block_fwd(FAKE, contiguous, FAKE, FAKE, contiguous, CP_BF16, 1, 2, 128, 8, 8, -1.0f, 0,
                          (float*)FAKE, contiguous, (float*)FAKE, NULL) == CP_ERR_INVALID_ARG);
  CHECK(cp_attn_block_fwd(FAKE, contiguous, FAKE, FAKE, contiguous, CP_BF16, 1, 2, 128, 8, 8, 0.1f, 0x80u,
                          (float*)FAKE, contiguous, (float*)FAKE, NULL) == CP_ERR_INVALID_ARG);
  CHECK(cp_attn_block_fwd(FAKE, contiguous, FAKE, FAKE, contiguous, CP_F32, 1, 2, 128, 8, 8, 0.1f,
                          CP_BLOCK_PACKED_V, (float*)FAKE, contiguous, (float*)FAKE, NULL) == CP_ERR_UNSUPPORTED);
  /* nothing to do is not an error */
  CHECK(cp_attn_block_fwd(NULL, contiguous, NULL, NULL, contiguous, CP_BF16, 0, 2, 128, 8, 8, 0.1f, 0, NULL,
                          contiguous, NULL, NULL) == CP_OK);

  /* ring: uneven blocks need CP_RING_ANYTHING; the message says so */
  {
    const void* kb[2] = {FAKE, FAKE};
    const void* vb[2] = {FAKE, FAKE};
    const int lens[2] = {8, 7};
    CHECK(cp_ring_attention(FAKE, contiguous, kb, vb, contiguous, lens, 2, CP_BF16, 1, 2, 128, 8, 0.1f, 0,
                            (float*)FAKE, contiguous, (float*)FAKE, NULL, 0, NULL) == CP_ERR_INVALID_ARG);
    CHECK(strstr(cp_last_error(), "CP_RING_ANYTHING") != NULL);
    CHECK(cp_ring_attention(FAKE, contiguous, kb, vb, contiguous, lens, 2, CP_BF16, 1, 2, 128, 8, 0.1f,
                            CP_RING_ANYTHING | CP_RING_SEPARATE_MERGE, (float*)FAKE, contiguous, (float*)FAKE,
                            NULL, 0, NULL) == CP_ERR_WORKSPACE);
  }

  /* merge, regroup, packs: host-side rejections */
  CHECK(cp_lse_merge((float*)FAKE, (float*)FAKE, (float*)FAKE, (float*)FAKE_AT(8192), contiguous, contiguous, 1,
                     2, 8, 128, NULL) == CP_ERR_INVALID_ARG); /* accumulator == block */
  CHECK(cp_ulysses_regroup(FAKE, FAKE_AT(1 << 30), 2, 1, 16, 24, 128, 5, CP_REGROUP_SEQ_TO_HEAD, NULL) ==
        CP_ERR_INVALID_ARG);
  CHECK(strstr(cp_last_error(), "divisible") != NULL);
  {
    const int heads[3] = {3, 3, 2};
    CHECK(cp_ulysses_pack_heads(FAKE, FAKE_AT(1 << 30), 3, 1, 16, 128, 3, heads, CP_REGROUP_SEQ_TO_HEAD, NULL) ==
          CP_ERR_UNSUPPORTED); /* elem_bytes 3 */
  }
  CHECK(cp_attn_pack_v(FAKE, contiguous, 1, 2, 128, 8, FAKE_AT(1 << 30), 16, NULL) == CP_ERR_INVALID_ARG);
  CHECK(cp_ulysses_regroup_pack_v(FAKE, 1, 16, 24, 128, 5, FAKE_AT(1 << 30), 1 << 20, NULL) == CP_ERR_INVALID_ARG);

  /* backward: float32 inputs are not supported */
  CHECK(cp_attn_bwd_prep(FAKE, contiguous, FAKE, contiguous, CP_F32, 1, 2, 8, 128, FAKE, 1 << 20, NULL) ==
        CP_ERR_UNSUPPORTED);

  if (failures == 0) printf("C ABI consumer: all checks passed\n");
  return failures == 0 ? 0 : 1;
}
