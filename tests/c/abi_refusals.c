/* The C ABI used from plain C (no C++ types in the header): the host-side refusals,
 * which need no GPU. Exit status 0 when every check holds. */
#include <stdio.h>
#include <string.h>

#include "gdn_block.h"

static int fails = 0;
#define CHECK(cond, what)                          \
  do {                                             \
    if (!(cond)) {                                 \
      fprintf(stderr, "FAILED: %s\n", what);       \
      ++fails;                                     \
    }                                              \
  } while (0)

int main(void) {
  gdn_block_config cfg;
  memset(&cfg, 0, sizeof(cfg));
  cfg.hidden = 100; /* not a multiple of 256 */
  cfg.num_k_heads = 2;
  cfg.head_k_dim = 32;
  cfg.num_v_heads = 3; /* not a multiple of num_k_heads */
  cfg.head_v_dim = 32;
  cfg.conv_width = 5;
  cfg.num_state_slots = 4;
  cfg.max_rows = 40;
  cfg.qkvz_format = GDN_FMT_MXFP6;
  cfg.ssm_state_dtype = GDN_STATE_F32;
  cfg.norm_eps = cfg.gated_norm_eps = cfg.l2norm_eps = 1e-6f;
  gdn_block_t blk = (gdn_block_t)1;
  const int rc = gdn_block_create(&cfg, &blk);
  CHECK(rc == GDN_E_UNSUPPORTED, "a bad config is refused");
  CHECK(blk == NULL, "the handle is NULL after a refusal");
  const char* msg = gdn_block_last_error(NULL);
  CHECK(msg != NULL && strstr(msg, "hidden") && strstr(msg, "num_v_heads") && strstr(msg, "conv_width") &&
            strstr(msg, "max_rows"),
        "every reason is listed");
  CHECK(gdn_block_create(NULL, &blk) == GDN_E_INVALID_ARG, "a NULL config is refused");
  CHECK(gdn_mxfp4_quantize((const void*)0x100000, 1, 48, (void*)0x100000, (void*)0x100000, GDN_MXSCALE_ROUNDED_MAX,
                           NULL) == GDN_E_INVALID_ARG,
        "cols must be a multiple of 32");
  CHECK(gdn_mxfp4_quantize((const void*)0x100000, 1, 32, (void*)0x100000, (void*)0x100000, 7, NULL) ==
            GDN_E_INVALID_ARG, "an unknown scale rule is refused");
  CHECK(gdn_block_set_spin_limit(NULL, 1) == GDN_E_INVALID_ARG, "a spin limit needs a handle");
  CHECK(gdn_mxfp6_round_weights(NULL, 1, 32, (void*)0x100000, (void*)0x100000, NULL) == GDN_E_INVALID_ARG,
        "NULL weights are refused");
  CHECK(gdn_block_decode(NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, NULL, NULL) == GDN_E_INVALID_ARG,
        "a NULL handle is refused");
  CHECK(gdn_block_verify(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, 2, NULL, NULL) == GDN_E_INVALID_ARG,
        "verify with a NULL handle is refused");
  CHECK(gdn_block_packed_weight_bytes(NULL) == 0, "no packed size without a handle");
  gdn_block_destroy(NULL);
  printf("%d failed\n", fails);
  return fails ? 1 : 0;
}
