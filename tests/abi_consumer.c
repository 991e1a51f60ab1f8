/* A plain C99 consumer of include/mtp_draft.h, built and run by
 * tests/test_abi_host.py on a host without a GPU. It shows that the header and
 * the shared library serve a C caller with no C++ or torch in between, and
 * checks the host-only parts of the ABI: the version, the status texts, the
 * workspace queries against the layout the header documents, the kernel-form
 * query, and that argument errors are reported before any device work (every
 * call below carries one, so none reaches the HIP runtime).
 * Exit status: 0 when every check holds, 1 otherwise (each failure printed). */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mtp_draft.h"

static int failures = 0;

#define CHECK(cond)                                               \
  do {                                                            \
    if (!(cond)) {                                                \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__,      \
              __LINE__, #cond);                                   \
      ++failures;                                                 \
    }                                                             \
  } while (0)

static size_t round_up_256(size_t v) { return (v + 255u) / 256u * 256u; }

int main(void) {
  int s;
  CHECK(mtp_abi_version() == MTP_ABI_VERSION);

  for (s = MTP_OK; s <= MTP_ERR_RANGE; ++s) {
    const char *t = mtp_status_string(s);
    CHECK(t != NULL && t[0] != '\0');
  }
  CHECK(mtp_status_string(-1) != NULL);
  CHECK(mtp_status_string(1000) != NULL);

  /* the draft step's workspace holds u [b, h] at MTP_STEP_WS_U_OFFSET and c
   * [b, 2h] after it, at the next multiple of 256 */
  {
    const int64_t shapes[][2] = {{1, 4096}, {8, 4096}, {3, 5120}, {4, 8192}, {1, 16}};
    size_t i;
    for (i = 0; i < sizeof shapes / sizeof shapes[0]; ++i) {
      const int64_t b = shapes[i][0], h = shapes[i][1];
      const size_t need = MTP_STEP_WS_U_OFFSET + round_up_256((size_t)(2 * b * h)) + (size_t)(4 * b * h);
      CHECK(mtp_draft_step_workspace_bytes(b, h) >= need);
    }
  }
  /* the combine's: c at MTP_COMBINE_WS_C_OFFSET, then u */
  CHECK(mtp_draft_combine_workspace_bytes(2, 4096) >= MTP_COMBINE_WS_C_OFFSET + 4u * 2 * 4096 + 2u * 2 * 4096);
  CHECK(mtp_lmhead_argmax_workspace_bytes(154880, 4096, 1, MTP_W_BF16) > 0);
  CHECK(mtp_quantize_nvfp4_workspace_bytes(154880, 4096) > 0);

  /* kernel forms: the VALU sweep at one vector, the matrix cores for wide
   * batches, -1 outside the limits */
  CHECK(mtp_lmhead_kernel_form(1, 4096, MTP_W_BF16) == 0);
  CHECK(mtp_lmhead_kernel_form(1, 4096, MTP_W_FP8_E4M3_ROW) == 0);
  CHECK(mtp_lmhead_kernel_form(1, 4096, MTP_W_NVFP4) == 0);
  CHECK(mtp_lmhead_kernel_form(8, 4096, MTP_W_BF16) == 1);
  CHECK(mtp_lmhead_kernel_form(8, 4096, MTP_W_FP8_E4M3_ROW) == 1);
  CHECK(mtp_lmhead_kernel_form(8, 4096, MTP_W_NVFP4) == 1);
  CHECK(mtp_lmhead_kernel_form(9, 4096, MTP_W_BF16) == -1);
  CHECK(mtp_lmhead_kernel_form(1, 4100, MTP_W_BF16) == -1);
  CHECK(mtp_lmhead_kernel_form(1, 4096, 7) == -1);

  /* argument errors come back as statuses, before any device work: each
   * call carries exactly one error, with fake, aligned device addresses 64 GB
   * apart for the rest (never dereferenced, since validation fails first) */
  {
#define P(i) ((void *)(uintptr_t)(0x7F0000000000ull + (uint64_t)(i) * (64ull << 30)))
    const size_t lm_ws = mtp_lmhead_argmax_workspace_bytes(1000, 4096, 1, MTP_W_BF16);
    const size_t st_ws = mtp_draft_step_workspace_bytes(1, 4096);
    int32_t tok_host[1] = {3};
    CHECK(mtp_lmhead_argmax(NULL, 1, 4096, MTP_W_BF16, P(1), NULL, NULL, 1000, 0, P(2), NULL, P(3), lm_ws,
                            NULL) == MTP_ERR_NULL);
    CHECK(mtp_lmhead_argmax(P(0), 1, 4096, 9, P(1), NULL, NULL, 1000, 0, P(2), NULL, P(3), lm_ws, NULL) ==
          MTP_ERR_DTYPE);
    CHECK(mtp_lmhead_argmax(P(0), 0, 4096, MTP_W_BF16, P(1), NULL, NULL, 1000, 0, P(2), NULL, P(3), lm_ws,
                            NULL) == MTP_ERR_SHAPE);
    CHECK(mtp_lmhead_argmax(P(0), 1, 4096, MTP_W_BF16, P(1), NULL, NULL, 1000, 0, P(2), NULL, P(3), lm_ws - 1,
                            NULL) == MTP_ERR_WORKSPACE);
    CHECK(mtp_draft_step(NULL, 10, tok_host, 0, P(1), P(2), P(3), P(4), P(5), 1, 4096, 1e-6f, 0.0f, MTP_W_BF16,
                         P(6), NULL, NULL, 1000, 0, P(7), NULL, NULL, NULL, P(8), st_ws, NULL) == MTP_ERR_NULL);
    tok_host[0] = 10; /* outside [0, embed_vocab) */
    CHECK(mtp_draft_step(P(0), 10, tok_host, 0, P(1), P(2), P(3), P(4), P(5), 1, 4096, 1e-6f, 0.0f, MTP_W_BF16,
                         P(6), NULL, NULL, 1000, 0, P(7), NULL, NULL, NULL, P(8), st_ws, NULL) == MTP_ERR_RANGE);
    CHECK(mtp_codec_encode_range(5, 0u, 16, (uint8_t *)P(9), NULL) == MTP_ERR_DTYPE);
#undef P
  }

  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("abi consumer: all checks passed (ABI %d)\n", mtp_abi_version());
  return 0;
}
