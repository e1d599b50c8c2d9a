/* Host-side driver for the sanitizer build of the C ABI (address and undefined-
 * behaviour sanitizers on the host code): status strings, workspace sizes over
 * the whole accepted shape range (where the size arithmetic could overflow), the
 * diagnostic hooks, and every entry point with arguments that fail validation.
 * Every call here returns before any HIP call that could reach a GPU, so the
 * driver runs the same with or without one.  Exit status 0 when every call
 * returned the expected status; the sanitizers abort on their first report. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mtp.h"

static int failures = 0;

#define EXPECT(call, want)                                                                   \
  do {                                                                                       \
    const mtp_status got_ = (call);                                                          \
    if (got_ != (want)) {                                                                    \
      fprintf(stderr, "line %d: %s returned %d, expected %d (%s)\n", __LINE__, #call, (int)got_, \
              (int)(want), mtp_last_error());                                                \
      ++failures;                                                                            \
    }                                                                                        \
  } while (0)

int main(void) {
  /* aligned and misaligned fake addresses: validation fails before they are used */
  void* const A = (void*)(uintptr_t)0x10000;
  void* const M = (void*)(uintptr_t)0x10008;
  const int32_t* const Ai = (const int32_t*)A;
  size_t n = 0;

  for (int s = -3; s < 24; ++s) {
    const char* str = mtp_status_string((mtp_status)s);
    if (!str || !strlen(str)) { fprintf(stderr, "empty status string %d\n", s); ++failures; }
  }
  if (!mtp_version() || !mtp_last_error()) ++failures;

  /* workspace sizes at the edges of the accepted shapes */
  const int32_t big = INT32_MAX, vmax = 1 << 30;
  for (int dt = 0; dt < 2; ++dt) {
    EXPECT(mtp_verify_workspace_size(big, 8, vmax, (mtp_dtype)dt, &n), MTP_OK);
    EXPECT(mtp_verify_target_only_workspace_size(big, 8, vmax, (mtp_dtype)dt, &n), MTP_OK);
    EXPECT(mtp_verify_gumbel_workspace_size(big, 8, vmax, (mtp_dtype)dt, &n), MTP_OK);
    EXPECT(mtp_gumbel_sample_workspace_size(big, vmax, (mtp_dtype)dt, &n), MTP_OK);
    EXPECT(mtp_tv_topk_workspace_size(big, 8, vmax, (mtp_dtype)dt, &n), MTP_OK);
    for (int sh = 0; sh < 2; ++sh) {
      EXPECT(mtp_tv_loss_workspace_size(big, 8, vmax, (mtp_dtype)dt, sh, &n), MTP_OK);
      EXPECT(mtp_tv_loss_fwd_bwd_workspace_size(big, 8, vmax, (mtp_dtype)dt, sh, &n), MTP_OK);
    }
    EXPECT(mtp_verify_workspace_size(1, 1, 1, (mtp_dtype)dt, &n), MTP_OK);
    EXPECT(mtp_tv_loss_workspace_size(1, 1, 1, (mtp_dtype)dt, 1, &n), MTP_OK);
  }
  EXPECT(mtp_verify_workspace_size(-1, 3, 100, MTP_BF16, &n), MTP_ERR_SHAPE);
  EXPECT(mtp_verify_workspace_size(4, 0, 100, MTP_BF16, &n), MTP_ERR_SHAPE);
  EXPECT(mtp_verify_workspace_size(4, 9, 100, MTP_BF16, &n), MTP_ERR_SHAPE);
  EXPECT(mtp_verify_workspace_size(4, 3, 0, MTP_BF16, &n), MTP_ERR_SHAPE);
  EXPECT(mtp_verify_workspace_size(4, 3, vmax + 1, MTP_BF16, &n), MTP_ERR_SHAPE);
  EXPECT(mtp_verify_workspace_size(4, 3, 100, (mtp_dtype)7, &n), MTP_ERR_DTYPE);
  EXPECT(mtp_verify_workspace_size(4, 3, 100, MTP_BF16, NULL), MTP_ERR_NULL);
  EXPECT(mtp_tv_loss_workspace_size(0, 3, 100, MTP_BF16, 1, &n), MTP_ERR_SHAPE);
  EXPECT(mtp_tv_loss_fwd_bwd_workspace_size(-5, 3, 100, MTP_BF16, 1, &n), MTP_ERR_SHAPE);
  EXPECT(mtp_tv_topk_workspace_size(4, 3, 100, MTP_BF16, NULL), MTP_ERR_NULL);
  EXPECT(mtp_gumbel_sample_workspace_size(-1, 100, MTP_BF16, &n), MTP_ERR_SHAPE);
  EXPECT(mtp_verify_max_vocab((mtp_dtype)9, (int32_t*)A), MTP_ERR_DTYPE);
  EXPECT(mtp_verify_max_vocab(MTP_BF16, NULL), MTP_ERR_NULL);

  /* the diagnostic hooks, and the layouts under the smallest chunk */
  const uint64_t wl = mtp_set_wait_limit(12345);
  if (mtp_set_wait_limit(wl) != 12345) ++failures;
  if (mtp_set_chunk_vectors(1) != 0) ++failures;
  EXPECT(mtp_verify_workspace_size(big, 8, vmax, MTP_F32, &n), MTP_OK);
  EXPECT(mtp_tv_loss_fwd_bwd_workspace_size(big, 4, vmax, MTP_F32, 1, &n), MTP_OK);
  if (mtp_set_chunk_vectors(0) != 1) ++failures;

  /* entry points with arguments that fail validation */
  uint8_t* const acc = (uint8_t*)A;
  int32_t* const i32 = (int32_t*)A;
  float* const f32 = (float*)A;
  /* row stride 104 bfloat16 logits (208 bytes) for V = 100 */
  EXPECT(mtp_verify(A, 104, A, 104, MTP_BF16, 2, 3, 100, Ai, 1, 0, acc, i32, i32, i32, f32, f32, f32, i32, NULL, 0,
                    NULL),
         MTP_ERR_WORKSPACE);
  EXPECT(mtp_verify(M, 104, A, 104, MTP_BF16, 2, 3, 100, Ai, 1, 0, acc, i32, i32, i32, f32, f32, f32, i32, A, 1 << 20,
                    NULL),
         MTP_ERR_ALIGN);
  EXPECT(mtp_verify(A, 101, A, 104, MTP_BF16, 2, 3, 100, Ai, 1, 0, acc, i32, i32, i32, f32, f32, f32, i32, A, 1 << 20,
                    NULL),
         MTP_ERR_ALIGN);
  EXPECT(mtp_verify(A, 104, A, 104, MTP_BF16, 2, 3, 100, NULL, 1, 0, acc, i32, i32, i32, f32, f32, f32, i32, A,
                    1 << 20, NULL),
         MTP_ERR_NULL);
  EXPECT(mtp_verify(A, 104, A, 104, MTP_BF16, 2, 3, 100, Ai, 1, 0, acc, i32, i32, i32, f32, f32, f32, i32, A, 16, NULL),
         MTP_ERR_WORKSPACE);
  EXPECT(mtp_verify(A, 104, A, 104, MTP_BF16, 2, 3, 100, Ai, 1, 0, acc, i32, i32, i32, f32, f32, f32, i32, M, 1 << 20,
                    NULL),
         MTP_ERR_WORKSPACE);
  EXPECT(mtp_verify(A, -8, A, 104, MTP_BF16, 2, 3, 100, Ai, 1, 0, acc, i32, i32, i32, f32, f32, f32, i32, A, 1 << 20,
                    NULL),
         MTP_ERR_SHAPE);
  EXPECT(mtp_verify(A, 8, A, 104, MTP_BF16, 2, 3, 100, Ai, 1, 0, acc, i32, i32, i32, f32, f32, f32, i32, A, 1 << 20,
                    NULL),
         MTP_ERR_SHAPE);   /* row stride below the vocabulary */
  EXPECT(mtp_verify(A, 104, A, 104, MTP_BF16, big, 8, 100, Ai, 1, 0, acc, i32, i32, i32, f32, f32, f32, i32, A,
                    1 << 20, NULL),
         MTP_ERR_WORKSPACE);   /* the largest batch: a workspace of terabytes */
  EXPECT(mtp_verify_noalloc(A, 8, A, 8, MTP_BF16, 2, 9, 100, Ai, 1, 0, acc, i32, i32, i32, f32, f32, f32, i32, NULL),
         MTP_ERR_SHAPE);
  EXPECT(mtp_verify_noalloc(A, 8, A, 8, MTP_BF16, big, 8, vmax, Ai, 1, 0, acc, i32, i32, i32, f32, f32, f32, i32, NULL),
         MTP_ERR_SHAPE);   /* beyond the stride, and far beyond the static scratch */
  EXPECT(mtp_verify_target_only(A, 104, A, 104, MTP_F32, 2, 3, 100, 1, 0, acc, i32, i32, i32, f32, acc, i32, f32, f32,
                                f32, i32, NULL, 0, NULL),
         MTP_ERR_WORKSPACE);
  EXPECT(mtp_verify_target_only(A, 104, A, 104, MTP_F32, 2, 3, 100, 1, 0, acc, i32, i32, NULL, f32, acc, i32, f32, f32,
                                f32, i32, A, 1 << 20, NULL),
         MTP_ERR_NULL);
  EXPECT(mtp_verify_gumbel(A, 104, A, 104, MTP_BF16, 2, 3, 100, Ai, 0.f, 1, 0, acc, i32, i32, i32, f32, f32, f32, i32, A,
                           1 << 20, NULL),
         MTP_ERR_SHAPE);   /* temperature 0 */
  EXPECT(mtp_gumbel_sample(A, 104, MTP_BF16, 3, 100, -1.f, 1, 0, i32, A, 1 << 20, NULL), MTP_ERR_SHAPE);
  EXPECT(mtp_gumbel_sample(M, 104, MTP_BF16, 3, 100, 1.f, 1, 0, i32, A, 1 << 20, NULL), MTP_ERR_ALIGN);
  EXPECT(mtp_tv_loss_fwd(A, 104, 0, A, 312, 104, MTP_BF16, 4, 3, 100, f32, f32, f32, NULL, 0, NULL), MTP_ERR_WORKSPACE);
  EXPECT(mtp_tv_loss_fwd(A, 104, 0, A, 312, 104, MTP_BF16, 4, 9, 100, f32, f32, f32, A, 1 << 20, NULL), MTP_ERR_SHAPE);
  EXPECT(mtp_tv_loss_fwd(M, 104, 0, A, 312, 104, MTP_BF16, 4, 3, 100, f32, f32, f32, A, 1 << 20, NULL), MTP_ERR_ALIGN);
  EXPECT(mtp_tv_loss_bwd(A, 104, 0, A, 312, 104, MTP_BF16, 4, 3, 100, NULL, f32, A, 312, 104, MTP_BF16, NULL),
         MTP_ERR_NULL);
  EXPECT(mtp_tv_loss_bwd(A, 104, 0, A, 312, 104, MTP_BF16, 4, 3, 100, f32, f32, A, 312, 104, (mtp_dtype)5, NULL),
         MTP_ERR_DTYPE);
  EXPECT(mtp_tv_loss_fwd_bwd(A, 104, 0, A, 312, 104, MTP_BF16, 4, 3, 100, f32, f32, f32, f32, A, 312, 104, MTP_BF16,
                             NULL, 0, NULL),
         MTP_ERR_WORKSPACE);
  EXPECT(mtp_tv_loss_fwd_bwd(A, 104, 0, A, 312, 104, MTP_BF16, 4, 3, 100, f32, f32, f32, f32, M, 312, 104, MTP_BF16,
                             A, 1 << 20, NULL),
         MTP_ERR_ALIGN);
  EXPECT(mtp_tv_loss_fwd_bwd(A, 104, 0, A, 312, 104, MTP_BF16, 4, 3, 100, f32, f32, f32, f32, A, -312, 104, MTP_BF16,
                             A, 1 << 20, NULL),
         MTP_ERR_SHAPE);
  EXPECT(mtp_tv_topk_fwd(Ai, f32, 16, 0, 0, A, 312, 104, MTP_BF16, 4, 3, 100, f32, f32, f32, A, 1 << 20, NULL),
         MTP_ERR_SHAPE);   /* K = 0 */
  EXPECT(mtp_tv_topk_bwd(Ai, NULL, 16, 0, 16, A, 312, 104, MTP_BF16, 4, 3, 100, f32, f32, A, 312, 104, MTP_BF16, NULL),
         MTP_ERR_NULL);
  EXPECT(mtp_workspace_error(NULL, (uint32_t*)A, NULL), MTP_ERR_NULL);

  if (failures) fprintf(stderr, "%d unexpected results\n", failures);
  else printf("host ABI driver: all calls returned the expected status\n");
  return failures ? 1 : 0;
}
