/* Drives every host-side argument check of the C ABI (include/kdkl.h)
 * without touching a device: run against a copy of the library whose host
 * code is built with AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_sanitized_host.py).  Fake device pointers are never
 * dereferenced: every call here returns before its first HIP call. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include "kdkl.h"

#define CHECK(expr, want)                                                                         \
  do {                                                                                            \
    int got_ = (int)(expr);                                                                       \
    if (got_ != (int)(want)) {                                                                    \
      fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, #expr, got_,   \
              (int)(want));                                                                       \
      return 1;                                                                                   \
    }                                                                                             \
  } while (0)

static kd_problem prob(int64_t T, int64_t H, int64_t V, int32_t K, float tau, int32_t cv, int32_t bt,
                       uint32_t flags) {
  kd_problem p = {T, H, V, K, tau, cv, bt, flags};
  return p;
}

int main(void) {
  const uint16_t* fh = (const uint16_t*)(uintptr_t)(1u << 20);
  const int32_t* fi = (const int32_t*)(uintptr_t)(1u << 20);
  const float* ff = (const float*)(uintptr_t)(1u << 20);
  float* fo = (float*)(uintptr_t)(1u << 20);
  void* fw = (void*)(uintptr_t)(1u << 20);
  size_t n = 0;
  int64_t bt = 0, cv = 0;
  int32_t nb = 0;

  /* sizes and tiling of valid problems, from T = 0 to the sweep's largest */
  const int64_t Ts[] = {0, 1, 255, 256, 4096, 8193, 262144};
  for (unsigned i = 0; i < sizeof(Ts) / sizeof(Ts[0]); ++i) {
    kd_problem p = prob(Ts[i], 2880, 201088, 64, 1.0f, 0, 0, 0);
    CHECK(kd_topk_kl_workspace_size(&p, &n), KD_OK);
    CHECK(kd_topk_kl_fwd_workspace_size(&p, &n), KD_OK);
    CHECK(kd_topk_kl_saved_size(&p, &n), KD_OK);
    CHECK(kd_topk_kl_tiling(&p, &bt, &cv, &nb), KD_OK);
    p.flags = KD_FLAG_SEQ_CHUNK | KD_FLAG_GRAD_BF16;
    CHECK(kd_topk_kl_workspace_size(&p, &n), KD_OK);
  }
  /* invalid and unsupported problems */
  kd_problem p = prob(4096, 2880, 201088, 64, 0.0f, 0, 0, 0);
  CHECK(kd_topk_kl_workspace_size(&p, &n), KD_ERR_ARG);
  p.tau = NAN;
  CHECK(kd_topk_kl_workspace_size(&p, &n), KD_ERR_ARG);
  p = prob(-1, 2880, 201088, 64, 1.0f, 0, 0, 0);
  CHECK(kd_topk_kl_workspace_size(&p, &n), KD_ERR_ARG);
  p = prob(4096, 2880, 50, 64, 1.0f, 0, 0, 0);
  CHECK(kd_topk_kl_workspace_size(&p, &n), KD_ERR_ARG);
  p = prob(4096, 2900, 201088, 64, 1.0f, 0, 0, 0);
  CHECK(kd_topk_kl_workspace_size(&p, &n), KD_ERR_UNSUPPORTED);
  p = prob(4096, 2880, 201088, 2000, 1.0f, 0, 0, 0);
  CHECK(kd_topk_kl_workspace_size(&p, &n), KD_ERR_UNSUPPORTED);
  p = prob(4096, 98304, 201088, 64, 1.0f, 0, 0, 0); /* fp32 dW chunk over 4 GiB */
  CHECK(kd_topk_kl_workspace_size(&p, &n), KD_ERR_UNSUPPORTED);
  p = prob(4096, 2880, 201088, 64, 1.0f, 300, 0, 0);
  CHECK(kd_topk_kl_workspace_size(&p, &n), KD_ERR_UNSUPPORTED);
  p = prob(4096, 2880, 201088, 64, 1.0f, 0, 0, 1u << 12);
  CHECK(kd_topk_kl_workspace_size(&p, &n), KD_ERR_ARG);
  CHECK(kd_topk_kl_workspace_size(NULL, &n), KD_ERR_ARG);
  CHECK(kd_topk_kl_workspace_size(&p, NULL), KD_ERR_ARG);
  CHECK(kd_topk_kl_tiling(&p, NULL, &cv, &nb), KD_ERR_ARG);

  /* the fused call: argument errors before any launch */
  p = prob(16, 64, 100, 4, 1.0f, 0, 0, 0);
  CHECK(kd_topk_kl_workspace_size(&p, &n), KD_OK);
  CHECK(kd_topk_kl_fwd_bwd(&p, fh, NULL, fi, ff, NULL, fo, NULL, NULL, NULL, fw, n, NULL), KD_ERR_ARG);
  CHECK(kd_topk_kl_fwd_bwd(&p, fh, fh, fi, ff, NULL, NULL, NULL, NULL, NULL, fw, n, NULL), KD_ERR_ARG);
  CHECK(kd_topk_kl_fwd_bwd(&p, fh, fh, fi, ff, NULL, fo, NULL, NULL, NULL, NULL, n, NULL), KD_ERR_ARG);
  CHECK(kd_topk_kl_fwd_bwd(&p, (const uint16_t*)((uintptr_t)fh + 2), fh, fi, ff, NULL, fo, NULL, NULL, NULL, fw,
                           n, NULL),
        KD_ERR_UNSUPPORTED);
  CHECK(kd_topk_kl_fwd_bwd(&p, fh, fh, fi, ff, NULL, fo, NULL, NULL, NULL, fw, 16, NULL), KD_ERR_WORKSPACE);
  CHECK(kd_topk_kl_fwd(&p, fh, fh, fi, ff, NULL, fo, NULL, NULL, fw, n, NULL), KD_ERR_ARG);
  CHECK(kd_topk_kl_bwd(&p, fh, fh, fi, ff, NULL, NULL, NULL, fo, fo, fw, n, NULL), KD_ERR_ARG);
  /* the allocation-free call: a problem beyond its scratch, then argument errors */
  p = prob(4096, 2880, 201088, 64, 1.0f, 0, 0, 0);
  CHECK(kd_topk_kl_fwd_bwd_noalloc(&p, fh, fh, fi, ff, NULL, fo, fw, fw, NULL, NULL), KD_ERR_WORKSPACE);
  CHECK(kd_topk_kl_fwd_bwd_noalloc(&p, fh, NULL, fi, ff, NULL, fo, fw, fw, NULL, NULL), KD_ERR_ARG);

  /* the logits variant and the top-K producer */
  kd_logits_problem lp = {16, 100, 4, 1.0f, 0};
  CHECK(kd_topk_kl_logits_workspace_size(&lp, &n), KD_OK);
  CHECK(kd_topk_kl_logits(&lp, fw, fi, ff, NULL, NULL, NULL, NULL, fw, n, NULL), KD_ERR_ARG);
  lp.K = 200;
  CHECK(kd_topk_kl_logits_workspace_size(&lp, &n), KD_ERR_ARG);
  kd_topk_problem tp = {16, 100, 4, 0};
  CHECK(kd_topk_select(&tp, fh, NULL, NULL, NULL), KD_ERR_ARG);
  tp.V = 101;
  CHECK(kd_topk_select(&tp, fh, (int32_t*)fw, fo, NULL), KD_ERR_UNSUPPORTED);

  /* status strings, including codes the enum does not name */
  for (int c = -1; c <= 8; ++c)
    if (!kd_status_string((kd_status)c)) return 1;
  if (kd_abi_version() != 5) return 1;
  printf("host ABI checks: ok\n");
  return 0;
}
