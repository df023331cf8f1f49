// Drives the C-ABI's host-side argument checks (every check entry, the status strings and the
// head-dim queries) with valid and invalid arguments.  Built with AddressSanitizer and
// UndefinedBehaviorSanitizer for the host only, so that an out-of-bounds read, an overflow or any
// other undefined behaviour in the checks fails the run.  The checks never dereference the tensor
// pointers (fake, aligned addresses here) and enqueue nothing; only ffpa_check_cu_seqlens reads
// memory, a host array of B + 1 offsets.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../include/ffpa.h"

static int failures = 0;
#define EXPECT(expr, want)                                                                           \
  do {                                                                                               \
    const long long got_ = (long long)(expr);                                                        \
    if (got_ != (long long)(want)) {                                                                 \
      std::printf("FAIL %s:%d: %s = %lld, want %lld (%s)\n", __FILE__, __LINE__, #expr, got_,      \
                  (long long)(want), ffpa_last_error_detail());                                      \
      ++failures;                                                                                    \
    }                                                                                                \
  } while (0)

static const void* P(uint64_t i) { return (const void*)(uintptr_t)(0x1000000000ull * i); }

int main() {
  const float nan = std::nanf("");
  const void *q = P(1), *k = P(2), *v = P(3), *o = P(4);
  const float* lse = (const float*)P(5);
  // dense forward
  EXPECT(ffpa_check_args(q, k, v, nullptr, o, lse, 2, 8, 2, 100, 130, 512, nan, 0, FFPA_BF16), FFPA_OK);
  for (int64_t D = 8; D <= 1024; D += 8) EXPECT(ffpa_check_args(q, k, v, nullptr, o, lse, 1, 2, 1, 5, 7, D, nan, 0, FFPA_FP16), FFPA_OK);
  EXPECT(ffpa_check_args(q, k, v, nullptr, o, lse, 1, 2, 1, 5, 7, 1032, nan, 0, FFPA_BF16), FFPA_ERR_UNSUPPORTED);
  EXPECT(ffpa_check_args(q, k, v, nullptr, o, lse, 1, 2, 1, 5, 7, 12, nan, 0, FFPA_BF16), FFPA_ERR_UNSUPPORTED);
  EXPECT(ffpa_check_args(q, k, v, nullptr, o, lse, 0, 2, 1, 5, 7, 64, nan, 0, FFPA_BF16), FFPA_ERR_VALUE);
  EXPECT(ffpa_check_args(q, k, v, nullptr, o, lse, 1, 3, 2, 5, 7, 64, nan, 0, FFPA_BF16), FFPA_ERR_VALUE);
  EXPECT(ffpa_check_args(q, k, v, nullptr, o, lse, 1, 2, 1, 5, 7, 64, INFINITY, 0, FFPA_BF16), FFPA_ERR_VALUE);
  EXPECT(ffpa_check_args(q, k, v, nullptr, o, lse, 1, 2, 1, 5, 7, 64, nan, 0, 7), FFPA_ERR_TYPE);
  EXPECT(ffpa_check_args((const char*)q + 2, k, v, nullptr, o, lse, 1, 2, 1, 5, 7, 64, nan, 0, FFPA_BF16), FFPA_ERR_VALUE);
  EXPECT(ffpa_check_args(q, k, v, nullptr, o, lse, INT64_MAX / 2, INT64_MAX / 2, 1, INT64_MAX / 2, 7, 64, nan, 0,
                         FFPA_BF16), FFPA_ERR_UNSUPPORTED);
  EXPECT(ffpa_check_args(q, k, v, nullptr, o, lse, 1, 1, 1, INT64_MAX, INT64_MAX, 1024, nan, 1, FFPA_BF16),
         FFPA_ERR_UNSUPPORTED);
  ffpa_mask_t m{P(6), FFPA_MASK_ADD_F32, 0, 0, 130, 1};
  EXPECT(ffpa_check_args(q, k, v, &m, o, lse, 2, 8, 2, 100, 130, 512, nan, 1, FFPA_BF16), FFPA_OK);
  m.stride_k = 2;
  EXPECT(ffpa_check_args(q, k, v, &m, o, lse, 2, 8, 2, 100, 130, 512, nan, 0, FFPA_BF16), FFPA_ERR_UNSUPPORTED);
  m.stride_k = 1;
  m.kind = 9;
  EXPECT(ffpa_check_args(q, k, v, &m, o, lse, 2, 8, 2, 100, 130, 512, nan, 0, FFPA_BF16), FFPA_ERR_TYPE);
  m.kind = FFPA_MASK_BOOL_U8;
  m.stride_q = -1;
  EXPECT(ffpa_check_args(q, k, v, &m, o, lse, 2, 8, 2, 100, 130, 512, nan, 0, FFPA_BF16), FFPA_ERR_VALUE);
  m.stride_q = INT64_MAX / 4;
  EXPECT(ffpa_check_args(q, k, v, &m, o, lse, 2, 8, 2, 100, 130, 512, nan, 0, FFPA_BF16) != FFPA_OK, 1);

  // strided layouts
  ffpa_layout_t lay{{8 * 100 * 512, 512, 8 * 512}, {2 * 130 * 512, 512, 2 * 512}, {2 * 130 * 512, 512, 2 * 512},
                    {8 * 100 * 512, 512, 8 * 512}};
  EXPECT(ffpa_check_strided_args(q, k, v, nullptr, o, lse, 2, 8, 2, 100, 130, 512, &lay, nan, 0, FFPA_BF16), FFPA_OK);
  lay.q[2] = 3;
  EXPECT(ffpa_check_strided_args(q, k, v, nullptr, o, lse, 2, 8, 2, 100, 130, 512, &lay, nan, 0, FFPA_BF16) != FFPA_OK, 1);
  lay.q[2] = INT64_MAX / 2;
  EXPECT(ffpa_check_strided_args(q, k, v, nullptr, o, lse, 2, 8, 2, 100, 130, 512, &lay, nan, 0, FFPA_BF16) != FFPA_OK, 1);
  EXPECT(ffpa_check_strided_args(q, k, v, nullptr, o, lse, 2, 8, 2, 100, 130, 512, nullptr, nan, 0, FFPA_BF16),
         FFPA_ERR_VALUE);
  ffpa_layout_t huge{{INT64_MAX / 8 * 8, 512, 8 * 512}, {INT64_MAX / 8 * 8, INT64_MAX / 16 * 8, 2 * 512},
                     {2 * 130 * 512, 512, 2 * 512}, {INT64_MAX / 8 * 8, 512, 8 * 512}};
  EXPECT(ffpa_check_strided_args(q, k, v, nullptr, o, lse, 2, 8, 2, 100, 130, 512, &huge, nan, 0, FFPA_BF16) != FFPA_OK,
         1);

  // packed variable-length sequences: the host offsets are read
  const int32_t cu[4] = {0, 70, 70, 200};
  EXPECT(ffpa_check_cu_seqlens(cu, 3, 200, 130), FFPA_OK);
  EXPECT(ffpa_check_cu_seqlens(cu, 3, 200, 100), FFPA_ERR_VALUE);
  EXPECT(ffpa_check_cu_seqlens(cu, 3, 199, 130), FFPA_ERR_VALUE);
  const int32_t bad[3] = {0, 50, 40};
  EXPECT(ffpa_check_cu_seqlens(bad, 2, 40, 100), FFPA_ERR_VALUE);
  std::vector<int32_t> big(1001);
  for (int i = 0; i <= 1000; ++i) big[i] = 3 * i;
  EXPECT(ffpa_check_cu_seqlens(big.data(), 1000, 3000, 3), FFPA_OK);
  const int32_t* cq = (const int32_t*)P(7);
  EXPECT(ffpa_check_varlen_args(q, k, v, cq, cq, o, lse, 3, 8, 2, 200, 200, 130, 130, 512, nan, 1, FFPA_BF16), FFPA_OK);
  EXPECT(ffpa_check_varlen_args(q, k, v, nullptr, cq, o, lse, 3, 8, 2, 200, 200, 130, 130, 512, nan, 1, FFPA_BF16),
         FFPA_ERR_VALUE);
  EXPECT(ffpa_check_varlen_args(q, k, v, cq, cq, o, lse, 3, 8, 2, INT64_MAX, 200, 130, 130, 512, nan, 0, FFPA_BF16) !=
             FFPA_OK, 1);

  // dropout
  const uint32_t* keep = (const uint32_t*)P(8);
  EXPECT(ffpa_check_dropout_args(q, k, v, nullptr, o, lse, 1, 2, 1, 96, 160, 512, nan, 0, FFPA_BF16, keep, 0.2f), FFPA_OK);
  EXPECT(ffpa_check_dropout_args(q, k, v, nullptr, o, lse, 1, 2, 1, 96, 160, 512, nan, 0, FFPA_BF16, keep, 1.0f),
         FFPA_ERR_VALUE);
  EXPECT(ffpa_check_dropout_args(q, k, v, nullptr, o, lse, 1, 2, 1, 96, 160, 512, nan, 0, FFPA_BF16, keep, nan),
         FFPA_ERR_VALUE);

  // fp8
  const float* f = (const float*)P(9);
  EXPECT(ffpa_check_fp8_args(q, k, v, f, f, f, nullptr, o, lse, 1, 8, 8, 4096, 4096, 512, nan, 0, FFPA_BF16), FFPA_OK);
  EXPECT(ffpa_check_fp8_args(q, k, v, f, f, f, nullptr, o, lse, 1, 8, 8, 4096, 4096, 520, nan, 0, FFPA_BF16),
         FFPA_ERR_UNSUPPORTED);
  EXPECT(ffpa_check_fp8_args(q, k, v, f, f, f, nullptr, o, lse, 1, 8, 8, 4096, 4096, 512, nan, 0, 5), FFPA_ERR_TYPE);

  // backward (host checks only: invalid arguments return before any HIP call)
  void *dq = (void*)P(10), *dk = (void*)P(11), *dv = (void*)P(12), *ws = (void*)P(13);
  EXPECT(ffpa_bwd(q, k, v, o, o, lse, nullptr, dq, dk, dv, 1, 2, 1, 100, 130, 100, nan, 0, FFPA_BF16, ws, 1 << 20,
                  nullptr), FFPA_ERR_UNSUPPORTED);
  EXPECT(ffpa_bwd(q, k, v, o, o, lse, nullptr, dq, dk, dv, 1, 2, 1, 100, 130, 512, nan, 0, FFPA_BF16, ws, 16, nullptr),
         FFPA_ERR_VALUE);
  EXPECT(ffpa_bwd(q, k, v, o, o, lse, nullptr, dq, dk, dv, INT64_MAX / 2, INT64_MAX / 2, 1, INT64_MAX / 2, 130, 512,
                  nan, 0, FFPA_BF16, ws, 1 << 20, nullptr), FFPA_ERR_UNSUPPORTED);
  EXPECT(ffpa_bwd_workspace_size(1, 8, 8, 4096, 4096, 512), 131072);
  EXPECT(ffpa_bwd_workspace_size(INT64_MAX / 2, INT64_MAX / 2, 1, INT64_MAX / 2, 7, 64), 0);
  EXPECT(ffpa_bwd_workspace_size(1, 8, 3, 4096, 4096, 512), 0);

  // strings and head-dim queries
  for (int s = -2; s < 8; ++s) EXPECT(std::strlen(ffpa_status_string(s)) > 0, 1);
  for (int64_t D = -8; D <= 1100; D += 4) {
    (void)ffpa_rows_per_block(D);
    (void)ffpa_kernel_head_dim(D);
    (void)ffpa_fp8_kernel_head_dim(D);
    const char* n = ffpa_kernel_name(D);
    if (n) (void)std::strlen(n);
  }
  std::printf("%d failures\n", failures);
  return failures == 0 ? 0 : 1;
}
