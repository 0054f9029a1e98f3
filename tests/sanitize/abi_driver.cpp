// Host-side checks of the C ABI (include/cat.h) under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Every validation path runs: malformed and
// unsupported problems, NULL and misaligned pointers, a plan of the wrong
// kind, every status string and the last-error text.  Valid problems run the
// plan's geometry and workspace layout and its host tables; without a GPU
// plan creation stops at the first device call with CAT_ERR_HIP (freeing
// what it built), with one the plan is built, queried and destroyed.  The
// driver prints the first failed expectation and returns 1; it returns 0
// when every expectation holds and no sanitizer fires.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "cat.h"

static int failures = 0;
#define EXPECT(c)                                                  \
  do {                                                             \
    if (!(c)) {                                                    \
      std::printf("expectation failed at line %d: %s\n", __LINE__, #c); \
      ++failures;                                                  \
    }                                                              \
  } while (0)

static cat_problem prob(int kind, int dtype, int64_t B, int64_t N, int64_t D, int64_t H, int64_t Hg = 0,
                        int64_t Wg = 0) {
  cat_problem p;
  std::memset(&p, 0, sizeof p);
  p.kind = kind;
  p.dtype = dtype;
  p.B = B;
  p.N = N;
  p.D = D;
  p.H = H;
  p.Hg = Hg;
  p.Wg = Wg;
  return p;
}

// Entries with a valid plan but bad pointers: rejected before any HIP call.
static void bad_pointers(cat_plan pl, bool is1d) {
  alignas(16) static unsigned char buf[256];
  void* mis = buf + 4;  // misaligned
  if (is1d) {
    EXPECT(cat_forward_1d(pl, nullptr, buf, buf, buf, buf, nullptr) == CAT_ERR_INVALID_ARG);
    EXPECT(cat_forward_1d(pl, mis, buf, buf, buf, buf, nullptr) == CAT_ERR_INVALID_ARG);
    EXPECT(cat_forward_bccb_2d(pl, buf, buf, buf, buf, buf, buf, nullptr) == CAT_ERR_PLAN_MISMATCH);
    EXPECT(cat_backward_1d(pl, nullptr, buf, buf, buf, buf, buf, buf, buf, nullptr) == CAT_ERR_INVALID_ARG);
    EXPECT(cat_step_mix_backward_1d(pl, nullptr, buf, buf, reinterpret_cast<float*>(buf), buf, buf, nullptr) ==
           CAT_ERR_INVALID_ARG);
    EXPECT(cat_forward_avgkey_1d(pl, buf, buf, buf, buf, mis, buf, nullptr) != CAT_OK);
    EXPECT(cat_forward_causal_1d(pl, buf, nullptr, buf, buf, buf, nullptr) != CAT_OK);
    EXPECT(cat_forward_1d_noalloc(pl, buf, buf, nullptr, buf, nullptr) == CAT_ERR_INVALID_ARG);
  } else {
    EXPECT(cat_forward_bccb_2d(pl, buf, buf, buf, nullptr, buf, buf, nullptr) == CAT_ERR_INVALID_ARG);
    EXPECT(cat_forward_1d(pl, buf, buf, buf, buf, buf, nullptr) == CAT_ERR_PLAN_MISMATCH);
    EXPECT(cat_backward_1d(pl, buf, buf, buf, buf, buf, buf, buf, buf, nullptr) == CAT_ERR_PLAN_MISMATCH);
    EXPECT(cat_forward_1d_noalloc(pl, buf, buf, buf, buf, nullptr) == CAT_ERR_PLAN_MISMATCH);
  }
  EXPECT(cat_step_mix(pl, nullptr, buf, buf, buf, nullptr) == CAT_ERR_INVALID_ARG);
}

int main() {
  // NULL plan and NULL outputs
  EXPECT(cat_plan_create(nullptr, nullptr) == CAT_ERR_INVALID_ARG);
  cat_plan pl = reinterpret_cast<cat_plan>(0x1);
  EXPECT(cat_plan_create(&pl, nullptr) == CAT_ERR_INVALID_ARG && pl == nullptr);
  EXPECT(cat_plan_destroy(nullptr) == CAT_OK);
  size_t ws = 0;
  EXPECT(cat_plan_workspace_size(nullptr, &ws) == CAT_ERR_INVALID_ARG);
  EXPECT(cat_forward_1d(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == CAT_ERR_INVALID_ARG);
  EXPECT(cat_backward_1d(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) ==
         CAT_ERR_INVALID_ARG);
  EXPECT(std::strlen(cat_last_error()) > 0);

  // malformed problems (CAT_ERR_INVALID_ARG) and unsupported ones
  const cat_problem invalid[] = {
      prob(CAT_1D, CAT_F32, -1, 64, 32, 2),      prob(CAT_1D, CAT_F32, 1, 0, 32, 2),
      prob(CAT_1D, CAT_F32, 1, 64, 30, 4),       prob(CAT_1D, CAT_F32, 1, 64, 36, 4),
      prob(CAT_1D, CAT_F32, 1, 64, 24, 24),      prob(7, CAT_F32, 1, 64, 32, 2),
      prob(CAT_1D, 9, 1, 64, 32, 2),             prob(CAT_BCCB_2D, CAT_F32, 1, 64, 32, 2, 4, 4),
      prob(CAT_BCCB_2D, CAT_F32, 1, 64, 32, 2, 0, 64),
  };
  for (const cat_problem& p : invalid) {
    pl = reinterpret_cast<cat_plan>(0x1);
    const cat_status st = cat_plan_create(&pl, &p);
    EXPECT(st != CAT_OK && pl == nullptr);
    EXPECT(std::strlen(cat_last_error()) > 0);
  }
  const cat_problem unsupported[] = {
      prob(CAT_1D, CAT_F32, 1, 131072, 32, 2),   prob(CAT_1D, CAT_F32, 1, 40000, 32, 2),
      prob(CAT_1D, CAT_F32, 1, 64, 512, 64),     prob(CAT_BCCB_2D, CAT_F32, 1, 100, 32, 2, 10, 10),
      prob(CAT_1D, CAT_BF16, 1 << 20, 1024, 4096, 32), prob(CAT_1D, CAT_F32, int64_t(1) << 40, int64_t(1) << 30, 64, 2),
      prob(CAT_1D, CAT_F32, int64_t(1) << 62, 4, 16, 2),
  };
  for (const cat_problem& p : unsupported) {
    pl = reinterpret_cast<cat_plan>(0x1);
    EXPECT(cat_plan_create(&pl, &p) == CAT_ERR_UNSUPPORTED && pl == nullptr);
  }

  // valid problems over every path: built (with a GPU) or stopped at the
  // first device call (without one)
  const cat_problem valid[] = {
      prob(CAT_1D, CAT_BF16, 16, 1024, 768, 12),   prob(CAT_1D, CAT_F32, 2, 197, 96, 3),
      prob(CAT_1D, CAT_BF16, 4, 256, 128, 4),      prob(CAT_1D, CAT_F32, 1, 65536, 32, 2),
      prob(CAT_1D, CAT_BF16, 1, 20000, 32, 2),     prob(CAT_1D, CAT_F32, 0, 64, 32, 2),
      prob(CAT_1D, CAT_F32, 3, 1, 16, 2),          prob(CAT_BCCB_2D, CAT_BF16, 8, 9216, 384, 6, 96, 96),
      prob(CAT_BCCB_2D, CAT_F32, 2, 12, 16, 2, 3, 4), prob(CAT_BCCB_2D, CAT_BF16, 1, 1024, 64, 2, 32, 32),
  };
  for (const cat_problem& p : valid) {
    pl = reinterpret_cast<cat_plan>(0x1);
    const cat_status st = cat_plan_create(&pl, &p);
    EXPECT(st == CAT_OK || st == CAT_ERR_HIP || st == CAT_ERR_ALLOC);
    if (st != CAT_OK) {
      EXPECT(pl == nullptr);
      continue;
    }
    EXPECT(cat_plan_workspace_size(pl, &ws) == CAT_OK && ws > 0);
    int64_t L = 0, L1 = 0, L2 = 0;
    EXPECT(cat_plan_geometry(pl, &L, &L1, &L2) == CAT_OK && L == L1 * L2 && L >= 1);
    int path = -1;
    EXPECT(cat_plan_conv_path(pl, &path) == CAT_OK && path >= 0 && path <= 3);
    if (p.B > 0) bad_pointers(pl, p.kind == CAT_1D);
    EXPECT(cat_plan_destroy(pl) == CAT_OK);
  }

  // status strings
  for (int c = -6; c <= 1; ++c) EXPECT(cat_status_string(static_cast<cat_status>(c)) != nullptr);
  if (failures == 0) std::printf("abi driver: all expectations held\n");
  return failures == 0 ? 0 : 1;
}
