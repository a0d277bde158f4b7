// host_driver.cpp -- runs the host side of the HIP library
// (bf16_forward_attention_amd/csrc/attn_fwd.hip, compiled in) under
// AddressSanitizer and UndefinedBehaviorSanitizer on the host: every entry
// point's argument checks (which return before any HIP call), the split
// plans over a sweep of shapes, and the status strings.  With no GPU the
// calls that pass their argument checks stop at the device check.  Built and
// run by tests/test_sanitize.py; exits non-zero on a failed check.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "attn_fwd.h"

static int failures = 0;
#define CHECK(cond)                                                             \
  do {                                                                          \
    if (!(cond)) {                                                              \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                               \
    }                                                                           \
  } while (0)

int main() {
  // fake, aligned, non-overlapping device addresses: nothing is dereferenced before the checks fail
  char* base = reinterpret_cast<char*>(uintptr_t(1) << 40);
  void *q = base, *k = base + (1 << 24), *v = base + (2 << 24), *o = base + (3 << 24);
  float* lse = reinterpret_cast<float*>(base + (4 << 24));
  void* ws = base + (5 << 24);
  const int64_t big = int64_t(1) << 40;
  // plain call
  CHECK(attn_fwd_bf16(nullptr, k, v, o, 1, 1, 1, 1, 0, 0, nullptr) == ATTN_ERR_NULL);
  CHECK(attn_fwd_bf16(q, k, v, o, 0, 1, 1, 1, 0, 0, nullptr) == ATTN_ERR_SIZE);
  CHECK(attn_fwd_bf16(q, k, v, o, big, big, big, big, 0, 0, nullptr) == ATTN_ERR_SIZE);
  CHECK(attn_fwd_bf16(q, k, v, o, 1, int64_t(1) << 19, 1, 1, 0, 0, nullptr) == ATTN_ERR_SIZE);
  CHECK(attn_fwd_bf16(q, k, v, o, 1, 1, 1, 1, 7, 0, nullptr) == ATTN_ERR_LAYOUT);
  CHECK(attn_fwd_bf16(q, k, v, o, 1, 1, 1, 1, 0, 9, nullptr) == ATTN_ERR_ROUND);
  CHECK(attn_fwd_bf16(static_cast<char*>(q) + 2, k, v, o, 1, 1, 1, 1, 0, 0, nullptr) == ATTN_ERR_ALIGN);
  CHECK(attn_fwd_bf16(q, k, v, q, 1, 1, 1, 1, 0, 0, nullptr) == ATTN_ERR_ALIAS);
  const int any_device = attn_fwd_bf16(q, k, v, o, 1, 1, 1, 1, 0, 0, nullptr);
  CHECK(any_device == ATTN_ERR_DEVICE);  // no GPU on the host this runs on
  // masked, grouped, lse
  CHECK(attn_fwd_bf16_masked(q, k, v, o, 1, 1, 1, 1, 0, 0, 5, nullptr) == ATTN_ERR_MASK);
  CHECK(attn_fwd_bf16_gqa(q, k, v, o, nullptr, 1, 4, 3, 1, 1, 0, 0, 0, nullptr) == ATTN_ERR_HEADS);
  CHECK(attn_fwd_bf16_gqa(q, k, v, o, reinterpret_cast<float*>(base + 2), 1, 4, 2, 1, 1, 0, 0, 0, nullptr) ==
        ATTN_ERR_ALIGN);
  CHECK(attn_fwd_bf16_gqa(q, k, v, o, static_cast<float*>(q), 1, 4, 2, 1, 1, 0, 0, 0, nullptr) == ATTN_ERR_ALIAS);
  CHECK(attn_fwd_bf16_gqa(q, k, v, o, lse, 1, 4, 2, 1, 1, 0, 0, 1, nullptr) == ATTN_ERR_DEVICE);
  // workspace and static-scratch variants
  CHECK(attn_fwd_bf16_ws(q, k, v, o, 1, 1, 1, 1, 0, 0, ws, -1, nullptr) == ATTN_ERR_SIZE);
  CHECK(attn_fwd_bf16_gqa_ws(q, k, v, o, lse, 1, 4, 2, 1, 1, 0, 0, 3, ws, 16, nullptr) == ATTN_ERR_MASK);
  CHECK(attn_fwd_bf16_gqa_noalloc(q, k, v, o, lse, 1, 4, 2, 1, 1, 0, 0, 3, nullptr) == ATTN_ERR_MASK);
  CHECK(attn_fwd_bf16_gqa_noalloc(q, k, v, o, lse, 1, 4, 2, 1, 1, 0, 0, 2, nullptr) == ATTN_ERR_DEVICE);
  int64_t bytes = -1;
  CHECK(attn_fwd_bf16_workspace_size(1, 1, 1, 1, nullptr) == ATTN_ERR_NULL);
  CHECK(attn_fwd_bf16_workspace_size(0, 1, 1, 1, &bytes) == ATTN_ERR_SIZE && bytes == 0);
  CHECK(attn_fwd_bf16_gqa_workspace_size(1, 1, 1, 1, 4, &bytes) == ATTN_ERR_MASK);
  // varlen
  int32_t* cu = reinterpret_cast<int32_t*>(base + (6 << 24));
  CHECK(attn_fwd_bf16_varlen(q, k, v, o, nullptr, nullptr, cu, 1, 1, 1, 1, 1, 1, 0, 0, nullptr) == ATTN_ERR_NULL);
  CHECK(attn_fwd_bf16_varlen(q, k, v, o, nullptr, cu, cu, 1, 1, 1, 0, 1, 1, 0, 0, nullptr) == ATTN_ERR_SIZE);
  CHECK(attn_fwd_bf16_varlen(q, k, v, o, nullptr, cu, cu, 1, 1, 1, 1, 1, 1, 0, 0, nullptr) == ATTN_ERR_DEVICE);
  // key shards
  float* part = reinterpret_cast<float*>(base + (8 << 24));
  CHECK(attn_fwd_bf16_partial(q, k, v, part, nullptr, 1, 1, 1, 1, 1, 0, 1, 0, 0, nullptr) == ATTN_ERR_NULL);
  CHECK(attn_fwd_bf16_partial(q, k, v, part, lse, 1, 1, 1, 1, 2, 1, 2, 0, 0, nullptr) == ATTN_ERR_SIZE);
  CHECK(attn_fwd_bf16_merge(part, lse, 0, o, nullptr, 1, 1, 1, 0, 0, nullptr) == ATTN_ERR_SIZE);
  CHECK(attn_fwd_bf16_merge(part, lse, 2, o, nullptr, 1, 1, 1, 0, 0, nullptr) == ATTN_ERR_DEVICE);
  // split plans over a sweep of shapes: every item accounted for, ranges cover the tiles
  int64_t p[4];
  for (int64_t n_work = 1; n_work <= 2000; n_work = n_work * 3 / 2 + 1)
    for (int64_t n_tiles = 1; n_tiles <= 4096; n_tiles = n_tiles * 2 + 3)
      for (int64_t n_cu : {1, 7, 80, 256, 304}) {
        CHECK(attn_fwd_bf16_split_plan(n_work, n_tiles, n_cu, p) == ATTN_OK);
        CHECK(p[0] + p[1] == n_work && p[2] >= 1 && p[2] * p[3] >= n_tiles && (p[2] - 1) * p[3] < n_tiles);
      }
  for (int64_t heads : {1, 3, 4, 64, 1000})
    for (int64_t Sq : {1, 255, 256, 4097, 16384})
      for (int64_t Sk : {1, 63, 2000, 32771})
        for (int mask = 0; mask < 3; ++mask) {
          CHECK(attn_fwd_bf16_split_plan_masked(heads, Sq, Sk, mask, 256, p) == ATTN_OK);
          CHECK(p[2] >= 1 && p[3] >= 1 && p[2] * (p[0] + p[1]) >= 1);
        }
  CHECK(attn_fwd_bf16_split_plan_masked(1, 1, 1, 3, 256, p) == ATTN_ERR_MASK);
  for (int st = -1; st < 20; ++st) CHECK(attn_fwd_bf16_strerror(st) != nullptr);
  CHECK(std::strcmp(attn_fwd_bf16_strerror(12345), "unknown status") == 0);
  CHECK(attn_fwd_bf16_abi_version() == ATTN_FWD_ABI_VERSION);
  if (failures)
    std::fprintf(stderr, "%d checks failed\n", failures);
  else
    std::printf("host driver: all checks passed\n");
  return failures ? 1 : 0;
}
