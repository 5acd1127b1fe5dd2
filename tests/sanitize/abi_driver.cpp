// Host-side driver of the C ABI for the sanitizer build of the library's
// host code (address and undefined-behaviour sanitizers).  Every call here
// returns before a kernel is enqueued: argument errors, workspace planning
// for many shapes, the host projection matrix, and whole forward / backward
// calls stopped at their first launcher by HYPERATTN_FAIL_AT (the planning
// of the causal recursion, odd splits and rectangular problems included).
// Dummy device pointers are never dereferenced.  Exit status 0 = every
// expectation held (the sanitizers abort on their own findings).
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "hyperattn.h"

static int failures = 0;
#define EXPECT(cond)                                                    \
  do {                                                                  \
    if (!(cond)) {                                                      \
      std::fprintf(stderr, "expectation failed line %d: %s (%s)\n", __LINE__, #cond, \
                   hyperattn_last_error());                             \
      ++failures;                                                       \
    }                                                                   \
  } while (0)

int main() {
  void* d = reinterpret_cast<void*>(uintptr_t(256));   // dummy device pointer, never used
  float* df = static_cast<float*>(d);
  // ---- workspace planning over many shapes ----
  const int ns[] = {0, 1, 2, 63, 64, 65, 100, 777, 1000, 1024, 4096, 4097, 131072};
  const int ss[] = {1, 7, 64, 100, 256, 4096};
  const int bs[] = {1, 24, 64, 96, 256, 512, 1 << 20};
  const int ms[] = {0, 1, 48, 256, 4096};
  size_t total = 0;
  for (int n : ns)
    for (int b : bs)
      for (int m : ms) {
        total += hyperattn_workspace_bytes(2, n, 64, 8, 2, b, m, 7, 0, 0, HA_BF16, 0);
        total += hyperattn_workspace_bytes(2, n, 128, 8, 2, b, m, 12, 0, 0, HA_F32, HA_FLAG_ROWNORM);
        total += hyperattn_workspace_bytes(1, n, 64, 4, 4, b, m, 7, 0, 0, HA_BF16, HA_FLAG_MATERIALIZE | HA_FLAG_UNFUSED);
        total += hyperattn_rect_workspace_bytes(1, n, 3 * n + 1, 64, 4, 2, b, m, 7, HA_BF16);
        for (int s : ss) {
          total += hyperattn_workspace_bytes(1, n, 64, 4, 2, b, m, 7, 1, s, HA_BF16, 0);
          total += hyperattn_backward_workspace_bytes(1, n, 64, 4, 2, b, m, 7, 1, s, HA_BF16);
          EXPECT(hyperattn_debug_levels(n, 1, s) >= 0);
        }
      }
  EXPECT(total > 0);
  EXPECT(hyperattn_workspace_bytes(1, 100, 96, 1, 1, 8, 0, 7, 0, 0, HA_BF16, 0) == 0);
  EXPECT(hyperattn_debug_levels(131072, 1, 4096) == 5 && hyperattn_debug_levels(5, 0, 0) == 1);
  EXPECT(hyperattn_sort_workspace_bytes(64, 131072, 1, 16) > 0);
  EXPECT(hyperattn_rownorm_samples_workspace_bytes(1, 32, 131072) > 0);

  // ---- host projections ----
  for (int dd : {1, 8, 64, 100, 128})
    for (int r = 1; r <= 16; r += 5) {
      std::vector<float> R(dd * r);
      EXPECT(hyperattn_projections_host(12345u, dd, r, R.data()) == HA_OK);
    }

  // ---- argument errors (nothing enqueued) ----
  EXPECT(hyperattn_forward(nullptr, nullptr, nullptr, HA_BF16, 1, 1024, 64, 4, 2, 64, 16, 7, 0, 0, 0, nullptr,
                           nullptr, nullptr, 0, nullptr) == HA_EINVAL);
  EXPECT(hyperattn_forward_ex(d, d, d, 9, 1, 1024, 64, 4, 2, 64, 16, 7, 0, 0, 0, 0, d, df, d, 1 << 30,
                              nullptr) == HA_EINVAL);
  EXPECT(hyperattn_forward_ex(d, d, d, HA_BF16, 1, 1024, 64, 4, 2, 64, 16, 7, 0, 0, 0, 0, d, df, d, 16,
                              nullptr) == HA_EWORKSPACE);
  EXPECT(hyperattn_forward_noalloc(d, d, d, HA_BF16, 1, 131072, 64, 32, 32, 256, 256, 7, 1, 4096, 0, d, df,
                                   nullptr) == HA_EWORKSPACE);
  EXPECT(hyperattn_forward_debug(d, d, d, HA_BF16, 1, 1024, 64, 4, 2, 64, 16, 7, 0, 0, 0, d, df, d, 1 << 30,
                                 nullptr, nullptr) == HA_EINVAL);
  EXPECT(hyperattn_sort(nullptr, 2, 100, 60, 50, 60, 1, 7, nullptr, nullptr, 0, nullptr) == HA_EINVAL);
  EXPECT(hyperattn_causal_leaves(nullptr, nullptr, nullptr, HA_BF16, 1, 100, 64, 1, 1, 30, nullptr, nullptr,
                                 nullptr) == HA_ESHAPE);
  EXPECT(hyperattn_attend(nullptr, nullptr, nullptr, HA_BF16, 1, 64, 64, 1, 1, 64, 4, nullptr, nullptr, nullptr,
                          4, nullptr, nullptr, nullptr) == HA_EINVAL);

  // ---- whole calls stopped before their first launch ----
  setenv("HYPERATTN_FAIL_AT", "proj", 1);
  struct Case { int n, b, m, causal, s, dtype, d; };
  const Case cases[] = {{1024, 64, 64, 0, 0, HA_F32, 64},   {131072, 256, 256, 0, 0, HA_BF16, 64},
                        {131072, 256, 256, 1, 4096, HA_BF16, 64}, {2048, 96, 48, 1, 256, HA_BF16, 128},
                        {1000, 64, 32, 1, 100, HA_BF16, 64}, {777, 128, 48, 1, 64, HA_F32, 128},
                        {1000, 40, 50, 0, 0, HA_BF16, 64},   {4096, 64, 0, 1, 4096, HA_BF16, 64}};
  std::vector<unsigned char> host_dump(1);
  for (const Case& c : cases) {
    EXPECT(hyperattn_forward(d, d, d, c.dtype, 1, c.n, c.d, 4, 2, c.b, c.m, 7, c.causal, c.s, 0, d, df, d,
                             size_t(1) << 40, nullptr) == HA_EHIP);
    EXPECT(std::strstr(hyperattn_last_error(), "injected failure before the proj launch") != nullptr);
    ha_debug_dump dump;
    std::memset(&dump, 0, sizeof(dump));
    dump.perm_q = static_cast<int32_t*>(d);
    EXPECT(hyperattn_forward_debug(d, d, d, c.dtype, 1, c.n, c.d, 4, 2, c.b, c.m, 7, c.causal, c.s, 0, d, df, d,
                                   size_t(1) << 40, nullptr, &dump) == HA_EHIP);
    if (c.dtype == HA_BF16)
      EXPECT(hyperattn_backward(d, d, d, d, df, d, HA_BF16, 1, c.n, c.d, 4, 2, c.b, c.m, 7, c.causal, c.s, 0, df,
                                df, df, d, size_t(1) << 40, nullptr) == HA_EHIP);
    if (!c.causal) {
      EXPECT(hyperattn_forward_ex(d, d, d, c.dtype, 1, c.n, c.d, 4, 2, c.b, c.m, 7, 0, 0, 0, HA_FLAG_ROWNORM, d,
                                  df, d, size_t(1) << 40, nullptr) == HA_EHIP);
      EXPECT(hyperattn_forward_rect(d, d, d, c.dtype, 1, c.n, 3 * c.n + 5, c.d, 4, 2, c.b, c.m, 7, 0, d, df, d,
                                    size_t(1) << 40, nullptr) == HA_EHIP);
    }
  }
  unsetenv("HYPERATTN_FAIL_AT");
  if (failures) {
    std::fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  std::printf("abi driver: all expectations held\n");
  return 0;
}
