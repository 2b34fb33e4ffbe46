// Optional event timing of moe_forward's phases (benchmarks only).  When
// enabled, a HIP event is recorded on the call's stream at every phase
// boundary; reading the marks waits for them and reports the time between
// consecutive marks.  Disabled by default: a single branch per boundary.
#include <mutex>
#include <string.h>
#include <vector>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {
struct Mark {
  const char* name;
  hipEvent_t ev;
  int first;   // first mark of a call
};
std::mutex g_mu;
std::vector<hipEvent_t> g_pool;
std::vector<Mark> g_marks;
bool g_on = false;
}  // namespace

void timing_mark(const char* name, hipStream_t s, int first) {
  if (!g_on) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_marks.size() >= g_pool.size()) return;   // pool exhausted: drop the mark
  hipEvent_t e = g_pool[g_marks.size()];
  if (hipEventRecord(e, s) == hipSuccess) g_marks.push_back({name, e, first});
}

}  // namespace moe

using namespace moe;

extern "C" int moe_timing_enable(int n) {
  std::lock_guard<std::mutex> lk(g_mu);
  for (hipEvent_t e : g_pool) hipEventDestroy(e);
  g_pool.clear();
  g_marks.clear();
  g_on = n > 0;
  for (int i = 0; i < n; ++i) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) {
      g_on = false;
      return MOE_EHIP;
    }
    g_pool.push_back(e);
  }
  return MOE_OK;
}

extern "C" int moe_timing_read(char* names, int name_len, float* ms, int max) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!names || !ms || name_len < 2 || max < 0) return MOE_EINVAL;
  const int m = (int)g_marks.size() < max ? (int)g_marks.size() : max;
  for (int i = 0; i < m; ++i) {
    strncpy(names + (size_t)i * name_len, g_marks[i].name, name_len - 1);
    names[(size_t)i * name_len + name_len - 1] = 0;
    ms[i] = -1.f;
    if (hipEventSynchronize(g_marks[i].ev) != hipSuccess) return MOE_EHIP;
    if (i > 0 && !g_marks[i].first) {
      float t = 0.f;
      if (hipEventElapsedTime(&t, g_marks[i - 1].ev, g_marks[i].ev) != hipSuccess) return MOE_EHIP;
      ms[i] = t;
    }
  }
  g_marks.clear();
  return m;
}
