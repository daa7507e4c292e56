// Launch profiling: while enabled, every kernel the library launches carries
// two HIP events attached to its dispatch (start and end of its execution on
// the launch stream), so a caller can read per-kernel GPU durations of the
// launches it made (moe_profile_* in include/moe.h). Process-global and not thread-safe by design: it is a
// measurement aid, off unless a caller turns it on.
#include <string.h>

#include <string>
#include <vector>

#include "../../include/moe.h"
#include "common.h"

namespace moe {
namespace {

struct Rec {
  const char* name;
  hipEvent_t a, b;
};

struct Summary {
  std::string name;
  int launches;
  double ms;
};

std::vector<hipEvent_t> g_pool;
std::vector<Rec> g_recs;
std::vector<Summary> g_sum;
size_t g_used = 0;
bool g_on = false;
bool g_open = false;
Rec g_cur;

}  // namespace

bool prof_open(const char* name, hipEvent_t* start, hipEvent_t* stop) {
  g_open = false;
  if (!g_on || g_used + 2 > g_pool.size()) return false;
  g_cur.name = name;
  g_cur.a = g_pool[g_used];
  g_cur.b = g_pool[g_used + 1];
  *start = g_cur.a;
  *stop = g_cur.b;
  g_open = true;
  return true;
}

void prof_close() {
  if (!g_open) return;
  g_open = false;
  g_used += 2;
  g_recs.push_back(g_cur);
}

}  // namespace moe

extern "C" {

int moe_profile_begin(int32_t max_launches) {
  using namespace moe;
  if (max_launches < 1) return MOE_ERR_INVALID_ARG;
  while (g_pool.size() < (size_t)2 * max_launches) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return MOE_ERR_HIP;
    g_pool.push_back(e);
  }
  g_recs.clear();
  g_sum.clear();
  g_used = 0;
  g_on = true;
  return MOE_OK;
}

int moe_profile_end(void) {
  using namespace moe;
  g_on = false;
  g_sum.clear();
  for (const Rec& r : g_recs) {
    if (hipEventSynchronize(r.b) != hipSuccess) return MOE_ERR_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return MOE_ERR_HIP;
    size_t i = 0;
    while (i < g_sum.size() && g_sum[i].name != r.name) ++i;
    if (i == g_sum.size()) g_sum.push_back(Summary{r.name, 0, 0.0});
    g_sum[i].launches += 1;
    g_sum[i].ms += ms;
  }
  g_recs.clear();
  return MOE_OK;
}

int32_t moe_profile_count(void) { return (int32_t)moe::g_sum.size(); }


int moe_profile_get(int32_t i, const char** name, int32_t* launches, double* total_ms) {
  using namespace moe;
  if (i < 0 || (size_t)i >= g_sum.size() || !name || !launches || !total_ms) return MOE_ERR_INVALID_ARG;
  *name = g_sum[i].name.c_str();
  *launches = g_sum[i].launches;
  *total_ms = g_sum[i].ms;
  return MOE_OK;
}

}  // extern "C"
