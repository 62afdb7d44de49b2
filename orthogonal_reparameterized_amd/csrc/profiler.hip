// Optional launch profiler: while enabled, every kernel launch of the library is bracketed by a HIP event pair
// recorded on the launch's own stream, tagged with its kernel class and its algorithmic flops and bytes.
#include <mutex>
#include <vector>

#include "../../include/poet.h"
#include "internal.h"

namespace poet {
namespace {

struct Rec {
  int kclass;
  hipEvent_t a, b;
  double flops, bytes;
};

std::mutex g_mu;
bool g_on = false;
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t get_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

int prof_begin(int kclass, hipStream_t st, double flops, double bytes) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on) return -1;
  Rec r{kclass, get_event(), get_event(), flops, bytes};
  if (!r.a || !r.b || hipEventRecord(r.a, st) != hipSuccess) return -1;
  g_recs.push_back(r);
  return (int)g_recs.size() - 1;
}

void prof_end(int rec, hipStream_t st) {
  if (rec < 0) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (rec < (int)g_recs.size()) (void)hipEventRecord(g_recs[rec].b, st);
}

}  // namespace poet

using namespace poet;

extern "C" {

void poet_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (on) {
    for (auto& r : g_recs) {
      g_pool.push_back(r.a);
      g_pool.push_back(r.b);
    }
    g_recs.clear();
  }
  g_on = on != 0;
}

poet_status poet_profile_query(int kclass, int64_t* launches, double* total_ms, double* flops, double* bytes) {
  if (kclass < 0 || kclass >= POET_K_NCLASS) return POET_E_ARG;
  std::lock_guard<std::mutex> lk(g_mu);
  int64_t n = 0;
  double ms = 0, fl = 0, by = 0;
  for (auto& r : g_recs) {
    if (r.kclass != kclass) continue;
    if (hipEventSynchronize(r.b) != hipSuccess) return POET_E_HIP;
    float t = 0.f;
    if (hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) return POET_E_HIP;
    ++n;
    ms += t;
    fl += r.flops;
    by += r.bytes;
  }
  if (launches) *launches = n;
  if (total_ms) *total_ms = ms;
  if (flops) *flops = fl;
  if (bytes) *bytes = by;
  return POET_OK;
}

}  // extern "C"
