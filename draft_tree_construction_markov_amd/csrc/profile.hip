// profile.hip -- optional per-kernel timing with HIP events.  When enabled,
// every launch of the library is bracketed by two events recorded on the
// launch stream, tagged with the kernel kind and its work units (e.g. the
// number of parents of a fused Markov launch).  Off by default; the event
// pool is created once, when profiling is first enabled.
#include <mutex>
#include <vector>

#include "../../include/pctree.h"
#include "pct_internal.h"

namespace pct {

namespace {
struct Rec {
  int kind;
  int64_t units;
  int ev;  // index of the start event; stop is ev + 1
};
std::mutex g_mu;
bool g_on = false;
std::vector<hipEvent_t> g_pool;
std::vector<Rec> g_recs;
int g_next = 0;
constexpr int kPoolEvents = 16384;
}  // namespace

ProfScope::ProfScope(int kind, int64_t units, hipStream_t s)
    : stream_(s), idx_(-1) {
  if (!g_on) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_next + 2 > (int)g_pool.size()) return;
  idx_ = g_next;
  g_next += 2;
  g_recs.push_back(Rec{kind, units, idx_});
  (void)hipEventRecord(g_pool[idx_], s);
}

ProfScope::~ProfScope() {
  if (idx_ < 0) return;
  (void)hipEventRecord(g_pool[idx_ + 1], stream_);
}

}  // namespace pct

using namespace pct;

extern "C" {

pct_status pct_profile_enable(int32_t enable) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (enable && g_pool.empty()) {
    g_pool.resize(kPoolEvents);
    for (auto& e : g_pool) {
      if (hipEventCreate(&e) != hipSuccess) {
        (void)hipGetLastError();
        g_pool.clear();
        return PCT_ERR_HIP;
      }
    }
  }
  g_on = enable != 0;
  return PCT_OK;
}

pct_status pct_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_recs.clear();
  g_next = 0;
  return PCT_OK;
}

pct_status pct_profile_read(int32_t kind, int64_t units, double* total_ms,
                            int64_t* launches) {
  if (!total_ms || !launches) return PCT_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(g_mu);
  double tot = 0.0;
  int64_t n = 0;
  for (const Rec& r : g_recs) {
    if (r.kind != kind || (units >= 0 && r.units != units)) continue;
    if (hipEventSynchronize(g_pool[r.ev + 1]) != hipSuccess) {
      (void)hipGetLastError();
      return PCT_ERR_HIP;
    }
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, g_pool[r.ev], g_pool[r.ev + 1]) !=
        hipSuccess) {
      (void)hipGetLastError();
      return PCT_ERR_HIP;
    }
    tot += ms;
    ++n;
  }
  *total_ms = tot;
  *launches = n;
  return PCT_OK;
}

}  // extern "C"
