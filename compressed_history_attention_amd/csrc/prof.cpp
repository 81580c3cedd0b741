// Per-stage HIP-event timing of the tuned path (profiling aid).
#include <string.h>

#include <atomic>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "prof.hpp"

namespace nkv {

namespace {
struct Rec {
  const char* name;
  hipEvent_t a, b;
};
// Events of enabled scopes from any host thread; the mutex covers the
// record list and the pool of reusable events.
std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Rec> g_pending;
std::vector<hipEvent_t> g_pool;

hipEvent_t get_event() {
  std::lock_guard<std::mutex> lock(g_mu);
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

bool prof_on() { return g_on; }

ProfScope::ProfScope(const char* name, hipStream_t s) : name_(name), s_(s), a_(nullptr) {
  if (!g_on) return;
  a_ = get_event();
  if (a_) (void)hipEventRecord(a_, s_);
}

ProfScope::~ProfScope() {
  if (!a_) return;
  hipEvent_t b = get_event();
  if (!b) return;
  (void)hipEventRecord(b, s_);
  std::lock_guard<std::mutex> lock(g_mu);
  g_pending.push_back(Rec{name_, a_, b});
}

}  // namespace nkv

using namespace nkv;

extern "C" {

void nkv_profile_enable(int on) { g_on = on != 0; }

int nkv_profile_read(nkv_prof_entry* out, int32_t max_entries) {
  std::lock_guard<std::mutex> lock(g_mu);
  std::map<std::string, std::pair<double, int>> acc;
  std::vector<std::string> order;
  int rc = 0;
  for (auto& r : g_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
      rc = -1;
    if (!acc.count(r.name)) order.push_back(r.name);
    auto& e = acc[r.name];
    e.first += ms;
    e.second += 1;
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_pending.clear();
  if (rc) return rc;
  int n = 0;
  for (auto& name : order) {
    if (n >= max_entries) break;
    memset(out[n].name, 0, sizeof(out[n].name));
    strncpy(out[n].name, name.c_str(), sizeof(out[n].name) - 1);
    out[n].ms = acc[name].first;
    out[n].count = acc[name].second;
    ++n;
  }
  return n;
}

}  // extern "C"
