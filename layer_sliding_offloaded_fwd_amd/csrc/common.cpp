// Error reporting, version string and the event-based kernel timer of libslide.
#include "common.h"

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <map>
#include <mutex>
#include <string>
#include <vector>

namespace slide {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SLIDE_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return SLIDE_OK;
}

// ---------------------------------------------------------------- profiler
namespace {
struct Pending {
  std::string name;
  hipEvent_t start, stop;
};
struct Stat {
  int64_t count = 0;
  double ms = 0;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<hipEvent_t> g_event_pool;
std::vector<Pending> g_pending;          // index = ProfScope::slot
std::map<std::string, Stat> g_stats;

hipEvent_t pool_get() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void drain_locked() {
  for (auto& p : g_pending) {
    if (!p.start || !p.stop) continue;
    hipEventSynchronize(p.stop);
    float ms = 0;
    if (hipEventElapsedTime(&ms, p.start, p.stop) == hipSuccess) {
      Stat& s = g_stats[p.name];
      s.count += 1;
      s.ms += ms;
    }
    g_event_pool.push_back(p.start);
    g_event_pool.push_back(p.stop);
  }
  g_pending.clear();
}
}  // namespace

ProfScope::ProfScope(const char* name, hipStream_t s) : stream(s) {
  if (!g_prof_on) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (g_pending.size() > 20000) drain_locked();
  Pending p{name, pool_get(), pool_get()};
  if (!p.start || !p.stop) return;
  hipEventRecord(p.start, stream);
  slot = (int)g_pending.size();
  g_pending.push_back(p);
}

ProfScope::~ProfScope() {
  if (slot < 0) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (slot < (int)g_pending.size()) hipEventRecord(g_pending[slot].stop, stream);
}

}  // namespace slide

using namespace slide;

extern "C" const char* slide_last_error(void) { return g_err; }
extern "C" const char* slide_version(void) { return "libslide 0.1 (gfx950)"; }

extern "C" int slide_prof_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = on != 0;
  return SLIDE_OK;
}

extern "C" int slide_prof_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  drain_locked();
  g_stats.clear();
  return SLIDE_OK;
}

extern "C" int slide_prof_read(char (*names)[64], int64_t* counts, double* total_ms,
                               int max_entries, int* n_out) {
  if (!names || !counts || !total_ms || !n_out || max_entries < 0)
    return fail(SLIDE_E_ARG, "slide_prof_read: null argument");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  drain_locked();
  int n = 0;
  for (auto& kv : g_stats) {
    if (n >= max_entries) break;
    snprintf(names[n], 64, "%s", kv.first.c_str());
    counts[n] = kv.second.count;
    total_ms[n] = kv.second.ms;
    ++n;
  }
  *n_out = n;
  return SLIDE_OK;
}
