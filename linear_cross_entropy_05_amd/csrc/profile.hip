// Optional per-kernel timing with HIP events (see flce_profile_begin in
// flce.h).  Off by default; when on, every launch the library makes is
// bracketed by two event records on the launch's own stream.
#include <vector>

#include "../../include/flce.h"
#include "flce_internal.h"

namespace flce {

namespace {
struct ProfState {
  bool on = false;
  std::vector<hipEvent_t> ev;
  std::vector<int> phase;  // phase of launch i: events 2 i, 2 i + 1
  size_t next = 0;
};
ProfState g_prof;
}  // namespace

ProfScope::ProfScope(int phase, hipStream_t s) : idx_(-1), s_(s) {
  if (!g_prof.on || 2 * g_prof.next + 1 >= g_prof.ev.size()) return;
  idx_ = (long)g_prof.next++;
  g_prof.phase[idx_] = phase;
  (void)hipEventRecord(g_prof.ev[2 * idx_], s_);
}

ProfScope::~ProfScope() {
  if (idx_ >= 0) (void)hipEventRecord(g_prof.ev[2 * idx_ + 1], s_);
}

}  // namespace flce

extern "C" {

int flce_profile_begin(int max_launches) {
  using flce::g_prof;
  if (g_prof.on || max_launches <= 0) return FLCE_ERR_ARG;
  g_prof.ev.assign(2 * (size_t)max_launches, nullptr);
  g_prof.phase.assign((size_t)max_launches, -1);
  for (auto& e : g_prof.ev)
    if (hipEventCreate(&e) != hipSuccess) return FLCE_ERR_LAUNCH;
  g_prof.next = 0;
  g_prof.on = true;
  return FLCE_OK;
}

int flce_profile_end(double* total_ms, int64_t* launches, int n) {
  using flce::g_prof;
  if (!g_prof.on) return FLCE_ERR_ARG;
  g_prof.on = false;
  for (int p = 0; p < n; ++p) {
    if (total_ms) total_ms[p] = 0.0;
    if (launches) launches[p] = 0;
  }
  int st = FLCE_OK;
  for (size_t i = 0; i < g_prof.next; ++i) {
    float ms = 0.f;
    if (hipEventSynchronize(g_prof.ev[2 * i + 1]) != hipSuccess ||
        hipEventElapsedTime(&ms, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]) != hipSuccess) {
      st = FLCE_ERR_LAUNCH;
      continue;
    }
    const int p = g_prof.phase[i];
    if (p >= 0 && p < n) {
      if (total_ms) total_ms[p] += ms;
      if (launches) launches[p] += 1;
    }
  }
  for (auto e : g_prof.ev) (void)hipEventDestroy(e);
  g_prof.ev.clear();
  g_prof.phase.clear();
  g_prof.next = 0;
  return st;
}

}  // extern "C"
