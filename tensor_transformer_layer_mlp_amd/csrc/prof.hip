// Per-launch HIP-event timing of the library's kernels, for benchmarks.  Off unless enabled.
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "prof.h"
#include "tpshard.h"

namespace tp {

namespace {

struct Rec {
  std::string tag;
  hipEvent_t a = nullptr, b = nullptr;
  double flop = 0, bytes = 0;
};

std::mutex g_mu;
bool g_on = false;
std::vector<Rec> g_recs;   // events are reused from one collection to the next
size_t g_used = 0;

}  // namespace

thread_local const char* g_site = nullptr;

bool prof_enabled() { return g_on; }

ProfSite::ProfSite(const char* site) : prev_(g_site) { g_site = site; }
ProfSite::~ProfSite() { g_site = prev_; }

ProfScope::ProfScope(const char* tag, hipStream_t s, double flop, double bytes) : slot_(-1), s_(s) {
  if (!g_on) return;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_used == g_recs.size()) {
    Rec r;
    if (hipEventCreate(&r.a) != hipSuccess || hipEventCreate(&r.b) != hipSuccess) return;
    g_recs.push_back(r);
  }
  Rec& r = g_recs[g_used];
  r.tag = g_site ? std::string(g_site) + "|" + tag : std::string(tag);
  r.flop = flop;
  r.bytes = bytes;
  if (hipEventRecord(r.a, s) != hipSuccess) return;
  slot_ = (int)g_used++;
}

ProfScope::~ProfScope() {
  if (slot_ < 0) return;
  std::lock_guard<std::mutex> lock(g_mu);
  (void)hipEventRecord(g_recs[slot_].b, s_);
}

}  // namespace tp

extern "C" {

int tp_prof_enable(int enable) {
  std::lock_guard<std::mutex> lock(tp::g_mu);
  tp::g_on = enable != 0;
  return TP_OK;
}

int tp_prof_collect(int max_entries, char* names, int name_len, int* launches, double* total_ms,
                    double* total_flop, double* total_bytes) {
  using namespace tp;
  std::lock_guard<std::mutex> lock(g_mu);
  if (max_entries < 0 || (max_entries > 0 && (!names || name_len < 2 || !launches || !total_ms ||
                                               !total_flop || !total_bytes)))
    return TP_EINVAL;
  std::vector<std::string> tags;
  std::vector<int> cnt;
  std::vector<double> ms, fl, by;
  int status = TP_OK;
  for (size_t i = 0; i < g_used; ++i) {
    Rec& r = g_recs[i];
    float t = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess)
      status = TP_EHIP;
    size_t k = 0;
    while (k < tags.size() && tags[k] != r.tag) ++k;
    if (k == tags.size()) {
      tags.push_back(r.tag);
      cnt.push_back(0);
      ms.push_back(0);
      fl.push_back(0);
      by.push_back(0);
    }
    cnt[k] += 1;
    ms[k] += t;
    fl[k] += r.flop;
    by[k] += r.bytes;
  }
  g_used = 0;
  if (status != TP_OK) return status;
  for (size_t k = 0; k < tags.size() && (int)k < max_entries; ++k) {
    strncpy(names + k * name_len, tags[k].c_str(), name_len - 1);
    names[k * name_len + name_len - 1] = '\0';
    launches[k] = cnt[k];
    total_ms[k] = ms[k];
    total_flop[k] = fl[k];
    total_bytes[k] = by[k];
  }
  return (int)tags.size();
}

}  // extern "C"
