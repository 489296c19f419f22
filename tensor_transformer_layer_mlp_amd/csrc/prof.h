// Optional per-launch timing with HIP events (used by benchmarks; off by default).
#pragma once

#include <hip/hip_runtime.h>

namespace tp {

bool prof_enabled();

// Names the call site of the launches that follow on this thread (e.g. "fc1") until it goes out of
// scope; the launches' records then carry "site|tag" instead of the bare kernel tag.
class ProfSite {
 public:
  explicit ProfSite(const char* site);
  ~ProfSite();
  ProfSite(const ProfSite&) = delete;
  ProfSite& operator=(const ProfSite&) = delete;

 private:
  const char* prev_;
};

// Brackets one kernel launch: records an event on `s` now and another when the scope ends.
// `tag` names the kernel instantiation; flop/bytes are the launch's algorithmic work.
class ProfScope {
 public:
  ProfScope(const char* tag, hipStream_t s, double flop, double bytes);
  ~ProfScope();
  ProfScope(const ProfScope&) = delete;
  ProfScope& operator=(const ProfScope&) = delete;

 private:
  int slot_;
  hipStream_t s_;
};

}  // namespace tp
