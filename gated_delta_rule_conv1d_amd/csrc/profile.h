// Opt-in per-kernel timing: when enabled, every kernel launch of the library
// is bracketed by hipEventRecord on the launch stream.  Off by default; the
// hooks then cost one relaxed atomic load per launch.  Safe to use from
// several host threads: the records are guarded by a mutex.
#pragma once

#include <hip/hip_runtime.h>

namespace gdn {

size_t prof_begin(const char* name, hipStream_t st);
void prof_end(size_t rec, hipStream_t st);

struct ProfScope {
  hipStream_t st;
  bool on;
  size_t rec;
  ProfScope(const char* name, hipStream_t s);
  ~ProfScope();
};

}  // namespace gdn

// use inside its own block: { GDN_PROF("kernel", st); kernel<<<...>>>(...); }
#define GDN_PROF(name, stream) ::gdn::ProfScope gdn_prof_scope_(name, stream)
