// Per-kernel HIP-event timing hook (diagnostics).  The events are created once
// and reused; reading the totals synchronises on them.  One mutex guards the
// records and the event pool, and each launch scope remembers its own record,
// so launches from several host threads each time their own kernel.
#include <atomic>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "gdn_internal.h"
#include "profile.h"

namespace gdn {
namespace {

struct Rec {
  const char* name;
  hipEvent_t a, b;
};

std::atomic<int> g_on{0};
std::mutex g_mu;                 // guards g_recs and g_pool
std::vector<Rec> g_recs;         // records of the current window
std::vector<hipEvent_t> g_pool;  // events available for reuse

hipEvent_t take() {
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

size_t prof_begin(const char* name, hipStream_t st) {
  std::lock_guard<std::mutex> lock(g_mu);
  Rec r{name, take(), take()};
  if (r.a) (void)hipEventRecord(r.a, st);
  g_recs.push_back(r);
  return g_recs.size() - 1;
}

void prof_end(size_t rec, hipStream_t st) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (rec < g_recs.size() && g_recs[rec].b) (void)hipEventRecord(g_recs[rec].b, st);
}

ProfScope::ProfScope(const char* name, hipStream_t s)
    : st(s), on(g_on.load(std::memory_order_relaxed) != 0), rec((size_t)-1) {
  if (on) rec = prof_begin(name, st);
}
ProfScope::~ProfScope() {
  if (on) prof_end(rec, st);
}

}  // namespace gdn

using namespace gdn;

extern "C" {

// Start (1) or stop (0) recording; starting clears earlier records.
void gdn_profile_enable(int on) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (on) {
    for (auto& r : g_recs) {
      if (r.a) g_pool.push_back(r.a);
      if (r.b) g_pool.push_back(r.b);
    }
    g_recs.clear();
  }
  g_on.store(on ? 1 : 0);
}

// Write "name count total_ms\n" lines (one per kernel name, first-seen order)
// into buf; waits for the recorded events.  Returns the number of bytes
// needed (excluding the terminating zero).
size_t gdn_profile_report(char* buf, size_t cap) {
  std::lock_guard<std::mutex> lock(g_mu);
  std::vector<std::string> names;
  std::vector<double> tot;
  std::vector<long> cnt;
  for (auto& r : g_recs) {
    if (!r.a || !r.b) continue;
    if (hipEventSynchronize(r.b) != hipSuccess) continue;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) continue;
    size_t i = 0;
    for (; i < names.size(); ++i)
      if (names[i] == r.name) break;
    if (i == names.size()) {
      names.emplace_back(r.name);
      tot.push_back(0.0);
      cnt.push_back(0);
    }
    tot[i] += ms;
    cnt[i] += 1;
  }
  std::string out;
  char line[256];
  for (size_t i = 0; i < names.size(); ++i) {
    snprintf(line, sizeof line, "%s %ld %.6f\n", names[i].c_str(), cnt[i], tot[i]);
    out += line;
  }
  if (buf && cap) {
    const size_t n = out.size() < cap - 1 ? out.size() : cap - 1;
    memcpy(buf, out.data(), n);
    buf[n] = 0;
  }
  return out.size();
}

}  // extern "C"
