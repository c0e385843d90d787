// Opt-in per-kernel timing with HIP events. When enabled, every kernel launch
// of the library is bracketed by a pair of events recorded on the launch
// stream; dsa_mla_trace_collect waits for them and reports, per kernel name,
// the number of launches and the summed event time.
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/dsa_mla.h"
#include "kernels.h"

namespace dsa {
namespace {
struct Rec {
  const char* name;
  hipEvent_t a, b;
};
std::mutex g_mu;
bool g_on = false;
std::vector<Rec> g_recs;
}  // namespace

KernelTrace::KernelTrace(const char* name, hipStream_t s) : name_(name), stream_(s), a_(nullptr) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on) return;
  hipEvent_t a;
  if (hipEventCreate(&a) != hipSuccess) return;
  if (hipEventRecord(a, s) != hipSuccess) {
    (void)hipEventDestroy(a);
    return;
  }
  a_ = a;
}

KernelTrace::~KernelTrace() {
  if (a_ == nullptr) return;
  hipEvent_t b;
  if (hipEventCreate(&b) != hipSuccess || hipEventRecord(b, stream_) != hipSuccess) {
    (void)hipEventDestroy((hipEvent_t)a_);
    return;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  g_recs.push_back(Rec{name_, (hipEvent_t)a_, b});
}

}  // namespace dsa

extern "C" {

int dsa_mla_trace_enable(int on) {
  std::lock_guard<std::mutex> lk(dsa::g_mu);
  const int prev = dsa::g_on ? 1 : 0;
  dsa::g_on = on != 0;
  return prev;
}

int dsa_mla_trace_collect(int max_kernels, char* names, int* counts, double* total_ms) {
  std::vector<dsa::Rec> recs;
  {
    std::lock_guard<std::mutex> lk(dsa::g_mu);
    recs.swap(dsa::g_recs);
  }
  std::vector<std::string> nm;
  std::vector<int> cnt;
  std::vector<double> tot;
  for (auto& r : recs) {
    float ms = 0.f;
    const bool ok = hipEventSynchronize(r.b) == hipSuccess && hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess;
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
    if (!ok) continue;
    size_t j = 0;
    while (j < nm.size() && nm[j] != r.name) ++j;
    if (j == nm.size()) {
      nm.emplace_back(r.name);
      cnt.push_back(0);
      tot.push_back(0.0);
    }
    cnt[j] += 1;
    tot[j] += ms;
  }
  const int n = (int)nm.size();
  for (int j = 0; j < n && j < max_kernels; ++j) {
    if (names) {
      std::strncpy(names + 32 * j, nm[j].c_str(), 31);
      names[32 * j + 31] = '\0';
    }
    if (counts) counts[j] = cnt[j];
    if (total_ms) total_ms[j] = tot[j];
  }
  return n;
}

}  // extern "C"
