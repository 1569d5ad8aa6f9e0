// Kernel timing: while enabled, each launch of the library (or of one kernel
// class only) is bracketed by two HIP events on its stream and recorded with
// its algorithmic work (model FLOPs and the minimum bytes the kernel must
// move). Disabled, a scope costs one relaxed load of a flag.
#include <atomic>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"
#include "kernels.h"

namespace nc {
namespace {

struct Rec {
  const char* name;
  double flops, bytes;
  int ev;  // index of the event pair
};

struct Prof {
  std::atomic<bool> on{false};
  std::mutex mu;
  std::vector<Rec> recs;
  std::vector<hipEvent_t> events;  // 2 per record, reused across enables
  std::string only;                // record only this kernel class (empty: all)
};

Prof& prof() {
  static Prof p;
  return p;
}

}  // namespace

ProfScope::ProfScope(const char* name, double flops, double bytes, hipStream_t st) : slot_(-1), st_(st) {
  Prof& p = prof();
  if (!p.on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> g(p.mu);
  if (!p.only.empty() && p.only != name) return;
  int i = (int)p.recs.size();
  while ((int)p.events.size() < 2 * (i + 1)) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return;
    p.events.push_back(e);
  }
  if (hipEventRecord(p.events[2 * i], st) != hipSuccess) return;
  p.recs.push_back(Rec{name, flops, bytes, i});
  slot_ = i;
}

ProfScope::~ProfScope() {
  if (slot_ < 0) return;
  Prof& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  (void)hipEventRecord(p.events[2 * slot_ + 1], st_);
}

}  // namespace nc

using namespace nc;

extern "C" {

nc_status nc_profile_enable(int on) {
  Prof& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  if (on) p.recs.clear();
  p.on.store(on != 0);
  return NC_OK;
}

nc_status nc_profile_only(const char* kernel_class) {
  Prof& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  p.only = kernel_class ? kernel_class : "";
  return NC_OK;
}

nc_status nc_profile_summary(char* buf, size_t len, size_t* written) {
  if (!written) return NC_ERR_INVALID_ARG;
  Prof& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  struct Agg {
    int n = 0;
    double ms = 0, flops = 0, bytes = 0;
  };
  std::map<std::string, Agg> agg;
  for (const Rec& r : p.recs) {
    hipEvent_t a = p.events[2 * r.ev], b = p.events[2 * r.ev + 1];
    hipError_t e = hipEventSynchronize(b);
    if (e != hipSuccess) return record_hip_error(e, "nc_profile_summary sync");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, a, b);
    if (e != hipSuccess) return record_hip_error(e, "nc_profile_summary elapsed");
    Agg& x = agg[r.name];
    x.n += 1;
    x.ms += ms;
    x.flops += r.flops;
    x.bytes += r.bytes;
  }
  std::string s = "{";
  bool first = true;
  char tmp[512];
  for (auto& kv : agg) {
    snprintf(tmp, sizeof(tmp), "%s\"%s\": {\"launches\": %d, \"ms\": %.6f, \"flops\": %.6e, \"bytes\": %.6e}",
             first ? "" : ", ", kv.first.c_str(), kv.second.n, kv.second.ms, kv.second.flops, kv.second.bytes);
    s += tmp;
    first = false;
  }
  s += "}";
  *written = s.size() + 1;
  if (!buf || len < s.size() + 1) return NC_ERR_INVALID_ARG;
  std::memcpy(buf, s.c_str(), s.size() + 1);
  return NC_OK;
}

}  // extern "C"
