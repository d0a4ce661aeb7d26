// Per-launch timing of the library's kernels with HIP events (the profiling
// pass of the RoundPipe paper, section 4.4, times layers with device events;
// here the same mechanism times every kernel launch so that a benchmark can
// price each kernel against its roofline while the real workload runs).
#pragma once

#include <string>
#include <vector>

#include "common.h"

namespace rp {

struct TraceRec {
  std::string name;
  double flops, bytes;
  hipEvent_t a, b;
};

struct Trace {
  bool on = false;
  size_t cap = 0;
  std::vector<TraceRec> recs;
  std::vector<hipEvent_t> pool;  // events owned by the trace, reused across sessions
  size_t pool_used = 0;
  ~Trace();
  hipEvent_t take();
};

// the trace of the context the calling thread entered last (nullptr: off)
void trace_bind(Trace* t);
Trace* trace_current();

// Records an event on `s` now and another when the scope ends; the pair is
// one launch of kernel `name` with the given algorithmic work.
class TraceScope {
 public:
  TraceScope(hipStream_t s, const char* name, double flops, double bytes);
  TraceScope(hipStream_t s, const std::string& name, double flops, double bytes)
      : TraceScope(s, name.c_str(), flops, bytes) {}
  ~TraceScope();
  TraceScope(const TraceScope&) = delete;
  TraceScope& operator=(const TraceScope&) = delete;

 private:
  Trace* t_ = nullptr;
  hipStream_t s_ = nullptr;
  size_t idx_ = 0;
};

}  // namespace rp
