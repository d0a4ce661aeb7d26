// Kernel-launch trace: event pairs around launches, read back after the
// stream has passed them.
#include "trace.h"

namespace rp {

namespace {
thread_local Trace* g_trace = nullptr;
}

void trace_bind(Trace* t) { g_trace = t; }
Trace* trace_current() { return g_trace; }

Trace::~Trace() {
  for (hipEvent_t e : pool) (void)hipEventDestroy(e);
}

hipEvent_t Trace::take() {
  if (pool_used == pool.size()) {
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    pool.push_back(e);
  }
  return pool[pool_used++];
}

TraceScope::TraceScope(hipStream_t s, const char* name, double flops, double bytes) {
  Trace* t = g_trace;
  if (!t || !t->on || t->recs.size() >= t->cap) return;
  hipEvent_t a = t->take(), b = t->take();
  if (!a || !b) return;
  if (hipEventRecord(a, s) != hipSuccess) return;
  t_ = t;
  s_ = s;
  idx_ = t->recs.size();
  t->recs.push_back(TraceRec{name, flops, bytes, a, b});
}

TraceScope::~TraceScope() {
  if (t_) (void)hipEventRecord(t_->recs[idx_].b, s_);
}

}  // namespace rp
