// The optimizer side of a RoundPipe worker ("Efficient Training on Multiple
// Consumer GPUs with RoundPipe", section 2.1.2 "Weight and Optimizer
// Offloading", section 4.3 "Fine-Grained Model Consistency"). Host code.
//
// Three copies of the trainable weights exist (section 4.3.1): the GPU's
// transient copy, a low-precision master copy in host memory that the GPU
// uploads from (and whose gradient buffer it downloads into), and the fp32
// optimizer copy with the Adam moments. The optimizer worker is one host
// thread that runs the queued steps in order (rule 5). Per layer, step t:
//   wait until the GPU has downloaded g_t into the master gradient buffer
//   (rule 3), G-cp: copy it into the optimizer copy, release the buffer for
//   the GPU's next download (rule 4); Adam on the fp32 copy; wait until the
//   GPU has uploaded layer l for iteration t + 1, which reads the weights of
//   step t - 1 (rule 1); P-cp: round the fp32 weights into the master copy
//   and release it for the GPU's upload of iteration t + 2 (rule 2).
// Each wait and release is per layer (section 4.3.2), so the first layers are
// ready for the next iteration while deeper layers are still being updated.
// Iteration t + 1 therefore trains on the weights produced after iteration
// t - 1: staleness-1 asynchronous updates (section 2.1.2).
//
// Adam (Kingma and Ba), with decoupled weight decay when weight_decay > 0:
//   g = grad_scale * G;  m = b1 m + (1 - b1) g;  v = b2 v + (1 - b2) g^2;
//   w -= lr * ((m / (1 - b1^s)) / (sqrt(v / (1 - b2^s)) + eps) + wd * w)
// with s the 1-based step count, every operation a single fp32 rounding in
// that order (no fused multiply-adds), the bias corrections formed in double.
#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <condition_variable>
#include <cstdio>
#include <cstring>
#include <deque>
#include <mutex>
#include <thread>
#include <vector>

#include "ops.h"

#pragma clang fp contract(off)

namespace {

struct Seg {
  void* master_w;          // bf16 or fp32 master weights (host)
  const float* master_g;   // fp32 master gradients (host)
  size_t n;
  size_t off;              // first element in the layer's optimizer arrays
};

struct LayerState {
  std::vector<Seg> segs;
  std::vector<float> w, m, v, g;  // optimizer copy
  int64_t steps = 0;              // Adam steps applied to this layer
  bool bound = false;
};

struct Job {
  int64_t iteration;
  rp_opt_hparams hp;
};

inline uint16_t bf16_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

inline float bf16_to_f(uint16_t h) {
  const uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

}  // namespace

struct rp_opt {
  int n_layers = 0;
  int dtype = RP_DTYPE_BF16;
  int n_threads = 1;
  std::vector<LayerState> layers;
  // protocol edges: largest iteration signalled per (edge, layer), -1 = none
  std::vector<int64_t> edge[4];
  std::mutex mu;
  std::condition_variable cv;
  std::deque<Job> queue;
  int64_t done_steps = 0, queued_steps = 0;
  bool stop = false;
  rp_status worker_status = RP_OK;
  char worker_error[256] = {0};
  std::thread worker;
  int64_t edge_timeout_ms = 0;  // 0: wait without limit

  void run();
  rp_status process(const Job& j);
  bool wait_edge(int e, int layer, int64_t it);
  void signal(int e, int layer, int64_t it) {
    {
      std::lock_guard<std::mutex> lk(mu);
      int64_t& v = edge[e][layer];
      v = std::max(v, it);
    }
    cv.notify_all();
  }
};

namespace {

// fp32 Adam over [lo, hi) of one layer, the formula above in fp32
void adam_range(LayerState& L, size_t lo, size_t hi, const rp_opt_hparams& hp, float bc1, float bc2) {
  const float b1 = hp.beta1, b2 = hp.beta2, c1 = (float)(1.0 - (double)hp.beta1),
              c2 = (float)(1.0 - (double)hp.beta2), lr = hp.lr, eps = hp.eps, wd = hp.weight_decay,
              gs = hp.grad_scale;
  float* w = L.w.data();
  float* m = L.m.data();
  float* v = L.v.data();
  const float* g = L.g.data();
  for (size_t i = lo; i < hi; ++i) {
    const float gi = gs * g[i];
    const float mi = b1 * m[i] + c1 * gi;
    const float vi = b2 * v[i] + c2 * (gi * gi);
    m[i] = mi;
    v[i] = vi;
    const float mhat = mi / bc1;
    const float vhat = vi / bc2;
    float upd = mhat / (std::sqrt(vhat) + eps);
    if (wd != 0.f) upd = upd + wd * w[i];
    w[i] = w[i] - lr * upd;
  }
}

template <class F>
void parallel_for(size_t n, int threads, F&& fn) {
  const size_t chunk = std::max<size_t>((n + threads - 1) / std::max(threads, 1), 1 << 16);
  const size_t parts = (n + chunk - 1) / chunk;
  if (parts <= 1) {
    fn(0, n);
    return;
  }
  std::vector<std::thread> ts;
  ts.reserve(parts - 1);
  for (size_t p = 1; p < parts; ++p) ts.emplace_back([&, p] { fn(p * chunk, std::min(n, (p + 1) * chunk)); });
  fn(0, std::min(n, chunk));
  for (auto& t : ts) t.join();
}

}  // namespace

bool rp_opt::wait_edge(int e, int layer, int64_t it) {
  std::unique_lock<std::mutex> lk(mu);
  auto ready = [&] { return stop || edge[e][layer] >= it; };
  if (edge_timeout_ms > 0) {
    if (!cv.wait_for(lk, std::chrono::milliseconds(edge_timeout_ms), ready)) return false;
  } else {
    cv.wait(lk, ready);
  }
  return !stop;
}

rp_status rp_opt::process(const Job& j) {
  const int64_t t = j.iteration;
  for (int l = 0; l < n_layers; ++l) {
    LayerState& L = layers[l];
    if (!L.bound) continue;
    // rule 3: g_t has landed in the master gradient buffer
    if (!wait_edge(RP_OPT_GRADS_DOWNLOADED, l, t)) {
      snprintf(worker_error, sizeof worker_error, "optimizer: layer %d step %lld: gradient download never signalled",
               l, (long long)t);
      return RP_ERR_STATE;
    }
    // G-cp, then rule 4: the GPU may download the next gradients
    for (const Seg& s : L.segs) std::memcpy(L.g.data() + s.off, s.master_g, s.n * sizeof(float));
    signal(RP_OPT_GCP_DONE, l, t);
    L.steps += 1;
    const double s = (double)L.steps;
    const float bc1 = (float)(1.0 - std::pow((double)j.hp.beta1, s));
    const float bc2 = (float)(1.0 - std::pow((double)j.hp.beta2, s));
    parallel_for(L.w.size(), n_threads, [&](size_t lo, size_t hi) { adam_range(L, lo, hi, j.hp, bc1, bc2); });
    // rule 1: iteration t + 1 has uploaded the weights of step t - 1
    if (!wait_edge(RP_OPT_PARAMS_UPLOADED, l, t + 1)) {
      snprintf(worker_error, sizeof worker_error, "optimizer: layer %d step %lld: upload of iteration %lld never "
               "signalled", l, (long long)t, (long long)(t + 1));
      return RP_ERR_STATE;
    }
    // P-cp, then rule 2: iteration t + 2 may upload
    for (const Seg& sg : L.segs) {
      const float* src = L.w.data() + sg.off;
      if (dtype == RP_DTYPE_BF16) {
        uint16_t* dst = static_cast<uint16_t*>(sg.master_w);
        parallel_for(sg.n, n_threads, [&](size_t lo, size_t hi) {
          for (size_t i = lo; i < hi; ++i) dst[i] = bf16_rne(src[i]);
        });
      } else {
        std::memcpy(sg.master_w, src, sg.n * sizeof(float));
      }
    }
    signal(RP_OPT_PCP_DONE, l, t);
  }
  return RP_OK;
}

void rp_opt::run() {
  for (;;) {
    Job j;
    {
      std::unique_lock<std::mutex> lk(mu);
      cv.wait(lk, [&] { return stop || !queue.empty(); });
      if (stop) return;
      j = queue.front();
    }
    // after a failed step the later ones are dropped: their inputs are suspect
    const rp_status st = worker_status == RP_OK ? process(j) : RP_OK;
    {
      std::lock_guard<std::mutex> lk(mu);
      queue.pop_front();
      done_steps += 1;
      if (st != RP_OK && worker_status == RP_OK) worker_status = st;
    }
    cv.notify_all();
  }
}

using namespace rp;

extern "C" {

rp_status rp_opt_create(int n_layers, int master_dtype, int n_threads, int64_t edge_timeout_ms, rp_opt** out) {
  RP_CHECK(out != nullptr, RP_ERR_INVALID, "opt_create: null output");
  RP_CHECK(n_layers >= 1 && n_layers <= 4096, RP_ERR_INVALID, "opt_create: n_layers out of range");
  RP_CHECK(master_dtype == RP_DTYPE_BF16 || master_dtype == RP_DTYPE_F32, RP_ERR_INVALID,
           "opt_create: master dtype must be bf16 or fp32");
  RP_CHECK(edge_timeout_ms >= 0, RP_ERR_INVALID, "opt_create: negative timeout");
  rp_opt* o = new rp_opt();
  o->n_layers = n_layers;
  o->dtype = master_dtype;
  o->n_threads = std::max(1, n_threads > 0 ? n_threads : (int)std::thread::hardware_concurrency());
  o->edge_timeout_ms = edge_timeout_ms;
  o->layers.resize(n_layers);
  for (auto& e : o->edge) e.assign(n_layers, -1);
  o->worker = std::thread([o] { o->run(); });
  *out = o;
  return RP_OK;
}

rp_status rp_opt_destroy(rp_opt* o) {
  if (!o) return RP_OK;
  {
    std::lock_guard<std::mutex> lk(o->mu);
    o->stop = true;
  }
  o->cv.notify_all();
  if (o->worker.joinable()) o->worker.join();
  delete o;
  return RP_OK;
}

rp_status rp_opt_bind_layer(rp_opt* o, int layer, const rp_opt_seg* segs, int n_segs) {
  RP_CHECK(o && segs && n_segs >= 1, RP_ERR_INVALID, "opt_bind_layer: bad arguments");
  RP_CHECK(layer >= 0 && layer < o->n_layers, RP_ERR_INVALID, "opt_bind_layer: layer %d out of range", layer);
  {
    std::lock_guard<std::mutex> lk(o->mu);
    RP_CHECK(o->queued_steps == o->done_steps, RP_ERR_STATE, "opt_bind_layer: steps are still running");
  }
  LayerState& L = o->layers[layer];
  L = LayerState();
  size_t off = 0;
  for (int i = 0; i < n_segs; ++i) {
    RP_CHECK(segs[i].master_w && segs[i].master_g, RP_ERR_INVALID, "opt_bind_layer: segment %d has a null buffer", i);
    L.segs.push_back(Seg{segs[i].master_w, segs[i].master_g, (size_t)segs[i].n, off});
    off += (size_t)segs[i].n;
  }
  L.w.resize(off);
  L.m.assign(off, 0.f);
  L.v.assign(off, 0.f);
  L.g.assign(off, 0.f);
  // the optimizer copy starts from the given fp32 values, else from the master
  for (int i = 0; i < n_segs; ++i) {
    float* dst = L.w.data() + L.segs[i].off;
    const size_t n = L.segs[i].n;
    if (segs[i].init) {
      std::memcpy(dst, segs[i].init, n * sizeof(float));
    } else if (o->dtype == RP_DTYPE_BF16) {
      const uint16_t* src = static_cast<const uint16_t*>(segs[i].master_w);
      for (size_t k = 0; k < n; ++k) dst[k] = bf16_to_f(src[k]);
    } else {
      std::memcpy(dst, segs[i].master_w, n * sizeof(float));
    }
  }
  L.bound = true;
  return RP_OK;
}

rp_status rp_opt_step(rp_opt* o, int64_t iteration, const rp_opt_hparams* hp) {
  RP_CHECK(o && hp, RP_ERR_INVALID, "opt_step: null argument");
  RP_CHECK(iteration >= 0, RP_ERR_INVALID, "opt_step: negative iteration");
  RP_CHECK(hp->lr >= 0.f && hp->beta1 >= 0.f && hp->beta1 < 1.f && hp->beta2 >= 0.f && hp->beta2 < 1.f &&
               hp->eps > 0.f,
           RP_ERR_INVALID, "opt_step: hyper-parameters out of range");
  {
    std::lock_guard<std::mutex> lk(o->mu);
    RP_CHECK(o->worker_status == RP_OK, o->worker_status, "%s", o->worker_error);
    o->queue.push_back(Job{iteration, *hp});
    o->queued_steps += 1;
  }
  o->cv.notify_all();
  return RP_OK;
}

rp_status rp_opt_signal(rp_opt* o, int edge, int layer, int64_t iteration) {
  RP_CHECK(o, RP_ERR_INVALID, "opt_signal: null optimizer");
  RP_CHECK(edge == RP_OPT_PARAMS_UPLOADED || edge == RP_OPT_GRADS_DOWNLOADED, RP_ERR_INVALID,
           "opt_signal: only the GPU side's edges are signalled from outside");
  RP_CHECK(layer >= -1 && layer < o->n_layers, RP_ERR_INVALID, "opt_signal: layer %d out of range", layer);
  if (layer < 0) {
    for (int l = 0; l < o->n_layers; ++l) o->signal(edge, l, iteration);
  } else {
    o->signal(edge, layer, iteration);
  }
  return RP_OK;
}

rp_status rp_opt_wait(rp_opt* o, int edge, int layer, int64_t iteration) {
  RP_CHECK(o, RP_ERR_INVALID, "opt_wait: null optimizer");
  RP_CHECK(edge == RP_OPT_PCP_DONE || edge == RP_OPT_GCP_DONE, RP_ERR_INVALID,
           "opt_wait: the GPU side waits for the optimizer's edges only");
  RP_CHECK(layer >= 0 && layer < o->n_layers, RP_ERR_INVALID, "opt_wait: layer %d out of range", layer);
  if (iteration < 0 || !o->layers[layer].bound) return RP_OK;
  {
    std::unique_lock<std::mutex> lk(o->mu);
    auto ready = [&] { return o->edge[edge][layer] >= iteration || o->worker_status != RP_OK; };
    if (o->edge_timeout_ms > 0) {
      RP_CHECK(o->cv.wait_for(lk, std::chrono::milliseconds(o->edge_timeout_ms), ready), RP_ERR_STATE,
               "opt_wait: edge %d of layer %d for step %lld not reached in %lld ms", edge, layer,
               (long long)iteration, (long long)o->edge_timeout_ms);
    } else {
      o->cv.wait(lk, ready);
    }
    RP_CHECK(o->worker_status == RP_OK, o->worker_status, "%s", o->worker_error);
  }
  return RP_OK;
}

rp_status rp_opt_sync(rp_opt* o) {
  RP_CHECK(o, RP_ERR_INVALID, "opt_sync: null optimizer");
  std::unique_lock<std::mutex> lk(o->mu);
  auto ready = [&] { return o->done_steps == o->queued_steps; };
  if (o->edge_timeout_ms > 0) {
    RP_CHECK(o->cv.wait_for(lk, std::chrono::milliseconds(o->edge_timeout_ms * 4), ready), RP_ERR_STATE,
             "opt_sync: queued steps did not finish");
  } else {
    o->cv.wait(lk, ready);
  }
  RP_CHECK(o->worker_status == RP_OK, o->worker_status, "%s", o->worker_error);
  return RP_OK;
}

rp_status rp_opt_read(rp_opt* o, int layer, int which, float* dst, uint64_t n) {
  RP_CHECK(o && dst, RP_ERR_INVALID, "opt_read: null argument");
  RP_CHECK(layer >= 0 && layer < o->n_layers && o->layers[layer].bound, RP_ERR_INVALID,
           "opt_read: layer %d not bound", layer);
  std::lock_guard<std::mutex> lk(o->mu);
  RP_CHECK(o->done_steps == o->queued_steps, RP_ERR_STATE, "opt_read: steps are still running");
  const LayerState& L = o->layers[layer];
  const std::vector<float>* src = which == 0 ? &L.w : which == 1 ? &L.m : which == 2 ? &L.v : nullptr;
  RP_CHECK(src != nullptr, RP_ERR_INVALID, "opt_read: which must be 0 (weights), 1 (m) or 2 (v)");
  RP_CHECK(n == src->size(), RP_ERR_INVALID, "opt_read: layer %d holds %zu elements, asked for %llu", layer,
           src->size(), (unsigned long long)n);
  std::memcpy(dst, src->data(), n * sizeof(float));
  return RP_OK;
}

}  // extern "C"
