// The worker context behind rp_ctx: configuration, streams, buffer bindings
// and the events that order compute against the four copy classes.
#pragma once

#include <map>
#include <vector>

#include "ops.h"
#include "trace.h"

struct rp_ctx;

namespace rp {

// Ordering state of one bound device buffer (a layer's weight block, an
// LM-head shard, ...). Events are created lazily and owned by the context.
struct Slot {
  const void* w = nullptr;       // weights (device)
  float* g = nullptr;            // fp32 gradient (device)
  size_t w_bytes = 0, g_bytes = 0;
  hipEvent_t w_ready = nullptr;     // recorded on w_h2d after the last upload chunk
  bool w_ready_pending = false;     // compute must wait on w_ready before reading
  int w_chunks_unissued = 0;        // upload chunks still deferred behind a ticket
  hipEvent_t w_consumed = nullptr;  // recorded on compute after the last read
  bool w_consumed_valid = false;
  hipEvent_t g_ready = nullptr;     // recorded on compute after the gradient is written
  bool g_ready_valid = false;
  hipEvent_t g_drained = nullptr;   // recorded on g_d2h after the last download chunk
  bool g_drained_pending = false;
  int g_chunks_unissued = 0;
  void* g_stage = nullptr;          // bf16 staging copy of g (bf16 downloads), owned by the context
};

struct LayerBinding {
  bool bound = false;
  Slot base;   // weight block + gradient block
  Slot lora;   // adapter block + adapter gradient block (lora_rank > 0)
};

struct Shape {
  int H, nq, nkv, d, F, E, topk, Fe, r;
  int Q, KV, QKV;  // q width, kv width, packed qkv width
  int dt;
  size_t es;       // element size
  bool qkn;        // per-head RMSNorm of q and k before RoPE
};

// Bump allocator over the caller's workspace; a dry run (base == nullptr)
// measures the size with exactly the same carving code.
struct Bump {
  char* base;
  size_t off = 0;
  explicit Bump(void* b) : base((char*)b) {}
  template <class P = void>
  P* take(size_t bytes) {
    off = align_up(off, 256);
    P* p = base ? reinterpret_cast<P*>(base + off) : nullptr;
    off += align_up(bytes, 256);
    return p;
  }
};

// A deferred parameter/gradient window (gated on an activation ticket)
struct XChunk {
  int dir;            // RP_H2D / RP_D2H
  Slot* slot;
  char* dev;
  char* host;
  uint64_t bytes;
};
struct XWindow {
  int dir;
  int64_t gate;       // ticket to wait for, -1 for none
  std::vector<XChunk> chunks;
};

}  // namespace rp

namespace rp {
// a default-priority stream on a hardware queue of its own (all CUs enabled)
rp_status new_queue_stream(int device, hipStream_t* out);
}  // namespace rp

struct rp_ctx {
  int device = 0;
  rp_layer_cfg cfg{};
  rp::Shape sh{};
  hipStream_t compute = nullptr, act_h2d = nullptr, act_d2h = nullptr, w_h2d = nullptr, g_d2h = nullptr;
  // a second compute stream of the context's own: memory-bound kernels of a
  // call run on it beside the call's matrix products on `compute`, and every
  // call joins it back into `compute` before it returns
  hipStream_t side = nullptr;
  std::vector<hipEvent_t> side_ev;  // fork/join events of the side stream (created once)
  // the device's fixed scratch of rp_op_attn_bwd_noalloc (looked up at creation)
  float* attn_scratch = nullptr;
  // transfer streams the context created (each on a hardware queue of its own)
  std::vector<hipStream_t> owned;
  std::vector<rp::LayerBinding> layers;   // indexed by layer id
  // LM head
  int vocab = 0, n_shards = 0;
  std::vector<rp::Slot> shards;
  std::vector<int> shard_lo;              // row offsets, n_shards + 1
  rp::Slot final_norm;                    // gamma_f / dgamma_f
  // activation tickets
  int64_t next_ticket = 0;
  std::map<int64_t, hipEvent_t> ticket_ev;
  std::vector<rp::XWindow> deferred;
  hipEvent_t last_act_d2h = nullptr;      // every call starts after the previous downloads
  bool last_act_d2h_valid = false;
  std::vector<hipEvent_t> all_events;    // every event created (destroyed with the context)
  std::vector<hipEvent_t> ev_free;       // recycled ticket events
  hipEvent_t ev_mark = nullptr;          // scratch: "compute reached this point"
  std::vector<void*> stages;             // bf16 gradient staging copies (freed with the context)
  // per workspace (by base pointer): the compute stream is done with it after
  // this event -- uploads into a workspace's checkpoint buffers wait for it
  std::map<const void*, hipEvent_t> ws_done;
  hipEvent_t ck_free[2] = {nullptr, nullptr};  // backward: checkpoint buffer i & 1 read
  // kept-activation bookkeeping for RP_USE_KEPT_ACTS
  const void* kept_ws = nullptr;
  int kept_l0 = -1, kept_l1 = -1, kept_batch = 0, kept_seq = 0;
  // per-launch kernel timing (rp_trace_begin / rp_trace_read)
  rp::Trace trace;

  hipEvent_t new_event();
};

namespace rp {

// stage executor (stage.cpp)
rp_status stage_fwd(rp_ctx* c, int l0, int l1, int batch, int seq, const void* x_in, void* y_out,
                    void* const* ckpt_host, const float* const* router, int flags, void* ws, size_t ws_bytes,
                    size_t* need);
rp_status stage_bwd(rp_ctx* c, int l0, int l1, int batch, int seq, const void* const* ckpt, const void* dy,
                    void* dx, const float* const* router, int flags, void* ws, size_t ws_bytes, size_t* need);
rp_status lmhead(rp_ctx* c, int batch, int seq, const void* x, const int32_t* labels, float* loss, void* dx,
                 void* ws, size_t ws_bytes, size_t* need);

// transfer engine (xfer.cpp)
rp_status act_copy(rp_ctx* c, int dir, void* dst, const void* src, size_t bytes, int64_t* ticket);
rp_status act_wait(rp_ctx* c, int where, int64_t ticket);
rp_status weight_stream_submit(rp_ctx* c, const rp_xfer* items, int n_items, int n_windows, uint64_t max_chunk,
                               const int64_t* gates, int64_t gate0);
rp_status wait_weights(rp_ctx* c, Slot& s);       // compute waits for a pending upload
rp_status mark_consumed(rp_ctx* c, Slot& s);      // after the last compute read
rp_status wait_grad_drained(rp_ctx* c, Slot& s);  // before compute overwrites a gradient
rp_status mark_grad_ready(rp_ctx* c, Slot& s);    // after compute wrote the gradient
bool is_pinned_host(const void* p);

// layout of the weight / gradient / LoRA blocks
rp_status block_layout(const rp_layer_cfg& cfg, int block, int tensor, size_t* off, size_t* bytes,
                       size_t* total);
Shape make_shape(const rp_layer_cfg& cfg);

}  // namespace rp
