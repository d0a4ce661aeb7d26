// C ABI of the stage library: validation, context life cycle, bindings and
// the thin entry points over the stage executor and the transfer engine.
#include <cstdarg>
#include <cstring>
#include <new>

#include "attn_flash.h"
#include "ctx.h"

namespace rp {

namespace {
thread_local char g_err[1024] = "";
constexpr int kMaxLayers = 4096;
}  // namespace

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}
const char* last_error() { return g_err; }

Shape make_shape(const rp_layer_cfg& c) {
  Shape s{};
  s.H = c.hidden; s.nq = c.n_q; s.nkv = c.n_kv; s.d = c.head_dim;
  s.F = c.ffn; s.E = c.n_experts; s.topk = c.top_k; s.Fe = c.expert_ffn; s.r = c.lora_rank;
  s.Q = c.n_q * c.head_dim; s.KV = c.n_kv * c.head_dim; s.QKV = s.Q + 2 * s.KV;
  s.dt = c.dtype;
  s.es = dtype_size(c.dtype);
  s.qkn = c.qk_norm != 0;
  return s;
}

rp_status block_layout(const rp_layer_cfg& cfg, int block, int tensor, size_t* off, size_t* bytes,
                       size_t* total) {
  const Shape s = make_shape(cfg);
  struct T { int id; size_t n; };
  std::vector<T> ts;
  size_t es;
  if (block == RP_BLOCK_WEIGHT || block == RP_BLOCK_GRAD) {
    es = block == RP_BLOCK_WEIGHT ? s.es : 4;
    const size_t H = s.H;
    const size_t gu = s.E > 0 ? (size_t)s.E * 2 * s.Fe * H : 2 * (size_t)s.F * H;
    const size_t dn = s.E > 0 ? (size_t)s.E * H * s.Fe : H * (size_t)s.F;
    ts = {{RP_T_GAMMA1, H}, {RP_T_WQKV, (size_t)s.QKV * H}, {RP_T_WO, H * s.Q}, {RP_T_GAMMA2, H},
          {RP_T_WGU, gu}, {RP_T_WD, dn}};
    // the QK-norm gains come last, so that the other offsets do not move
    if (s.qkn) {
      ts.push_back({RP_T_QNORM, (size_t)s.d});
      ts.push_back({RP_T_KNORM, (size_t)s.d});
    }
  } else if (block == RP_BLOCK_LORA) {
    RP_CHECK(s.r > 0, RP_ERR_INVALID, "layout: no LoRA block when lora_rank == 0");
    es = 4;
    const size_t r = s.r, H = s.H;
    ts = {{RP_T_AQ, r * H}, {RP_T_BQ, (size_t)s.Q * r}, {RP_T_AK, r * H}, {RP_T_BK, (size_t)s.KV * r},
          {RP_T_AV, r * H}, {RP_T_BV, (size_t)s.KV * r}, {RP_T_AO, r * s.Q}, {RP_T_BO, H * r}};
  } else {
    set_error("layout: unknown block %d", block);
    return RP_ERR_INVALID;
  }
  size_t o = 0;
  bool found = false;
  for (const T& t : ts) {
    o = align_up(o, 256);
    if (t.id == tensor) {
      if (off) *off = o;
      if (bytes) *bytes = t.n * es;
      found = true;
    }
    o += t.n * es;
  }
  if (total) *total = align_up(o, 256);
  RP_CHECK(found || tensor < 0, RP_ERR_INVALID, "layout: block %d has no tensor %d", block, tensor);
  return RP_OK;
}

}  // namespace rp

hipEvent_t rp_ctx::new_event() {
  if (!ev_free.empty()) {
    hipEvent_t e = ev_free.back();
    ev_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return nullptr;
  all_events.push_back(e);
  return e;
}

using namespace rp;

#define CTX_CHECK(c) RP_CHECK((c) != nullptr, RP_ERR_INVALID, "null context")

// Entering a context makes its device current (one thread may drive several).
#define CTX_ENTER(c)           \
  CTX_CHECK(c);                \
  RP_HIP(hipSetDevice((c)->device)); \
  ::rp::trace_bind(&(c)->trace)

extern "C" {

const char* rp_status_string(rp_status s) {
  switch (s) {
    case RP_OK: return "RP_OK";
    case RP_ERR_INVALID: return "RP_ERR_INVALID";
    case RP_ERR_UNSUPPORTED: return "RP_ERR_UNSUPPORTED";
    case RP_ERR_WORKSPACE: return "RP_ERR_WORKSPACE";
    case RP_ERR_NOT_PINNED: return "RP_ERR_NOT_PINNED";
    case RP_ERR_HIP: return "RP_ERR_HIP";
    case RP_ERR_STATE: return "RP_ERR_STATE";
  }
  return "RP_ERR_UNKNOWN";
}

const char* rp_last_error(void) { return last_error(); }

const char* rp_version(void) { return "roundpipe-stage-gfx950 0.1"; }

rp_status rp_block_layout(const rp_layer_cfg* cfg, int block, int tensor, size_t* offset, size_t* bytes,
                          size_t* total) {
  RP_CHECK(cfg, RP_ERR_INVALID, "layout: null cfg");
  return block_layout(*cfg, block, tensor, offset, bytes, total);
}

rp_status rp_ctx_create(int device, const rp_layer_cfg* cfg, const rp_streams* streams, rp_ctx** out) {
  RP_CHECK(cfg && out, RP_ERR_INVALID, "ctx_create: null argument");
  *out = nullptr;
  const rp_layer_cfg& c = *cfg;
  RP_CHECK(c.dtype == RP_DTYPE_F32 || c.dtype == RP_DTYPE_BF16, RP_ERR_INVALID, "ctx_create: bad dtype %d",
           c.dtype);
  RP_CHECK(c.hidden > 0 && c.hidden % 64 == 0, RP_ERR_UNSUPPORTED, "ctx_create: hidden must be a multiple of 64");
  RP_CHECK(c.n_q > 0 && c.n_kv > 0 && c.n_q % c.n_kv == 0, RP_ERR_UNSUPPORTED,
           "ctx_create: n_q must be a positive multiple of n_kv");
  RP_CHECK(c.head_dim == 64 || c.head_dim == 128, RP_ERR_UNSUPPORTED, "ctx_create: head_dim must be 64 or 128");
  RP_CHECK(c.n_experts == 0 || (c.n_experts <= 256 && c.top_k >= 1 && c.top_k <= 16 && c.top_k <= c.n_experts &&
                                 c.expert_ffn > 0 && c.expert_ffn % 8 == 0 && c.ffn == 0 &&
                                 c.dtype == RP_DTYPE_BF16),
           RP_ERR_UNSUPPORTED,
           "ctx_create: MoE layers need bf16, up to 256 experts, 1 <= top_k <= 16, expert_ffn a multiple of 8 "
           "and ffn == 0");
  RP_CHECK(c.lora_rank == 0 || (c.lora_rank > 0 && c.lora_rank % 8 == 0 && c.lora_rank <= 128 &&
                                 c.dtype == RP_DTYPE_BF16),
           RP_ERR_UNSUPPORTED, "ctx_create: LoRA rank must be a multiple of 8 up to 128, with bf16 layers");
  RP_CHECK(c.n_experts > 0 || (c.ffn > 0 && c.ffn % 8 == 0), RP_ERR_UNSUPPORTED,
           "ctx_create: ffn must be a positive multiple of 8");
  RP_CHECK(c.rms_eps > 0.f && c.rope_base > 1.f, RP_ERR_INVALID, "ctx_create: bad rms_eps or rope_base");
  int n_dev = 0;
  RP_HIP(hipGetDeviceCount(&n_dev));
  RP_CHECK(device >= 0 && device < n_dev, RP_ERR_INVALID, "ctx_create: device %d of %d", device, n_dev);
  RP_HIP(hipSetDevice(device));
  rp_ctx* x = new (std::nothrow) rp_ctx();
  RP_CHECK(x, RP_ERR_INVALID, "ctx_create: out of host memory");
  x->device = device;
  x->cfg = c;
  x->sh = make_shape(c);
  if (streams) {
    x->compute = (hipStream_t)streams->compute;
    x->act_h2d = (hipStream_t)streams->act_h2d;
    x->act_d2h = (hipStream_t)streams->act_d2h;
    x->w_h2d = (hipStream_t)streams->w_h2d;
    x->g_d2h = (hipStream_t)streams->g_d2h;
  }
  // missing streams: created here, each on its own hardware queue (a stream
  // with a CU mask never shares its queue; all CUs enabled). Such a stream is
  // a blocking stream: work enqueued on the legacy default stream before a
  // call runs before the call's kernels, and default-stream work enqueued
  // after it waits for them.
  for (hipStream_t* ps : {&x->compute, &x->act_h2d, &x->act_d2h, &x->w_h2d, &x->g_d2h, &x->side}) {
    if (*ps) continue;
    rp_status st = new_queue_stream(device, ps);
    if (st != RP_OK) {
      (void)rp_ctx_destroy(x);
      return st;
    }
    x->owned.push_back(*ps);
  }
  {
    // the allocation-free attention backward's scratch: its address on this
    // device, with the device current
    rp_status st = attn_scratch(device, &x->attn_scratch);
    if (st != RP_OK) {
      (void)rp_ctx_destroy(x);
      return st;
    }
  }
  x->layers.resize(kMaxLayers);  // fixed: deferred transfers keep pointers into it
  *out = x;
  return RP_OK;
}

rp_status rp_ctx_streams(const rp_ctx* c, rp_streams* out) {
  CTX_CHECK(c);
  RP_CHECK(out != nullptr, RP_ERR_INVALID, "ctx_streams: null output");
  out->compute = c->compute;
  out->act_h2d = c->act_h2d;
  out->act_d2h = c->act_d2h;
  out->w_h2d = c->w_h2d;
  out->g_d2h = c->g_d2h;
  return RP_OK;
}

rp_status rp_ctx_sync(rp_ctx* c) {
  CTX_ENTER(c);
  hipStream_t ss[6] = {c->compute, c->act_h2d, c->act_d2h, c->w_h2d, c->g_d2h, c->side};
  for (hipStream_t s : ss) RP_HIP(hipStreamSynchronize(s));
  RP_HIP(hipGetLastError());
  RP_CHECK(c->deferred.empty(), RP_ERR_STATE, "ctx_sync: %zu transfer windows still wait for activation tickets",
           c->deferred.size());
  return RP_OK;
}

rp_status rp_ctx_destroy(rp_ctx* c) {
  if (!c) return RP_OK;
  if (trace_current() == &c->trace) trace_bind(nullptr);
  rp_status st = RP_OK;
  if (hipSetDevice(c->device) == hipSuccess) {
    hipStream_t ss[6] = {c->compute, c->act_h2d, c->act_d2h, c->w_h2d, c->g_d2h, c->side};
    for (hipStream_t s : ss)
      if (s && hipStreamSynchronize(s) != hipSuccess) st = RP_ERR_HIP;
    for (hipStream_t d : c->owned) (void)hipStreamDestroy(d);
    for (hipEvent_t e : c->all_events) (void)hipEventDestroy(e);
    for (void* p : c->stages) (void)hipFree(p);
  }
  delete c;
  return st;
}

rp_status rp_bind_layer(rp_ctx* c, int layer, const void* w_dev, float* grad_dev, const float* lora_dev,
                        float* lora_grad_dev) {
  CTX_CHECK(c);
  RP_CHECK(layer >= 0 && layer < kMaxLayers, RP_ERR_INVALID, "bind_layer: layer %d out of range", layer);
  RP_CHECK(w_dev && ((uintptr_t)w_dev & 255) == 0, RP_ERR_INVALID, "bind_layer: weights null or not 256-aligned");
  RP_CHECK(!grad_dev || ((uintptr_t)grad_dev & 255) == 0, RP_ERR_INVALID, "bind_layer: gradient not 256-aligned");
  LayerBinding& b = c->layers[layer];
  RP_CHECK(b.base.w_chunks_unissued == 0 && b.base.g_chunks_unissued == 0 && b.lora.w_chunks_unissued == 0 &&
               b.lora.g_chunks_unissued == 0,
           RP_ERR_STATE, "bind_layer: layer %d has deferred transfers", layer);
  if (c->cfg.lora_rank > 0) {
    RP_CHECK(lora_dev && ((uintptr_t)lora_dev & 255) == 0, RP_ERR_INVALID,
             "bind_layer: LoRA layers need a 256-aligned adapter block");
    RP_CHECK(!lora_grad_dev || ((uintptr_t)lora_grad_dev & 255) == 0, RP_ERR_INVALID,
             "bind_layer: adapter gradient not 256-aligned");
    size_t lt = 0;
    RP_TRY(block_layout(c->cfg, RP_BLOCK_LORA, -1, nullptr, nullptr, &lt));
    b.lora.w = lora_dev;
    b.lora.g = lora_grad_dev;
    b.lora.w_bytes = lt;
    b.lora.g_bytes = lora_grad_dev ? lt : 0;
  } else {
    RP_CHECK(!lora_dev && !lora_grad_dev, RP_ERR_INVALID, "bind_layer: adapters given for a context without LoRA");
  }
  size_t wt = 0, gt = 0;
  RP_TRY(block_layout(c->cfg, RP_BLOCK_WEIGHT, -1, nullptr, nullptr, &wt));
  RP_TRY(block_layout(c->cfg, RP_BLOCK_GRAD, -1, nullptr, nullptr, &gt));
  b.bound = true;
  b.base.w = w_dev;
  b.base.g = grad_dev;
  b.base.w_bytes = wt;
  b.base.g_bytes = grad_dev ? gt : 0;
  return RP_OK;
}

rp_status rp_bind_lmhead(rp_ctx* c, int vocab, int n_shards, const void* const* w_shard, float* const* dw_shard,
                         const void* gamma_f, float* dgamma_f) {
  CTX_CHECK(c);
  RP_CHECK(vocab > 0 && n_shards >= 1 && n_shards <= 64 && n_shards <= vocab, RP_ERR_INVALID,
           "bind_lmhead: bad vocab/n_shards");
  RP_CHECK(w_shard, RP_ERR_INVALID, "bind_lmhead: null shard list");
  RP_CHECK(c->deferred.empty(), RP_ERR_STATE, "bind_lmhead: transfers are deferred");
  const int base = vocab / n_shards, extra = vocab % n_shards;
  std::vector<int> lo(n_shards + 1, 0);
  for (int s = 0; s < n_shards; ++s) lo[s + 1] = lo[s] + base + (s < extra ? 1 : 0);
  if (c->sh.dt == RP_DTYPE_BF16)
    for (int s = 0; s < n_shards; ++s)
      RP_CHECK((lo[s + 1] - lo[s]) % 8 == 0, RP_ERR_UNSUPPORTED, "bind_lmhead: bf16 shard rows must be a multiple of 8");
  for (int s = 0; s < n_shards; ++s) {
    RP_CHECK(w_shard[s] && ((uintptr_t)w_shard[s] & 15) == 0, RP_ERR_INVALID, "bind_lmhead: shard %d null/misaligned", s);
    RP_CHECK(!dw_shard || !dw_shard[s] || ((uintptr_t)dw_shard[s] & 15) == 0, RP_ERR_INVALID,
             "bind_lmhead: gradient %d misaligned", s);
  }
  c->vocab = vocab;
  c->n_shards = n_shards;
  c->shard_lo = lo;
  c->shards.assign(n_shards, Slot{});
  for (int s = 0; s < n_shards; ++s) {
    Slot& sl = c->shards[s];
    const size_t rows = lo[s + 1] - lo[s];
    sl.w = w_shard[s];
    sl.g = dw_shard ? dw_shard[s] : nullptr;
    sl.w_bytes = rows * c->sh.H * c->sh.es;
    sl.g_bytes = sl.g ? rows * c->sh.H * 4 : 0;
  }
  c->final_norm = Slot{};
  if (gamma_f) {
    c->final_norm.w = gamma_f;
    c->final_norm.g = dgamma_f;
    c->final_norm.w_bytes = (size_t)c->sh.H * c->sh.es;
    c->final_norm.g_bytes = dgamma_f ? (size_t)c->sh.H * 4 : 0;
  }
  return RP_OK;
}

rp_status rp_workspace_size(const rp_ctx* cc, int op, int batch, int seq, int n_layers, int flags, size_t* bytes) {
  rp_ctx* c = const_cast<rp_ctx*>(cc);
  CTX_CHECK(c);
  RP_CHECK(bytes, RP_ERR_INVALID, "workspace_size: null output");
  RP_CHECK(batch >= 1 && seq >= 1 && n_layers >= 1, RP_ERR_INVALID, "workspace_size: bad sizes");
  switch (op) {
    case RP_OP_STAGE_FWD:
      return stage_fwd(c, 0, n_layers, batch, seq, nullptr, nullptr, nullptr, nullptr, flags, nullptr, 0, bytes);
    case RP_OP_STAGE_BWD:
      return stage_bwd(c, 0, n_layers, batch, seq, nullptr, nullptr, nullptr, nullptr, flags, nullptr, 0, bytes);
    case RP_OP_FUSED:
      return stage_bwd(c, 0, n_layers, batch, seq, nullptr, nullptr, nullptr, nullptr, RP_USE_KEPT_ACTS, nullptr, 0,
                       bytes);
    case RP_OP_LMHEAD:
      return lmhead(c, batch, seq, nullptr, nullptr, nullptr, nullptr, nullptr, 0, bytes);
    case RP_OP_MOE_ROUTE: {
      RP_CHECK(c->sh.E > 0, RP_ERR_STATE, "workspace_size: MoE routing in a dense context");
      const int64_t T = (int64_t)batch * seq;
      *bytes = 2 * align_up((size_t)moe_max_tiles(T, c->sh.topk, c->sh.E) * 4, 256);
      return RP_OK;
    }
  }
  set_error("workspace_size: unknown op %d", op);
  return RP_ERR_INVALID;
}

rp_status rp_stage_fwd(rp_ctx* c, int l0, int l1, int batch, int seq, const void* x_in, void* y_out,
                       void* const* ckpt_host, const float* const* router, int flags, void* ws, size_t ws_bytes) {
  CTX_ENTER(c);
  RP_CHECK((flags & ~RP_KEEP_ACTS) == 0, RP_ERR_INVALID, "stage_fwd: unknown flags 0x%x", flags);
  if (flags & RP_KEEP_ACTS) {
    // the kept internals sit in front of the backward temporaries of a fused stage
    size_t need = 0;
    RP_TRY(stage_bwd(c, 0, l1 - l0, batch, seq, nullptr, nullptr, nullptr, nullptr, RP_USE_KEPT_ACTS, nullptr, 0,
                     &need));
    RP_CHECK(ws_bytes >= need, RP_ERR_WORKSPACE, "stage_fwd(keep): workspace %zu < %zu bytes (fused size)",
             ws_bytes, need);
  }
  return stage_fwd(c, l0, l1, batch, seq, x_in, y_out, ckpt_host, router, flags, ws, ws_bytes, nullptr);
}

rp_status rp_stage_bwd_recompute(rp_ctx* c, int l0, int l1, int batch, int seq, const void* const* ckpt,
                                 const void* dy, void* dx, const float* const* router, int flags, void* ws,
                                 size_t ws_bytes) {
  CTX_ENTER(c);
  RP_CHECK((flags & ~(RP_USE_KEPT_ACTS | RP_CKPT_DEVICE | RP_ACCUM_GRADS)) == 0, RP_ERR_INVALID,
           "stage_bwd: unknown flags 0x%x", flags);
  return stage_bwd(c, l0, l1, batch, seq, ckpt, dy, dx, router, flags, ws, ws_bytes, nullptr);
}

rp_status rp_lmhead_ce_fwd_bwd(rp_ctx* c, int batch, int seq, const void* x, const int32_t* labels, float* loss,
                               void* dx, void* ws, size_t ws_bytes) {
  CTX_ENTER(c);
  return lmhead(c, batch, seq, x, labels, loss, dx, ws, ws_bytes, nullptr);
}

rp_status rp_embed_fwd(rp_ctx* c, int n_tokens, int vocab, const int32_t* ids, const void* table, void* x0) {
  CTX_ENTER(c);
  RP_CHECK(n_tokens >= 0 && vocab > 0 && ids && table && x0, RP_ERR_INVALID, "embed_fwd: bad arguments");
  return embed_fwd(c->sh.dt, ids, table, x0, n_tokens, vocab, c->sh.H, c->compute);
}

rp_status rp_embed_bwd(rp_ctx* c, int n_tokens, int vocab, const int32_t* ids, const void* dx0, float* dtable) {
  CTX_ENTER(c);
  RP_CHECK(n_tokens >= 0 && vocab > 0 && ids && dx0 && dtable, RP_ERR_INVALID, "embed_bwd: bad arguments");
  return embed_bwd(c->sh.dt, ids, dx0, dtable, n_tokens, vocab, c->sh.H, c->compute);
}

rp_status rp_act_copy(rp_ctx* c, int dir, void* dst, const void* src, size_t bytes, int64_t* ticket) {
  CTX_ENTER(c);
  return act_copy(c, dir, dst, src, bytes, ticket);
}

rp_status rp_act_wait(rp_ctx* c, int where, int64_t ticket) {
  CTX_ENTER(c);
  RP_CHECK(where == RP_ON_COMPUTE || where == RP_ON_ACT_H2D || where == RP_ON_ACT_D2H, RP_ERR_INVALID,
           "act_wait: bad stream selector %d", where);
  return act_wait(c, where, ticket);
}

rp_status rp_act_next_ticket(const rp_ctx* c, int64_t* next) {
  CTX_CHECK(c);
  RP_CHECK(next != nullptr, RP_ERR_INVALID, "act_next_ticket: null output");
  *next = c->next_ticket;
  return RP_OK;
}

rp_status rp_op_gemm_bf16(rp_ctx* c, int M, int N, int K, const void* A, int lda, int a_kmajor, const void* B,
                          int ldb, int b_kmajor, void* C, int ldc, int out_f32, int accumulate) {
  CTX_ENTER(c);
  GemmDesc d;
  d.M = M; d.N = N; d.K = K;
  d.A = A; d.lda = lda; d.a_kmajor = a_kmajor != 0;
  d.B = B; d.ldb = ldb; d.b_kmajor = b_kmajor != 0;
  d.C = C; d.ldc = ldc;
  d.in_dtype = RP_DTYPE_BF16;
  d.out_dtype = out_f32 ? RP_DTYPE_F32 : RP_DTYPE_BF16;
  d.accumulate = accumulate != 0;
  RP_CHECK(ldc >= N, RP_ERR_INVALID, "op_gemm: ldc < N");
  return gemm(d, c->compute);
}

rp_status rp_op_copy(rp_ctx* c, void* dst, const void* src, size_t bytes) {
  CTX_ENTER(c);
  RP_CHECK(bytes == 0 || (dst && src), RP_ERR_INVALID, "op_copy: null pointer");
  return copy16(dst, src, bytes, c->compute);
}

rp_status rp_op_transpose_bf16(rp_ctx* c, int rows, int cols, const void* src, int64_t lds, void* dst, int64_t ldd) {
  CTX_ENTER(c);
  RP_CHECK(rows >= 0 && cols >= 0 && lds >= cols && ldd >= rows, RP_ERR_INVALID, "op_transpose: bad sizes");
  RP_CHECK(rows == 0 || cols == 0 || (src && dst), RP_ERR_INVALID, "op_transpose: null pointer");
  return transpose_bf16(src, lds, dst, ldd, rows, cols, c->compute);
}

rp_status rp_op_attn_fwd(rp_ctx* c, int batch, int seq, const void* qkv, void* o, float* lse) {
  CTX_ENTER(c);
  RP_CHECK(batch >= 1 && seq >= 1 && qkv && o && lse, RP_ERR_INVALID, "op_attn_fwd: bad arguments");
  AttnDesc a;
  a.dt = c->sh.dt; a.batch = batch; a.seq = seq; a.n_q = c->sh.nq; a.n_kv = c->sh.nkv; a.d = c->sh.d;
  return attn_fwd(a, qkv, o, lse, c->compute);
}

rp_status rp_op_attn_bwd(rp_ctx* c, int batch, int seq, const void* qkv, const void* o, const void* dout,
                         const float* lse, void* dqkv, void* ws, size_t ws_bytes) {
  CTX_ENTER(c);
  RP_CHECK(batch >= 1 && seq >= 1 && qkv && o && dout && lse && dqkv && ws, RP_ERR_INVALID,
           "op_attn_bwd: bad arguments");
  AttnDesc a;
  a.dt = c->sh.dt; a.batch = batch; a.seq = seq; a.n_q = c->sh.nq; a.n_kv = c->sh.nkv; a.d = c->sh.d;
  RP_CHECK(ws_bytes >= attn_bwd_ws_bytes(a), RP_ERR_WORKSPACE, "op_attn_bwd: workspace too small");
  return attn_bwd(a, qkv, o, dout, lse, (float*)ws, dqkv, c->compute);
}

rp_status rp_op_attn_bwd_noalloc(rp_ctx* c, int batch, int seq, const void* qkv, const void* o, const void* dout,
                                 const float* lse, void* dqkv) {
  CTX_ENTER(c);
  RP_CHECK(batch >= 1 && seq >= 1 && qkv && o && dout && lse && dqkv, RP_ERR_INVALID,
           "op_attn_bwd_noalloc: bad arguments");
  AttnDesc a;
  a.dt = c->sh.dt; a.batch = batch; a.seq = seq; a.n_q = c->sh.nq; a.n_kv = c->sh.nkv; a.d = c->sh.d;
  RP_CHECK(attn_bwd_ws_bytes(a) <= kAttnScratchFloats * sizeof(float), RP_ERR_UNSUPPORTED,
           "op_attn_bwd_noalloc: n_q * batch * seq = %lld exceeds the fixed scratch of %zu rows",
           (long long)a.n_q * batch * seq, kAttnScratchFloats);
  RP_CHECK(c->attn_scratch != nullptr, RP_ERR_STATE, "op_attn_bwd_noalloc: no scratch address");
  return attn_bwd(a, qkv, o, dout, lse, c->attn_scratch, dqkv, c->compute);
}

rp_status rp_op_moe_route(rp_ctx* c, int batch, int seq, const float* logits, int32_t* idx, float* wgt,
                          int32_t* cnt, int32_t* off, int32_t* perm_row, float* perm_w, int32_t* inv, void* ws,
                          size_t ws_bytes) {
  CTX_ENTER(c);
  RP_CHECK(c->sh.E > 0, RP_ERR_STATE, "op_moe_route: dense context");
  RP_CHECK(batch >= 1 && seq >= 1, RP_ERR_INVALID, "op_moe_route: bad sizes");
  const int64_t T = (int64_t)batch * seq;
  RP_CHECK(T * c->sh.topk <= INT32_MAX, RP_ERR_UNSUPPORTED, "op_moe_route: too many tokens");
  RP_CHECK(logits && idx && wgt && cnt && off && perm_row && perm_w && inv && ws, RP_ERR_INVALID,
           "op_moe_route: null pointer");
  size_t need = 0;
  RP_TRY(rp_workspace_size(c, RP_OP_MOE_ROUTE, batch, seq, 1, 0, &need));
  RP_CHECK(ws_bytes >= need, RP_ERR_WORKSPACE, "op_moe_route: workspace %zu < %zu bytes", ws_bytes, need);
  MoeRouting m;
  m.max_tiles = moe_max_tiles(T, c->sh.topk, c->sh.E);
  m.idx = idx;
  m.wgt = wgt;
  m.cnt = cnt;
  m.off = off;
  m.tile_e = (int*)ws;
  m.tile_m0 = (int*)((char*)ws + need / 2);
  m.perm_row = perm_row;
  m.perm_w = perm_w;
  m.inv = inv;
  return moe_route(m, logits, (int)T, c->sh.E, c->sh.topk, c->compute);
}

rp_status rp_trace_begin(rp_ctx* c, int max_launches) {
  CTX_ENTER(c);
  RP_CHECK(max_launches >= 1, RP_ERR_INVALID, "trace_begin: max_launches must be >= 1");
  RP_CHECK(!c->trace.on, RP_ERR_STATE, "trace_begin: a trace is already running");
  // events of the previous session are reused once the stream has passed them
  RP_HIP(hipStreamSynchronize(c->compute));
  c->trace.recs.clear();
  c->trace.pool_used = 0;
  c->trace.cap = (size_t)max_launches;
  c->trace.on = true;
  return RP_OK;
}

rp_status rp_trace_end(rp_ctx* c) {
  CTX_ENTER(c);
  c->trace.on = false;
  return RP_OK;
}

rp_status rp_trace_read(rp_ctx* c, rp_trace_rec* out, int cap, int* n) {
  CTX_ENTER(c);
  RP_CHECK(n, RP_ERR_INVALID, "trace_read: null count");
  RP_CHECK(!c->trace.on, RP_ERR_STATE, "trace_read: call rp_trace_end first");
  const size_t nr = c->trace.recs.size();
  *n = (int)nr;
  RP_CHECK(out || nr == 0 || cap == 0, RP_ERR_INVALID, "trace_read: null output");
  if (cap <= 0) return RP_OK;
  RP_CHECK((size_t)cap >= nr, RP_ERR_INVALID, "trace_read: %zu records exceed cap %d", nr, cap);
  for (size_t i = 0; i < nr; ++i) {
    const TraceRec& r = c->trace.recs[i];
    RP_HIP(hipEventSynchronize(r.b));
    float ms = 0.f;
    RP_HIP(hipEventElapsedTime(&ms, r.a, r.b));
    rp_trace_rec& o = out[i];
    memset(&o, 0, sizeof(o));
    snprintf(o.name, sizeof(o.name), "%s", r.name.c_str());
    o.flops = r.flops;
    o.bytes = r.bytes;
    o.ms = ms;
  }
  return RP_OK;
}

}  // extern "C"
