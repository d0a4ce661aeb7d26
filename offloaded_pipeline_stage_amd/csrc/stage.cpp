// Stage executor: the decoder-layer forward, recompute + backward and the
// vocabulary-sharded LM head, expressed as a sequence of kernel launches on
// the context's compute stream, with the checkpoint copies on the activation
// streams (RoundPipe paper, section 2.1.1 full recomputation with layer
// inputs offloaded to host; section 3.2 fused first backward stage;
// section 4.2.1 compute synchronised with the activation streams by events).
#include <algorithm>
#include <cstring>
#include <functional>

#include "ctx.h"

namespace rp {
namespace {

// internals of one layer's forward, kept for its backward
struct Acts {
  void* x = nullptr;      // layer input [T, H]
  float* rstd1 = nullptr; // [T]
  void* a = nullptr;      // RMSNorm1(x) [T, H]
  void* qkv = nullptr;    // [T, QKV], q and k rotated
  void* qkraw = nullptr;  // QK-norm: pre-norm q and k heads [T * (nq + nkv), d]
  float* qkrstd = nullptr; // QK-norm: [T * (nq + nkv)]
  void* o = nullptr;      // attention output [T, Q]
  float* lse = nullptr;   // [nq, T]
  void* h1 = nullptr;     // x + o Wo^T [T, H]
  float* rstd2 = nullptr; // [T]
  void* b = nullptr;      // RMSNorm2(h1) [T, H]
  void* gu = nullptr;     // gate/up pre-activations [T, 2F] (MoE: [T k, 2Fe] grouped rows)
  void* m = nullptr;      // silu(g) * u [T, F] (MoE: [T k, Fe])
  MoeRouting mr;          // MoE routing of this layer's tokens
  // LoRA: s * (a A^T) for q|k|v [T, 3r] and s * (o Ao^T) [T, r], s = alpha / r
  void* us_qkv = nullptr;
  void* us_o = nullptr;
};

// bf16 copies of one layer's LoRA adapters, in the orientation the products use
struct LoraBf16 {
  void* aqkv = nullptr;  // [3r, H]: A_q, A_k, A_v stacked
  void* bq = nullptr;    // [Q, r]
  void* bk = nullptr;    // [KV, r]
  void* bv = nullptr;    // [KV, r]
  void* ao = nullptr;    // [r, Q]
  void* bo = nullptr;    // [H, r]
};

struct BwdTmp {
  void* dgu = nullptr;     // [T, 2F]
  float* gbuf = nullptr;   // fp32 [T, H] (db, then da)
  float* dh1f = nullptr;   // fp32 [T, H]
  void* dh1 = nullptr;     // [T, H]
  void* dO = nullptr;      // [T, Q]
  void* dqkv = nullptr;    // [T, QKV]
  float* Dbuf = nullptr;   // [nq, T]
  float* dm_tmp = nullptr; // fp32 [T, F] (unfused fp32 path)
  float* part = nullptr;   // RMSNorm dgamma partials
  void* g_qkv = nullptr;   // LoRA: dq|dk|dv times B_q|B_k|B_v [T, 3r]
  void* g_o = nullptr;     // LoRA: dh1 B_o [T, r]
  float* splitk = nullptr; // split-K partials of the adapter-gradient products
  size_t splitk_bytes = 0;
  void* dbe = nullptr;     // MoE: input gradients per grouped row [T k, H]
  void* gp[2] = {nullptr, nullptr};  // inter-layer gradients
  void* ck[2] = {nullptr, nullptr};  // uploaded checkpoints
  float* qkpart = nullptr;           // QK-norm gain-gradient partials
};

struct Layout {
  float2* rope = nullptr;
  LoraBf16 lw;
  void* ye = nullptr;     // MoE: expert outputs [T k, H] (grouped rows)
  void* lora_d = nullptr; // LoRA with the rotation fused: us_x B_x^T for q|k|v [T, QKV]
  std::vector<Acts> acts;
  void* xb[2] = {nullptr, nullptr};
  BwdTmp bt;
};

// whether the QKV product applies RoPE in its epilogue: bf16 heads of 128 and
// no QK-norm between the product and the rotation
bool fused_rope(const Shape& s) { return s.dt == RP_DTYPE_BF16 && s.d == 128 && !s.qkn; }

void carve_acts(Bump& bp, const Shape& s, int64_t T, Acts& A) {
  A.x = bp.take(T * s.H * s.es);
  A.rstd1 = bp.take<float>(T * 4);
  A.a = bp.take(T * s.H * s.es);
  A.qkv = bp.take(T * s.QKV * s.es);
  if (s.qkn) {
    A.qkraw = bp.take(T * (s.Q + s.KV) * s.es);
    A.qkrstd = bp.take<float>(T * (s.nq + s.nkv) * 4);
  }
  A.o = bp.take(T * s.Q * s.es);
  A.lse = bp.take<float>((size_t)s.nq * T * 4);
  A.h1 = bp.take(T * s.H * s.es);
  A.rstd2 = bp.take<float>(T * 4);
  A.b = bp.take(T * s.H * s.es);
  const int64_t rows = s.E > 0 ? T * s.topk : T;  // MLP rows (grouped rows for MoE)
  const int64_t F = s.E > 0 ? s.Fe : s.F;
  A.gu = bp.take(rows * 2 * F * s.es);
  A.m = bp.take(rows * F * s.es);
  if (s.E > 0) {
    MoeRouting& m = A.mr;
    m.max_tiles = moe_max_tiles(T, s.topk, s.E);
    m.idx = bp.take<int>(rows * 4);
    m.wgt = bp.take<float>(rows * 4);
    m.cnt = bp.take<int>((size_t)s.E * 4);
    m.off = bp.take<int>((size_t)(s.E + 1) * 4);
    m.tile_e = bp.take<int>((size_t)m.max_tiles * 4);
    m.tile_m0 = bp.take<int>((size_t)m.max_tiles * 4);
    m.perm_row = bp.take<int>(rows * 4);
    m.perm_w = bp.take<float>(rows * 4);
    m.inv = bp.take<int>(rows * 4);
  }
  if (s.r > 0) {
    A.us_qkv = bp.take(T * 3 * s.r * s.es);
    A.us_o = bp.take(T * s.r * s.es);
  }
}

// split-K partial scratch of the adapter-gradient products
constexpr size_t kLoraSplitBytes = 64u << 20;

// mode bits: 1 = keep all layers' internals, 2 = backward temporaries, 4 = fwd ping-pong
void carve(Bump& bp, const Shape& s, int64_t T, int seq, int n_layers, bool keep, bool bwd, bool fwd_pp,
           Layout& L) {
  L.rope = bp.take<float2>((size_t)seq * (s.d / 2) * sizeof(float2));
  if (s.r > 0) {
    const size_t r = s.r, e = s.es;
    L.lw.aqkv = bp.take(3 * r * s.H * e);
    L.lw.bq = bp.take((size_t)s.Q * r * e);
    L.lw.bk = bp.take((size_t)s.KV * r * e);
    L.lw.bv = bp.take((size_t)s.KV * r * e);
    L.lw.ao = bp.take(r * s.Q * e);
    L.lw.bo = bp.take((size_t)s.H * r * e);
  }
  L.acts.assign(keep ? n_layers : 1, Acts{});
  for (auto& a : L.acts) carve_acts(bp, s, T, a);
  if (s.E > 0) L.ye = bp.take(T * s.topk * s.H * s.es);
  if (s.r > 0 && fused_rope(s)) L.lora_d = bp.take(T * s.QKV * s.es);
  if (fwd_pp) {
    L.xb[0] = bp.take(T * s.H * s.es);
    L.xb[1] = bp.take(T * s.H * s.es);
  }
  if (bwd) {
    BwdTmp& b = L.bt;
    if (s.E > 0) {
      b.dgu = bp.take(T * s.topk * 2 * s.Fe * s.es);
      b.dbe = bp.take(T * s.topk * s.H * s.es);
    } else {
      b.dgu = bp.take(T * 2 * s.F * s.es);
    }
    b.gbuf = bp.take<float>(T * s.H * 4);
    b.dh1f = bp.take<float>(T * s.H * 4);
    b.dh1 = bp.take(T * s.H * s.es);
    b.dO = bp.take(T * s.Q * s.es);
    b.dqkv = bp.take(T * s.QKV * s.es);
    b.Dbuf = bp.take<float>((size_t)s.nq * T * 4);
    if (s.dt == RP_DTYPE_F32) b.dm_tmp = bp.take<float>(T * s.F * 4);
    b.part = bp.take<float>(rmsnorm_bwd_part_bytes((int)T, s.H));
    if (s.qkn) b.qkpart = bp.take<float>(qknorm_part_bytes((int)T, s.nq + s.nkv, s.d));
    if (s.r > 0) {
      b.g_qkv = bp.take(T * 3 * s.r * s.es);
      b.g_o = bp.take(T * s.r * s.es);
      b.splitk = bp.take<float>(kLoraSplitBytes);
      b.splitk_bytes = kLoraSplitBytes;
    }
    b.gp[0] = bp.take(T * s.H * s.es);
    b.gp[1] = bp.take(T * s.H * s.es);
    b.ck[0] = bp.take(T * s.H * s.es);
    b.ck[1] = bp.take(T * s.H * s.es);
  }
}

inline const char* wptr(const Slot& s, const rp_layer_cfg& cfg, int tensor) {
  size_t off = 0, bytes = 0;
  block_layout(cfg, RP_BLOCK_WEIGHT, tensor, &off, &bytes, nullptr);
  return (const char*)s.w + off;
}
inline float* gptr(const Slot& s, const rp_layer_cfg& cfg, int tensor) {
  size_t off = 0, bytes = 0;
  block_layout(cfg, RP_BLOCK_GRAD, tensor, &off, &bytes, nullptr);
  return (float*)((char*)s.g + off);
}

inline const float* lptr(const Slot& s, const rp_layer_cfg& cfg, int tensor) {
  size_t off = 0, bytes = 0;
  block_layout(cfg, RP_BLOCK_LORA, tensor, &off, &bytes, nullptr);
  return (const float*)((const char*)s.w + off);
}
inline float* lgptr(const Slot& s, const rp_layer_cfg& cfg, int tensor) {
  size_t off = 0, bytes = 0;
  block_layout(cfg, RP_BLOCK_LORA, tensor, &off, &bytes, nullptr);
  return (float*)((char*)s.g + off);
}

// the layer's fp32 adapters -> bf16 operand copies
rp_status lora_cast(rp_ctx* c, const Slot& ls, const LoraBf16& lw, hipStream_t st) {
  const Shape& s = c->sh;
  const rp_layer_cfg& cfg = c->cfg;
  const size_t r = s.r, rh = r * s.H;
  char* aqkv = (char*)lw.aqkv;
  RP_TRY(cast_from_f32(s.dt, lptr(ls, cfg, RP_T_AQ), aqkv, rh, st));
  RP_TRY(cast_from_f32(s.dt, lptr(ls, cfg, RP_T_AK), aqkv + rh * s.es, rh, st));
  RP_TRY(cast_from_f32(s.dt, lptr(ls, cfg, RP_T_AV), aqkv + 2 * rh * s.es, rh, st));
  RP_TRY(cast_from_f32(s.dt, lptr(ls, cfg, RP_T_BQ), lw.bq, (size_t)s.Q * r, st));
  RP_TRY(cast_from_f32(s.dt, lptr(ls, cfg, RP_T_BK), lw.bk, (size_t)s.KV * r, st));
  RP_TRY(cast_from_f32(s.dt, lptr(ls, cfg, RP_T_BV), lw.bv, (size_t)s.KV * r, st));
  RP_TRY(cast_from_f32(s.dt, lptr(ls, cfg, RP_T_AO), lw.ao, r * s.Q, st));
  RP_TRY(cast_from_f32(s.dt, lptr(ls, cfg, RP_T_BO), lw.bo, (size_t)s.H * r, st));
  return RP_OK;
}

GemmDesc mk(int M, int N, int K, const void* A, int64_t lda, bool ak, const void* B, int64_t ldb, bool bk,
            void* C, int64_t ldc, int in_dt, int out_dt, int epi = EPI_STORE) {
  GemmDesc d;
  d.M = M; d.N = N; d.K = K;
  d.A = A; d.lda = lda; d.a_kmajor = ak;
  d.B = B; d.ldb = ldb; d.b_kmajor = bk;
  d.C = C; d.ldc = ldc;
  d.in_dtype = in_dt; d.out_dtype = out_dt; d.epi = epi;
  return d;
}

// forward of one layer: x -> y. With y == nullptr (recomputation before the
// backward) the down projection is skipped: the backward reads the layer's
// internals, never its output. LoRA layers add s (x A^T) B^T to the q, k, v
// and o projections (s = alpha / r), in place on the bf16 projection output.
rp_status layer_fwd(rp_ctx* c, const LayerBinding& lb, const LoraBf16& lw, void* ye, void* lora_d,
                     const float* router, int T,
                    int seq, const void* x, const Acts& A, void* y, const float2* rope, hipStream_t st,
                    bool keep_gu, const std::function<rp_status()>& after_qkv = {}) {
  const Shape& s = c->sh;
  const int dt = s.dt;
  const rp_layer_cfg& cfg = c->cfg;
  const Slot& w = lb.base;
  const int r = s.r;
  const float ls = r > 0 ? cfg.lora_alpha / (float)r : 0.f;
  RP_TRY(rmsnorm_fwd(dt, x, wptr(w, cfg, RP_T_GAMMA1), A.a, A.rstd1, T, s.H, cfg.rms_eps, st));
  // the rotation of q and k rides in the product's epilogue unless the
  // QK-norm must come between the product and the rotation. LoRA deltas
  // (us_x = s a A_x^T, then us_x B_x^T per part) are computed first and added
  // in that epilogue before the rotation; unfused they are added in place.
  const bool rope_fused = fused_rope(s);
  if (r > 0) {
    RP_TRY(lora_cast(c, lb.lora, lw, st));
    GemmDesc gu = mk(T, 3 * r, s.H, A.a, s.H, true, lw.aqkv, s.H, true, A.us_qkv, 3 * r, dt, dt);
    gu.alpha = ls;
    RP_TRY(gemm(gu, st));
    if (rope_fused) {
      const void* bx[3] = {lw.bq, lw.bk, lw.bv};
      const int nx[3] = {s.Q, s.KV, s.KV}, cx[3] = {0, s.Q, s.Q + s.KV};
      for (int xi = 0; xi < 3; ++xi)
        RP_TRY(gemm(mk(T, nx[xi], r, (const char*)A.us_qkv + (size_t)xi * r * s.es, 3 * r, true, bx[xi], r, true,
                       (char*)lora_d + (size_t)cx[xi] * s.es, s.QKV, dt, dt),
                    st));
    }
  }
  GemmDesc gqkv = mk(T, s.QKV, s.H, A.a, s.H, true, wptr(w, cfg, RP_T_WQKV), s.H, true, A.qkv, s.QKV, dt, dt,
                     rope_fused ? EPI_ROPE : EPI_STORE);
  if (rope_fused) {
    gqkv.rope_tab = rope;
    gqkv.rope_seq = seq;
    gqkv.rope_heads = s.nq + s.nkv;
    if (r > 0) {
      gqkv.R = lora_d;
      gqkv.ldr = s.QKV;
    }
  }
  RP_TRY(gemm(gqkv, st));
  if (after_qkv) RP_TRY(after_qkv());
  if (r > 0 && !rope_fused) {
    // q|k|v += us_x B_x^T in place
    const void* bx[3] = {lw.bq, lw.bk, lw.bv};
    const int nx[3] = {s.Q, s.KV, s.KV}, cx[3] = {0, s.Q, s.Q + s.KV};
    for (int xi = 0; xi < 3; ++xi) {
      char* col = (char*)A.qkv + (size_t)cx[xi] * s.es;
      GemmDesc g = mk(T, nx[xi], r, (const char*)A.us_qkv + (size_t)xi * r * s.es, 3 * r, true, bx[xi], r, true, col,
                      s.QKV, dt, dt, EPI_RESID);
      g.R = col; g.ldr = s.QKV;
      RP_TRY(gemm(g, st));
    }
  }
  if (s.qkn)
    RP_TRY(qknorm_rope_fwd(dt, A.qkv, s.QKV, A.qkraw, A.qkrstd, wptr(w, cfg, RP_T_QNORM), wptr(w, cfg, RP_T_KNORM), T,
                           seq, s.nq, s.nkv, s.d, rope, cfg.rms_eps, st));
  else if (!rope_fused)
    RP_TRY(rope_apply(dt, A.qkv, s.QKV, T, seq, s.nq + s.nkv, s.d, rope, false, st));
  AttnDesc ad;
  ad.dt = dt; ad.batch = T / seq; ad.seq = seq; ad.n_q = s.nq; ad.n_kv = s.nkv; ad.d = s.d;
  RP_TRY(attn_fwd(ad, A.qkv, A.o, A.lse, st));
  GemmDesc go = mk(T, s.H, s.Q, A.o, s.Q, true, wptr(w, cfg, RP_T_WO), s.Q, true, A.h1, s.H, dt, dt, EPI_RESID);
  go.R = x; go.ldr = s.H;
  RP_TRY(gemm(go, st));
  if (r > 0) {
    // us_o = s o A_o^T ; h1 += us_o B_o^T
    GemmDesc gu = mk(T, r, s.Q, A.o, s.Q, true, lw.ao, s.Q, true, A.us_o, r, dt, dt);
    gu.alpha = ls;
    RP_TRY(gemm(gu, st));
    GemmDesc g = mk(T, s.H, r, A.us_o, r, true, lw.bo, r, true, A.h1, s.H, dt, dt, EPI_RESID);
    g.R = A.h1; g.ldr = s.H;
    RP_TRY(gemm(g, st));
  }
  RP_TRY(rmsnorm_fwd(dt, A.h1, wptr(w, cfg, RP_T_GAMMA2), A.b, A.rstd2, T, s.H, cfg.rms_eps, st));
  if (s.E > 0) {
    // MoE: route, then per expert gu = b_e W_gu,e^T with the SwiGLU epilogue
    // (rows of b gathered through the routing), ye = m_e W_d,e^T, and
    // y = h1 + sum_s w_s ye[row(t, s)]
    const int k = s.topk, Fe = s.Fe;
    RP_TRY(moe_route(A.mr, router, T, s.E, k, st));
    GemmGroup grp;
    grp.tile_e = A.mr.tile_e; grp.tile_m0 = A.mr.tile_m0; grp.off = A.mr.off; grp.cnt = A.mr.cnt;
    grp.max_tiles_m = A.mr.max_tiles;
    grp.rows = A.mr.perm_row;
    grp.a_rows = T;
    grp.b_stride = (int64_t)2 * Fe * s.H;
    GemmDesc gg = mk(T * k, 2 * Fe, s.H, A.b, s.H, true, wptr(w, cfg, RP_T_WGU), s.H, true, A.gu, 2 * Fe, dt, dt,
                     EPI_SWIGLU);
    gg.C2 = A.m; gg.ldc2 = Fe;
    gg.c_unused = !keep_gu;
    gg.group = &grp;
    RP_TRY(gemm_grouped(gg, st));
    if (y == nullptr) return RP_OK;
    GemmGroup g2 = grp;
    g2.rows = nullptr;
    g2.a_rows = (int64_t)T * k;
    g2.b_stride = (int64_t)s.H * Fe;
    GemmDesc gd = mk(T * k, s.H, Fe, A.m, Fe, true, wptr(w, cfg, RP_T_WD), Fe, true, ye, s.H, dt, dt);
    gd.group = &g2;
    RP_TRY(gemm_grouped(gd, st));
    return moe_combine(A.h1, ye, A.mr, T, k, s.H, y, st);
  }
  GemmDesc gg = mk(T, 2 * s.F, s.H, A.b, s.H, true, wptr(w, cfg, RP_T_WGU), s.H, true, A.gu, 2 * s.F, dt, dt,
                   EPI_SWIGLU);
  gg.C2 = A.m; gg.ldc2 = s.F;
  gg.c_unused = !keep_gu;  // the pre-activations are read only by a backward
  RP_TRY(gemm(gg, st));
  if (y == nullptr) return RP_OK;
  GemmDesc gd = mk(T, s.H, s.F, A.m, s.F, true, wptr(w, cfg, RP_T_WD), s.F, true, y, s.H, dt, dt, EPI_RESID);
  gd.R = A.h1; gd.ldr = s.H;
  RP_TRY(gemm(gd, st));
  return RP_OK;
}

// `to` waits for the work enqueued on `from` so far. The event is recorded
// and waited on at once, so one event serves every such fork and join.
rp_status stream_fork(rp_ctx* c, hipStream_t from, hipStream_t to) {
  if (c->side_ev.empty()) {
    hipEvent_t e = c->new_event();
    RP_CHECK(e != nullptr, RP_ERR_HIP, "event creation failed");
    c->side_ev.push_back(e);
  }
  RP_HIP(hipEventRecord(c->side_ev[0], from));
  RP_HIP(hipStreamWaitEvent(to, c->side_ev[0], 0));
  return RP_OK;
}

// a weight-gradient product dW = X^T Y (X M-major; Y M-major, or K-major
// when b_kmajor: Y^T stored [N, K]; fp32 out), added to dW when
// accumulating over micro-batches
rp_status wgrad(int M, int N, int K, const void* A, int64_t lda, const void* Bm, int64_t ldb, float* C, int64_t ldc,
                int dt, const BwdTmp& B, float alpha, bool accum, hipStream_t st, bool b_kmajor = false) {
  GemmDesc g = mk(M, N, K, A, lda, false, Bm, ldb, b_kmajor, C, ldc, dt, RP_DTYPE_F32);
  g.accumulate = accum;
  g.alpha = alpha;
  if (B.splitk) {
    g.split_k = 0;  // automatic for the skinny adapter products
    g.partial = B.splitk;
    g.partial_bytes = B.splitk_bytes;
  }
  return gemm(g, st);
}

// backward of one layer from its forward internals: dy -> dx and the weight
// gradients (every weight and gain for a full fine-tune; with LoRA the base is
// frozen and only the adapters get gradients), written or, with accum, added
// to the gradient block
rp_status layer_bwd(rp_ctx* c, LayerBinding& lb, const LoraBf16& lw, int T, int seq, const void* x, const Acts& A,
                    const BwdTmp& B, const void* dy, void* dx, const float2* rope, bool accum, hipStream_t st) {
  const Shape& s = c->sh;
  const int dt = s.dt;
  const rp_layer_cfg& cfg = c->cfg;
  Slot& w = lb.base;
  const int r = s.r;
  const bool full = r == 0;  // full fine-tune: base weights are trainable
  const float ls = r > 0 ? cfg.lora_alpha / (float)r : 0.f;
  Slot& gs = full ? w : lb.lora;  // the slot whose gradient block this backward writes
  const int F2 = 2 * s.F;
  RP_TRY(wait_grad_drained(c, gs));
  if (r > 0) RP_TRY(lora_cast(c, lb.lora, lw, st));
  if (s.E > 0) {
    // MoE with frozen experts: input gradient only. Per expert
    // dgu = SwiGLU'(w_s dy_e W_d,e) (routing weight as a row factor, rows of
    // dy gathered through the routing), dbe = dgu W_gu,e, db = sum_s dbe.
    const int k = s.topk, Fe = s.Fe;
    GemmGroup grp;
    grp.tile_e = A.mr.tile_e; grp.tile_m0 = A.mr.tile_m0; grp.off = A.mr.off; grp.cnt = A.mr.cnt;
    grp.max_tiles_m = A.mr.max_tiles;
    grp.rows = A.mr.perm_row;
    grp.a_rows = T;
    grp.b_stride = (int64_t)s.H * Fe;
    GemmDesc g1 = mk(T * k, Fe, s.H, dy, s.H, true, wptr(w, cfg, RP_T_WD), Fe, false, B.dgu, 2 * Fe, dt, dt,
                     EPI_SWIGLU_BWD);
    g1.R = A.gu; g1.ldr = 2 * Fe;
    g1.row_scale = A.mr.perm_w;
    g1.group = &grp;
    RP_TRY(gemm_grouped(g1, st));
    GemmGroup g2 = grp;
    g2.rows = nullptr;
    g2.a_rows = (int64_t)T * k;
    g2.b_stride = (int64_t)2 * Fe * s.H;
    GemmDesc gb = mk(T * k, s.H, 2 * Fe, B.dgu, 2 * Fe, true, wptr(w, cfg, RP_T_WGU), s.H, false, B.dbe, s.H, dt, dt);
    gb.group = &g2;
    RP_TRY(gemm_grouped(gb, st));
    RP_TRY(moe_uncombine(B.dbe, A.mr, T, k, s.H, B.gbuf, st));
  } else {
    // dWgu = dgu^T b reads b as a K-major operand once b is transposed: on
    // the side stream, beside the products before it, into dh1, which is
    // free until the RMSNorm backward below
    const bool b_tr = full && dt == RP_DTYPE_BF16 && T % 8 == 0 && s.H % 8 == 0;
    if (b_tr) {
      RP_TRY(stream_fork(c, st, c->side));
      RP_TRY(transpose_bf16(A.b, s.H, B.dh1, T, T, s.H, c->side));
    }
    // MLP: dm = dy Wd -> dgu (fused SwiGLU backward)
    GemmDesc g1 = mk(T, s.F, s.H, dy, s.H, true, wptr(w, cfg, RP_T_WD), s.F, false, B.dgu, F2, dt, dt,
                     EPI_SWIGLU_BWD);
    g1.R = A.gu; g1.ldr = F2; g1.tmp = B.dm_tmp;
    RP_TRY(gemm(g1, st));
    // dWd = dy^T m
    if (full) RP_TRY(wgrad(s.H, s.F, T, dy, s.H, A.m, s.F, gptr(w, cfg, RP_T_WD), s.F, dt, B, 1.f, accum, st));
    // db = dgu Wgu
    RP_TRY(gemm(mk(T, s.H, F2, B.dgu, F2, true, wptr(w, cfg, RP_T_WGU), s.H, false, B.gbuf, s.H, dt, RP_DTYPE_F32),
                st));
    // dWgu = dgu^T b
    if (b_tr) {
      RP_TRY(stream_fork(c, c->side, st));
      RP_TRY(wgrad(F2, s.H, T, B.dgu, F2, B.dh1, T, gptr(w, cfg, RP_T_WGU), s.H, dt, B, 1.f, accum, st, true));
    } else if (full) {
      RP_TRY(wgrad(F2, s.H, T, B.dgu, F2, A.b, s.H, gptr(w, cfg, RP_T_WGU), s.H, dt, B, 1.f, accum, st));
    }
  }
  // dh1 = dy + RMSNorm2^T db ; dgamma2
  RP_TRY(rmsnorm_bwd(dt, B.gbuf, A.h1, wptr(w, cfg, RP_T_GAMMA2), A.rstd2, dy, dt, B.dh1f, B.dh1,
                     full ? gptr(w, cfg, RP_T_GAMMA2) : nullptr, accum, B.part, T, s.H, st));
  // attention output projection: dO = dh1 Wo ; dWo = dh1^T o
  RP_TRY(gemm(mk(T, s.Q, s.H, B.dh1, s.H, true, wptr(w, cfg, RP_T_WO), s.Q, false, B.dO, s.Q, dt, dt), st));
  if (full) RP_TRY(wgrad(s.H, s.Q, T, B.dh1, s.H, A.o, s.Q, gptr(w, cfg, RP_T_WO), s.Q, dt, B, 1.f, accum, st));
  if (r > 0) {
    const Slot& L = lb.lora;
    // g_o = dh1 B_o ; dO += s g_o A_o ; dA_o = s g_o^T o ; dB_o = dh1^T us_o
    RP_TRY(gemm(mk(T, r, s.H, B.dh1, s.H, true, lw.bo, r, false, B.g_o, r, dt, dt), st));
    GemmDesc g = mk(T, s.Q, r, B.g_o, r, true, lw.ao, s.Q, false, B.dO, s.Q, dt, dt, EPI_RESID);
    g.R = B.dO; g.ldr = s.Q; g.alpha = ls;
    RP_TRY(gemm(g, st));
    RP_TRY(wgrad(r, s.Q, T, B.g_o, r, A.o, s.Q, lgptr(L, cfg, RP_T_AO), s.Q, dt, B, ls, accum, st));
    RP_TRY(wgrad(s.H, r, T, B.dh1, s.H, A.us_o, r, lgptr(L, cfg, RP_T_BO), r, dt, B, 1.f, accum, st));
  }
  AttnDesc ad;
  ad.dt = dt; ad.batch = T / seq; ad.seq = seq; ad.n_q = s.nq; ad.n_kv = s.nkv; ad.d = s.d;
  // without QK-norm the rotation's backward rides in the attention
  // backward's dQ and dK stores where the flash kernels run
  const bool fused_rope = rope && !s.qkn && attn_bwd_fuses_rope(ad) && ((uintptr_t)rope & 15) == 0;
  RP_TRY(attn_bwd(ad, A.qkv, A.o, B.dO, A.lse, B.Dbuf, B.dqkv, st, fused_rope ? rope : nullptr));
  if (s.qkn) {
    // the gains are base weights: trained in a full fine-tune, frozen with LoRA;
    // gamma_k's gradient directly follows gamma_q's in the gradient block
    float* dg = full ? gptr(w, cfg, RP_T_QNORM) : nullptr;
    RP_CHECK(!dg || gptr(w, cfg, RP_T_KNORM) == dg + s.d, RP_ERR_STATE, "qk-norm: gain gradients not adjacent");
    RP_TRY(qknorm_rope_bwd(dt, B.dqkv, s.QKV, A.qkraw, A.qkrstd, wptr(w, cfg, RP_T_QNORM), wptr(w, cfg, RP_T_KNORM),
                           T, seq, s.nq, s.nkv, s.d, rope, dg, accum, B.qkpart, st));
  } else if (!fused_rope) {
    RP_TRY(rope_apply(dt, B.dqkv, s.QKV, T, seq, s.nq + s.nkv, s.d, rope, true, st));
  }
  // da = dqkv Wqkv ; dWqkv = dqkv^T a
  RP_TRY(gemm(mk(T, s.H, s.QKV, B.dqkv, s.QKV, true, wptr(w, cfg, RP_T_WQKV), s.H, false, B.gbuf, s.H, dt,
                 RP_DTYPE_F32), st));
  if (full) RP_TRY(wgrad(s.QKV, s.H, T, B.dqkv, s.QKV, A.a, s.H, gptr(w, cfg, RP_T_WQKV), s.H, dt, B, 1.f, accum, st));
  if (r > 0) {
    const Slot& L = lb.lora;
    // g_x = d{q,k,v} B_x ; da += s [g_q g_k g_v] [A_q; A_k; A_v] ;
    // dA_x = s g_x^T a ; dB_x = d{q,k,v}^T us_x
    const void* bx[3] = {lw.bq, lw.bk, lw.bv};
    const int nx[3] = {s.Q, s.KV, s.KV}, cx[3] = {0, s.Q, s.Q + s.KV};
    const int ta[3] = {RP_T_AQ, RP_T_AK, RP_T_AV}, tb[3] = {RP_T_BQ, RP_T_BK, RP_T_BV};
    for (int xi = 0; xi < 3; ++xi) {
      const char* dcol = (const char*)B.dqkv + (size_t)cx[xi] * s.es;
      char* gcol = (char*)B.g_qkv + (size_t)xi * r * s.es;
      RP_TRY(gemm(mk(T, r, nx[xi], dcol, s.QKV, true, bx[xi], r, false, gcol, 3 * r, dt, dt), st));
    }
    GemmDesc g = mk(T, s.H, 3 * r, B.g_qkv, 3 * r, true, lw.aqkv, s.H, false, B.gbuf, s.H, dt, RP_DTYPE_F32);
    g.accumulate = true;
    g.alpha = ls;
    RP_TRY(gemm(g, st));
    for (int xi = 0; xi < 3; ++xi) {
      const char* dcol = (const char*)B.dqkv + (size_t)cx[xi] * s.es;
      const char* gcol = (const char*)B.g_qkv + (size_t)xi * r * s.es;
      const char* ucol = (const char*)A.us_qkv + (size_t)xi * r * s.es;
      RP_TRY(wgrad(r, s.H, T, gcol, 3 * r, A.a, s.H, lgptr(L, cfg, ta[xi]), s.H, dt, B, ls, accum, st));
      RP_TRY(wgrad(nx[xi], r, T, dcol, s.QKV, ucol, 3 * r, lgptr(L, cfg, tb[xi]), r, dt, B, 1.f, accum, st));
    }
  }
  // dx = dh1 + RMSNorm1^T da ; dgamma1
  RP_TRY(rmsnorm_bwd(dt, B.gbuf, x, wptr(w, cfg, RP_T_GAMMA1), A.rstd1, B.dh1f, RP_DTYPE_F32, nullptr, dx,
                     full ? gptr(w, cfg, RP_T_GAMMA1) : nullptr, accum, B.part, T, s.H, st));
  RP_TRY(mark_consumed(c, w));
  if (r > 0) RP_TRY(mark_consumed(c, lb.lora));
  RP_TRY(mark_grad_ready(c, gs));
  return RP_OK;
}

// A call that used workspace ws records when the compute stream is done with
// it. The table is bounded: past 64 workspaces it starts over, and a
// workspace without an entry is treated as in use up to the current point.
rp_status ws_mark(rp_ctx* c, const void* ws) {
  if (c->ws_done.size() >= 64 && !c->ws_done.count(ws)) {
    for (auto& kv : c->ws_done) c->ev_free.push_back(kv.second);
    c->ws_done.clear();
  }
  hipEvent_t& e = c->ws_done[ws];
  if (!e) e = c->new_event();
  RP_HIP(hipEventRecord(e, c->compute));
  return RP_OK;
}

rp_status check_range(rp_ctx* c, int l0, int l1, int batch, int seq) {
  RP_CHECK(l0 >= 0 && l1 > l0 && l1 <= (int)c->layers.size(), RP_ERR_INVALID,
           "layer range [%d, %d) invalid or not bound", l0, l1);
  for (int l = l0; l < l1; ++l)
    RP_CHECK(c->layers[l].bound, RP_ERR_INVALID, "layer %d is not bound", l);
  RP_CHECK(batch >= 1 && seq >= 1, RP_ERR_INVALID, "batch and seq must be >= 1");
  RP_CHECK((int64_t)batch * seq < (int64_t)1 << 30, RP_ERR_UNSUPPORTED, "too many tokens");
  return RP_OK;
}

}  // namespace

rp_status stage_fwd(rp_ctx* c, int l0, int l1, int batch, int seq, const void* x_in, void* y_out,
                    void* const* ckpt_host, const float* const* router, int flags, void* ws, size_t ws_bytes,
                    size_t* need) {
  const Shape& s = c->sh;
  const bool keep = flags & RP_KEEP_ACTS;
  const int n = l1 - l0;
  const int64_t T = (int64_t)batch * seq;
  Layout L;
  Bump bp(need ? nullptr : ws);
  carve(bp, s, T, seq, n, keep, keep, !keep, L);
  if (need) {
    *need = bp.off;
    return RP_OK;
  }
  RP_TRY(check_range(c, l0, l1, batch, seq));
  RP_CHECK(x_in && y_out && ws, RP_ERR_INVALID, "stage_fwd: null pointer");
  RP_CHECK(x_in != y_out, RP_ERR_INVALID, "stage_fwd: y_out may not alias x_in");
  if (s.E > 0) {
    RP_CHECK(router != nullptr, RP_ERR_INVALID, "stage_fwd: MoE layers need router logits");
    for (int i = 0; i < n; ++i) RP_CHECK(router[i] != nullptr, RP_ERR_INVALID, "stage_fwd: router %d is null", i);
  }
  RP_CHECK(ws_bytes >= bp.off, RP_ERR_WORKSPACE, "stage_fwd: workspace %zu < %zu bytes", ws_bytes, bp.off);
  if (ckpt_host)
    for (int i = 0; i < n; ++i)
      RP_CHECK(ckpt_host[i] && is_pinned_host(ckpt_host[i]), RP_ERR_NOT_PINNED,
               "stage_fwd: checkpoint %d is not pinned host memory", i);
  hipStream_t st = c->compute;
  if (c->last_act_d2h_valid) RP_HIP(hipStreamWaitEvent(st, c->last_act_d2h, 0));
  RP_TRY(rope_table(L.rope, seq, s.d, c->cfg.rope_base, st));
  const size_t xbytes = (size_t)T * s.H * s.es;
  if (keep) RP_HIP(hipMemcpyAsync(L.acts[0].x, x_in, xbytes, hipMemcpyDeviceToDevice, st));
  std::vector<hipEvent_t> d2h_done(n, nullptr);
  for (int i = 0; i < n; ++i) {
    const int l = l0 + i;
    LayerBinding& lb = c->layers[l];
    Slot& w = lb.base;
    RP_TRY(wait_weights(c, w));
    if (s.r > 0) RP_TRY(wait_weights(c, lb.lora));
    const Acts& A = keep ? L.acts[i] : L.acts[0];
    const void* x = keep ? A.x : (i == 0 ? x_in : L.xb[(i - 1) & 1]);
    void* y = (i == n - 1) ? y_out : (keep ? L.acts[i + 1].x : L.xb[i & 1]);
    // the checkpoint download of this layer's input, issued once the layer's
    // QKV product is enqueued: the runtime copies device to host with a
    // blit kernel that takes CUs while it runs, and started with the layer
    // it starved the first RMSNorm; the input stays intact until the layer's
    // residual add, after the download has been ordered
    auto download_ckpt = [&]() -> rp_status {
      if (!ckpt_host) return RP_OK;
      int64_t tk;
      RP_TRY(act_copy(c, RP_D2H, ckpt_host[i], x, xbytes, &tk));
      d2h_done[i] = c->ticket_ev[tk];
      // later calls rewrite this workspace: they start after the download
      if (!c->last_act_d2h) c->last_act_d2h = c->new_event();
      RP_HIP(hipEventRecord(c->last_act_d2h, c->act_d2h));
      c->last_act_d2h_valid = true;
      return RP_OK;
    };
    // the ping-pong buffer written by this layer held the input of layer
    // i - 1, whose checkpoint download must have finished
    if (!keep && ckpt_host && i >= 1 && i != n - 1) RP_HIP(hipStreamWaitEvent(st, d2h_done[i - 1], 0));
    RP_TRY(layer_fwd(c, lb, L.lw, L.ye, L.lora_d, s.E > 0 ? router[i] : nullptr, (int)T, seq, x, A, y, L.rope, st,
                     keep, download_ckpt));
    RP_TRY(mark_consumed(c, w));
    if (s.r > 0) RP_TRY(mark_consumed(c, lb.lora));
  }
  if (keep) {
    c->kept_ws = ws;
    c->kept_l0 = l0; c->kept_l1 = l1; c->kept_batch = batch; c->kept_seq = seq;
  } else if (c->kept_ws == ws) {
    c->kept_ws = nullptr;
  }
  return ws_mark(c, ws);
}

rp_status stage_bwd(rp_ctx* c, int l0, int l1, int batch, int seq, const void* const* ckpt, const void* dy,
                    void* dx, const float* const* router, int flags, void* ws, size_t ws_bytes, size_t* need) {
  const Shape& s = c->sh;
  const bool kept = flags & RP_USE_KEPT_ACTS;
  const bool ck_dev = flags & RP_CKPT_DEVICE;
  const bool accum = flags & RP_ACCUM_GRADS;
  const int n = l1 - l0;
  const int64_t T = (int64_t)batch * seq;
  Layout L;
  Bump bp(need ? nullptr : ws);
  carve(bp, s, T, seq, n, kept, true, false, L);
  if (need) {
    *need = bp.off;
    return RP_OK;
  }
  RP_TRY(check_range(c, l0, l1, batch, seq));
  RP_CHECK(dy && dx && ws, RP_ERR_INVALID, "stage_bwd: null pointer");
  RP_CHECK(s.E == 0 || s.r > 0, RP_ERR_UNSUPPORTED,
           "stage_bwd: MoE expert weights are frozen here; MoE layers train through LoRA adapters");
  if (s.E > 0 && !kept) {
    RP_CHECK(router != nullptr, RP_ERR_INVALID, "stage_bwd: recomputing MoE layers needs router logits");
    for (int i = 0; i < n; ++i) RP_CHECK(router[i] != nullptr, RP_ERR_INVALID, "stage_bwd: router %d is null", i);
  }
  RP_CHECK(ws_bytes >= bp.off, RP_ERR_WORKSPACE, "stage_bwd: workspace %zu < %zu bytes", ws_bytes, bp.off);
  if (kept) {
    RP_CHECK(c->kept_ws == ws && c->kept_l0 == l0 && c->kept_l1 == l1 && c->kept_batch == batch &&
                 c->kept_seq == seq, RP_ERR_STATE,
             "stage_bwd: no activations kept for layers [%d, %d) on this workspace", l0, l1);
  } else {
    RP_CHECK(ckpt != nullptr, RP_ERR_INVALID, "stage_bwd: checkpoints required without RP_USE_KEPT_ACTS");
    for (int i = 0; i < n; ++i) {
      RP_CHECK(ckpt[i] != nullptr, RP_ERR_INVALID, "stage_bwd: checkpoint %d is null", i);
      if (!ck_dev)
        RP_CHECK(is_pinned_host(ckpt[i]), RP_ERR_NOT_PINNED, "stage_bwd: checkpoint %d is not pinned", i);
    }
  }
  for (int l = l0; l < l1; ++l) {
    if (s.r > 0)
      RP_CHECK(c->layers[l].lora.w != nullptr && c->layers[l].lora.g != nullptr, RP_ERR_INVALID,
               "stage_bwd: layer %d has no LoRA adapter / adapter-gradient buffer", l);
    else
      RP_CHECK(c->layers[l].base.g != nullptr, RP_ERR_INVALID, "stage_bwd: layer %d has no gradient buffer", l);
  }
  hipStream_t st = c->compute;
  if (c->last_act_d2h_valid) RP_HIP(hipStreamWaitEvent(st, c->last_act_d2h, 0));
  RP_TRY(rope_table(L.rope, seq, s.d, c->cfg.rope_base, st));
  const size_t xbytes = (size_t)T * s.H * s.es;
  // checkpoint uploads: layer i's input into ck[i & 1], one layer ahead
  bool ck_read[2] = {false, false};  // buffer i & 1 has been read by this call
  auto upload = [&](int i) -> rp_status {
    if (kept || ck_dev) return RP_OK;
    if (ck_read[i & 1]) RP_HIP(hipStreamWaitEvent(c->act_h2d, c->ck_free[i & 1], 0));
    int64_t tk;
    return act_copy(c, RP_H2D, L.bt.ck[i & 1], ckpt[i], xbytes, &tk);
  };
  // the checkpoints may have been written to host memory by this context's
  // earlier downloads (the forward stage): uploads start after those
  if (!kept && !ck_dev && c->last_act_d2h_valid) RP_HIP(hipStreamWaitEvent(c->act_h2d, c->last_act_d2h, 0));
  // the upload buffers live in ws, which earlier work on the compute stream
  // (the previous call on the same workspace) may still be reading: uploads
  // into them start after that work
  if (!kept && !ck_dev) {
    auto it = c->ws_done.find(ws);
    if (it != c->ws_done.end()) {
      RP_HIP(hipStreamWaitEvent(c->act_h2d, it->second, 0));
    } else {
      if (!c->ev_mark) c->ev_mark = c->new_event();
      RP_HIP(hipEventRecord(c->ev_mark, st));
      RP_HIP(hipStreamWaitEvent(c->act_h2d, c->ev_mark, 0));
    }
  }
  // act_copy(H2D) makes the compute stream wait at issue time, so the
  // prefetch of layer i - 1 is issued after layer i's compute is enqueued.
  if (!kept && !ck_dev) RP_TRY(upload(n - 1));
  const void* g_in = dy;
  for (int i = n - 1; i >= 0; --i) {
    const int l = l0 + i;
    LayerBinding& lb = c->layers[l];
    RP_TRY(wait_weights(c, lb.base));
    if (s.r > 0) RP_TRY(wait_weights(c, lb.lora));
    const Acts& A = kept ? L.acts[i] : L.acts[0];
    const void* x;
    if (kept) {
      x = A.x;
    } else {
      x = ck_dev ? ckpt[i] : L.bt.ck[i & 1];
      // recompute the forward from the checkpoint (same kernels as the forward)
      RP_TRY(layer_fwd(c, lb, L.lw, L.ye, L.lora_d, s.E > 0 ? router[i] : nullptr, (int)T, seq, x, A, nullptr, L.rope,
                       st, true));
    }
    // inter-layer gradients alternate gp[0], gp[1]; the stage input's goes to dx
    void* g_out = (i == 0) ? dx : L.bt.gp[(n - 1 - i) & 1];
    RP_TRY(layer_bwd(c, lb, L.lw, (int)T, seq, x, A, L.bt, g_in, g_out, L.rope, accum, st));
    if (!kept && !ck_dev) {
      if (!c->ck_free[i & 1]) c->ck_free[i & 1] = c->new_event();
      RP_HIP(hipEventRecord(c->ck_free[i & 1], st));
      ck_read[i & 1] = true;
      if (i >= 1) RP_TRY(upload(i - 1));
    }
    g_in = g_out;
  }
  return ws_mark(c, ws);
}

// ---------------------------------------------------------------------------
// LM head
// ---------------------------------------------------------------------------
rp_status lmhead(rp_ctx* c, int batch, int seq, const void* x, const int32_t* labels, float* loss, void* dx,
                 void* ws, size_t ws_bytes, size_t* need) {
  const Shape& s = c->sh;
  const int64_t T = (int64_t)batch * seq;
  const int ns = c->n_shards;
  int vs_max = 0;
  for (int i = 0; i < ns; ++i) vs_max = std::max(vs_max, c->shard_lo[i + 1] - c->shard_lo[i]);
  const bool fnorm = c->final_norm.w != nullptr;
  Bump bp(need ? nullptr : ws);
  void* z = fnorm ? bp.take(T * s.H * s.es) : nullptr;
  float* rstd = bp.take<float>(T * 4);
  float* logits = bp.take<float>((size_t)ns * T * vs_max * 4);
  float2* parts = bp.take<float2>((size_t)ns * T * sizeof(float2));
  float* zlab = bp.take<float>(T * 4);
  float* lse = bp.take<float>(T * 4);
  float* inv_n = bp.take<float>(4);
  void* dzb[2] = {bp.take(T * vs_max * s.es), bp.take(T * vs_max * s.es)};
  float* dxf = bp.take<float>(T * s.H * 4);
  float* part = bp.take<float>(rmsnorm_bwd_part_bytes((int)T, s.H));
  // x^T [H, T] for the weight-gradient products (bf16, sizes in multiples of 8)
  const bool xt_fit = s.dt == RP_DTYPE_BF16 && T % 8 == 0 && s.H % 8 == 0;
  void* zt = xt_fit ? bp.take(T * s.H * s.es) : nullptr;
  if (need) {
    *need = bp.off;
    return RP_OK;
  }
  RP_CHECK(ns > 0, RP_ERR_STATE, "lmhead: no LM head bound");
  RP_CHECK(batch >= 1 && seq >= 1, RP_ERR_INVALID, "lmhead: batch and seq must be >= 1");
  RP_CHECK(x && labels && loss && dx && ws, RP_ERR_INVALID, "lmhead: null pointer");
  RP_CHECK(ws_bytes >= bp.off, RP_ERR_WORKSPACE, "lmhead: workspace %zu < %zu bytes", ws_bytes, bp.off);
  hipStream_t st = c->compute;
  const int dt = s.dt;
  if (c->last_act_d2h_valid) RP_HIP(hipStreamWaitEvent(st, c->last_act_d2h, 0));
  const void* zz = x;
  if (fnorm) {
    RP_TRY(wait_weights(c, c->final_norm));
    RP_TRY(rmsnorm_fwd(dt, x, c->final_norm.w, z, rstd, (int)T, s.H, c->cfg.rms_eps, st));
    zz = z;
  }
  // Each shard's statistics run in line after its logits product (beside
  // the next one they slowed it by as much as they take alone, and the two
  // stream hops cost more); each shard's dz runs on the side stream beside
  // the previous shard's input- and weight-gradient products (dz alternates
  // between two buffers).
  hipStream_t sd = c->side;
  if ((int)c->side_ev.size() < 2 * ns + 3) {
    c->side_ev.resize(2 * ns + 3, nullptr);
    for (hipEvent_t& e : c->side_ev)
      if (!e) {
        e = c->new_event();
        RP_CHECK(e != nullptr, RP_ERR_HIP, "lmhead: event creation failed");
      }
  }
  auto fork = [&](hipStream_t from, hipStream_t to, int k) -> rp_status {  // `to` waits for `from`'s work so far
    RP_HIP(hipEventRecord(c->side_ev[k], from));
    RP_HIP(hipStreamWaitEvent(to, c->side_ev[k], 0));
    return RP_OK;
  };
  // dW_s = dz^T x reads x as a K-major operand once x is transposed (once
  // per call, on the side stream beside the first logits product), so that
  // only dz goes through transposing LDS reads; otherwise both operands are
  // read M-major.
  const bool xt = xt_fit && ((uintptr_t)zz & 15) == 0;
  if (xt) {
    RP_TRY(fork(st, sd, 2 * ns + 2));
    RP_TRY(transpose_bf16(zz, s.H, zt, T, (int)T, s.H, sd));
  }
  RP_TRY(fill_zero(zlab, T * 4, st));
  for (int i = 0; i < ns; ++i) {
    const int lo = c->shard_lo[i], vs = c->shard_lo[i + 1] - lo;
    Slot& w = c->shards[i];
    RP_TRY(wait_weights(c, w));
    float* lg = logits + (size_t)i * T * vs_max;
    RP_TRY(gemm(mk((int)T, vs, s.H, zz, s.H, true, w.w, s.H, true, lg, vs, dt, RP_DTYPE_F32), st));
    RP_TRY(ce_shard_stats(lg, vs, (int)T, vs, lo, labels, c->vocab, parts + (size_t)i * T, zlab, st));
  }
  RP_TRY(fork(sd, st, ns));
  RP_TRY(ce_combine((int)T, ns, parts, zlab, labels, c->vocab, lse, loss, inv_n, st));
  auto grad = [&](int i, hipStream_t on) -> rp_status {
    const int lo = c->shard_lo[i], vs = c->shard_lo[i + 1] - lo;
    return ce_grad(dt, logits + (size_t)i * T * vs_max, vs, (int)T, vs, lo, labels, c->vocab, lse, inv_n,
                   dzb[i & 1], vs, on);
  };
  RP_TRY(grad(0, st));
  for (int i = 0; i < ns; ++i) {
    const int lo = c->shard_lo[i], vs = c->shard_lo[i + 1] - lo;
    Slot& w = c->shards[i];
    RP_CHECK(w.g != nullptr, RP_ERR_INVALID, "lmhead: shard %d has no gradient buffer", i);
    if (i + 1 < ns) {
      // shard i + 1's dz, into the buffer shard i - 1's products read
      RP_TRY(fork(st, sd, ns + 1 + i));
      RP_TRY(grad(i + 1, sd));
    }
    RP_TRY(wait_grad_drained(c, w));
    const void* dz = dzb[i & 1];
    // dX = sum over shards of dz_s W_s: the first shard's product writes dxf
    // (no separate clearing pass), the others add to it
    GemmDesc gx = mk((int)T, s.H, vs, dz, vs, true, w.w, s.H, false, dxf, s.H, dt, RP_DTYPE_F32);
    gx.accumulate = i > 0;
    RP_TRY(gemm(gx, st));
    if (xt)
      RP_TRY(gemm(mk(vs, s.H, (int)T, dz, vs, false, zt, T, true, w.g, s.H, dt, RP_DTYPE_F32), st));
    else
      RP_TRY(gemm(mk(vs, s.H, (int)T, dz, vs, false, zz, s.H, false, w.g, s.H, dt, RP_DTYPE_F32), st));
    RP_TRY(mark_consumed(c, w));
    RP_TRY(mark_grad_ready(c, w));
    if (i + 1 < ns) RP_TRY(fork(sd, st, 2 * ns + 1));  // shard i + 1's dz is ready
  }
  if (fnorm) {
    RP_CHECK(c->final_norm.g != nullptr, RP_ERR_INVALID, "lmhead: final norm has no gradient buffer");
    RP_TRY(wait_grad_drained(c, c->final_norm));
    RP_TRY(rmsnorm_bwd(dt, dxf, x, c->final_norm.w, rstd, nullptr, RP_DTYPE_F32, nullptr, dx, c->final_norm.g,
                       false, part, (int)T, s.H, st));
    RP_TRY(mark_consumed(c, c->final_norm));
    RP_TRY(mark_grad_ready(c, c->final_norm));
  } else {
    RP_TRY(cast_from_f32(dt, dxf, dx, (size_t)T * s.H, st));
  }
  return ws_mark(c, ws);
}

}  // namespace rp
