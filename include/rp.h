/*
 * rp.h -- C ABI of one RoundPipe GPU worker stage on MI355X (gfx950).
 *
 * A RoundPipe GPU worker is stateless: model weights, layer-input
 * checkpoints and gradients live in host memory, and whatever stage the
 * controller dispatches is executed by streaming its weights in, computing,
 * and streaming activations and gradients back out ("Efficient Training on
 * Multiple Consumer GPUs with RoundPipe", section 3.1 "Computation Dispatch
 * Paradigm"; section 4.2 "Data Transfer Overlap"). A stage is a contiguous
 * range of decoder layers (section 3.2, forward partition F_i and backward
 * partition B_j); the first backward stage B_1 is fused with its own forward,
 * which doubles as the recomputation (section 3.2, asymmetric stage
 * splitting); every other backward stage recomputes its layers from the saved
 * layer inputs (section 2.1.1, full activation recomputation).
 *
 * This library is that worker's hot path. Its calls map onto the pages'
 * statement of a stage:
 *   rp_stage_fwd            -- forward of layers [l0, l1): activation in, out
 *   rp_stage_bwd_recompute  -- recompute + backward of [l0, l1): dy in, dx out,
 *                              weight gradients out
 *   rp_lmhead_ce_fwd_bwd    -- vocabulary-sharded LM head + cross-entropy,
 *                              forward and backward (the LM head is the
 *                              heaviest single stage, section 2.3, and is split
 *                              before transfer scheduling, section 4.2.2)
 *   rp_weight_stream_submit -- parameter uploads / gradient downloads packed
 *                              into the idle windows after critical-path
 *                              activation copies (section 4.2.2)
 *   rp_act_copy             -- the critical-path activation copies themselves
 *
 * Conventions (all calls):
 *   - Every call that touches the GPU only ENQUEUES work on the context's
 *     streams and returns. RP_OK means "validated and enqueued". Device-side
 *     failures surface as RP_ERR_HIP from a later call or from rp_ctx_sync.
 *   - Arguments are validated synchronously before anything is enqueued; on
 *     an error nothing is enqueued and rp_last_error() describes the problem.
 *   - The caller owns every buffer (device, pinned host, workspace) and keeps
 *     it alive and unmodified until rp_ctx_sync returns (or until the work
 *     that reads it is known complete). The library owns only its own events.
 *   - A context is used from one host thread at a time. No C++ exception
 *     crosses this ABI.
 *   - Streams are the caller's (e.g. created by torch). The library never
 *     changes their priority: every copy class has its own stream, and the
 *     priority of activation copies over weight/gradient copies is enforced by
 *     issue order, event gating and bounded chunk sizes (section 4.2.2), not by
 *     stream priorities.
 *   - Layouts: activations are token-major row-major [T, H] with
 *     T = batch * seq, tokens ordered (batch row, position). Weight matrices
 *     are [out, in] row-major (y = x W^T). Gradients are fp32 in the same
 *     layout as the weights they belong to.
 */
#ifndef RP_H_
#define RP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------------ */
/* status                                                                    */
/* ------------------------------------------------------------------------ */

typedef enum rp_status {
  RP_OK = 0,
  RP_ERR_INVALID = 1,     /* null/misaligned pointer, bad range or size        */
  RP_ERR_UNSUPPORTED = 2, /* shape/option outside what the kernels implement   */
  RP_ERR_WORKSPACE = 3,   /* workspace smaller than rp_workspace_size()         */
  RP_ERR_NOT_PINNED = 4,  /* host pointer is not page-locked (pinned) memory    */
  RP_ERR_HIP = 5,         /* HIP runtime error                                  */
  RP_ERR_STATE = 6        /* call order violated (e.g. no kept activations)     */
} rp_status;

/* Human-readable name of a status code (static string). */
const char* rp_status_string(rp_status s);
/* Description of the most recent error on the calling thread (static
 * thread-local buffer, valid until the next failing call on this thread). */
const char* rp_last_error(void);
/* Library version string. */
const char* rp_version(void);

/* ------------------------------------------------------------------------ */
/* configuration                                                             */
/* ------------------------------------------------------------------------ */

typedef enum rp_dtype { RP_DTYPE_F32 = 0, RP_DTYPE_BF16 = 1 } rp_dtype;

/* Shape of every decoder layer of a context (the GQA transformer layer of the
 * paper's appendix B.1: two RMSNorms, q/k/v/o projections, causal attention
 * with RoPE, SwiGLU MLP -- or a top-k mixture of SwiGLU experts, appendix C.2
 * -- with optional LoRA adapters on q, k, v, o for the LoRA fine-tune of
 * section 5.1).
 *   hidden        H; multiple of 64
 *   n_q, n_kv     query / key-value heads; n_q % n_kv == 0
 *   head_dim      d; 64 or 128 (bf16 kernels: 128 only)
 *   ffn           dense SwiGLU width F (multiple of 8); 0 iff n_experts > 0
 *   n_experts     E experts (0 = dense MLP), top_k experts per token
 *   expert_ffn    per-expert SwiGLU width (multiple of 8)
 *   lora_rank     r (0 = no adapters; then all weights are trainable; with
 *                 adapters only the adapters are trainable), lora_alpha
 *   rms_eps       RMSNorm epsilon
 *   rope_base     RoPE base (rotate-half pairs (i, i + d/2), angle
 *                 pos * base^(-2i/d), positions restart per batch row)
 *   dtype         rp_dtype of weights and activations; arithmetic inside the
 *                 kernels is fp32 (bf16 operands, fp32 accumulation). */
typedef struct rp_layer_cfg {
  int32_t hidden;
  int32_t n_q;
  int32_t n_kv;
  int32_t head_dim;
  int32_t ffn;
  int32_t n_experts;
  int32_t top_k;
  int32_t expert_ffn;
  int32_t lora_rank;
  float lora_alpha;
  float rms_eps;
  float rope_base;
  int32_t dtype;
  int32_t qk_norm; /* 1: per-head RMSNorm of q and k before RoPE (Qwen3-style),
                      gains gamma_q, gamma_k [head_dim]; 0: none */
} rp_layer_cfg;

/* The streams a context issues on (hipStream_t values, passed as void*).
 * compute  -- all kernels
 * act_h2d  -- activation / checkpoint uploads (critical path)
 * act_d2h  -- activation / checkpoint downloads (critical path)
 * w_h2d    -- parameter uploads (low priority by scheduling)
 * g_d2h    -- gradient downloads (low priority by scheduling)
 * A stream left NULL is created by the context (and destroyed with it) on a
 * hardware queue of its own, at the default priority. Recommended: streams
 * that share a hardware queue execute in one order, so a transfer stream
 * waiting for a copy on the compute stream's queue would hold the compute
 * kernels queued behind it. The streams the context creates are blocking
 * streams: work on the legacy default stream enqueued before a call runs
 * before the call's kernels, and default-stream work enqueued after a call
 * waits for them, with no event from the caller. A caller working on another
 * stream orders it with an event (rp_ctx_streams gives the compute stream).
 * Caller-provided streams stay the caller's. */
typedef struct rp_streams {
  void* compute;
  void* act_h2d;
  void* act_d2h;
  void* w_h2d;
  void* g_d2h;
} rp_streams;

/* ------------------------------------------------------------------------ */
/* weight-block layout                                                       */
/* ------------------------------------------------------------------------ */

/* One layer's weights are one contiguous block (the unit streamed per layer,
 * section 4.2: "per-stage parameter uploads"). Tensors in order, each starting
 * at a 256-byte aligned offset, elements of the context dtype:
 *   RP_T_GAMMA1  [H]
 *   RP_T_WQKV    [(n_q + 2 n_kv) d, H]   rows: Wq, then Wk, then Wv
 *   RP_T_WO      [H, n_q d]
 *   RP_T_GAMMA2  [H]
 *   RP_T_WGU     dense: [2F, H] rows Wg then Wu;  MoE: [E][2 Fe, H]
 *   RP_T_WD      dense: [H, F];                   MoE: [E][H, Fe]
 * The gradient block has the same tensors and order in fp32, each at a
 * 256-byte aligned offset (RP_BLOCK_GRAD). With LoRA, the adapters form a
 * separate fp32 block (RP_BLOCK_LORA, and the same layout for its gradient):
 *   RP_T_AQ [r, H]  RP_T_BQ [n_q d, r]  RP_T_AK [r, H]  RP_T_BK [n_kv d, r]
 *   RP_T_AV [r, H]  RP_T_BV [n_kv d, r] RP_T_AO [r, n_q d]  RP_T_BO [H, r]
 * and the base weights are frozen (no weight-gradient block is written). */
typedef enum rp_tensor {
  RP_T_GAMMA1 = 0, RP_T_WQKV = 1, RP_T_WO = 2, RP_T_GAMMA2 = 3, RP_T_WGU = 4, RP_T_WD = 5,
  RP_T_QNORM = 6, RP_T_KNORM = 7, /* qk_norm only: gamma_q, gamma_k [head_dim], after WD */
  RP_T_AQ = 16, RP_T_BQ = 17, RP_T_AK = 18, RP_T_BK = 19,
  RP_T_AV = 20, RP_T_BV = 21, RP_T_AO = 22, RP_T_BO = 23
} rp_tensor;

typedef enum rp_block { RP_BLOCK_WEIGHT = 0, RP_BLOCK_GRAD = 1, RP_BLOCK_LORA = 2 } rp_block;

/* Offset and size in bytes of one tensor inside a block; *total gets the
 * block's total size (may be NULL). Returns RP_ERR_INVALID for a tensor that
 * the block does not contain. Pure host function. */
rp_status rp_block_layout(const rp_layer_cfg* cfg, int block, int tensor,
                          size_t* offset, size_t* bytes, size_t* total);

/* ------------------------------------------------------------------------ */
/* context and bindings                                                      */
/* ------------------------------------------------------------------------ */

typedef struct rp_ctx rp_ctx;

/* Create a context on HIP device `device` for layers of shape *cfg. Returns
 * RP_ERR_UNSUPPORTED for shapes the kernels do not implement. */
rp_status rp_ctx_create(int device, const rp_layer_cfg* cfg, const rp_streams* streams,
                        rp_ctx** out);
/* The streams the context issues on (its own where the caller passed NULL). */
rp_status rp_ctx_streams(const rp_ctx* ctx, rp_streams* out);
/* Waits for the context's outstanding work, then frees it (NULL is a no-op). */
rp_status rp_ctx_destroy(rp_ctx* ctx);
/* Blocks until every stream of the context is idle; reports device errors. */
rp_status rp_ctx_sync(rp_ctx* ctx);

/* Bind the device buffers of layer `layer` (0 <= layer < 4096):
 *   w_dev          weight block (RP_BLOCK_WEIGHT layout), 256-byte aligned
 *   grad_dev       fp32 gradient block (RP_BLOCK_GRAD), or NULL when the layer
 *                  is frozen (LoRA) -- required for full fine-tuning
 *   lora_dev       fp32 adapter block (RP_BLOCK_LORA) when lora_rank > 0
 *   lora_grad_dev  fp32 adapter-gradient block when lora_rank > 0
 * Rebinding a layer is allowed once the work that used the old buffers has
 * been enqueued (the library keeps the stream ordering). */
rp_status rp_bind_layer(rp_ctx* ctx, int layer, const void* w_dev, float* grad_dev,
                        const float* lora_dev, float* lora_grad_dev);

/* Bind the LM head: vocabulary `vocab` split into `n_shards` (1..64)
 * contiguous shards, shard s covering rows [lo_s, hi_s) where the first
 * vocab % n_shards shards have one extra row. w_shard[s] is [hi_s - lo_s, H]
 * (context dtype), dw_shard[s] the fp32 gradient of the same shape.
 * gamma_f / dgamma_f: optional final RMSNorm gain [H] (context dtype) and its
 * fp32 gradient; both NULL for an LM head without final norm. */
rp_status rp_bind_lmhead(rp_ctx* ctx, int vocab, int n_shards,
                         const void* const* w_shard, float* const* dw_shard,
                         const void* gamma_f, float* dgamma_f);

/* ------------------------------------------------------------------------ */
/* workspace                                                                 */
/* ------------------------------------------------------------------------ */

typedef enum rp_op {
  RP_OP_STAGE_FWD = 0,
  RP_OP_STAGE_BWD = 1,
  RP_OP_LMHEAD = 2,
  RP_OP_FUSED = 3, /* rp_stage_fwd(RP_KEEP_ACTS) followed by
                      rp_stage_bwd_recompute(RP_USE_KEPT_ACTS) on one workspace */
  RP_OP_MOE_ROUTE = 4 /* rp_op_moe_route (MoE contexts; n_layers, flags ignored) */
} rp_op;

/* Bytes of device workspace the call needs for T = batch * seq tokens and
 * n_layers layers (flags as passed to the call). The caller allocates it
 * (256-byte aligned) and passes it to the call; the library keeps nothing in
 * it between calls except the kept activations of RP_KEEP_ACTS. */
rp_status rp_workspace_size(const rp_ctx* ctx, int op, int batch, int seq, int n_layers,
                            int flags, size_t* bytes);

/* ------------------------------------------------------------------------ */
/* stage calls                                                               */
/* ------------------------------------------------------------------------ */

enum {
  RP_KEEP_ACTS = 1,     /* fwd: keep every layer's internals in ws for a fused
                           backward stage (section 3.2, fused B_1)            */
  RP_USE_KEPT_ACTS = 2, /* bwd: use the internals kept by the preceding
                           rp_stage_fwd(RP_KEEP_ACTS) on this ws, skip the
                           recomputation                                     */
  RP_CKPT_DEVICE = 4,   /* bwd: ckpt[] are device pointers (default: pinned
                           host pointers, uploaded on act_h2d one layer ahead) */
  RP_ACCUM_GRADS = 8    /* bwd: add the weight gradients to the bound gradient
                           blocks instead of overwriting them: a stage that
                           runs several micro-batches passes it from the second
                           on and downloads the sum once (section 4.2, one
                           gradient download per stage)                      */
};

/* Forward of layers [l0, l1) (each bound) on `batch` rows of `seq` tokens.
 *   x_in         device [T, H], context dtype: the stage input
 *   y_out        device [T, H]: the stage output (may not alias x_in)
 *   ckpt_host    NULL, or l1 - l0 pinned host pointers [T, H]: the input of
 *                every layer is downloaded there on act_d2h (the layer-input
 *                checkpoints kept in host memory, section 2.1.1)
 *   router       MoE only: l1 - l0 device pointers to fp32 router logits
 *                [T, E] (NULL for dense layers)
 *   flags        RP_KEEP_ACTS or 0
 *   ws, ws_bytes workspace of rp_workspace_size(RP_OP_STAGE_FWD or RP_OP_FUSED)
 * Waits (on the compute stream) for pending weight uploads of the layers. */
rp_status rp_stage_fwd(rp_ctx* ctx, int l0, int l1, int batch, int seq,
                       const void* x_in, void* y_out, void* const* ckpt_host,
                       const float* const* router, int flags, void* ws, size_t ws_bytes);

/* Recompute + backward of layers [l0, l1), last layer first.
 *   ckpt         l1 - l0 pointers to the layers' inputs [T, H] (pinned host,
 *                or device with RP_CKPT_DEVICE); ignored with RP_USE_KEPT_ACTS
 *   dy           device [T, H]: gradient w.r.t. the stage output
 *   dx           device [T, H]: gradient w.r.t. the stage input (written)
 *   router       as for rp_stage_fwd
 * Weight gradients of each layer are written (overwritten, or with
 * RP_ACCUM_GRADS added in fp32) into its bound fp32 gradient block, or
 * LoRA-gradient block for LoRA layers. Host gradient buffers are always
 * overwritten by downloads; accumulation there is the controller's business. */
rp_status rp_stage_bwd_recompute(rp_ctx* ctx, int l0, int l1, int batch, int seq,
                                 const void* const* ckpt, const void* dy, void* dx,
                                 const float* const* router, int flags, void* ws,
                                 size_t ws_bytes);

/* LM head + mean cross-entropy, forward and backward, over the bound shards.
 *   x       device [T, H] (context dtype): the last layer's output
 *   labels  device int32 [T]; -1 marks an ignored row; others in [0, vocab)
 *           (out-of-range labels are treated as ignored)
 *   loss    device fp32 [1]: sum over labelled rows of (logsumexp - logit of
 *           the label) / number of labelled rows
 *   dx      device [T, H] (context dtype): dloss/dx
 * The per-shard weight gradients go to the bound dw_shard[s] (overwritten),
 * the final-norm gain gradient to dgamma_f. The shards are processed in
 * order, each waiting for its own pending weight upload. */
rp_status rp_lmhead_ce_fwd_bwd(rp_ctx* ctx, int batch, int seq, const void* x,
                               const int32_t* labels, float* loss, void* dx, void* ws,
                               size_t ws_bytes);

/* Token embedding of the full-model case: x0[t] = table[ids[t]] and its
 * backward dtable = scatter-add of dx0 over ids (overwrites dtable, fp32).
 * table: device [vocab, H] context dtype; ids int32 [T]. An id outside
 * [0, vocab) (a padding id) gives a zero row of x0 and adds nothing to
 * dtable. */
rp_status rp_embed_fwd(rp_ctx* ctx, int n_tokens, int vocab, const int32_t* ids,
                       const void* table, void* x0);
rp_status rp_embed_bwd(rp_ctx* ctx, int n_tokens, int vocab, const int32_t* ids,
                       const void* dx0, float* dtable);

/* ------------------------------------------------------------------------ */
/* stage partition                                                           */
/* ------------------------------------------------------------------------ */

/* Automatic stage partitioning (section 4.4). Host-only; no device work.
 * Inputs, per layer l < L (front to back): f[l] forward time, b[l] backward
 * time with the recomputation, mf[l] / mb[l] memory in a forward / backward
 * stage; h and mh: the LM head's time and memory; mem_cap: the memory limit
 * of one stage; n_micro (M) micro-batches per iteration on n_gpus (N) GPUs.
 * The LM head always sits in the fused first backward stage B_1 = the last
 * b1 layers, which costs h + their backward times (its forward doubles as
 * the recomputation). Forward stages cover layers [0, L - b1) front to back,
 * the remaining backward stages the same layers back to front. Minimises
 * (M S + N (N - 1)) t_max over t_max candidates = every contiguous sum of f,
 * of b, and h + every suffix sum of b: per candidate, B_1 takes as many
 * layers as fit, then both layer ranges are packed greedily into the fewest
 * stages (section 4.4.2, O(L^3)). Ties keep the smallest candidate.
 * Outputs: fwd_sizes[0 .. *n_fwd) layer counts of F_1.., *b1_out, and
 * bwd_sizes[0 .. *n_bwd) layer counts of B_2.. (B_2 covers the layers just
 * below B_1); both arrays need room for L entries. *objective gets the
 * minimised value. RP_ERR_UNSUPPORTED when nothing fits the memory cap. */
rp_status rp_partition(int L, const double* f, const double* b, double h, const double* mf,
                       const double* mb, double mh, double mem_cap, int n_micro, int n_gpus,
                       int* fwd_sizes, int* n_fwd, int* b1_out, int* bwd_sizes, int* n_bwd,
                       double* objective);

/* ------------------------------------------------------------------------ */
/* optimizer worker                                                          */
/* ------------------------------------------------------------------------ */

/* The host-side optimizer of section 2.1.2 with the Layerwise Model
 * Consistency Protocol of section 4.3. Host-only; no device work.
 *
 * Per layer there is a low-precision master copy in host memory (the bytes
 * the GPU uploads; bf16 or fp32) with its fp32 master gradient buffer (the
 * bytes the GPU downloads into), and an fp32 optimizer copy with the Adam
 * moments held by the optimizer. One worker thread runs the queued steps in
 * order (rule 5). Step t, layer by layer from layer 0:
 *   wait GRADS_DOWNLOADED(l, t)         rule 3: g_t is in the master buffer
 *   G-cp, signal GCP_DONE(l, t)         rule 4: the GPU may download g_{t+1}
 *   Adam on the fp32 copy
 *   wait PARAMS_UPLOADED(l, t + 1)      rule 1: iteration t + 1 has uploaded
 *                                        the master weights of step t - 1
 *   P-cp (round to the master dtype), signal PCP_DONE(l, t)
 *                                        rule 2: iteration t + 2 may upload
 * The GPU side (the caller) signals PARAMS_UPLOADED(l, i) once its upload of
 * layer l for iteration i has completed and GRADS_DOWNLOADED(l, i) once g_i
 * is in the master buffer; before uploading layer l for iteration i it waits
 * PCP_DONE(l, i - 2), before downloading g_i it waits GCP_DONE(l, i - 1).
 * Iteration i thus trains on the weights of step i - 2 (staleness 1). At the
 * end of training the caller signals PARAMS_UPLOADED(-1, last + 1) (layer -1:
 * every layer) so that the last step can write its weights.
 *
 * Adam with decoupled weight decay, each operation one fp32 rounding:
 *   g = grad_scale G; m = b1 m + (1 - b1) g; v = b2 v + (1 - b2) g g;
 *   w = w - lr ((m / (1 - b1^s)) / (sqrt(v / (1 - b2^s)) + eps) + wd w)
 * s = steps applied to the layer so far (1-based); 1 - b^s formed in double.
 * P-cp to bf16 rounds to nearest even. */
typedef struct rp_opt rp_opt;
typedef struct rp_opt_hparams {
  float lr, beta1, beta2, eps, weight_decay, grad_scale;
} rp_opt_hparams;
/* One tensor of a layer: n elements of master weights (master dtype) and of
 * master fp32 gradients, both host memory owned by the caller and kept alive
 * while the optimizer exists; init: NULL (the optimizer copy starts from the
 * master weights) or n fp32 starting values. */
typedef struct rp_opt_seg {
  void* master_w;
  const float* master_g;
  const float* init;
  uint64_t n;
} rp_opt_seg;
enum {
  RP_OPT_PARAMS_UPLOADED = 0,  /* signalled by the GPU side */
  RP_OPT_GRADS_DOWNLOADED = 1, /* signalled by the GPU side */
  RP_OPT_PCP_DONE = 2,         /* signalled by the optimizer, waited by the GPU side */
  RP_OPT_GCP_DONE = 3          /* signalled by the optimizer, waited by the GPU side */
};
/* n_threads <= 0: all hardware threads. edge_timeout_ms > 0 bounds every
 * wait (the worker's and rp_opt_wait's): a missing signal then fails the
 * step with RP_ERR_STATE instead of blocking forever; 0 waits without limit. */
rp_status rp_opt_create(int n_layers, int master_dtype, int n_threads, int64_t edge_timeout_ms,
                        rp_opt** out);
rp_status rp_opt_destroy(rp_opt* opt);
/* Bind (or rebind, with no step running) layer `layer`'s tensors. */
rp_status rp_opt_bind_layer(rp_opt* opt, int layer, const rp_opt_seg* segs, int n_segs);
/* Queue the optimizer step of iteration `iteration` and return. */
rp_status rp_opt_step(rp_opt* opt, int64_t iteration, const rp_opt_hparams* hp);
/* GPU side of the protocol: signal PARAMS_UPLOADED / GRADS_DOWNLOADED for a
 * layer (-1: all), and wait for PCP_DONE / GCP_DONE of a layer (returns at
 * once for iteration < 0). A failed step's error is returned by later
 * rp_opt_wait, rp_opt_step and rp_opt_sync calls. */
rp_status rp_opt_signal(rp_opt* opt, int edge, int layer, int64_t iteration);
rp_status rp_opt_wait(rp_opt* opt, int edge, int layer, int64_t iteration);
/* Wait until every queued step has finished. */
rp_status rp_opt_sync(rp_opt* opt);
/* Copy a layer's optimizer state out, with no step running: which = 0
 * fp32 weights, 1 first moment, 2 second moment; n = the layer's elements. */
rp_status rp_opt_read(rp_opt* opt, int layer, int which, float* dst, uint64_t n);

/* ------------------------------------------------------------------------ */
/* transfers                                                                 */
/* ------------------------------------------------------------------------ */

enum { RP_H2D = 0, RP_D2H = 1 };

/* Critical-path activation copy between pinned host memory and the device.
 * H2D runs on act_h2d and the compute stream waits for it before any later
 * kernel; D2H runs on act_d2h after the compute stream's work enqueued so
 * far. Every activation copy gets a ticket (increasing from 0 per context),
 * written to *ticket (may be NULL); weight/gradient windows can be gated on
 * tickets. Host pointers must be pinned (RP_ERR_NOT_PINNED otherwise). */
rp_status rp_act_copy(rp_ctx* ctx, int dir, void* dst, const void* src, size_t bytes,
                      int64_t* ticket);

/* Ordering on activation copies (section 4.2.1: the compute stream syncs with
 * the activation streams per micro-batch through events). rp_act_wait makes
 * later work on the chosen stream wait until activation copy `ticket` has
 * completed: RP_ON_ACT_H2D orders an upload after the download that fills its
 * host buffer (an activation that passes through host memory between two
 * stages), RP_ON_COMPUTE orders kernels after a copy. RP_ERR_STATE for a
 * ticket not yet issued, or one of more than 256 copies ago (its event has
 * been recycled). rp_act_next_ticket gives the ticket the next rp_act_copy
 * will get, so that a caller can gate transfer windows on copies it is about
 * to issue. */
enum { RP_ON_COMPUTE = 0, RP_ON_ACT_H2D = 1, RP_ON_ACT_D2H = 2 };
rp_status rp_act_wait(rp_ctx* ctx, int where, int64_t ticket);
rp_status rp_act_next_ticket(const rp_ctx* ctx, int64_t* next);

/* RP_GRAD_D2H_BF16 downloads an fp32 gradient range rounded to bf16 (nearest
 * even): the host buffer receives bytes / 2. This is the pages' low-precision
 * gradient on the link (section 4.3.1, the low-precision master copy, whose
 * G-cp casts it back); offset and bytes must be multiples of 32. At submit
 * time the range is rounded on the compute stream, behind the work already
 * enqueued there (so submit it after the call that writes the gradient),
 * into a bf16 staging copy of the gradient buffer that the context
 * allocates on first use (half the buffer's size) and frees with the
 * context; the download window copies from that by DMA. All transfers,
 * activation and checkpoint downloads included, go by DMA. */
typedef enum rp_xfer_kind { RP_PARAM_H2D = 0, RP_GRAD_D2H = 1, RP_GRAD_D2H_BF16 = 2 } rp_xfer_kind;
typedef enum rp_xfer_target {
  RP_TGT_LAYER = 0,  /* id = layer; bytes of the weight / gradient block      */
  RP_TGT_LMHEAD = 1, /* id = shard; bytes of the shard's weight / gradient    */
  RP_TGT_LORA = 2,   /* id = layer; bytes of the LoRA / LoRA-gradient block   */
  RP_TGT_FINAL_NORM = 3 /* id = 0; the final-norm gain / its gradient         */
} rp_xfer_target;

/* One parameter upload or gradient download: `bytes` at `offset` inside the
 * bound device buffer of (target, id), from/to pinned host memory `host`
 * (host points at the first byte to move). */
typedef struct rp_xfer {
  int32_t kind;
  int32_t target;
  int32_t id;
  int32_t reserved;
  uint64_t offset;
  uint64_t bytes;
  void* host;
} rp_xfer;

/* Schedule parameter uploads and gradient downloads (section 4.2.2):
 * per direction, items larger than ceil(total / n_windows) bytes -- or than
 * max_chunk (if non-zero) -- are split into chunks of that threshold rounded
 * up to 256 bytes (the last chunk takes the remainder); chunks are sorted by
 * size (descending, stable) and each is assigned to the window with the least
 * bytes so far (ties: lowest window). Window w is issued on w_h2d / g_d2h
 * after activation ticket gate_ticket + w has completed (gate_ticket < 0: no
 * gating; a ticket not yet issued defers the window until rp_act_copy issues
 * it). A PARAM_H2D upload waits until the compute work that last read its
 * buffer is done; its target is marked ready when all its chunks landed, and
 * stage calls wait for that. A GRAD_D2H download waits for the backward that
 * wrote the gradient; the next backward writing that buffer waits for it. */
rp_status rp_weight_stream_submit(rp_ctx* ctx, const rp_xfer* items, int n_items,
                                  int n_windows, uint64_t max_chunk, int64_t gate_ticket);
/* The same with one gate per window: window w waits for activation ticket
 * gates[w] (n_windows entries; negative: not gated; a ticket not yet issued
 * defers the window as above). A stage that runs M micro-batches gates window
 * j on the activation copy of its micro-batch j, so that every window follows
 * the critical-path copy it belongs to (section 4.2.2, one window per
 * micro-batch), also when a micro-batch issues several copies. */
rp_status rp_weight_stream_submit_gated(rp_ctx* ctx, const rp_xfer* items, int n_items,
                                        int n_windows, uint64_t max_chunk,
                                        const int64_t* gates);

/* The planner alone (pure host function, for tests): split + LPT-assign
 * n_items sizes into n_windows windows with the rule above (`align`-byte
 * chunk rounding, 256 in rp_weight_stream_submit). Writes up to cap chunks in
 * item order: item index, offset, bytes, window. *n_chunks gets the count
 * (RP_ERR_INVALID if it exceeds cap). */
rp_status rp_xfer_plan(const uint64_t* sizes, int n_items, int n_windows, uint64_t max_chunk,
                       uint64_t align, int cap, int32_t* item, uint64_t* offset,
                       uint64_t* bytes, int32_t* window, int* n_chunks);

/* ------------------------------------------------------------------------ */
/* kernel-level entry points (single kernels, for parity tests and rooflines) */
/* ------------------------------------------------------------------------ */

/* C[M, N] (+)= sum_k A(m, k) B(n, k), bf16 operands, fp32 accumulation.
 * A(m, k) = A[m * lda + k] if a_kmajor else A[k * lda + m]; likewise B with
 * b_kmajor. out_f32: C is fp32 (accumulate != 0 adds to it) else bf16 (round
 * to nearest even). Requires K % 8 == 0, lda/ldb/ldc % 8 == 0, 16-byte
 * aligned pointers. Enqueued on the compute stream. */
rp_status rp_op_gemm_bf16(rp_ctx* ctx, int M, int N, int K, const void* A, int lda,
                          int a_kmajor, const void* B, int ldb, int b_kmajor, void* C,
                          int ldc, int out_f32, int accumulate);

/* Causal GQA attention forward on a packed qkv buffer [T, (n_q + 2 n_kv) d]
 * (q, k already rotated): o [T, n_q d] and lse [n_q, T] (fp32, natural log of
 * the softmax denominator of the scaled scores). Context dtype and heads. */
rp_status rp_op_attn_fwd(rp_ctx* ctx, int batch, int seq, const void* qkv, void* o,
                         float* lse);
/* Its backward: from qkv, o, do [T, n_q d] and lse, writes dqkv
 * [T, (n_q + 2 n_kv) d] (dq, dk, dv; the kv-head gradients summed over the
 * query heads that share them). ws: rp_workspace_size(RP_OP_STAGE_BWD, ...)
 * bytes at least. */
rp_status rp_op_attn_bwd(rp_ctx* ctx, int batch, int seq, const void* qkv, const void* o,
                         const void* dout, const float* lse, void* dqkv, void* ws,
                         size_t ws_bytes);

/* rp_op_attn_bwd without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation). The per-row terms D = rowsum(dO * O) that the
 * workspace holds go to a fixed device array of the library instead:
 * 2^21 fp32 (8 MiB) on each GPU the library runs on, held until the process
 * ends, so n_q * batch * seq <= 2^21 (RP_ERR_UNSUPPORTED above that). Nothing
 * is allocated. The array is shared by every call on the GPU and keeps the
 * last call's contents; each call writes every entry it reads, so it needs no
 * clearing, but calls that overlap on one GPU (other streams or contexts)
 * race on it. Arguments and results otherwise as rp_op_attn_bwd. */
rp_status rp_op_attn_bwd_noalloc(rp_ctx* ctx, int batch, int seq, const void* qkv, const void* o,
                                 const void* dout, const float* lse, void* dqkv);

/* MoE routing alone, for checking its integer outputs bit for bit (the
 * top-k expert selection of the paperlayer.ai summary, appendix C.2, which
 * activates E_act of E_total experts per token; the grouped order is the
 * permutation that lets each expert's rows run as one product). For the
 * context's E experts and top_k = k, T = batch * seq tokens:
 *   logits    device fp32 [T, E] router logits (an input of the layer)
 *   idx       device int32 [T, k]: the k largest logits of each token, by
 *             value descending; equal logits are taken lower index first
 *   wgt       device fp32 [T, k]: softmax over the k selected logits
 *   cnt       device int32 [E]: (token, slot) pairs routed to each expert
 *   off       device int32 [E + 1]: first grouped row of each expert
 *             (off[0] = 0, off[E] = T k)
 *   perm_row  device int32 [T k]: the token of each grouped row; expert e's
 *             rows off[e] .. off[e+1]-1 list its pairs in increasing
 *             (token, slot) order (a stable counting sort)
 *   perm_w    device fp32 [T k]: the routing weight of each grouped row
 *   inv       device int32 [T k]: the grouped row of pair (token, slot)
 *   ws        rp_workspace_size(RP_OP_MOE_ROUTE, batch, seq) bytes: the tile
 *             map of the grouped products
 * RP_ERR_STATE for a dense context. Enqueued on the compute stream. */
rp_status rp_op_moe_route(rp_ctx* ctx, int batch, int seq, const float* logits, int32_t* idx,
                          float* wgt, int32_t* cnt, int32_t* off, int32_t* perm_row,
                          float* perm_w, int32_t* inv, void* ws, size_t ws_bytes);

/* Plain device-to-device copy of `bytes` (a multiple of 16; both pointers
 * 16-byte aligned, non-overlapping device memory), 16 bytes per lane. Its
 * known traffic is the scale for HBM byte counters (FETCH_SIZE, WRITE_SIZE)
 * read on the library's other kernels. Enqueued on the compute stream;
 * RP_ERR_INVALID on misaligned arguments. */
rp_status rp_op_copy(rp_ctx* ctx, void* dst, const void* src, size_t bytes);

/* bf16 transpose, dst[c * ldd + r] = src[r * lds + c] for r < rows,
 * c < cols (elements of dst outside that range untouched). The step that
 * makes the activation operand of a weight-gradient product (dW = dY^T X,
 * where dY and X are stored token-major) K-major ahead of the GEMM, so that
 * only dY is read through transposing LDS reads. rows, cols, lds
 * and ldd multiples of 8; pointers 16-byte aligned device memory, src and dst
 * not overlapping. Enqueued on the compute stream; RP_ERR_UNSUPPORTED when
 * the size or alignment rules are not met. */
rp_status rp_op_transpose_bf16(rp_ctx* ctx, int rows, int cols, const void* src, int64_t lds,
                               void* dst, int64_t ldd);

/* ------------------------------------------------------------------------ */
/* kernel trace                                                              */
/* ------------------------------------------------------------------------ */

/* The RoundPipe paper times every layer with device events in its profiling
 * pass (section 4.4, "Profiling"). The same mechanism here times every kernel
 * launch the library enqueues on the compute stream, so that each kernel can
 * be priced against its roofline while the real stage runs.
 *
 * rp_trace_begin waits for the compute stream, then records a HIP event pair
 * around each of the next max_launches launches made through this context
 * (later launches go unrecorded). rp_trace_end stops recording;
 * rp_trace_read then waits for the recorded events and writes one record per
 * launch, in issue order, to out[0 .. *n). With cap == 0 it only reports the
 * count in *n; cap < count is RP_ERR_INVALID. Event pairs add a few
 * microseconds per launch. */
typedef struct rp_trace_rec {
  char name[96];  /* kernel (template instance) name                        */
  double flops;   /* algorithmic FLOPs of the launch (matrix products)      */
  double bytes;   /* algorithmic HBM bytes of the launch (row/elementwise)  */
  float ms;       /* event-to-event duration on the compute stream          */
  int32_t reserved;
} rp_trace_rec;

rp_status rp_trace_begin(rp_ctx* ctx, int max_launches);
rp_status rp_trace_end(rp_ctx* ctx);
rp_status rp_trace_read(rp_ctx* ctx, rp_trace_rec* out, int cap, int* n);

#ifdef __cplusplus
}
#endif

#endif /* RP_H_ */
