"""Throughput of one RoundPipe GPU-worker step on one MI355X.

A step is one pass of the worker's hot path over one microbatch of the
Llama-3.1-8B-shaped stage (hidden 4096, 32 query / 8 key-value heads of 128,
SwiGLU FFN 14336, 1 x 8192 tokens, bf16 weights and activations, fp32
gradients):

  rp_stage_fwd            layer forward; its input checkpoint goes to pinned
                          host memory (activation offload)
  rp_lmhead_ce_fwd_bwd    4-shard LM head (4096 x 128256) + mean cross-entropy,
                          forward and backward -> dy
  rp_stage_bwd_recompute  checkpoint back from host, recompute the layer,
                          backward -> dx and the fp32 weight gradients

`value` is trained tokens per second with weights resident in HBM (inputs in
HBM when the timed region starts): the compute of the step. By default the
same step also runs as the workload states it, every weight uploaded from
pinned host memory and every fp32 gradient downloaded to it through
rp_weight_stream_submit, reported under "streamed" (never as `value`) with
the transfers alone, the overlap efficiency
(t_compute + t_transfers - t_step) / min(t_compute, t_transfers) and the link
rates against the box's measured pinned-copy peak ("link_peak"); then with
the gradients on the link in bf16 ("streamed_bf16_grads"), and, under
"priority", the latency of an activation upload alone, behind an ungated
weight upload, and with that upload gated on the activation copy's ticket.

With --ablation it also runs the pages' priority-aware transfer ablation on
Llama-3.1-8B-shaped layers (section 5.8.2): a forward + backward pass over
4 one-layer stages of 4 micro-batches each, every weight, activation and
gradient through pinned host memory, for micro-batch sizes 1..10 sequences of
2048 tokens, under the policies no_prefetch, prefetch and windowed
(offloaded_pipeline_stage_amd/microbatch.py). Reported under "ablation".

Each kernel launch in the timed region is timed by the library's own HIP
event pairs on the compute stream (rp_trace_*); the dominant kernel is priced
against the MI355X peak for its bound. The CPU oracle is timed in fp32 on the
full layer at the workload's length and on a row sample of the LM head for
the cpu_baseline field.

`roofline.traffic` comes from two rocprofv3 counter runs of this script
(FETCH_SIZE, then WRITE_SIZE, with --copy-calibration-mib for the scale),
reduced by offloaded_pipeline_stage_amd/pmc.py into
profiles/<workload>_step_traffic.txt.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-streamed]
                       [--no-cpu-baseline] [--cpu-head-rows R] [--trace-json PATH]
                       [--copy-calibration-mib M] [--configs] [--ablation] [--optimizer]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
from collections import defaultdict

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "trained tokens/sec per GPU (fwd+recompute+bwd) + MFMA util, 8B-shaped stage"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBPS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def layer_flops(cfg, recompute: bool) -> dict:
    """Matrix-product FLOPs of one layer (causal attention counts the causal
    pairs): forward, and backward (dX + dW products, attention dS/dP/dQ/dK/dV
    counted as twice the forward's two products)."""
    T, H, Q, KV, F = cfg.tokens, cfg.hidden, cfg.q_dim, cfg.kv_dim, cfg.ffn
    lin = 2.0 * T * H * (Q + 2 * KV) + 2.0 * T * Q * H + 2.0 * T * H * 2 * F + 2.0 * T * F * H
    pairs = cfg.batch * cfg.seq * (cfg.seq + 1) / 2.0
    att = 4.0 * cfg.head_dim * cfg.n_q * pairs
    fwd = lin + att
    bwd = 2 * lin + 2 * att
    return {"fwd": fwd, "recompute": fwd if recompute else 0.0, "bwd": bwd}


def lmhead_flops(cfg) -> float:
    return 3 * 2.0 * cfg.tokens * cfg.hidden * cfg.vocab


def layer_cost(cfg):
    """(forward, backward) matrix-product FLOPs of one layer, dense or MoE
    (active experts only), full fine-tuning or LoRA (frozen base: no weight
    gradient products); causal attention counts the causal pairs, its
    backward twice its forward."""
    T, H, Q, KV = cfg.tokens, cfg.hidden, cfg.q_dim, cfg.kv_dim
    attn_lin = 2.0 * T * H * (Q + 2 * KV) + 2.0 * T * Q * H
    if cfg.n_experts > 0:
        mlp = cfg.top_k * (2.0 * T * H * 2 * cfg.expert_ffn + 2.0 * T * cfg.expert_ffn * H)
    else:
        mlp = 2.0 * T * H * 2 * cfg.ffn + 2.0 * T * cfg.ffn * H
    att = 4.0 * cfg.head_dim * cfg.n_q * cfg.batch * cfg.seq * (cfg.seq + 1) / 2.0
    lin = attn_lin + mlp
    bwd = (lin if cfg.lora_rank > 0 else 2 * lin) + 2 * att
    return lin + att, bwd


class Step:
    """Buffers and calls of one worker step through the C ABI."""

    def __init__(self, cfg, streamed: bool, grad_bf16: bool = False):
        from offloaded_pipeline_stage_amd import binding as B
        from offloaded_pipeline_stage_amd.worker import Worker
        self.B = B
        self.cfg = cfg
        self.streamed = streamed
        # gradients on the link in bf16 (the pages' precision) instead of fp32
        self.grad_kind = B.RP_GRAD_D2H_BF16 if grad_bf16 else B.RP_GRAD_D2H
        gdt = torch.bfloat16 if grad_bf16 else torch.float32
        dev = torch.device("cuda", 0)
        T, H = cfg.tokens, cfg.hidden
        t0 = time.time()
        lw = synth.layer_weights(cfg, 0)
        head = synth.lmhead_weights(cfg)
        self.wk = Worker(cfg)
        ctx = self.wk.ctx
        if streamed:
            # weights live in pinned host memory; two device copies of the layer
            # (ids 0 and 1) alternate between steps so that the next step's
            # upload overlaps this step's compute
            self.host_layer = self.wk.pack_layer(lw, pinned=True)
            for l in (0, 1):
                self.wk.add_layer(l, resident=False)
            self.wk.add_lmhead(None, resident=False)
            rows = self.wk.shard_rows()
            self.host_shards, lo = [], 0
            for r in rows:
                self.host_shards.append(head["w"][lo:lo + r].contiguous().pin_memory())
                lo += r
            gb = self.wk.g_bytes // (2 if grad_bf16 else 1)
            self.host_grad = [torch.empty(gb, dtype=torch.uint8).pin_memory() for _ in (0, 1)]
            self.host_dshards = [torch.empty(r, H, dtype=gdt).pin_memory() for r in rows]
        else:
            self.wk.add_layer(0, lw)
            self.wk.add_lmhead(head["w"])
        del lw, head
        bf = dict(dtype=torch.bfloat16, device=dev)
        self.x = synth.activation(cfg, "x").to(dev)
        self.labels = synth.uniform_labels(cfg).to(dev)
        self.y = torch.empty(T, H, **bf)
        self.dy = torch.empty(T, H, **bf)
        self.dx = torch.empty(T, H, **bf)
        self.loss = torch.zeros(1, dtype=torch.float32, device=dev)
        self.ckpt = [torch.empty(T, H, dtype=torch.bfloat16).pin_memory()]
        self.ws_f = ctx.workspace(B.RP_OP_STAGE_FWD, cfg.batch, cfg.seq, 1)
        self.ws_b = ctx.workspace(B.RP_OP_STAGE_BWD, cfg.batch, cfg.seq, 1)
        self.ws_h = ctx.workspace(B.RP_OP_LMHEAD, cfg.batch, cfg.seq)
        self.n = 0
        log(f"[bench] setup {time.time() - t0:.1f}s; workspaces "
            f"{(self.ws_f.numel() + self.ws_b.numel() + self.ws_h.numel()) / 2**30:.2f} GiB")

    def _shard_items(self, kind):
        B, out = self.B, []
        hs = self.host_shards if kind == B.RP_PARAM_H2D else self.host_dshards
        for sh, h in enumerate(hs):
            nb = h.numel() * (4 if kind != B.RP_PARAM_H2D else h.element_size())  # device-side bytes
            out.append((kind, B.RP_TGT_LMHEAD, sh, 0, nb, h))
        return out

    def run(self):
        B, cfg, wk = self.B, self.cfg, self.wk
        ctx = wk.ctx
        b, s = cfg.batch, cfg.seq
        layer = self.n & 1 if self.streamed else 0
        sub = lambda items: ctx.weight_stream_submit(items, n_windows=1, max_chunk=64 << 20)  # noqa: E731
        if self.streamed and self.n == 0:
            sub([(B.RP_PARAM_H2D, B.RP_TGT_LAYER, layer, 0, wk.w_bytes, self.host_layer)]
                + self._shard_items(B.RP_PARAM_H2D))
        ctx.stage_fwd(layer, layer + 1, b, s, self.x, self.y, self.ws_f, ckpt_host=self.ckpt)
        if self.streamed:
            # the next step's layer weights go up (into the other device copy)
            # while this step computes
            sub([(B.RP_PARAM_H2D, B.RP_TGT_LAYER, layer ^ 1, 0, wk.w_bytes, self.host_layer)])
        ctx.lmhead_ce_fwd_bwd(b, s, self.y, self.labels, self.loss, self.dy, self.ws_h)
        if self.streamed:
            # shard gradients down; the next step's shards up once read
            sub(self._shard_items(self.grad_kind) + self._shard_items(B.RP_PARAM_H2D))
        ctx.stage_bwd_recompute(layer, layer + 1, b, s, self.dy, self.dx, self.ws_b, ckpt=self.ckpt)
        if self.streamed:
            sub([(self.grad_kind, B.RP_TGT_LAYER, layer, 0, wk.g_bytes, self.host_grad[layer])])
        self.n += 1

    def run_transfers_only(self):
        """The streamed step's uploads and downloads alone (the same items and
        chunking, no kernels): the time the host link needs for one step."""
        B, wk = self.B, self.wk
        items = ([(B.RP_PARAM_H2D, B.RP_TGT_LAYER, 0, 0, wk.w_bytes, self.host_layer)]
                 + self._shard_items(B.RP_PARAM_H2D) + self._shard_items(self.grad_kind)
                 + [(self.grad_kind, B.RP_TGT_LAYER, 1, 0, wk.g_bytes, self.host_grad[1])])
        wk.ctx.weight_stream_submit(items, n_windows=1, max_chunk=64 << 20)

    def sync(self):
        self.wk.ctx.sync()
        torch.cuda.synchronize()


def summarize_trace(recs, steps):
    agg = defaultdict(lambda: [0, 0.0, 0.0, 0.0])
    for name, fl, by, ms in recs:
        a = agg[name]
        a[0] += 1
        a[1] += fl
        a[2] += by
        a[3] += ms
    return agg


def roofline(agg, dtype, traffic_file):
    """The dominant kernel (most time per step) against its MI355X peak.
    `traffic` is its calibrated HBM bytes per launch from the committed
    FETCH_SIZE/WRITE_SIZE summary, or None when that summary is absent or
    was taken from another version of the kernel's source."""
    from offloaded_pipeline_stage_amd import pmc
    name, (cnt, fl, by, ms) = max(agg.items(), key=lambda kv: kv[1][3])
    sec = ms / 1e3
    traffic = pmc.traffic_for(traffic_file, name)
    traffic = None if traffic is None else round(traffic)
    if fl > 0:
        peak = PEAK_BF16_TFLOPS if dtype == "bf16" else PEAK_F32_TFLOPS
        ach = fl / sec / 1e12
        return {"kernel": name, "bound": "mfma", "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(ach / peak, 4), "traffic": traffic, "launches": cnt,
                "avg_launch_ms": round(ms / cnt, 4), "flops_per_launch": fl / cnt}
    ach = by / sec / 1e9
    return {"kernel": name, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBPS, 4), "traffic": traffic, "launches": cnt,
            "avg_launch_ms": round(ms / cnt, 4), "bytes_per_launch": by / cnt}


def copy_calibration(ctx, mib: int):
    """One plain device-to-device copy of `mib` MiB through the library's
    16-byte-per-lane copy kernel (rp_op_copy), the reference that the
    FETCH_SIZE / WRITE_SIZE counter runs are scaled by."""
    src = torch.ones(mib << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    ctx.op_copy(dst, src)
    ctx.sync()
    del src, dst
    torch.cuda.empty_cache()


def priority_probe(cfg, chunk_mib: int = 16, reps: int = 5):
    """Copy priority (the pages' multi-stream transfer scheduling): latency of
    one [T, H] activation upload as the compute stream sees it, alone, behind
    an ungated weight upload of two layers (chunked), and with that upload
    gated on the activation copy's ticket. Median over `reps` of each."""
    from offloaded_pipeline_stage_amd import binding as B
    from offloaded_pipeline_stage_amd.worker import Worker
    wk = Worker(cfg)
    lw = synth.layer_weights(cfg, 0)
    host_w = wk.pack_layer(lw, pinned=True)
    del lw
    for l in (0, 1):
        wk.add_layer(l, resident=False)
    ctx = wk.ctx
    comp = ctx.streams["compute"]
    T, H = cfg.tokens, cfg.hidden
    x_host = synth.activation(cfg, "x").pin_memory()
    x_dev = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    items = [(B.RP_PARAM_H2D, B.RP_TGT_LAYER, l, 0, wk.w_bytes, host_w) for l in (0, 1)]
    chunk = chunk_mib << 20

    def once(mode):
        ctx.sync()
        t_mark = ctx.act_copy(B.RP_H2D, x_dev, x_host, 256)  # the ticket counter's current value
        ctx.sync()
        if mode == "ungated":
            ctx.weight_stream_submit(items, n_windows=1, max_chunk=chunk)
        elif mode == "gated":
            ctx.weight_stream_submit(items, n_windows=1, max_chunk=chunk, gate_ticket=t_mark + 1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(comp)
        ctx.act_copy(B.RP_H2D, x_dev, x_host)  # the compute stream waits for it
        e1.record(comp)
        ctx.sync()
        return e0.elapsed_time(e1)

    out = {"act_copy_MB": round(T * H * 2 / 1e6, 1), "weight_stream_GB": round(2 * wk.w_bytes / 1e9, 3),
           "chunk_MiB": chunk_mib}
    for mode in ("alone", "ungated", "gated"):
        once(mode)
        ts = sorted(once(mode) for _ in range(reps))
        out[f"{mode}_ms"] = round(ts[len(ts) // 2], 3)
    return out


def transfer_ablation(mbs_list=tuple(range(1, 11)), n_layers: int = 4, n_micro: int = 4, seq: int = 2048,
                      reps: int = 2):
    """Throughput (tokens/s) of one forward + backward pass over `n_layers`
    one-layer stages of `n_micro` micro-batches per transfer policy and
    micro-batch size. Every stage streams a full layer's weights in and (for
    the backward) its fp32 gradients out; all layers share one host weight
    block, which moves the same bytes as distinct ones."""
    from offloaded_pipeline_stage_amd.microbatch import POLICIES, MicrobatchPass
    from offloaded_pipeline_stage_amd.worker import Worker
    cfg = synth.config("llama3_8b", seq=seq)
    packer = Worker(cfg)
    host_w = packer.pack_layer(synth.layer_weights(cfg, 0), pinned=True)
    packer.ctx.close()
    max_mbs = max(mbs_list)
    out = {"workload": f"Llama-3.1-8B-shaped layers, {n_layers} forward + {n_layers} backward one-layer stages, "
                       f"{n_micro} micro-batches per stage, micro-batch = mbs sequences of {seq} tokens",
           "weights_GB_per_stage": None, "grads_GB_per_bwd_stage": None, "mbs": list(mbs_list)}
    for pol in POLICIES:
        mp = MicrobatchPass(cfg, [host_w] * n_layers, n_micro=n_micro, max_mbs=max_mbs, policy=pol)
        out["weights_GB_per_stage"] = round(mp.wk.w_bytes / 1e9, 3)
        out["grads_GB_per_bwd_stage"] = round(mp.wk.g_bytes / 1e9, 3)
        src = synth.normal(tuple(mp.act[0][0].shape), cfg.seed, "ablation_in").to(mp.act[0][0].dtype)
        for buf in mp.act[0] + mp.grad[n_layers]:
            buf.copy_(src)
        vals = []
        for mbs in mbs_list:
            mp.run(mbs)  # warm-up
            mp.sync()
            t0 = time.perf_counter()
            for _ in range(reps):
                mp.run(mbs)
            mp.sync()
            dt = (time.perf_counter() - t0) / reps
            vals.append(round(mp.tokens(mbs) / dt, 1))
            log(f"[ablation] {pol} mbs={mbs}: {dt * 1e3:.1f} ms/pass, {vals[-1]:.0f} tokens/s")
        out[pol] = vals
        mp.close()
        del mp
        torch.cuda.empty_cache()
    out["windowed_over_no_prefetch"] = [round(w / n, 3) for w, n in zip(out["windowed"], out["no_prefetch"])]
    out["windowed_over_prefetch"] = [round(w / p, 3) for w, p in zip(out["windowed"], out["prefetch"])]
    return out


def optimizer_step_time(n_layers: int = 4, reps: int = 3):
    """Host optimizer step (rp_opt_*: G-cp, fp32 Adam, P-cp to the bf16 master
    copy) over n_layers Llama-3.1-8B-shaped layers, every protocol edge
    already signalled, on the host's threads. Reported per billion parameters
    and projected to the 8B and 32B models' decoder parameters."""
    import os as _os
    from offloaded_pipeline_stage_amd import binding as B
    from offloaded_pipeline_stage_amd.optimizer import AdamParams, OptimizerWorker
    cfg = synth.config("llama3_8b")
    per_layer = [B.block_layout(cfg, B.RP_BLOCK_WEIGHT, t)[1] // 2 for t in
                 (B.RP_T_GAMMA1, B.RP_T_WQKV, B.RP_T_WO, B.RP_T_GAMMA2, B.RP_T_WGU, B.RP_T_WD)]
    threads = len(_os.sched_getaffinity(0))
    opt = OptimizerWorker(n_layers, torch.bfloat16, n_threads=threads)
    for l in range(n_layers):
        segs = []
        for n in per_layer:
            segs.append((torch.full((n,), 0.01, dtype=torch.bfloat16), torch.full((n,), 1e-3), None))
        opt.bind_segments(l, segs)
    n_params = n_layers * sum(per_layer)
    hp = AdamParams(lr=1e-5, weight_decay=0.01)
    times = []
    for it in range(reps + 1):
        opt.signal(B.RP_OPT_GRADS_DOWNLOADED, -1, it)
        opt.signal(B.RP_OPT_PARAMS_UPLOADED, -1, it + 1)
        t0 = time.perf_counter()
        opt.step(it, hp)
        opt.sync()
        if it > 0:
            times.append(time.perf_counter() - t0)
    opt.close()
    dt = sorted(times)[len(times) // 2]
    s_per_b = dt / (n_params / 1e9)
    return {"params": n_params, "threads": threads, "s_per_step": round(dt, 3),
            "s_per_1B_params": round(s_per_b, 3),
            "projected_llama3_8b_layers_s": round(s_per_b * 32 * sum(per_layer) / 1e9, 2),
            "projected_32B_params_s": round(s_per_b * 32, 2),
            "note": "median of 3 steps after one warm-up; the pages quote 9.6 s for a 32B model's CPU step "
                    "(ZeRO-Offload, on other hardware) as context"}


def config_sweep(reps: int = 3):
    """Per-call and per-configuration throughput with resident weights, each
    configuration's own call sequence: wall time with the context synced
    (median of `reps` after one warm-up), tokens/s = T / time, and
    matrix-product TFLOP/s."""
    from offloaded_pipeline_stage_amd import binding as B
    from offloaded_pipeline_stage_amd.worker import Worker

    def timed(ctx, fn):
        fn()
        ctx.sync()
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            ctx.sync()
            ts.append((time.perf_counter() - t0) * 1e3)
        return sorted(ts)[len(ts) // 2]

    def entry(cfg, ms, flops):
        return {"ms": round(ms, 3), "tokens_per_s": round(cfg.tokens / (ms / 1e3), 1),
                "tflops": round(flops / (ms / 1e3) / 1e12, 1)}

    out = {}
    dev = torch.device("cuda", 0)
    for name, n_fwd in (("tiny", 0), ("qwen3_1p7b", 4), ("llama3_8b", 1), ("qwen3_32b", 2), ("qwen3_235b_moe", 1)):
        cfg = synth.config(name)
        log(f"[bench] sweep {name}")
        T, H, b, s = cfg.tokens, cfg.hidden, cfg.batch, cfg.seq
        dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
        f_l, b_l = layer_cost(cfg)
        wk = Worker(cfg)
        ctx = wk.ctx
        moe = cfg.n_experts > 0
        n_layers = max(n_fwd, 1) + (1 if name in ("qwen3_1p7b", "qwen3_32b") else 0)
        if name == "tiny":
            n_layers = 2
        for l in range(n_layers):
            lw = synth.layer_weights(cfg, l)
            wk.add_layer(l, lw, lora=synth.lora_weights(cfg, l, b_zero=False) if cfg.lora_rank > 0 else None)
            del lw
        router = [synth.router_logits(cfg, l).to(dev) for l in range(n_layers)] if moe else None
        x = synth.activation(cfg, "x").to(dev)
        dy = synth.activation(cfg, "dy").to(dev)
        y, dx = torch.empty(T, H, dtype=dt, device=dev), torch.empty(T, H, dtype=dt, device=dev)
        res = {"tokens": T}
        if name == "tiny":
            # fused stage over both layers with the final-norm LM head
            head = synth.lmhead_weights(cfg)
            wk.add_lmhead(head["w"], head["gamma_f"])
            labels = synth.shifted_labels(synth.token_ids(cfg)).reshape(-1).to(dev)
            loss = torch.zeros(1, device=dev)
            ws = ctx.workspace(B.RP_OP_FUSED, b, s, 2)
            ws_h = ctx.workspace(B.RP_OP_LMHEAD, b, s)

            def fused():
                ctx.stage_fwd(0, 2, b, s, x, y, ws, flags=B.RP_KEEP_ACTS)
                ctx.lmhead_ce_fwd_bwd(b, s, y, labels, loss, dy, ws_h)
                ctx.stage_bwd_recompute(0, 2, b, s, dy, dx, ws, flags=B.RP_USE_KEPT_ACTS)
            res["fused_2_layers_with_lm_head"] = entry(cfg, timed(ctx, fused), 2 * (f_l + b_l) + lmhead_flops(cfg))
            res["note"] = "fp32: the generic FMA GEMM path, not MFMA"
        elif name == "llama3_8b":
            head = synth.lmhead_weights(cfg)
            wk.add_lmhead(head["w"])
            del head
            labels = synth.uniform_labels(cfg).to(dev)
            loss = torch.zeros(1, device=dev)
            ck = [torch.empty(T, H, dtype=dt).pin_memory()]
            ws_f = ctx.workspace(B.RP_OP_STAGE_FWD, b, s, 1)
            ws_b = ctx.workspace(B.RP_OP_STAGE_BWD, b, s, 1)
            ws_h = ctx.workspace(B.RP_OP_LMHEAD, b, s)
            t_f = timed(ctx, lambda: ctx.stage_fwd(0, 1, b, s, x, y, ws_f, ckpt_host=ck))
            t_h = timed(ctx, lambda: ctx.lmhead_ce_fwd_bwd(b, s, y, labels, loss, dy, ws_h))
            t_b = timed(ctx, lambda: ctx.stage_bwd_recompute(0, 1, b, s, dy, dx, ws_b, ckpt=ck))
            res["fwd_1_layer"] = entry(cfg, t_f, f_l)
            res["lm_head_4_shards"] = entry(cfg, t_h, lmhead_flops(cfg))
            res["bwd_recompute_1_layer"] = entry(cfg, t_b, f_l + b_l)
            res["fwd_plus_bwd_recompute_1_layer"] = entry(cfg, t_f + t_b, 2 * f_l + b_l)
            del ws_f, ws_b
            torch.cuda.empty_cache()
            ws = ctx.workspace(B.RP_OP_FUSED, b, s, 1)

            def fused():
                ctx.stage_fwd(0, 1, b, s, x, y, ws, flags=B.RP_KEEP_ACTS)
                ctx.lmhead_ce_fwd_bwd(b, s, y, labels, loss, dy, ws_h)
                ctx.stage_bwd_recompute(0, 1, b, s, dy, dx, ws, flags=B.RP_USE_KEPT_ACTS)
            res["fused_b1_layer_with_lm_head"] = entry(cfg, timed(ctx, fused), f_l + b_l + lmhead_flops(cfg))
            t_model = 32 * (t_f + t_b) + t_h
            res["extrapolated_full_8b_model"] = {
                "ms": round(t_model, 1), "tokens_per_s": round(T / (t_model / 1e3), 1),
                "note": "extrapolation: T / (32 (t_fwd + t_bwd_recompute) + t_lm_head), weights resident"}
        else:
            ws_f = ctx.workspace(B.RP_OP_STAGE_FWD, b, s, max(n_fwd, 1))
            ws_b = ctx.workspace(B.RP_OP_STAGE_BWD, b, s, 1)
            lb = n_layers - 1  # the backward layer
            rf = router[:n_fwd] if moe else None
            rb = [router[lb]] if moe else None
            t_f = timed(ctx, lambda: ctx.stage_fwd(0, n_fwd, b, s, x, y, ws_f, router=rf))
            t_b = timed(ctx, lambda: ctx.stage_bwd_recompute(lb, lb + 1, b, s, dy, dx, ws_b, ckpt=[x], router=rb,
                                                              flags=B.RP_CKPT_DEVICE))
            res[f"fwd_{n_fwd}_layers"] = entry(cfg, t_f, n_fwd * f_l)
            res["bwd_recompute_1_layer"] = entry(cfg, t_b, f_l + b_l)
            res["stage_total"] = entry(cfg, t_f + t_b, (n_fwd + 1) * f_l + b_l)
        out[name] = res
        del wk, ctx
        torch.cuda.empty_cache()
    return out


def link_peak(nbytes: int = 1 << 30, chunk: int = 64 << 20, reps: int = 3):
    """The host link's pinned-copy rate on this machine: plain asynchronous copies
    between pinned host memory and the device, in chunks of the size the
    streamed step uses, on two independent non-blocking streams: one
    direction at a time, then both directions at once. Best of `reps`, GB/s.
    (A measurement of the link itself, outside the library's ordering rules:
    its activation downloads follow the compute stream, which waits for its
    activation uploads.)"""
    host_up = torch.ones(nbytes, dtype=torch.uint8).pin_memory()
    host_dn = torch.empty(nbytes, dtype=torch.uint8).pin_memory()
    dev_up = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dev_dn = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    s_up, s_dn = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()

    def up():
        with torch.cuda.stream(s_up):
            for o in range(0, nbytes, chunk):
                dev_up[o:o + chunk].copy_(host_up[o:o + chunk], non_blocking=True)

    def down():
        with torch.cuda.stream(s_dn):
            for o in range(0, nbytes, chunk):
                host_dn[o:o + chunk].copy_(dev_dn[o:o + chunk], non_blocking=True)

    def timed(fn):
        best = float("inf")
        for _ in range(reps + 1):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            best = min(best, time.perf_counter() - t0)
        return best

    t_up, t_dn = timed(up), timed(down)
    t_both = timed(lambda: (up(), down()))
    del host_up, host_dn, dev_up, dev_dn
    torch.cuda.empty_cache()
    return {"h2d_GBps": round(nbytes / t_up / 1e9, 1), "d2h_GBps": round(nbytes / t_dn / 1e9, 1),
            "both_directions_GBps": round(2 * nbytes / t_both / 1e9, 1), "bytes_per_direction": nbytes,
            "chunk_bytes": chunk}


def time_steps(st, steps: int, warmup: int) -> float:
    """ms per step of a Step over `steps` after `warmup`."""
    for _ in range(warmup):
        st.run()
    st.sync()
    t0 = time.perf_counter()
    for _ in range(steps):
        st.run()
    st.sync()
    return (time.perf_counter() - t0) * 1e3 / steps


def streamed_figures(cfg, steps: int, warmup: int, ms_resident: float, peak: dict, grad_bf16: bool = False):
    """The step with every weight uploaded from pinned host memory and every
    gradient downloaded to it (the workload as stated: bf16 weights streamed
    in, fp32 gradients out), against the resident step (compute alone) and
    the same transfers alone (link alone). link_bound_ms is the busier
    direction at its measured peak (the directions overlapping fully),
    link_serial_ms both directions one after the other."""
    st = Step(cfg, streamed=True, grad_bf16=grad_bf16)
    ms_s = time_steps(st, steps, warmup)
    st.sync()
    xs = []
    for _ in range(3):
        t0 = time.perf_counter()
        st.run_transfers_only()
        st.sync()
        xs.append((time.perf_counter() - t0) * 1e3)
    ms_x = sorted(xs)[1]
    h2d = st.wk.w_bytes + sum(h.numel() * h.element_size() for h in st.host_shards)
    d2h = (st.wk.g_bytes + sum(h.numel() * 4 for h in st.host_dshards)) // (2 if grad_bf16 else 1)
    del st
    torch.cuda.empty_cache()
    t_up, t_dn = h2d / (peak["h2d_GBps"] * 1e9), d2h / (peak["d2h_GBps"] * 1e9)
    return {"tokens_per_s": round(cfg.tokens / (ms_s / 1e3), 1), "ms_per_step": round(ms_s, 3),
            "over_resident": round(ms_s / ms_resident, 3),
            "h2d_GB_per_step": round(h2d / 1e9, 3), "d2h_GB_per_step": round(d2h / 1e9, 3),
            "transfers_alone_ms": round(ms_x, 3),
            "link_bound_ms": round(max(t_up, t_dn) * 1e3, 3),
            "link_serial_ms": round((t_up + t_dn) * 1e3, 3),
            "overlap_efficiency": round((ms_resident + ms_x - ms_s) / min(ms_resident, ms_x), 3),
            "h2d_GBps": round(h2d / 1e9 / (ms_s / 1e3), 1), "d2h_GBps": round(d2h / 1e9 / (ms_s / 1e3), 1),
            "h2d_frac_of_peak": round(h2d / 1e9 / (ms_s / 1e3) / peak["h2d_GBps"], 3),
            "d2h_frac_of_peak": round(d2h / 1e9 / (ms_s / 1e3) / peak["d2h_GBps"], 3),
            "link_GBps": round((h2d + d2h) / 1e9 / (ms_s / 1e3), 1)}


def cpu_baseline(cfg, head_rows: int):
    """The oracle, as it stands, on the host cores in fp32 (the workload's
    gradient precision): the full layer at the workload's sequence length
    (forward, then recompute + backward), and the LM head + cross-entropy on
    `head_rows` of its token rows. The LM head's work per token does not
    depend on the sequence length, so its time is scaled by tokens /
    head_rows; tokens/s = tokens / (layer time + scaled LM-head time)."""
    from oracle import stage as O
    f32 = torch.float32
    lw = synth.layer_weights(cfg, 0)
    x = synth.activation(cfg, "x")
    dy = synth.activation(cfg, "dy")
    t0 = time.time()
    y, ck = O.stage_forward(x, [lw], cfg, dtype=f32)
    O.stage_backward_recompute(ck, [lw], dy, cfg, dtype=f32)
    t_layer = time.time() - t0
    del y, ck
    w = synth.lmhead_weights(cfg)["w"]
    labels = synth.uniform_labels(cfg)[:head_rows]
    t0 = time.time()
    O.lmhead_fwd_bwd(x[:head_rows], w, labels, cfg.n_shards, dtype=f32)
    t_head = time.time() - t0
    t_step = t_layer + t_head * cfg.tokens / head_rows
    import platform
    cpu = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return {"value": round(cfg.tokens / t_step, 2), "unit": "tokens/s", "cores": torch.get_num_threads(),
            "kind": "oracle",
            "sample": f"fp32 torch on the host ({cpu}): the full layer at 1 x {cfg.seq} tokens, forward then "
                      f"recompute + backward, {t_layer:.1f} s; the {cfg.n_shards}-shard LM head + CE forward/backward "
                      f"on {head_rows} of the {cfg.tokens} token rows, {t_head:.1f} s, scaled by "
                      f"{cfg.tokens // head_rows} (its work per token does not depend on the sequence length)"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter,
                                 allow_abbrev=False)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama3_8b")
    ap.add_argument("--no-streamed", action="store_true",
                    help="skip the weight-streaming step (run by default, reported under 'streamed')")
    ap.add_argument("--streamed-only", action="store_true",
                    help="run only the streamed step with fp32 gradients (for copy traces); prints its figures")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-head-rows", type=int, default=1024,
                    help="token rows of the LM head in the CPU oracle's timed sample")
    ap.add_argument("--trace-json", default=None, help="write the per-kernel table here")
    ap.add_argument("--configs", action="store_true",
                    help="also time every configuration's own call sequence (resident weights)")
    ap.add_argument("--optimizer", action="store_true",
                    help="also time the host optimizer step (Adam, G-cp, P-cp) on Llama-8B-shaped layers")
    ap.add_argument("--ablation", action="store_true",
                    help="also run the transfer-policy ablation over micro-batch sizes")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run one device copy of this size (for the HBM counter runs)")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {a.gpus}); "
              f"the worker step is the per-GPU unit and is reported at N=1 only.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (HIP device)", file=sys.stderr)
        sys.exit(1)
    from offloaded_pipeline_stage_amd import binding
    binding.lib()  # fails loudly when librp.so is missing

    cfg = synth.config(a.workload)
    traffic_file = os.path.join(ROOT, "profiles", f"{a.workload}_step_traffic.txt")
    if a.streamed_only:
        st = Step(cfg, streamed=True)
        ms_s = time_steps(st, a.steps, a.warmup)
        print(json.dumps({"streamed_only": {"ms_per_step": round(ms_s, 3), "steps": a.steps, "warmup": a.warmup,
                                            "tokens_per_s": round(cfg.tokens / (ms_s / 1e3), 1)}}), flush=True)
        return
    step = Step(cfg, streamed=False)
    if a.copy_calibration_mib > 0:
        copy_calibration(step.wk.ctx, a.copy_calibration_mib)
    for _ in range(a.warmup):
        step.run()
    step.sync()
    ctx = step.wk.ctx
    ctx.trace_begin(100000)
    step.sync()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        step.run()
    step.sync()
    t1 = time.perf_counter()
    recs = ctx.trace_end()
    ms_step = (t1 - t0) * 1e3 / a.steps
    tok_s = cfg.tokens / (ms_step / 1e3)
    agg = summarize_trace(recs, a.steps)
    lf = layer_flops(cfg, recompute=True)
    step_flops = lf["fwd"] + lf["recompute"] + lf["bwd"] + lmhead_flops(cfg)
    traced_flops = sum(v[1] for v in agg.values()) / a.steps
    kernels = sorted(((k, v[3] / a.steps) for k, v in agg.items()), key=lambda kv: -kv[1])
    out = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights, uniform labels)",
        "config": {"workload": "Llama-3.1-8B-shaped stage: 1 layer fwd + recompute+bwd, 4-shard LM head + CE",
                   "batch": cfg.batch, "seq": cfg.seq, "hidden": cfg.hidden, "n_q": cfg.n_q, "n_kv": cfg.n_kv,
                   "head_dim": cfg.head_dim, "ffn": cfg.ffn, "vocab": cfg.vocab, "n_shards": cfg.n_shards,
                   "weights": "resident in HBM"},
        "step_tflop": round(step_flops / 1e12, 3),
        "tflops": round(step_flops / (ms_step / 1e3) / 1e12, 1),
        "mfma_util": round(step_flops / (ms_step / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "traced_tflop_per_step": round(traced_flops / 1e12, 3),
        "roofline": roofline(agg, cfg.dtype, traffic_file),
        "kernels_ms_per_step": {k: round(v, 3) for k, v in kernels[:12]},
    }
    if a.trace_json:
        with open(a.trace_json, "w") as f:
            json.dump({k: {"launches": v[0], "flops": v[1], "bytes": v[2], "ms": v[3]} for k, v in agg.items()},
                      f, indent=1)
    del step
    torch.cuda.empty_cache()

    if not a.no_streamed:
        peak = link_peak()
        out["link_peak"] = peak
        out["streamed"] = streamed_figures(cfg, a.steps, a.warmup, ms_step, peak)
        log(f"[bench] streamed {out['streamed']}")
        # the same step with the gradients on the link in bf16 (the pages'
        # precision; the workload's own gradients are fp32)
        out["streamed_bf16_grads"] = streamed_figures(cfg, a.steps, a.warmup, ms_step, peak, grad_bf16=True)
        out["priority"] = priority_probe(cfg)
        torch.cuda.empty_cache()

    if a.configs:
        out["configs"] = config_sweep()
    if a.ablation:
        out["ablation"] = transfer_ablation()
    if a.optimizer:
        out["optimizer"] = optimizer_step_time()
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, a.cpu_head_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
