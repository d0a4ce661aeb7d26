"""A whole decoder model trained through RoundPipe's stage structure on one
GPU worker ("Efficient Training on Multiple Consumer GPUs with RoundPipe").

* Profiling (section 4.4): the first iterations run one layer per stage and
  time every layer's forward, backward (with recomputation) and the LM head
  with events on the compute stream.
* Partitioning (section 4.4.2): rp_partition turns those times and a memory
  model into forward stages F_1 .. F_Sf, the fused first backward stage B_1
  (the last b1 layers, whose forward doubles as the recomputation, with the
  LM head) and backward stages B_2 .. B_Sb.
* An iteration (section 3.2): embedding; every forward stage, which downloads
  each layer's input to pinned host memory (the checkpoints, section 2.1.1);
  B_1; every other backward stage, which recomputes from those checkpoints;
  the embedding backward.

With one GPU every stage runs on the same worker in order and the bubble
formula gives zero. Splitting changes only where the work runs, so every
partition yields bit-identical loss and gradients. Weights stay resident
here: their streaming per stage is covered by the micro-batch pass. This
module orders library calls; all arithmetic is in librp.so.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence, Tuple

import torch

from . import binding as B
from .worker import Worker


@dataclass(frozen=True)
class Partition:
    fwd: Tuple[int, ...]   # layer counts of F_1 .. F_Sf, front to back
    b1: int                # layers in the fused stage B_1 (the last b1 layers)
    bwd: Tuple[int, ...]   # layer counts of B_2 .. B_Sb, from just below B_1 down

    def stages(self, n_layers: int):
        """[(kind, l0, l1)] in execution order."""
        out, lo = [], 0
        for n in self.fwd:
            out.append(("F", lo, lo + n))
            lo += n
        if lo != n_layers - self.b1 or self.b1 < 1 or sum(self.bwd) != lo:
            raise ValueError(f"partition {self} does not cover {n_layers} layers")
        out.append(("B1", lo, n_layers))
        hi = lo
        for n in self.bwd:
            out.append(("B", hi - n, hi))
            hi -= n
        return out

    @staticmethod
    def fused(n_layers: int) -> "Partition":
        return Partition((), n_layers, ())

    @staticmethod
    def one_layer_per_stage(n_layers: int) -> "Partition":
        return Partition((1,) * (n_layers - 1), 1, (1,) * (n_layers - 1))


class RoundPipeModel:
    """layers: per-layer weight dicts; head: {"w": [V, H], "gamma_f": [H] or
    None, "embed": [V, H] or None} (the synth layouts)."""

    def __init__(self, cfg, layers: Sequence[Dict[str, torch.Tensor]], head: Dict[str, torch.Tensor],
                 device: int = 0):
        self.cfg = cfg
        self.L = len(layers)
        self.dev = torch.device("cuda", device)
        self.wk = Worker(cfg, device)
        self.ctx = self.wk.ctx
        for l, w in enumerate(layers):
            self.wk.add_layer(l, w)
        self.wk.add_lmhead(head["w"], head.get("gamma_f"))
        dt = self.wk.dt
        self.table = head["embed"].to(dt).to(self.dev) if head.get("embed") is not None else None
        self.dtable = torch.zeros_like(self.table, dtype=torch.float32) if self.table is not None else None
        T, H = cfg.tokens, cfg.hidden
        self.ckpt = [torch.empty(T, H, dtype=dt).pin_memory() for _ in range(self.L)]
        z = lambda: torch.empty(T, H, dtype=dt, device=self.dev)  # noqa: E731
        self.x0, self.act, self.dact, self.y, self.dy = z(), [z(), z()], [z(), z()], z(), z()
        self.loss = torch.zeros(1, dtype=torch.float32, device=self.dev)
        self._ws: Dict[Tuple[int, int], torch.Tensor] = {}

    # ------------------------------------------------------------ workspaces
    def _workspace(self, op: int, n: int) -> torch.Tensor:
        key = (op, n)
        if key not in self._ws:
            self._ws[key] = self.ctx.workspace(op, self.cfg.batch, self.cfg.seq, n)
        return self._ws[key]

    def memory_model(self) -> Tuple[List[float], List[float], float]:
        """Bytes a layer adds to a forward / backward stage (weights, gradient
        block, the call's workspace per layer) and the LM head's share."""
        c, b, s = self.ctx, self.cfg.batch, self.cfg.seq
        wl, gl = self.wk.w_bytes, self.wk.g_bytes
        mf = wl + c.workspace_size(B.RP_OP_STAGE_FWD, b, s, 1)
        mb = wl + gl + c.workspace_size(B.RP_OP_FUSED, b, s, 1)
        head = self.wk.head
        mh = sum(t.numel() * t.element_size() for t in head["w"] + head["dw"]) + \
            c.workspace_size(B.RP_OP_LMHEAD, b, s)
        return [float(mf)] * self.L, [float(mb)] * self.L, float(mh)

    # ------------------------------------------------------------ one iteration
    def step(self, ids: torch.Tensor, labels: torch.Tensor, x_in: Optional[torch.Tensor] = None,
             part: Optional[Partition] = None, events: Optional[list] = None):
        """Enqueue one forward + backward over the model. ids [T] int32 (with an
        embedding) or x_in [T, H] (without); labels [T] int32. Loss in
        self.loss; gradients in the layers' blocks, the LM head's buffers and
        self.dtable. events: list that receives (stage, l0, l1, start, end)
        compute-stream events when given."""
        ctx, cfg = self.ctx, self.cfg
        b, s = cfg.batch, cfg.seq
        part = part or Partition.fused(self.L)
        comp = self.ctx.streams["compute"]

        def mark():
            if events is None:
                return None
            e = torch.cuda.Event(enable_timing=True)
            e.record(comp)
            return e

        if self.table is not None:
            ctx.embed_fwd(ids, self.table, self.x0)
            x = self.x0
        else:
            x = x_in
        stages = part.stages(self.L)
        cur, pp = x, 0
        for kind, l0, l1 in stages:
            n = l1 - l0
            e0 = mark()
            if kind == "F":
                out = self.act[pp]
                ctx.stage_fwd(l0, l1, b, s, cur, out, self._workspace(B.RP_OP_STAGE_FWD, n),
                              ckpt_host=self.ckpt[l0:l1])
                cur, pp = out, pp ^ 1
            elif kind == "B1":
                ws = self._workspace(B.RP_OP_FUSED, n)
                ctx.stage_fwd(l0, l1, b, s, cur, self.y, ws, flags=B.RP_KEEP_ACTS)
                ctx.lmhead_ce_fwd_bwd(b, s, self.y, labels, self.loss, self.dy,
                                      self._workspace(B.RP_OP_LMHEAD, 1))
                g_out = self.dact[0] if l0 == 0 else self.dact[1]
                ctx.stage_bwd_recompute(l0, l1, b, s, self.dy, g_out, ws, flags=B.RP_USE_KEPT_ACTS)
                g_cur, gq = g_out, 0 if l0 != 0 else 1
            else:
                dst = self.dact[gq]
                ctx.stage_bwd_recompute(l0, l1, b, s, g_cur, dst, self._workspace(B.RP_OP_STAGE_BWD, n),
                                        ckpt=self.ckpt[l0:l1])
                g_cur, gq = dst, gq ^ 1
            if events is not None:
                events.append((kind, l0, l1, e0, mark()))
        if self.table is not None:
            ctx.embed_bwd(ids, g_cur, self.dtable)
        self.dx = g_cur
        return self.loss

    # ------------------------------------------------------------ profiling + plan
    def profile(self, ids, labels, x_in=None, reps: int = 2):
        """Per-layer forward and backward times and the LM head's (ms), from a
        one-layer-per-stage iteration timed with compute-stream events (the
        last of reps runs). The B_1 stage of that partition holds the top
        layer together with the LM head, so the top layer takes the times of
        the layer below it (the layers are alike) and the LM head the rest."""
        part = Partition.one_layer_per_stage(self.L)
        ev = []
        for _ in range(reps):
            ev = []
            self.step(ids, labels, x_in, part, events=ev)
        self.ctx.sync()
        torch.cuda.synchronize(self.dev)
        f = [0.0] * self.L
        bw = [0.0] * self.L
        b1_ms = 0.0
        for kind, l0, l1, e0, e1 in ev:
            ms = e0.elapsed_time(e1)
            if kind == "F":
                f[l0] = ms
            elif kind == "B":
                bw[l0] = ms
            else:
                b1_ms = ms
        # B_1 costs h + b[top] in the partition model (its forward is the
        # recomputation), so the LM head's share is what B_1 took beyond that
        top = self.L - 1
        if self.L > 1:
            f[top] = f[top - 1]
            bw[top] = bw[top - 1]
        else:
            f[top] = bw[top] = b1_ms / 3.0
        h = max(b1_ms - bw[top], 0.0)
        return f, bw, h

    def plan(self, f, bw, h, n_micro: int, n_gpus: int, mem_cap: float) -> Tuple[float, Partition]:
        mf, mb, mh = self.memory_model()
        obj, fwd, b1, bwd = B.partition(f, bw, h, mf, mb, mh, mem_cap, n_micro, n_gpus)
        return obj, Partition(fwd, b1, bwd)

    def layer_grads(self, l: int):
        return self.wk.unpack_grads(self.wk.layers[l]["g"])

    def close(self):
        self.ctx.close()
