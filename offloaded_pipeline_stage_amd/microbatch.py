"""A worker's stages over several micro-batches, with the next stage's weights
streaming in and the previous stage's gradients streaming out during the
current stage's compute ("Efficient Training on Multiple Consumer GPUs with
RoundPipe", section 4.2 "Data Transfer Overlap"), under the three transfer
policies that its priority-aware transfer ablation compares (section 5.8.2).

One pass runs the forward stages F_0 .. F_{K-1} and then the backward stages
B_{K-1} .. B_0, one decoder layer per stage, each over M micro-batches of
`mbs` rows. As on a RoundPipe worker, every activation and activation
gradient goes through pinned host memory between stages: it is uploaded one
micro-batch ahead of its compute and downloaded behind it (section 4.2.1).
Weights come from pinned host blocks; the fp32 weight gradients of a backward
stage are summed over its micro-batches on the device (RP_ACCUM_GRADS) and go
back to pinned host blocks once per stage.

Policies:
  no_prefetch  one device weight slot. A stage's weights go up only after the
               previous stage has finished with the slot, and a stage's
               gradients go down before the next backward may reuse the block:
               transfers never overlap compute.
  prefetch     two weight slots. The next stage's weights go up in one piece as
               soon as this stage starts, ungated, and the stage's gradients go
               down in one piece when it ends. The copy engine serves its
               queues first in, first out, so this stage's activation uploads
               wait behind the weights (head-of-line blocking).
  windowed     two weight slots. The next stage's weights and the previous
               stage's gradients are split and LPT-packed into M windows
               (section 4.2.2); window j is gated on micro-batch j + 1's
               activation upload, so every activation copy goes first.

Every policy computes the same thing, call for call: only the transfer order
differs, and the results are bit-identical. This module orders library calls;
all arithmetic is in librp.so.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import torch

from . import binding as B
from .worker import Worker

POLICIES = ("no_prefetch", "prefetch", "windowed")

# a host buffer's producing download is waited for only while its ticket's
# event is still kept by the library (it keeps the last 256); an older one has
# completed, since the upload stream has since waited on newer downloads of
# the same in-order download stream
_TICKET_HORIZON = 200


class MicrobatchPass:
    """Buffers and call order of one forward + backward pass over K one-layer
    stages, M micro-batches each, for micro-batch sizes up to `max_mbs` rows
    of cfg.seq tokens.

    host_layers: K pinned weight blocks (Worker.pack_layer(..., pinned=True)).
    """

    def __init__(self, cfg, host_layers: Sequence[torch.Tensor], n_micro: int, max_mbs: int,
                 policy: str, max_chunk: int = 64 << 20, device: int = 0):
        if policy not in POLICIES:
            raise ValueError(f"unknown policy {policy!r}; one of {POLICIES}")
        if n_micro < 1 or max_mbs < 1 or not host_layers:
            raise ValueError("need at least one layer, one micro-batch and one row per micro-batch")
        if cfg.lora_rank or cfg.n_experts:
            raise ValueError("the micro-batch pass runs dense full fine-tune layers")
        self.cfg = cfg.with_(batch=max_mbs)
        self.policy = policy
        self.M = n_micro
        self.K = len(host_layers)
        self.max_mbs = max_mbs
        self.max_chunk = max_chunk
        self.dev = torch.device("cuda", device)
        self.wk = Worker(self.cfg, device)
        self.ctx = self.wk.ctx
        self.host_w = list(host_layers)
        for w in self.host_w:
            if not w.is_pinned() or w.numel() != self.wk.w_bytes:
                raise ValueError("host layers must be pinned weight blocks of the context's layout")
        self.n_slots = 1 if policy == "no_prefetch" else 2
        for s in range(self.n_slots):
            self.wk.add_layer(s, resident=False)
        T, H, M, K = self.cfg.tokens, self.cfg.hidden, n_micro, self.K
        dt = self.wk.dt
        pin = lambda: torch.empty(T, H, dtype=dt).pin_memory()  # noqa: E731
        # act[l][j]: input of layer l for micro-batch j (act[K]: the pass output)
        self.act = [[pin() for _ in range(M)] for _ in range(K + 1)]
        # grad[l][j]: gradient w.r.t. act[l][j] (grad[K]: the given dy)
        self.grad = [[pin() for _ in range(M)] for _ in range(K + 1)]
        self.wgrad = [torch.empty(self.wk.g_bytes, dtype=torch.uint8).pin_memory() for _ in range(K)]
        dv = lambda: torch.empty(T, H, dtype=dt, device=self.dev)  # noqa: E731
        # two device sets (consecutive stages alternate) of per-micro-batch buffers
        self.d_in = [[dv() for _ in range(M)] for _ in range(2)]
        self.d_in2 = [[dv() for _ in range(M)] for _ in range(2)]
        self.d_out = [[dv() for _ in range(M)] for _ in range(2)]
        self.ws_f = self.ctx.workspace(B.RP_OP_STAGE_FWD, max_mbs, self.cfg.seq, 1)
        self.ws_b = self.ctx.workspace(B.RP_OP_STAGE_BWD, max_mbs, self.cfg.seq, 1)
        self.produced: Dict[int, int] = {}  # id(host buffer) -> ticket of the download that fills it
        torch.cuda.synchronize(self.dev)

    # ---------------------------------------------------------------- helpers
    def tokens(self, mbs: int) -> int:
        return self.M * mbs * self.cfg.seq

    def _view(self, t: torch.Tensor, rows: int) -> torch.Tensor:
        return t[:rows]

    def _upload_item(self, stage: int, layer: int):
        return (B.RP_PARAM_H2D, B.RP_TGT_LAYER, self._slot(stage), 0, self.wk.w_bytes, self.host_w[layer])

    def _grad_item(self, stage: int, layer: int):
        return (B.RP_GRAD_D2H, B.RP_TGT_LAYER, self._slot(stage), 0, self.wk.g_bytes, self.wgrad[layer])

    def _slot(self, stage: int) -> int:
        return stage % self.n_slots

    def _stage_ops(self, kind: str, layer: int, par: int, rows: int):
        """The stage's activation copies and compute calls in issue order:
        ("h2d", dev, host, micro-batch), ("d2h", host, dev, micro-batch) or
        ("compute", micro-batch)."""
        M, ops = self.M, []
        v = self._view

        def uploads(j):
            # the layer input (the checkpoint, for a backward stage), then dy
            ops.append(("h2d", v(self.d_in[par][j], rows), v(self.act[layer][j], rows), j))
            if kind == "B":
                ops.append(("h2d", v(self.d_in2[par][j], rows), v(self.grad[layer + 1][j], rows), j))

        uploads(0)
        for j in range(M):
            ops.append(("compute", j))
            if j + 1 < M:
                uploads(j + 1)
            dst = self.act[layer + 1][j] if kind == "F" else self.grad[layer][j]
            ops.append(("d2h", v(dst, rows), v(self.d_out[par][j], rows), j))
        return ops

    @staticmethod
    def window_gates(ops, t0: int, n_windows: int) -> List[int]:
        """Ticket that gates window j: the last activation upload of micro-batch
        j + 1 (of the last micro-batch for the final window), with tickets
        numbered from t0 in the order of the copies in `ops`."""
        last_up: Dict[int, int] = {}
        t = t0
        for op in ops:
            if op[0] == "compute":
                continue
            if op[0] == "h2d":
                last_up[op[3]] = t
            t += 1
        return [last_up[min(j + 1, n_windows - 1)] for j in range(n_windows)]

    def _submit(self, items, gates: Optional[List[int]] = None):
        if not items:
            return
        if gates is None:
            self.ctx.weight_stream_submit(items, n_windows=1, max_chunk=self.max_chunk)
        else:
            self.ctx.weight_stream_submit_gated(items, gates, max_chunk=self.max_chunk)

    # ---------------------------------------------------------------- a pass
    def run(self, mbs: int):
        """Enqueue one pass at micro-batch size mbs (rows of cfg.seq tokens);
        the caller syncs. Inputs: act[0][j] and grad[K][j] (first mbs rows);
        outputs: act[K][j], grad[0][j] and the per-layer gradient blocks."""
        if not 1 <= mbs <= self.max_mbs:
            raise ValueError(f"mbs {mbs} outside [1, {self.max_mbs}]")
        ctx, M, K, seq = self.ctx, self.M, self.K, self.cfg.seq
        rows = mbs * seq
        stages = [("F", l) for l in range(K)] + [("B", l) for l in reversed(range(K))]
        self._submit([self._upload_item(0, stages[0][1])])
        pending_grads = []  # gradient downloads still to be scheduled (windowed policy)
        last_d2h: Dict[int, int] = {}  # stage -> ticket of its last activation download
        for k, (kind, layer) in enumerate(stages):
            par = k & 1
            ops = self._stage_ops(kind, layer, par, rows)
            if k >= 2 and last_d2h[k - 2] >= ctx.act_next_ticket() - _TICKET_HORIZON:
                # this stage reuses the device buffers of stage k - 2: its uploads
                # (and through them its compute) start after that stage's last
                # download, which itself followed all of that stage's compute. An
                # older ticket needs no wait: stage k - 1's uploads already waited
                # on stage k - 2's downloads, ahead of everything on the stream.
                ctx.act_wait(B.RP_ON_ACT_H2D, last_d2h[k - 2])
            nxt = [self._upload_item(k + 1, stages[k + 1][1])] if k + 1 < len(stages) else []
            if self.policy == "windowed":
                t0 = ctx.act_next_ticket()
                self._submit(nxt + pending_grads, self.window_gates(ops, t0, M))
                pending_grads = []
            elif self.policy == "prefetch":
                self._submit(nxt)
            slot = self._slot(k)
            for op in ops:
                if op[0] == "compute":
                    j = op[1]
                    x, y = self.d_in[par][j], self.d_out[par][j]
                    if kind == "F":
                        ctx.stage_fwd(slot, slot + 1, mbs, seq, x, y, self.ws_f)
                    else:
                        flags = B.RP_CKPT_DEVICE | (B.RP_ACCUM_GRADS if j > 0 else 0)
                        ctx.stage_bwd_recompute(slot, slot + 1, mbs, seq, self.d_in2[par][j], y, self.ws_b,
                                                ckpt=[x], flags=flags)
                elif op[0] == "h2d":
                    _, dst, src, _ = op
                    prod = self.produced.get(src.data_ptr())
                    if prod is not None and prod >= ctx.act_next_ticket() - _TICKET_HORIZON:
                        ctx.act_wait(B.RP_ON_ACT_H2D, prod)
                    ctx.act_copy(B.RP_H2D, dst, src)
                else:
                    _, dst, src, _ = op
                    self.produced[dst.data_ptr()] = last_d2h[k] = ctx.act_copy(B.RP_D2H, dst, src)
            if kind == "B":
                g = [self._grad_item(k, layer)]
                if self.policy == "windowed" and k + 1 < len(stages):
                    pending_grads = g
                else:
                    self._submit(g)
            if self.policy == "no_prefetch" and nxt:
                # waits for this stage's last use of the one weight slot
                self._submit(nxt)

    def sync(self):
        self.ctx.sync()
        torch.cuda.synchronize(self.dev)

    def close(self):
        self.ctx.close()
