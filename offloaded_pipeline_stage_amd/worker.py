"""Drive one GPU worker's stages through the C ABI.

Packs per-layer weight dictionaries (names wq, wk, wv, wo, wg, wu, wd,
gamma1, gamma2; LoRA aq..bo) into the library's block layout, holds the
device/pinned buffers, and unpacks the fp32 gradient blocks. All arithmetic
is in librp.so; this is marshalling.
"""
from __future__ import annotations

from typing import Dict, List, Optional

import torch

from . import binding as B

LAYER_NAMES = ("gamma1", "wq", "wk", "wv", "wo", "gamma2", "wg", "wu", "wd")


def storage_dtype(cfg) -> torch.dtype:
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


class Worker:
    def __init__(self, cfg, device: int = 0):
        self.cfg = cfg
        self.dev = torch.device("cuda", device)
        self.ctx = B.Context(cfg, device)
        self.dt = storage_dtype(cfg)
        self.w_bytes = self.ctx.block_bytes(B.RP_BLOCK_WEIGHT)
        self.g_bytes = self.ctx.block_bytes(B.RP_BLOCK_GRAD)
        self.layers: Dict[int, dict] = {}
        self.head: Optional[dict] = None

    # ------------------------------------------------------------------ layers
    def layer_tensors(self, w: Dict[str, torch.Tensor]) -> Dict[int, torch.Tensor]:
        cfg = self.cfg
        if cfg.n_experts > 0:
            gu = torch.cat([w["wg"], w["wu"]], dim=1)  # [E, 2Fe, H]
        else:
            gu = torch.cat([w["wg"], w["wu"]], dim=0)  # [2F, H]
        t = {
            B.RP_T_GAMMA1: w["gamma1"], B.RP_T_WQKV: torch.cat([w["wq"], w["wk"], w["wv"]], dim=0),
            B.RP_T_WO: w["wo"], B.RP_T_GAMMA2: w["gamma2"], B.RP_T_WGU: gu, B.RP_T_WD: w["wd"],
        }
        if getattr(cfg, "qk_norm", False):
            t[B.RP_T_QNORM] = w["qnorm"]
            t[B.RP_T_KNORM] = w["knorm"]
        return t

    def pack_layer(self, w: Dict[str, torch.Tensor], pinned: bool = False) -> torch.Tensor:
        """Packed weight block, on the device or in pinned host memory."""
        host = torch.zeros(self.w_bytes, dtype=torch.uint8)
        self.ctx.pack(B.RP_BLOCK_WEIGHT, {k: v.to(self.dt).cpu() for k, v in self.layer_tensors(w).items()}, host)
        if pinned:
            return host.pin_memory()
        return host.to(self.dev)

    LORA_IDS = (("aq", B.RP_T_AQ), ("bq", B.RP_T_BQ), ("ak", B.RP_T_AK), ("bk", B.RP_T_BK),
                ("av", B.RP_T_AV), ("bv", B.RP_T_BV), ("ao", B.RP_T_AO), ("bo", B.RP_T_BO))

    def pack_lora(self, lora: Dict[str, torch.Tensor], pinned: bool = False) -> torch.Tensor:
        """fp32 adapter block (A_q, B_q, ..., B_o at the library's offsets)."""
        host = torch.zeros(self.ctx.block_bytes(B.RP_BLOCK_LORA), dtype=torch.uint8)
        self.ctx.pack(B.RP_BLOCK_LORA, {tid: lora[n].float().cpu() for n, tid in self.LORA_IDS}, host)
        return host.pin_memory() if pinned else host.to(self.dev)

    def add_layer(self, layer: int, w: Optional[Dict[str, torch.Tensor]] = None, resident: bool = True,
                  grads: bool = True, wbuf: Optional[torch.Tensor] = None,
                  lora: Optional[Dict[str, torch.Tensor]] = None):
        """Allocate (and fill, if resident) the layer's device buffers and bind them.
        LoRA contexts freeze the base: no base-gradient block, an adapter block
        and its fp32 gradient block instead."""
        if wbuf is None:
            wbuf = self.pack_layer(w) if resident else torch.empty(self.w_bytes, dtype=torch.uint8, device=self.dev)
        lbuf = lgbuf = gbuf = None
        if self.cfg.lora_rank > 0:
            nb = self.ctx.block_bytes(B.RP_BLOCK_LORA)
            lbuf = self.pack_lora(lora) if lora is not None else torch.zeros(nb, dtype=torch.uint8, device=self.dev)
            lgbuf = torch.zeros(nb, dtype=torch.uint8, device=self.dev) if grads else None
        elif grads:
            gbuf = torch.zeros(self.g_bytes, dtype=torch.uint8, device=self.dev)
        self.ctx.bind_layer(layer, wbuf, gbuf, lbuf, lgbuf)
        self.layers[layer] = {"w": wbuf, "g": gbuf, "lora": lbuf, "lora_g": lgbuf}
        # torch filled / copied these on its own stream; the library's streams
        # must not see them before that work is done
        torch.cuda.current_stream(self.dev).synchronize()
        return wbuf, gbuf

    def unpack_lora_grads(self, lgbuf: torch.Tensor) -> Dict[str, torch.Tensor]:
        cfg = self.cfg
        r, H, Q, KV = cfg.lora_rank, cfg.hidden, cfg.q_dim, cfg.kv_dim
        shapes = {"aq": (r, H), "bq": (Q, r), "ak": (r, H), "bk": (KV, r), "av": (r, H), "bv": (KV, r),
                  "ao": (r, Q), "bo": (H, r)}
        out = {}
        for n, tid in self.LORA_IDS:
            off, nb = self.ctx.layout(B.RP_BLOCK_LORA, tid)
            out[n] = lgbuf[off:off + nb].view(torch.float32).view(*shapes[n])
        return out

    def unpack_grads(self, gbuf: torch.Tensor) -> Dict[str, torch.Tensor]:
        cfg = self.cfg
        g = {}
        tids = [B.RP_T_GAMMA1, B.RP_T_WQKV, B.RP_T_WO, B.RP_T_GAMMA2, B.RP_T_WGU, B.RP_T_WD]
        if getattr(cfg, "qk_norm", False):
            tids += [B.RP_T_QNORM, B.RP_T_KNORM]
        for tid in tids:
            off, nb = self.ctx.layout(B.RP_BLOCK_GRAD, tid)
            g[tid] = gbuf[off:off + nb].view(torch.float32)
        H, Q, KV = cfg.hidden, cfg.q_dim, cfg.kv_dim
        qkv = g[B.RP_T_WQKV].view(Q + 2 * KV, H)
        out = {"gamma1": g[B.RP_T_GAMMA1], "wq": qkv[:Q], "wk": qkv[Q:Q + KV], "wv": qkv[Q + KV:],
               "wo": g[B.RP_T_WO].view(H, Q), "gamma2": g[B.RP_T_GAMMA2]}
        if getattr(cfg, "qk_norm", False):
            out.update(qnorm=g[B.RP_T_QNORM], knorm=g[B.RP_T_KNORM])
        if cfg.n_experts > 0:
            E, Fe = cfg.n_experts, cfg.expert_ffn
            gu = g[B.RP_T_WGU].view(E, 2 * Fe, H)
            out.update(wg=gu[:, :Fe], wu=gu[:, Fe:], wd=g[B.RP_T_WD].view(E, H, Fe))
        else:
            F = cfg.ffn
            gu = g[B.RP_T_WGU].view(2 * F, H)
            out.update(wg=gu[:F], wu=gu[F:], wd=g[B.RP_T_WD].view(H, F))
        return out

    # ------------------------------------------------------------------ LM head
    def shard_rows(self) -> List[int]:
        V, S = self.cfg.vocab, self.cfg.n_shards
        return [V // S + (1 if s < V % S else 0) for s in range(S)]

    def add_lmhead(self, w: Optional[torch.Tensor], gamma_f: Optional[torch.Tensor] = None, resident: bool = True):
        rows = self.shard_rows()
        H = self.cfg.hidden
        shards, dshards, lo = [], [], 0
        for r in rows:
            if resident:
                shards.append(w[lo:lo + r].to(self.dt).to(self.dev).contiguous())
            else:
                shards.append(torch.empty(r, H, dtype=self.dt, device=self.dev))
            dshards.append(torch.zeros(r, H, dtype=torch.float32, device=self.dev))
            lo += r
        gf = dgf = None
        if gamma_f is not None:
            gf = gamma_f.to(self.dt).to(self.dev)
            dgf = torch.zeros(H, dtype=torch.float32, device=self.dev)
        self.ctx.bind_lmhead(self.cfg.vocab, shards, dshards, gf, dgf)
        self.head = {"w": shards, "dw": dshards, "gamma_f": gf, "dgamma_f": dgf}
        torch.cuda.current_stream(self.dev).synchronize()
        return self.head

    # ------------------------------------------------------------------ calls
    def fused_stage(self, l0: int, l1: int, x: torch.Tensor, labels: torch.Tensor, ws_fused: torch.Tensor,
                    ws_head: torch.Tensor, y: torch.Tensor, dy: torch.Tensor, dx: torch.Tensor,
                    loss: torch.Tensor):
        """The fused first backward stage B_1: forward of [l0, l1) keeping its
        internals, LM head + cross-entropy, then backward of [l0, l1) reusing them."""
        b, s = self.cfg.batch, self.cfg.seq
        self.ctx.stage_fwd(l0, l1, b, s, x, y, ws_fused, flags=B.RP_KEEP_ACTS)
        self.ctx.lmhead_ce_fwd_bwd(b, s, y, labels, loss, dy, ws_head)
        self.ctx.stage_bwd_recompute(l0, l1, b, s, dy, dx, ws_fused, flags=B.RP_USE_KEPT_ACTS)
