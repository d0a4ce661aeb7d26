"""The host-side optimizer worker and its per-layer consistency protocol
(rp_opt_* in librp.so; "Efficient Training on Multiple Consumer GPUs with
RoundPipe", sections 2.1.2 and 4.3). This module marshals arguments: Adam,
the weight and gradient copies and the event ordering run in the library.

A layer's trainable tensors are taken from the packed block layouts: the
master weights are a layer's weight block (bf16 or fp32, pinned host memory,
the bytes the GPU uploads) and the master gradients its fp32 gradient block
(the bytes the GPU downloads into).
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

from . import binding as B

LAYER_TENSORS = (B.RP_T_GAMMA1, B.RP_T_WQKV, B.RP_T_WO, B.RP_T_GAMMA2, B.RP_T_WGU, B.RP_T_WD)


@dataclass
class AdamParams:
    lr: float = 1e-4
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0
    grad_scale: float = 1.0

    def c(self) -> B.rp_opt_hparams:
        return B.rp_opt_hparams(self.lr, self.beta1, self.beta2, self.eps, self.weight_decay, self.grad_scale)


class OptimizerWorker:
    """n_layers layers; master_dtype torch.bfloat16 or torch.float32;
    n_threads <= 0 uses every hardware thread; timeout_ms > 0 bounds every
    protocol wait (0: unbounded)."""

    def __init__(self, n_layers: int, master_dtype: torch.dtype = torch.bfloat16, n_threads: int = 0,
                 timeout_ms: int = 0):
        dt = {torch.bfloat16: B.RP_DTYPE_BF16, torch.float32: B.RP_DTYPE_F32}[master_dtype]
        h = C.c_void_p()
        B.check(B.lib().rp_opt_create(n_layers, dt, n_threads, timeout_ms, C.byref(h)))
        self.h = h
        self.n_layers = n_layers
        self.master_dtype = master_dtype
        self._keep = {}
        self.sizes = [0] * n_layers

    def bind_segments(self, layer: int, segs: Sequence[tuple]):
        """segs: (master weights tensor, master gradient tensor (fp32), fp32 init or None),
        each flat with the same element count."""
        arr = (B.rp_opt_seg * len(segs))()
        n_tot = 0
        for i, (w, g, init) in enumerate(segs):
            n = w.numel()
            if g.numel() != n or g.dtype != torch.float32 or w.dtype != self.master_dtype:
                raise ValueError("segment: master weights (master dtype) and fp32 gradients of equal size")
            if init is not None and (init.numel() != n or init.dtype != torch.float32):
                raise ValueError("segment: init must be fp32 of the same size")
            arr[i] = B.rp_opt_seg(w.data_ptr(), g.data_ptr(), init.data_ptr() if init is not None else None, n)
            n_tot += n
        B.check(B.lib().rp_opt_bind_layer(self.h, layer, arr, len(segs)))
        self._keep[layer] = [t for seg in segs for t in seg if t is not None]
        self.sizes[layer] = n_tot

    def bind_blocks(self, cfg, layer: int, w_block: torch.Tensor, g_block: torch.Tensor,
                    init: Optional[torch.Tensor] = None):
        """A layer of configuration cfg from its packed weight block (uint8,
        master dtype inside) and fp32 gradient block (uint8); init: optional
        fp32 values of the trainable tensors in block order, concatenated."""
        segs, pos = [], 0
        tids = LAYER_TENSORS + ((B.RP_T_QNORM, B.RP_T_KNORM) if getattr(cfg, "qk_norm", False) else ())
        for tid in tids:
            wo, wn, _ = B.block_layout(cfg, B.RP_BLOCK_WEIGHT, tid)
            go, gn, _ = B.block_layout(cfg, B.RP_BLOCK_GRAD, tid)
            w = w_block[wo:wo + wn].view(self.master_dtype)
            g = g_block[go:go + gn].view(torch.float32)
            ini = None
            if init is not None:
                ini = init[pos:pos + w.numel()]
                pos += w.numel()
            segs.append((w, g, ini))
        self.bind_segments(layer, segs)

    def step(self, iteration: int, hp: AdamParams):
        B.check(B.lib().rp_opt_step(self.h, iteration, C.byref(hp.c())))

    def signal(self, edge: int, layer: int, iteration: int):
        B.check(B.lib().rp_opt_signal(self.h, edge, layer, iteration))

    def wait(self, edge: int, layer: int, iteration: int):
        B.check(B.lib().rp_opt_wait(self.h, edge, layer, iteration))

    def sync(self):
        B.check(B.lib().rp_opt_sync(self.h))

    def read(self, layer: int, which: int = 0) -> torch.Tensor:
        out = torch.empty(self.sizes[layer], dtype=torch.float32)
        B.check(B.lib().rp_opt_read(self.h, layer, which, out.data_ptr(), out.numel()))
        return out

    def close(self):
        if self.h:
            B.lib().rp_opt_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
