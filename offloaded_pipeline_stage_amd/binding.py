"""ctypes binding of librp.so -- argument marshalling only.

Every computation runs in the library's HIP kernels; this module converts
Python/torch arguments into the C ABI declared in include/rp.h. torch provides
device memory, pinned host memory and streams. The library must have been
built (python -m offloaded_pipeline_stage_amd.build); loading fails loudly
otherwise -- there is no fallback path.
"""
from __future__ import annotations

import atexit
import ctypes as C
import weakref
import os
from typing import Dict, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librp.so")

RP_OK, RP_ERR_INVALID, RP_ERR_UNSUPPORTED, RP_ERR_WORKSPACE, RP_ERR_NOT_PINNED, RP_ERR_HIP, RP_ERR_STATE = range(7)
RP_DTYPE_F32, RP_DTYPE_BF16 = 0, 1
RP_T_GAMMA1, RP_T_WQKV, RP_T_WO, RP_T_GAMMA2, RP_T_WGU, RP_T_WD = 0, 1, 2, 3, 4, 5
RP_T_QNORM, RP_T_KNORM = 6, 7
RP_T_AQ, RP_T_BQ, RP_T_AK, RP_T_BK, RP_T_AV, RP_T_BV, RP_T_AO, RP_T_BO = range(16, 24)
RP_BLOCK_WEIGHT, RP_BLOCK_GRAD, RP_BLOCK_LORA = 0, 1, 2
RP_OP_STAGE_FWD, RP_OP_STAGE_BWD, RP_OP_LMHEAD, RP_OP_FUSED, RP_OP_MOE_ROUTE = 0, 1, 2, 3, 4
RP_KEEP_ACTS, RP_USE_KEPT_ACTS, RP_CKPT_DEVICE, RP_ACCUM_GRADS = 1, 2, 4, 8
RP_H2D, RP_D2H = 0, 1
RP_ON_COMPUTE, RP_ON_ACT_H2D, RP_ON_ACT_D2H = 0, 1, 2
RP_OPT_PARAMS_UPLOADED, RP_OPT_GRADS_DOWNLOADED, RP_OPT_PCP_DONE, RP_OPT_GCP_DONE = 0, 1, 2, 3
RP_PARAM_H2D, RP_GRAD_D2H, RP_GRAD_D2H_BF16 = 0, 1, 2
RP_TGT_LAYER, RP_TGT_LMHEAD, RP_TGT_LORA, RP_TGT_FINAL_NORM = 0, 1, 2, 3


class rp_layer_cfg(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("n_q", C.c_int32), ("n_kv", C.c_int32), ("head_dim", C.c_int32),
                ("ffn", C.c_int32), ("n_experts", C.c_int32), ("top_k", C.c_int32), ("expert_ffn", C.c_int32),
                ("lora_rank", C.c_int32), ("lora_alpha", C.c_float), ("rms_eps", C.c_float),
                ("rope_base", C.c_float), ("dtype", C.c_int32), ("qk_norm", C.c_int32)]


class rp_streams(C.Structure):
    _fields_ = [("compute", C.c_void_p), ("act_h2d", C.c_void_p), ("act_d2h", C.c_void_p),
                ("w_h2d", C.c_void_p), ("g_d2h", C.c_void_p)]


class rp_xfer(C.Structure):
    _fields_ = [("kind", C.c_int32), ("target", C.c_int32), ("id", C.c_int32), ("reserved", C.c_int32),
                ("offset", C.c_uint64), ("bytes", C.c_uint64), ("host", C.c_void_p)]


class rp_opt_hparams(C.Structure):
    _fields_ = [("lr", C.c_float), ("beta1", C.c_float), ("beta2", C.c_float), ("eps", C.c_float),
                ("weight_decay", C.c_float), ("grad_scale", C.c_float)]


class rp_opt_seg(C.Structure):
    _fields_ = [("master_w", C.c_void_p), ("master_g", C.c_void_p), ("init", C.c_void_p), ("n", C.c_uint64)]


class rp_trace_rec(C.Structure):
    _fields_ = [("name", C.c_char * 96), ("flops", C.c_double), ("bytes", C.c_double), ("ms", C.c_float),
                ("reserved", C.c_int32)]


_P = C.c_void_p
_SIGS = {
    "rp_status_string": (C.c_char_p, [C.c_int]),
    "rp_last_error": (C.c_char_p, []),
    "rp_version": (C.c_char_p, []),
    "rp_block_layout": (C.c_int, [C.POINTER(rp_layer_cfg), C.c_int, C.c_int, C.POINTER(C.c_size_t),
                                  C.POINTER(C.c_size_t), C.POINTER(C.c_size_t)]),
    "rp_ctx_create": (C.c_int, [C.c_int, C.POINTER(rp_layer_cfg), C.POINTER(rp_streams), C.POINTER(_P)]),
    "rp_ctx_destroy": (C.c_int, [_P]),
    "rp_ctx_streams": (C.c_int, [_P, C.POINTER(rp_streams)]),
    "rp_ctx_sync": (C.c_int, [_P]),
    "rp_bind_layer": (C.c_int, [_P, C.c_int, _P, _P, _P, _P]),
    "rp_bind_lmhead": (C.c_int, [_P, C.c_int, C.c_int, C.POINTER(_P), C.POINTER(_P), _P, _P]),
    "rp_workspace_size": (C.c_int, [_P, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.POINTER(C.c_size_t)]),
    "rp_stage_fwd": (C.c_int, [_P, C.c_int, C.c_int, C.c_int, C.c_int, _P, _P, C.POINTER(_P), C.POINTER(_P),
                               C.c_int, _P, C.c_size_t]),
    "rp_stage_bwd_recompute": (C.c_int, [_P, C.c_int, C.c_int, C.c_int, C.c_int, C.POINTER(_P), _P, _P,
                                         C.POINTER(_P), C.c_int, _P, C.c_size_t]),
    "rp_lmhead_ce_fwd_bwd": (C.c_int, [_P, C.c_int, C.c_int, _P, _P, _P, _P, _P, C.c_size_t]),
    "rp_embed_fwd": (C.c_int, [_P, C.c_int, C.c_int, _P, _P, _P]),
    "rp_embed_bwd": (C.c_int, [_P, C.c_int, C.c_int, _P, _P, _P]),
    "rp_act_copy": (C.c_int, [_P, C.c_int, _P, _P, C.c_size_t, C.POINTER(C.c_int64)]),
    "rp_partition": (C.c_int, [C.c_int, C.POINTER(C.c_double), C.POINTER(C.c_double), C.c_double,
                               C.POINTER(C.c_double), C.POINTER(C.c_double), C.c_double, C.c_double, C.c_int,
                               C.c_int, C.POINTER(C.c_int), C.POINTER(C.c_int), C.POINTER(C.c_int),
                               C.POINTER(C.c_int), C.POINTER(C.c_int), C.POINTER(C.c_double)]),
    "rp_opt_create": (C.c_int, [C.c_int, C.c_int, C.c_int, C.c_int64, C.POINTER(_P)]),
    "rp_opt_destroy": (C.c_int, [_P]),
    "rp_opt_bind_layer": (C.c_int, [_P, C.c_int, C.POINTER(rp_opt_seg), C.c_int]),
    "rp_opt_step": (C.c_int, [_P, C.c_int64, C.POINTER(rp_opt_hparams)]),
    "rp_opt_signal": (C.c_int, [_P, C.c_int, C.c_int, C.c_int64]),
    "rp_opt_wait": (C.c_int, [_P, C.c_int, C.c_int, C.c_int64]),
    "rp_opt_sync": (C.c_int, [_P]),
    "rp_opt_read": (C.c_int, [_P, C.c_int, C.c_int, _P, C.c_uint64]),
    "rp_act_wait": (C.c_int, [_P, C.c_int, C.c_int64]),
    "rp_act_next_ticket": (C.c_int, [_P, C.POINTER(C.c_int64)]),
    "rp_weight_stream_submit": (C.c_int, [_P, C.POINTER(rp_xfer), C.c_int, C.c_int, C.c_uint64, C.c_int64]),
    "rp_weight_stream_submit_gated": (C.c_int, [_P, C.POINTER(rp_xfer), C.c_int, C.c_int, C.c_uint64,
                                                C.POINTER(C.c_int64)]),
    "rp_xfer_plan": (C.c_int, [C.POINTER(C.c_uint64), C.c_int, C.c_int, C.c_uint64, C.c_uint64, C.c_int,
                               C.POINTER(C.c_int32), C.POINTER(C.c_uint64), C.POINTER(C.c_uint64),
                               C.POINTER(C.c_int32), C.POINTER(C.c_int)]),
    "rp_op_gemm_bf16": (C.c_int, [_P, C.c_int, C.c_int, C.c_int, _P, C.c_int, C.c_int, _P, C.c_int, C.c_int, _P,
                                  C.c_int, C.c_int, C.c_int]),
    "rp_op_attn_fwd": (C.c_int, [_P, C.c_int, C.c_int, _P, _P, _P]),
    "rp_op_copy": (C.c_int, [_P, _P, _P, C.c_size_t]),
    "rp_op_transpose_bf16": (C.c_int, [_P, C.c_int, C.c_int, _P, C.c_int64, _P, C.c_int64]),
    "rp_op_attn_bwd": (C.c_int, [_P, C.c_int, C.c_int, _P, _P, _P, _P, _P, _P, C.c_size_t]),
    "rp_op_attn_bwd_noalloc": (C.c_int, [_P, C.c_int, C.c_int, _P, _P, _P, _P, _P]),
    "rp_op_moe_route": (C.c_int, [_P, C.c_int, C.c_int, _P, _P, _P, _P, _P, _P, _P, _P, _P, C.c_size_t]),
    "rp_trace_begin": (C.c_int, [_P, C.c_int]),
    "rp_trace_end": (C.c_int, [_P]),
    "rp_trace_read": (C.c_int, [_P, C.POINTER(rp_trace_rec), C.c_int, C.POINTER(C.c_int)]),
}
EXPORTS = tuple(_SIGS)

_lib = None


def lib() -> C.CDLL:
    """Load librp.so (built in-tree). Raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m offloaded_pipeline_stage_amd.build`")
        h = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib = h
    return _lib


class RPError(RuntimeError):
    def __init__(self, status: int, msg: str):
        self.status = status
        name = lib().rp_status_string(status).decode()
        super().__init__(f"{name}: {msg}")


def check(status: int) -> None:
    if status != RP_OK:
        raise RPError(status, lib().rp_last_error().decode())


def ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def ptr_array(ts):
    if ts is None:
        return None
    arr = (_P * len(ts))()
    for i, t in enumerate(ts):
        arr[i] = None if t is None else (t if isinstance(t, int) else t.data_ptr())
    return arr


def make_cfg(cfg) -> rp_layer_cfg:
    """rp_layer_cfg from any object with the StageConfig attribute names."""
    return rp_layer_cfg(cfg.hidden, cfg.n_q, cfg.n_kv, cfg.head_dim, cfg.ffn, cfg.n_experts, cfg.top_k,
                        cfg.expert_ffn, cfg.lora_rank, float(cfg.lora_alpha), float(cfg.rms_eps),
                        float(cfg.rope_base), RP_DTYPE_BF16 if cfg.dtype == "bf16" else RP_DTYPE_F32,
                        1 if getattr(cfg, "qk_norm", False) else 0)


def block_layout(cfg, block: int, tensor: int):
    c = make_cfg(cfg)
    off, nb, tot = C.c_size_t(), C.c_size_t(), C.c_size_t()
    check(lib().rp_block_layout(C.byref(c), block, tensor, C.byref(off), C.byref(nb), C.byref(tot)))
    return off.value, nb.value, tot.value


def block_bytes(cfg, block: int) -> int:
    c = make_cfg(cfg)
    tot = C.c_size_t()
    check(lib().rp_block_layout(C.byref(c), block, -1, None, None, C.byref(tot)))
    return tot.value


def xfer_plan(sizes: Sequence[int], n_windows: int, max_chunk: int = 0, align: int = 256):
    n = len(sizes)
    cap = max(16, 4 * n + 4 * n_windows + 64)
    while True:
        arr = (C.c_uint64 * max(n, 1))(*sizes)
        it = (C.c_int32 * cap)()
        of = (C.c_uint64 * cap)()
        by = (C.c_uint64 * cap)()
        wi = (C.c_int32 * cap)()
        nc = C.c_int()
        st = lib().rp_xfer_plan(arr, n, n_windows, max_chunk, align, cap, it, of, by, wi, C.byref(nc))
        if st == RP_ERR_INVALID and nc.value > cap:
            cap = nc.value
            continue
        check(st)
        return [(it[k], of[k], by[k], wi[k]) for k in range(nc.value)]


# contexts still open at interpreter exit are destroyed before the HIP runtime
# shuts down (their transfer streams belong to the library)
_LIVE = weakref.WeakSet()


def partition(f: Sequence[float], b: Sequence[float], h: float, mf: Sequence[float], mb: Sequence[float],
              mh: float, mem_cap: float, n_micro: int, n_gpus: int):
    """Stage partition (rp_partition): returns (objective, forward stage sizes,
    b1, backward stage sizes after B_1)."""
    L = len(f)
    if not (len(b) == len(mf) == len(mb) == L):
        raise ValueError("per-layer arrays must have the same length")
    D = C.c_double * max(L, 1)
    I = C.c_int * max(L, 1)
    fs, bs = I(), I()
    nf, b1, nb, obj = C.c_int(), C.c_int(), C.c_int(), C.c_double()
    check(lib().rp_partition(L, D(*f), D(*b), h, D(*mf), D(*mb), mh, mem_cap, n_micro, n_gpus, fs, C.byref(nf),
                             C.byref(b1), bs, C.byref(nb), C.byref(obj)))
    return obj.value, tuple(fs[:nf.value]), b1.value, tuple(bs[:nb.value])


@atexit.register
def _close_live():
    for c in list(_LIVE):
        try:
            c.close()
        except Exception:
            pass


class Context:
    """Owns an rp_ctx. Unless `streams` names them, every stream is the
    library's own, each on a hardware queue of its own: kernels run on its
    compute stream, copies on its transfer streams. Those are blocking
    streams, so torch work on the default stream is ordered against the
    library's kernels by the runtime; a call made while torch's current stream
    is another stream first makes the compute stream wait for it."""

    def __init__(self, cfg, device: int = 0, streams: Optional[Dict[str, torch.cuda.Stream]] = None):
        self.cfg = cfg
        self.device = device
        names = ("compute", "act_h2d", "act_d2h", "w_h2d", "g_d2h")
        given = dict(streams or {})
        s = rp_streams(*[given[n].cuda_stream if n in given else None for n in names])
        self._c = make_cfg(cfg)
        h = _P()
        check(lib().rp_ctx_create(device, C.byref(self._c), C.byref(s), C.byref(h)))
        self.h = h
        _LIVE.add(self)
        used = rp_streams()
        check(lib().rp_ctx_streams(h, C.byref(used)))
        self.streams = {n: given.get(n) or torch.cuda.ExternalStream(getattr(used, n), device=device)
                        for n in names}
        # every tensor handed to an enqueueing call stays referenced until
        # sync(): the library reads and writes them asynchronously on its own
        # streams, so torch must not recycle their memory before then
        self._keep = []

    # -- life cycle
    def _hold(self, *objs):
        for o in objs:
            if o is None:
                continue
            if isinstance(o, (list, tuple)):
                self._hold(*o)
            elif isinstance(o, torch.Tensor):
                self._keep.append(o)

    def _order(self):
        """Order the library's compute stream after torch's current stream
        when that is neither the default stream nor the compute stream, so
        that tensors torch has just filled or produced there are complete
        before a call reads or overwrites them. Default-stream work needs no
        event: the library's streams are blocking streams. (An event on the
        default stream would also wait for the library's in-flight transfers.)"""
        cur = torch.cuda.current_stream(self.device)
        comp = self.streams["compute"]
        if cur.cuda_stream not in (0, comp.cuda_stream):
            comp.wait_stream(cur)

    def sync(self):
        check(lib().rp_ctx_sync(self.h))
        self._keep.clear()

    def close(self):
        if self.h:
            _LIVE.discard(self)
            check(lib().rp_ctx_destroy(self.h))
            self.h = None

    def __del__(self):
        try:
            if getattr(self, "h", None):
                _LIVE.discard(self)
                lib().rp_ctx_destroy(self.h)
                self.h = None
        except Exception:
            pass

    # -- layouts and packing
    def layout(self, block: int, tensor: int):
        return block_layout(self.cfg, block, tensor)[:2]

    def block_bytes(self, block: int) -> int:
        return block_bytes(self.cfg, block)

    def pack(self, block: int, tensors: Dict[int, torch.Tensor], out: torch.Tensor) -> torch.Tensor:
        """Copy tensors into a flat byte buffer at the library's block offsets."""
        for tid, t in tensors.items():
            off, nb = self.layout(block, tid)
            src = t.contiguous().reshape(-1).view(torch.uint8)
            assert src.numel() == nb, (tid, src.numel(), nb)
            out[off:off + nb].copy_(src)
        return out

    # -- bindings
    def bind_layer(self, layer: int, w: torch.Tensor, g: Optional[torch.Tensor] = None,
                   lora: Optional[torch.Tensor] = None, lora_g: Optional[torch.Tensor] = None):
        check(lib().rp_bind_layer(self.h, layer, ptr(w), ptr(g), ptr(lora), ptr(lora_g)))
        self._bound = getattr(self, "_bound", {})
        self._bound[("layer", layer)] = (w, g, lora, lora_g)  # bindings live as long as the context

    def bind_lmhead(self, vocab: int, shards: Sequence[torch.Tensor], dshards: Optional[Sequence[torch.Tensor]],
                    gamma_f: Optional[torch.Tensor] = None, dgamma_f: Optional[torch.Tensor] = None):
        check(lib().rp_bind_lmhead(self.h, vocab, len(shards), ptr_array(shards),
                                   ptr_array(dshards) if dshards is not None else None, ptr(gamma_f), ptr(dgamma_f)))
        self._bound = getattr(self, "_bound", {})
        self._bound["lmhead"] = (list(shards), list(dshards or []), gamma_f, dgamma_f)

    def workspace_size(self, op: int, batch: int, seq: int, n_layers: int = 1, flags: int = 0) -> int:
        n = C.c_size_t()
        check(lib().rp_workspace_size(self.h, op, batch, seq, n_layers, flags, C.byref(n)))
        return n.value

    def workspace(self, op: int, batch: int, seq: int, n_layers: int = 1, flags: int = 0) -> torch.Tensor:
        n = self.workspace_size(op, batch, seq, n_layers, flags)
        return torch.empty(max(n, 256), dtype=torch.uint8, device=torch.device("cuda", self.device))

    # -- stage calls
    def stage_fwd(self, l0, l1, batch, seq, x, y, ws, ckpt_host=None, router=None, flags=0):
        self._order()
        check(lib().rp_stage_fwd(self.h, l0, l1, batch, seq, ptr(x), ptr(y), ptr_array(ckpt_host),
                                 ptr_array(router), flags, ptr(ws), ws.numel()))
        self._hold(x, y, ws, ckpt_host, router)

    def stage_bwd_recompute(self, l0, l1, batch, seq, dy, dx, ws, ckpt=None, router=None, flags=0):
        self._order()
        check(lib().rp_stage_bwd_recompute(self.h, l0, l1, batch, seq, ptr_array(ckpt), ptr(dy), ptr(dx),
                                           ptr_array(router), flags, ptr(ws), ws.numel()))
        self._hold(dy, dx, ws, ckpt, router)

    def lmhead_ce_fwd_bwd(self, batch, seq, x, labels, loss, dx, ws):
        self._order()
        check(lib().rp_lmhead_ce_fwd_bwd(self.h, batch, seq, ptr(x), ptr(labels), ptr(loss), ptr(dx), ptr(ws),
                                         ws.numel()))
        self._hold(x, labels, loss, dx, ws)

    def embed_fwd(self, ids, table, x0):
        self._order()
        check(lib().rp_embed_fwd(self.h, ids.numel(), table.shape[0], ptr(ids), ptr(table), ptr(x0)))
        self._hold(ids, table, x0)

    def embed_bwd(self, ids, dx0, dtable):
        self._order()
        check(lib().rp_embed_bwd(self.h, ids.numel(), dtable.shape[0], ptr(ids), ptr(dx0), ptr(dtable)))
        self._hold(ids, dx0, dtable)

    # -- transfers
    def act_copy(self, direction: int, dst: torch.Tensor, src: torch.Tensor, nbytes: Optional[int] = None) -> int:
        t = C.c_int64()
        nb = nbytes if nbytes is not None else src.numel() * src.element_size()
        self._order()
        check(lib().rp_act_copy(self.h, direction, ptr(dst), ptr(src), nb, C.byref(t)))
        self._hold(dst, src)
        return t.value

    def act_wait(self, where: int, ticket: int):
        check(lib().rp_act_wait(self.h, where, ticket))

    def act_next_ticket(self) -> int:
        t = C.c_int64()
        check(lib().rp_act_next_ticket(self.h, C.byref(t)))
        return t.value

    @staticmethod
    def _xfer_array(items):
        arr = (rp_xfer * max(len(items), 1))()
        for i, (kind, tgt, ident, off, nb, host) in enumerate(items):
            addr = host if isinstance(host, int) else host.data_ptr()
            arr[i] = rp_xfer(kind, tgt, ident, 0, off, nb, addr)
        return arr

    def weight_stream_submit(self, items, n_windows: int = 1, max_chunk: int = 0, gate_ticket: int = -1):
        """items: (kind, target, id, offset, bytes, host tensor or address)."""
        arr = self._xfer_array(items)
        self._order()
        check(lib().rp_weight_stream_submit(self.h, arr, len(items), n_windows, max_chunk, gate_ticket))
        self._hold([it[5] for it in items])

    def weight_stream_submit_gated(self, items, gates: Sequence[int], max_chunk: int = 0):
        """One window per entry of `gates` (the activation ticket it waits for, -1 for none)."""
        arr = self._xfer_array(items)
        g = (C.c_int64 * len(gates))(*gates)
        self._order()
        check(lib().rp_weight_stream_submit_gated(self.h, arr, len(items), len(gates), max_chunk, g))
        self._hold([it[5] for it in items])

    # -- kernel trace
    def trace_begin(self, max_launches: int = 100000):
        check(lib().rp_trace_begin(self.h, max_launches))

    def trace_end(self):
        """Stop recording and return [(kernel name, flops, bytes, ms)] in issue order."""
        check(lib().rp_trace_end(self.h))
        n = C.c_int()
        check(lib().rp_trace_read(self.h, None, 0, C.byref(n)))
        arr = (rp_trace_rec * max(n.value, 1))()
        check(lib().rp_trace_read(self.h, arr, n.value, C.byref(n)))
        return [(arr[i].name.decode(), arr[i].flops, arr[i].bytes, arr[i].ms) for i in range(n.value)]

    # -- single kernels
    def op_gemm_bf16(self, M, N, K, A, lda, a_kmajor, B, ldb, b_kmajor, Cm, ldc, out_f32, accumulate=False):
        self._order()
        check(lib().rp_op_gemm_bf16(self.h, M, N, K, ptr(A), lda, int(a_kmajor), ptr(B), ldb, int(b_kmajor),
                                    ptr(Cm), ldc, int(out_f32), int(accumulate)))
        self._hold(A, B, Cm)

    def op_transpose_bf16(self, src, dst):
        """dst[:cols, :rows] = src[:rows, :cols].T for 2-D bf16 device tensors
        with unit column stride."""
        rows, cols = src.shape
        if dst.dtype != torch.bfloat16 or src.dtype != torch.bfloat16 or src.stride(1) != 1 or dst.stride(1) != 1:
            raise ValueError("op_transpose_bf16: bf16 tensors with unit column stride")
        if dst.shape[0] < cols or dst.shape[1] < rows:
            raise ValueError("op_transpose_bf16: dst too small")
        self._order()
        check(lib().rp_op_transpose_bf16(self.h, rows, cols, ptr(src), src.stride(0), ptr(dst), dst.stride(0)))
        self._hold(src, dst)

    def op_copy(self, dst, src):
        self._order()
        n = src.numel() * src.element_size()
        if dst.numel() * dst.element_size() < n:
            raise ValueError("op_copy: dst smaller than src")
        check(lib().rp_op_copy(self.h, ptr(dst), ptr(src), n))
        self._hold(dst, src)

    def op_attn_fwd(self, batch, seq, qkv, o, lse):
        self._order()
        check(lib().rp_op_attn_fwd(self.h, batch, seq, ptr(qkv), ptr(o), ptr(lse)))
        self._hold(qkv, o, lse)

    def op_attn_bwd_noalloc(self, batch, seq, qkv, o, dout, lse, dqkv):
        self._order()
        check(lib().rp_op_attn_bwd_noalloc(self.h, batch, seq, ptr(qkv), ptr(o), ptr(dout), ptr(lse), ptr(dqkv)))
        self._hold(qkv, o, dout, lse, dqkv)

    def op_moe_route(self, batch, seq, logits, idx, wgt, cnt, off, perm_row, perm_w, inv, ws):
        self._order()
        check(lib().rp_op_moe_route(self.h, batch, seq, ptr(logits), ptr(idx), ptr(wgt), ptr(cnt), ptr(off),
                                    ptr(perm_row), ptr(perm_w), ptr(inv), ptr(ws), ws.numel()))
        self._hold(logits, idx, wgt, cnt, off, perm_row, perm_w, inv, ws)

    def op_attn_bwd(self, batch, seq, qkv, o, dout, lse, dqkv, ws):
        self._order()
        check(lib().rp_op_attn_bwd(self.h, batch, seq, ptr(qkv), ptr(o), ptr(dout), ptr(lse), ptr(dqkv), ptr(ws),
                                   ws.numel()))
        self._hold(qkv, o, dout, lse, dqkv, ws)
