"""Plain CPU statement of one RoundPipe stage's math -- TEST INFRASTRUCTURE ONLY.

Nothing in the product imports this module. It is the slow, obviously correct
definition the HIP path is checked against.

A stage is a contiguous range of decoder layers run forward (the forward
partition of section 3.2 of the RoundPipe paper), or run again from its saved
layer input and then backward (full activation recomputation, section 2.1.1;
the fused first backward stage of section 3.2 reuses its own forward for the
recompute). The decoder layer itself is the GQA transformer layer that the
paper's appendix B (paperlayer.ai summary, "B.1 Activation Size" and "B.2")
lists: two RMSNorms, four attention projections, attention, and a SwiGLU MLP
of three projections (a top-k mixture of SwiGLU experts for MoE models,
appendix C.2), with LoRA adapters for the LoRA fine-tune of section 5.1.

Readings of what the pages leave open (plainest reading the rest supports):

* pre-norm residual layer, no biases, no QK-norm, untied LM head;
* RMSNorm(x) = x * gamma / sqrt(mean(x^2) + eps);
* RoPE in the rotate-half convention, angle(p, i) = p * base^(-2i/d) for
  i < d/2, positions 0..S-1 restarting in every batch row;
* causal attention includes the diagonal, scale 1/sqrt(d), no attention across
  batch rows; query head h reads kv head floor(h * n_kv / n_q);
* MoE: router logits are a given fp32 input; the k largest (ties: lower index)
  are kept and their softmax weights the experts' SwiGLU outputs;
* LoRA: W x + (alpha / r) * B (A x) on q, k, v, o; base weights frozen;
* LM head: optional final RMSNorm, logits = z W^T, loss = mean over labelled
  rows (label -1 = ignored) of logsumexp(logits) - logits[label]; the vocabulary
  may be split into contiguous shards whose (max, sum-exp) partials are merged;
* gradients are the exact derivative of the forward above (computed with torch
  autograd, a library primitive), w.r.t. the stage input and every trainable
  tensor; the backward of a stage is seeded with an upstream gradient dy, i.e.
  it differentiates sum(y * dy).

Everything runs in the dtype of the inputs handed in (callers pass fp64 for
checking, fp32 where the workload is fp32).
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import torch

Tensor = torch.Tensor

# ---------------------------------------------------------------------------
# building blocks
# ---------------------------------------------------------------------------


def rmsnorm(x: Tensor, gamma: Tensor, eps: float) -> Tensor:
    """RMSNorm over the last dim (appendix B.1 "two layer norms"; RMS form)."""
    ms = (x * x).mean(dim=-1, keepdim=True)
    return x / torch.sqrt(ms + eps) * gamma


def rope_angles(seq: int, head_dim: int, base: float, dtype=torch.float64) -> Tensor:
    """theta[p, i] = p * base^(-2i/d), p < seq, i < d/2 (rotate-half RoPE)."""
    i = torch.arange(head_dim // 2, dtype=torch.float64)
    inv = base ** (-2.0 * i / head_dim)
    p = torch.arange(seq, dtype=torch.float64)
    return (p[:, None] * inv[None, :]).to(dtype)


def rope(u: Tensor, positions: Tensor, base: float) -> Tensor:
    """Rotate the pairs (i, i + d/2) of every head by theta[p, i].

    u: [T, n_heads, d]; positions: [T] integer positions.
    """
    d = u.shape[-1]
    half = d // 2
    th = rope_angles(int(positions.max()) + 1, d, base, u.dtype)[positions.long()]
    c = torch.cos(th)[:, None, :]
    s = torch.sin(th)[:, None, :]
    u1, u2 = u[..., :half], u[..., half:]
    return torch.cat([u1 * c - u2 * s, u2 * c + u1 * s], dim=-1)


def causal_attention(q: Tensor, k: Tensor, v: Tensor, batch: int, seq: int) -> Tensor:
    """softmax(q k^T / sqrt(d) + causal mask) v, one batch row and head at a time.

    q: [T, n_q, d]; k, v: [T, n_kv, d]; T = batch * seq, rows ordered (b, s).
    Query head h uses kv head floor(h * n_kv / n_q).
    """
    T, n_q, d = q.shape
    n_kv = k.shape[1]
    out = torch.empty_like(q)
    mask = torch.ones(seq, seq, dtype=torch.bool).tril()
    scale = 1.0 / math.sqrt(d)
    for b in range(batch):
        rows = slice(b * seq, (b + 1) * seq)
        for h in range(n_q):
            hk = (h * n_kv) // n_q
            s = (q[rows, h, :] @ k[rows, hk, :].T) * scale
            s = s.masked_fill(~mask, float("-inf"))
            p = torch.softmax(s, dim=-1)
            out[rows, h, :] = p @ v[rows, hk, :]
    return out


def silu(g: Tensor) -> Tensor:
    return g * torch.sigmoid(g)


def swiglu(b: Tensor, wg: Tensor, wu: Tensor, wd: Tensor) -> Tensor:
    """(silu(b Wg^T) * (b Wu^T)) Wd^T -- the SwiGLU MLP of appendix B.1."""
    return (silu(b @ wg.T) * (b @ wu.T)) @ wd.T


def topk_route(logits: Tensor, k: int) -> Tuple[Tensor, Tensor]:
    """Indices of the k largest logits per row (ties: lower expert index) and
    their softmax weights (softmax over the selected k only)."""
    order = torch.sort(logits, dim=-1, descending=True, stable=True).indices
    idx = order[:, :k]
    sel = torch.gather(logits, 1, idx)
    w = torch.softmax(sel, dim=-1)
    return idx, w


def moe_mlp(b: Tensor, logits: Tensor, wg: Tensor, wu: Tensor, wd: Tensor,
            k: int) -> Tensor:
    """sum over the k routed experts e of w[t, e] * SwiGLU_e(b[t]).

    wg, wu: [E, Fe, H]; wd: [E, H, Fe]. Appendix C.2: only the E_act selected
    experts contribute FLOPs, every expert's weights are present.
    """
    idx, w = topk_route(logits.to(b.dtype) if logits.dtype != b.dtype else logits, k)
    w = w.to(b.dtype)
    out = torch.zeros_like(b)
    for e in range(wg.shape[0]):
        tok, slot = (idx == e).nonzero(as_tuple=True)
        if tok.numel() == 0:
            continue
        ye = swiglu(b[tok], wg[e], wu[e], wd[e])
        out = out.index_add(0, tok, ye * w[tok, slot][:, None])
    return out


def lora_delta(x: Tensor, a: Tensor, bmat: Tensor, scale: float) -> Tensor:
    """scale * (x A^T) B^T for A [r, in], B [out, r]."""
    return scale * ((x @ a.T) @ bmat.T)


# ---------------------------------------------------------------------------
# decoder layer and stage
# ---------------------------------------------------------------------------


def _positions(batch: int, seq: int) -> Tensor:
    return torch.arange(seq).repeat(batch)


def attention_block(x: Tensor, w: Dict[str, Tensor], cfg, lora: Optional[Dict[str, Tensor]] = None):
    """The attention half of the layer and the MLP's input: returns
    (a, q, k, v, o, h1, b) with a = RMSNorm1(x), rotated q/k, v, attention
    output o, h1 = x + o Wo^T (+ LoRA) and b = RMSNorm2(h1)."""
    T, H = x.shape
    nq, nkv, d = cfg.n_q, cfg.n_kv, cfg.head_dim
    pos = _positions(cfg.batch, T // cfg.batch)
    scale = (cfg.lora_alpha / cfg.lora_rank) if lora is not None else 0.0

    a = rmsnorm(x, w["gamma1"], cfg.rms_eps)
    q = a @ w["wq"].T
    kk = a @ w["wk"].T
    v = a @ w["wv"].T
    if lora is not None:
        q = q + lora_delta(a, lora["aq"], lora["bq"], scale)
        kk = kk + lora_delta(a, lora["ak"], lora["bk"], scale)
        v = v + lora_delta(a, lora["av"], lora["bv"], scale)
    q, kk = q.reshape(T, nq, d), kk.reshape(T, nkv, d)
    if getattr(cfg, "qk_norm", False):
        # Qwen3-style QK-norm: RMSNorm of every query and key head over its d
        # dims, own gains per q and k, before the rotation
        q = rmsnorm(q, w["qnorm"], cfg.rms_eps)
        kk = rmsnorm(kk, w["knorm"], cfg.rms_eps)
    q = rope(q, pos, cfg.rope_base)
    kk = rope(kk, pos, cfg.rope_base)
    v = v.reshape(T, nkv, d)
    o = causal_attention(q, kk, v, cfg.batch, T // cfg.batch).reshape(T, nq * d)
    proj = o @ w["wo"].T
    if lora is not None:
        proj = proj + lora_delta(o, lora["ao"], lora["bo"], scale)
    h1 = x + proj
    bn = rmsnorm(h1, w["gamma2"], cfg.rms_eps)
    return a, q, kk, v, o, h1, bn


def layer_forward(x: Tensor, w: Dict[str, Tensor], cfg, lora: Optional[Dict[str, Tensor]] = None,
                  router: Optional[Tensor] = None, keep: bool = False):
    """One pre-norm decoder layer, x [T, H] -> y [T, H].

    With keep=True also returns the internals (normed inputs, rotated q/k, v,
    attention output, residual h1, MLP input).
    """
    T = x.shape[0]
    nq, nkv, d = cfg.n_q, cfg.n_kv, cfg.head_dim
    a, q, kk, v, o, h1, bn = attention_block(x, w, cfg, lora)
    if cfg.is_moe:
        mlp = moe_mlp(bn, router, w["wg"], w["wu"], w["wd"], cfg.top_k)
    else:
        mlp = swiglu(bn, w["wg"], w["wu"], w["wd"])
    y = h1 + mlp
    if not keep:
        return y
    return y, {"a": a, "q": q.reshape(T, nq * d), "k": kk.reshape(T, nkv * d),
               "v": v.reshape(T, nkv * d), "o": o, "h1": h1, "b": bn}


def layer_forward_rows(x: Tensor, w: Dict[str, Tensor], cfg, rows: Sequence[int],
                       lora: Optional[Dict[str, Tensor]] = None,
                       router: Optional[Tensor] = None) -> Tensor:
    """The same layer as layer_forward, evaluated only at the token rows
    `rows`: keys and values are projected for every token (a query attends to
    all earlier tokens of its batch row), everything else only for the listed
    rows. Returns y[rows] [len(rows), H]. Lets the full-size workloads be
    checked one output row at a time."""
    T, H = x.shape
    nq, nkv, d = cfg.n_q, cfg.n_kv, cfg.head_dim
    seq = T // cfg.batch
    pos = _positions(cfg.batch, seq)
    scale = (cfg.lora_alpha / cfg.lora_rank) if lora is not None else 0.0
    a = rmsnorm(x, w["gamma1"], cfg.rms_eps)
    kk = a @ w["wk"].T
    v = a @ w["wv"].T
    if lora is not None:
        kk = kk + lora_delta(a, lora["ak"], lora["bk"], scale)
        v = v + lora_delta(a, lora["av"], lora["bv"], scale)
    kk = kk.reshape(T, nkv, d)
    qkn = getattr(cfg, "qk_norm", False)
    if qkn:
        kk = rmsnorm(kk, w["knorm"], cfg.rms_eps)
    kk = rope(kk, pos, cfg.rope_base)
    v = v.reshape(T, nkv, d)
    group = nq // nkv
    out = []
    for t in rows:
        at = a[t:t + 1]
        q = at @ w["wq"].T
        if lora is not None:
            q = q + lora_delta(at, lora["aq"], lora["bq"], scale)
        q = q.reshape(1, nq, d)
        if qkn:
            q = rmsnorm(q, w["qnorm"], cfg.rms_eps)
        q = rope(q, pos[t:t + 1], cfg.rope_base)[0]
        r0 = (t // seq) * seq
        # the query heads of kv head g are g*group .. (g+1)*group - 1, i.e.
        # query head h reads kv head floor(h * n_kv / n_q)
        qg = q.reshape(nkv, group, d)                       # [n_kv, group, d]
        kt = kk[r0:t + 1].permute(1, 2, 0)                  # [n_kv, d, L]
        vt = v[r0:t + 1].permute(1, 0, 2)                   # [n_kv, L, d]
        p = torch.softmax((qg @ kt) / math.sqrt(d), dim=-1)  # [n_kv, group, L]
        o = (p @ vt).reshape(1, nq * d)
        proj = o @ w["wo"].T
        if lora is not None:
            proj = proj + lora_delta(o, lora["ao"], lora["bo"], scale)
        h1 = x[t:t + 1] + proj
        bn = rmsnorm(h1, w["gamma2"], cfg.rms_eps)
        if cfg.is_moe:
            mlp = moe_mlp(bn, router[t:t + 1], w["wg"], w["wu"], w["wd"], cfg.top_k)
        else:
            mlp = swiglu(bn, w["wg"], w["wu"], w["wd"])
        out.append(h1 + mlp)
    return torch.cat(out, dim=0)


def mlp_weight_grad_columns(b: Tensor, dy: Tensor, w: Dict[str, Tensor], cols: Sequence[int]):
    """Gradients of sum(y * dy) for the dense SwiGLU MLP
    y = h1 + (silu(b Wg^T) * (b Wu^T)) Wd^T, at the FFN columns `cols` only:
    dWd[:, cols], dWg[cols, :], dWu[cols, :]. Column f of the FFN involves
    only row f of Wg / Wu and column f of Wd, so each is exact on its own."""
    g = b @ w["wg"][cols].T
    u = b @ w["wu"][cols].T
    sg = torch.sigmoid(g)
    m = g * sg * u
    dm = dy @ w["wd"][:, cols]
    dg = dm * u * (sg + g * sg * (1 - sg))      # d silu(g) / dg = sg (1 + g (1 - sg))
    du = dm * g * sg
    return dy.T @ m, dg.T @ b, du.T @ b


def lmhead_rows(x: Tensor, w: Tensor, labels: Tensor, rows: Sequence[int], vocab_rows: Sequence[int],
                chunk: int = 1024):
    """Full-size LM-head checks without the [T, V] gradient: the mean
    cross-entropy over all labelled rows (logits built a row chunk at a time),
    dloss/dx at the token rows `rows`, and dloss/dW at the vocabulary rows
    `vocab_rows`. Same definition as lmhead_loss_unsharded (no final norm)."""
    T = x.shape[0]
    valid = labels >= 0
    n_valid = int(valid.sum())
    lse = torch.empty(T, dtype=x.dtype)
    total = torch.zeros((), dtype=x.dtype)
    for c0 in range(0, T, chunk):
        z = x[c0:c0 + chunk] @ w.T
        lse[c0:c0 + chunk] = torch.logsumexp(z, dim=-1)
        lab = labels[c0:c0 + chunk]
        ok = lab >= 0
        zl = z.gather(1, torch.where(ok, lab, torch.zeros_like(lab)).long()[:, None])[:, 0]
        total = total + torch.where(ok, lse[c0:c0 + chunk] - zl, torch.zeros((), dtype=x.dtype)).sum()
    loss = total / n_valid
    dx = []
    for t in rows:
        p = torch.softmax(x[t] @ w.T, dim=0)
        if labels[t] >= 0:
            p[int(labels[t])] -= 1.0
            dx.append((p @ w) / n_valid)
        else:
            dx.append(torch.zeros(w.shape[1], dtype=x.dtype))
    dw = []
    for vr in vocab_rows:
        pv = torch.exp(x @ w[vr] - lse)            # softmax column vr over all tokens
        pv = pv - (labels == vr).to(x.dtype)
        pv = torch.where(valid, pv, torch.zeros((), dtype=x.dtype))
        dw.append((pv @ x) / n_valid)
    return loss, torch.stack(dx), torch.stack(dw)


def trainable_names(cfg) -> List[str]:
    """Dense full fine-tune: every weight and gain. LoRA: the adapters only."""
    if cfg.lora_rank > 0:
        return ["aq", "bq", "ak", "bk", "av", "bv", "ao", "bo"]
    names = ["gamma1", "wq", "wk", "wv", "wo", "gamma2", "wg", "wu", "wd"]
    if getattr(cfg, "qk_norm", False):
        names += ["qnorm", "knorm"]
    return names


def _cast(d: Optional[Dict[str, Tensor]], dtype) -> Optional[Dict[str, Tensor]]:
    if d is None:
        return None
    return {k: v.to(dtype) for k, v in d.items()}


def stage_forward(x: Tensor, layers: Sequence[Dict[str, Tensor]], cfg,
                  loras: Optional[Sequence[Dict[str, Tensor]]] = None,
                  routers: Optional[Sequence[Tensor]] = None,
                  dtype=torch.float64) -> Tuple[Tensor, List[Tensor]]:
    """Forward of a contiguous layer range; returns the output and every
    layer's input (the checkpoints that are offloaded to host, section 2.1.1)."""
    h = x.to(dtype)
    ckpts = []
    with torch.no_grad():
        for i, w in enumerate(layers):
            ckpts.append(h)
            h = layer_forward(h, _cast(w, dtype), cfg,
                              _cast(loras[i], dtype) if loras else None,
                              routers[i] if routers else None)
    return h, ckpts


def layer_backward(x: Tensor, w: Dict[str, Tensor], dy: Tensor, cfg,
                   lora: Optional[Dict[str, Tensor]] = None,
                   router: Optional[Tensor] = None, dtype=torch.float64):
    """Recompute the layer forward from its input x, then differentiate
    sum(y * dy): returns (dx, {trainable name: grad}, recomputed y)."""
    xx = x.to(dtype).detach().requires_grad_(True)
    ww = {k: v.to(dtype).detach() for k, v in w.items()}
    ll = {k: v.to(dtype).detach() for k, v in lora.items()} if lora is not None else None
    names = trainable_names(cfg)
    src = ll if cfg.lora_rank > 0 else ww
    for n in names:
        src[n].requires_grad_(True)
    with torch.enable_grad():
        y = layer_forward(xx, ww, cfg, ll, router)
        grads = torch.autograd.grad((y * dy.to(dtype)).sum(), [xx] + [src[n] for n in names])
    return grads[0], dict(zip(names, grads[1:])), y.detach()


def layer_backward_rows(x: Tensor, w: Dict[str, Tensor], rows: Sequence[int], dy_rows: Tensor, cfg,
                        lora: Optional[Dict[str, Tensor]] = None,
                        router: Optional[Tensor] = None, dtype=torch.float64):
    """The exact layer gradients for an upstream gradient that is zero outside
    the token rows `rows` (dy[rows[i]] = dy_rows[i]): differentiates
    sum_i y[rows[i]] * dy_rows[i], with y[rows] from layer_forward_rows.
    Returns (dx for every row [T, H], {trainable name: full gradient}).

    Only the listed rows receive an upstream gradient, yet dx is non-zero at
    every row at or before a listed row of its batch row (keys and values feed
    the later queries), and every weight gradient is complete. So a full-size
    layer is checked element by element without the T x T forward."""
    xx = x.to(dtype).detach().requires_grad_(True)
    ww = {k: v.to(dtype).detach() for k, v in w.items()}
    ll = {k: v.to(dtype).detach() for k, v in lora.items()} if lora is not None else None
    names = trainable_names(cfg)
    src = ll if cfg.lora_rank > 0 else ww
    for n in names:
        src[n].requires_grad_(True)
    rr = router.to(dtype) if router is not None else None
    with torch.enable_grad():
        yr = layer_forward_rows(xx, ww, cfg, rows, ll, rr)
        grads = torch.autograd.grad((yr * dy_rows.to(dtype)).sum(), [xx] + [src[n] for n in names])
    return grads[0], dict(zip(names, grads[1:]))


def stage_backward_recompute(ckpts: Sequence[Tensor], layers: Sequence[Dict[str, Tensor]],
                             dy: Tensor, cfg, loras=None, routers=None, dtype=torch.float64):
    """Backward stage with full recomputation: for the layers in reverse order,
    recompute the forward from the saved layer input and back-propagate."""
    g = dy.to(dtype)
    per_layer = [None] * len(layers)
    for i in reversed(range(len(layers))):
        g, gr, _ = layer_backward(ckpts[i], layers[i], g, cfg,
                                  loras[i] if loras else None,
                                  routers[i] if routers else None, dtype)
        per_layer[i] = gr
    return g, per_layer


# ---------------------------------------------------------------------------
# LM head + cross-entropy, vocabulary-sharded
# ---------------------------------------------------------------------------


def shard_bounds(vocab: int, n_shards: int) -> List[Tuple[int, int]]:
    """Contiguous vocabulary ranges; the first vocab % n_shards shards get one
    extra row (equal ranges when n_shards divides vocab)."""
    base, extra = divmod(vocab, n_shards)
    out, lo = [], 0
    for s in range(n_shards):
        hi = lo + base + (1 if s < extra else 0)
        out.append((lo, hi))
        lo = hi
    return out


def lmhead_loss_sharded(x: Tensor, w: Tensor, labels: Tensor, n_shards: int,
                        gamma_f: Optional[Tensor] = None, eps: float = 1e-6) -> Tensor:
    """Mean cross-entropy with the vocabulary split into shards.

    Per shard s: m_s = row max of its logits, l_s = sum exp(logits - m_s);
    then m = max_s m_s, l = sum_s l_s exp(m_s - m), LSE = m + ln l. The
    label's logit is taken from the shard that owns it. The paper splits the
    LM head, its heaviest single tensor, before scheduling (section 4.2.2).
    """
    z = rmsnorm(x, gamma_f, eps) if gamma_f is not None else x
    valid = labels >= 0
    ms, ls, zlab = [], [], torch.zeros(x.shape[0], dtype=x.dtype)
    for lo, hi in shard_bounds(w.shape[0], n_shards):
        logit = z @ w[lo:hi].T
        m_s = logit.max(dim=-1).values
        ms.append(m_s)
        ls.append(torch.exp(logit - m_s[:, None]).sum(dim=-1))
        own = valid & (labels >= lo) & (labels < hi)
        col = torch.where(own, labels - lo, torch.zeros_like(labels)).long()
        zlab = zlab + torch.where(own, logit.gather(1, col[:, None])[:, 0],
                                  torch.zeros((), dtype=x.dtype))
    m = torch.stack(ms).max(dim=0).values
    l = sum(l_s * torch.exp(m_s - m) for m_s, l_s in zip(ms, ls))
    lse = m + torch.log(l)
    n_valid = int(valid.sum())
    return torch.where(valid, lse - zlab, torch.zeros((), dtype=x.dtype)).sum() / n_valid


def lmhead_loss_unsharded(x: Tensor, w: Tensor, labels: Tensor,
                          gamma_f: Optional[Tensor] = None, eps: float = 1e-6) -> Tensor:
    """Same loss, one logsumexp over the whole vocabulary."""
    z = rmsnorm(x, gamma_f, eps) if gamma_f is not None else x
    logit = z @ w.T
    valid = labels >= 0
    lse = torch.logsumexp(logit, dim=-1)
    col = torch.where(valid, labels, torch.zeros_like(labels)).long()
    zl = logit.gather(1, col[:, None])[:, 0]
    return torch.where(valid, lse - zl, torch.zeros((), dtype=x.dtype)).sum() / int(valid.sum())


def lmhead_fwd_bwd(x: Tensor, w: Tensor, labels: Tensor, n_shards: int,
                   gamma_f: Optional[Tensor] = None, eps: float = 1e-6,
                   dtype=torch.float64):
    """Loss, dloss/dx, dloss/dW (full [V, H]) and dloss/dgamma_f (or None)."""
    xx = x.to(dtype).detach().requires_grad_(True)
    ww = w.to(dtype).detach().requires_grad_(True)
    gg = gamma_f.to(dtype).detach().requires_grad_(True) if gamma_f is not None else None
    with torch.enable_grad():
        loss = lmhead_loss_sharded(xx, ww, labels, n_shards, gg, eps)
        ins = [xx, ww] + ([gg] if gg is not None else [])
        grads = torch.autograd.grad(loss, ins)
    return (loss.detach(), grads[0], grads[1], grads[2] if gg is not None else None)


# ---------------------------------------------------------------------------
# embedding (full tiny model only)
# ---------------------------------------------------------------------------


def embed(ids: Tensor, table: Tensor) -> Tensor:
    """x0[t] = E[ids[t]] for the flattened (b, s) token order."""
    return table[ids.reshape(-1).long()]


def embed_backward(ids: Tensor, dx0: Tensor, vocab: int) -> Tensor:
    """dE[v] = sum of dx0[t] over the tokens t with ids[t] == v."""
    out = torch.zeros(vocab, dx0.shape[1], dtype=dx0.dtype)
    return out.index_add(0, ids.reshape(-1).long(), dx0)


def full_model_fwd_bwd(ids: Tensor, labels: Tensor, layers, head, cfg, dtype=torch.float64):
    """End-to-end loss and gradients of the tiny full model in one autograd
    graph: embedding, every layer, final norm, LM head, mean cross-entropy."""
    table = head["embed"].to(dtype).detach().requires_grad_(True)
    ww = [{k: v.to(dtype).detach().requires_grad_(True) for k, v in l.items()} for l in layers]
    wl = head["w"].to(dtype).detach().requires_grad_(True)
    gf = head["gamma_f"].to(dtype).detach().requires_grad_(True)
    with torch.enable_grad():
        h = embed(ids, table)
        for w in ww:
            h = layer_forward(h, w, cfg)
        loss = lmhead_loss_sharded(h, wl, labels.reshape(-1), cfg.n_shards, gf, cfg.rms_eps)
        names = trainable_names(cfg)
        flat = [table, wl, gf] + [w[n] for w in ww for n in names]
        grads = torch.autograd.grad(loss, flat)
    out = {"embed": grads[0], "w": grads[1], "gamma_f": grads[2], "layers": []}
    it = iter(grads[3:])
    for _ in ww:
        out["layers"].append({n: next(it) for n in names})
    return loss.detach(), out
