"""Pins of the CPU oracle's stage math against things other than itself:
finite differences, closed forms, library routines and brute force.
CPU only."""
import math

import pytest
import torch
import torch.nn.functional as F

import synth
from oracle import stage as O

D64 = torch.float64


def tiny_cfg(**kw):
    base = dict(name="fd", hidden=16, n_q=2, n_kv=1, head_dim=8, ffn=24, batch=2, seq=8,
                dtype="f32", vocab=32, n_shards=1, rms_eps=1e-6, rope_base=10000.0, seed=7)
    base.update(kw)
    return synth.StageConfig(**base)


def f64(d):
    return {k: v.to(D64) for k, v in d.items()}


# ---------------------------------------------------------------------------
# finite-difference gradient checks (fp64, central, h = 1e-6)
# ---------------------------------------------------------------------------


def _fd_check(fn, tensors, grads, n_elem=6, h=1e-6, tol=1e-6, seed=0):
    """Compare autograd grads with central differences on sampled elements and
    on one random direction per tensor."""
    g = torch.Generator().manual_seed(seed)
    for t, gr in zip(tensors, grads):
        flat = t.view(-1)
        idx = torch.randint(0, flat.numel(), (n_elem,), generator=g)
        for i in idx.tolist():
            old = flat[i].item()
            flat[i] = old + h
            fp = fn().item()
            flat[i] = old - h
            fm = fn().item()
            flat[i] = old
            fd = (fp - fm) / (2 * h)
            an = gr.view(-1)[i].item()
            scale = max(abs(an), gr.abs().max().item() * 1e-3, 1e-8)
            assert abs(fd - an) / scale < tol, (i, fd, an)
        direc = torch.randn(t.shape, generator=g, dtype=D64)
        t0 = t.clone()
        t.copy_(t0 + h * direc)
        fp = fn().item()
        t.copy_(t0 - h * direc)
        fm = fn().item()
        t.copy_(t0)
        fd = (fp - fm) / (2 * h)
        an = (gr * direc).sum().item()
        assert abs(fd - an) / max(abs(an), 1e-8) < tol, (fd, an)


@pytest.mark.parametrize("variant", ["dense", "gqa", "lora", "moe", "qknorm"])
def test_layer_fd(variant):
    kw = {}
    if variant == "dense":
        kw = dict(n_q=2, n_kv=2)
    if variant == "qknorm":
        kw = dict(qk_norm=True)
    if variant == "lora":
        kw = dict(lora_rank=3, lora_alpha=6.0)
    if variant == "moe":
        kw = dict(ffn=0, n_experts=4, top_k=2, expert_ffn=12)
    cfg = tiny_cfg(**kw)
    w = f64(synth.layer_weights(cfg, 0, gamma="perturbed"))
    for k in ("wq", "wk", "wv", "wo", "wg", "wu", "wd"):
        w[k] = w[k] * 10  # std 0.2: keep attention and MLP non-trivial at H=16
    lora = f64(synth.lora_weights(cfg, 0, b_zero=False)) if cfg.lora_rank else None
    router = synth.router_logits(cfg, 0).to(D64) if cfg.is_moe else None
    x = synth.activation(cfg, "x").to(D64)
    dy = synth.activation(cfg, "dy").to(D64)
    dx, grads, _ = O.layer_backward(x, w, dy, cfg, lora, router)
    src = lora if cfg.lora_rank else w
    names = O.trainable_names(cfg)

    def fn():
        return (O.layer_forward(x, w, cfg, lora, router) * dy).sum()

    _fd_check(fn, [x] + [src[n] for n in names], [dx] + [grads[n] for n in names])


def test_lmhead_fd():
    cfg = tiny_cfg()
    x = synth.activation(cfg, "x").to(D64)
    w = synth.normal((cfg.vocab, cfg.hidden), 3, "w", 0.3).to(D64)
    gf = synth.normal((cfg.hidden,), 3, "gf", 0.1, mean=1.0).to(D64)
    labels = synth.uniform_int((cfg.tokens,), cfg.vocab, 3, "lab")
    labels[3] = -1
    loss, dx, dw, dg = O.lmhead_fwd_bwd(x, w, labels, 3, gf, 1e-6)

    def fn():
        return O.lmhead_loss_sharded(x, w, labels, 3, gf, 1e-6)

    _fd_check(fn, [x, w, gf], [dx, dw, dg])


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------


def test_qk_norm_scale_invariance_and_unit_heads():
    """QK-norm (Qwen3-style): with eps = 0 the per-head RMSNorm removes any
    positive scale of the q and k projections, so scaling W_q and W_k leaves
    the layer unchanged, while without QK-norm the same scaling changes it;
    with unit gains every rotated head has norm sqrt(d) (rotation keeps norms)."""
    cfg = tiny_cfg(qk_norm=True, rms_eps=0.0)
    w = f64(synth.layer_weights(cfg, 0, gamma="perturbed"))
    for k in ("wq", "wk", "wv", "wo", "wg", "wu", "wd"):
        w[k] = w[k] * 10
    x = synth.activation(cfg, "x").to(D64)
    y = O.layer_forward(x, w, cfg)
    w2 = dict(w, wq=w["wq"] * 3.7, wk=w["wk"] * 0.45)
    assert torch.allclose(O.layer_forward(x, w2, cfg), y, rtol=1e-12, atol=1e-12)
    plain = tiny_cfg(rms_eps=0.0)
    assert not torch.allclose(O.layer_forward(x, w2, plain), O.layer_forward(x, w, plain), rtol=1e-6, atol=1e-6)
    w1 = dict(w, qnorm=torch.ones_like(w["qnorm"]), knorm=torch.ones_like(w["knorm"]))
    _, q, k, _, _, _, _ = O.attention_block(x, w1, cfg)
    d = cfg.head_dim
    assert torch.allclose(q.norm(dim=-1), torch.full(q.shape[:2], math.sqrt(d), dtype=D64), rtol=1e-12)
    assert torch.allclose(k.norm(dim=-1), torch.full(k.shape[:2], math.sqrt(d), dtype=D64), rtol=1e-12)


def test_qk_norm_matches_library_rms_norm():
    """The per-head normalisation equals torch's rms_norm over each head's d
    dims (the rotation undone with the RoPE at position 0 of every row: seq 1)."""
    cfg = tiny_cfg(qk_norm=True, seq=1, batch=6)
    w = f64(synth.layer_weights(cfg, 0, gamma="perturbed"))
    x = synth.activation(cfg, "x").to(D64)
    a, q, k, _, _, _, _ = O.attention_block(x, w, cfg)
    T, d = x.shape[0], cfg.head_dim
    ref_q = F.rms_norm((a @ w["wq"].T).reshape(T, cfg.n_q, d), (d,), w["qnorm"], cfg.rms_eps)
    ref_k = F.rms_norm((a @ w["wk"].T).reshape(T, cfg.n_kv, d), (d,), w["knorm"], cfg.rms_eps)
    assert torch.allclose(q, ref_q, rtol=1e-12, atol=1e-14)
    assert torch.allclose(k, ref_k, rtol=1e-12, atol=1e-14)



@pytest.mark.parametrize("vocab,expect", [(4096, 8.317766166719343), (128256, 11.761783545564427)])
def test_zero_lmhead_loss_is_log_vocab(vocab, expect):
    T, H = 6, 8
    x = torch.randn(T, H, dtype=D64)
    w = torch.zeros(vocab, H, dtype=D64)
    labels = torch.randint(0, vocab, (T,))
    loss = O.lmhead_loss_sharded(x, w, labels, 4)
    assert abs(loss.item() - expect) < 1e-9
    assert abs(expect - math.log(vocab)) < 1e-9


def test_lmhead_grad_rows_sum_to_zero_and_zero_weight_closed_form():
    T, H, V = 10, 8, 40
    x = torch.randn(T, H, dtype=D64)
    w = torch.randn(V, H, dtype=D64) * 0.5
    labels = torch.randint(0, V, (T,))
    _, _, dw, _ = O.lmhead_fwd_bwd(x, w, labels, 3)
    # sum_v dlogits[t, v] = 0 for every row => the columns of dW sum to zero.
    assert dw.sum(0).abs().max().item() < 1e-12
    # W = 0: dlogits = (1/V - onehot) / N, so dW = dlogits^T x.
    _, dx0, dw0, _ = O.lmhead_fwd_bwd(x, torch.zeros(V, H, dtype=D64), labels, 2)
    dz = (torch.full((T, V), 1.0 / V, dtype=D64) - F.one_hot(labels, V).to(D64)) / T
    assert torch.allclose(dw0, dz.T @ x, atol=1e-14)
    assert dx0.abs().max().item() == 0.0


def test_attention_seq1_returns_v_and_zero_q_running_mean():
    T, nq, nkv, d = 5, 4, 2, 8
    q = torch.randn(T, nq, d, dtype=D64)
    k = torch.randn(T, nkv, d, dtype=D64)
    v = torch.randn(T, nkv, d, dtype=D64)
    out1 = O.causal_attention(q, k, v, batch=T, seq=1)  # every row its own sequence
    for h in range(nq):
        assert torch.allclose(out1[:, h], v[:, (h * nkv) // nq], atol=0, rtol=0)
    out0 = O.causal_attention(torch.zeros_like(q), k, v, batch=1, seq=T)
    mean = torch.cumsum(v, 0) / torch.arange(1, T + 1, dtype=D64)[:, None, None]
    for h in range(nq):
        assert torch.allclose(out0[:, h], mean[:, (h * nkv) // nq], atol=1e-14)


def test_rope_properties():
    d, base = 16, 10000.0
    u = torch.randn(7, 3, d, dtype=D64)
    pos = torch.tensor([0, 1, 2, 5, 9, 100, 4095])
    r = O.rope(u, pos, base)
    half = d // 2
    # pair norms preserved
    n0 = u[..., :half] ** 2 + u[..., half:] ** 2
    n1 = r[..., :half] ** 2 + r[..., half:] ** 2
    assert torch.allclose(n0, n1, atol=1e-12)
    # position 0 is the identity
    assert torch.equal(r[0], u[0])
    # complex form: (u1 + i u2) * exp(i theta)
    th = torch.arange(half, dtype=D64)
    th = pos[:, None].to(D64) * base ** (-2 * th / d)
    c = torch.complex(u[..., :half], u[..., half:]) * torch.polar(torch.ones_like(th), th)[:, None, :]
    assert torch.allclose(torch.cat([c.real, c.imag], -1), r, atol=1e-12)
    # relative position: <R_m q, R_n k> = <R_{m-n} q, k>
    q = torch.randn(1, 1, d, dtype=D64)
    k = torch.randn(1, 1, d, dtype=D64)
    for m, n in [(7, 3), (100, 37), (12, 12)]:
        lhs = (O.rope(q, torch.tensor([m]), base) * O.rope(k, torch.tensor([n]), base)).sum()
        rhs = (O.rope(q, torch.tensor([m - n]), base) * k).sum()
        assert abs(lhs - rhs) < 1e-12
    # backward = rotation by -theta (orthogonal: transpose = inverse)
    uu = u.clone().requires_grad_(True)
    g = torch.randn_like(u)
    (gu,) = torch.autograd.grad((O.rope(uu, pos, base) * g).sum(), [uu])
    back = O.rope(gu, pos, base)
    assert torch.allclose(back, g, atol=1e-12)


def test_rmsnorm_constant_and_library():
    for c in [3.0, -0.5, 1e-3]:
        x = torch.full((2, 64), c, dtype=D64)
        y = O.rmsnorm(x, torch.ones(64, dtype=D64), 1e-6)
        expect = math.copysign(1.0, c) / math.sqrt(1 + 1e-6 / c ** 2)
        assert torch.allclose(y, torch.full_like(y, expect), atol=1e-14)
    x = torch.randn(5, 32, dtype=D64)
    gm = torch.randn(32, dtype=D64)
    assert torch.allclose(O.rmsnorm(x, gm, 1e-6), F.rms_norm(x, (32,), gm, 1e-6), atol=1e-14)


def test_attention_matches_library_sdpa_gqa():
    B, S, nq, nkv, d = 2, 11, 8, 2, 16
    T = B * S
    q = torch.randn(T, nq, d, dtype=D64)
    k = torch.randn(T, nkv, d, dtype=D64)
    v = torch.randn(T, nkv, d, dtype=D64)
    ours = O.causal_attention(q, k, v, B, S)
    rep = nq // nkv
    qq = q.reshape(B, S, nq, d).transpose(1, 2)
    kk = k.reshape(B, S, nkv, d).transpose(1, 2).repeat_interleave(rep, dim=1)
    vv = v.reshape(B, S, nkv, d).transpose(1, 2).repeat_interleave(rep, dim=1)
    ref = F.scaled_dot_product_attention(qq, kk, vv, is_causal=True)
    assert torch.allclose(ours, ref.transpose(1, 2).reshape(T, nq, d), atol=1e-13)


def test_attention_causality():
    B, S, nq, nkv, d = 1, 12, 2, 1, 8
    q = torch.randn(S, nq, d, dtype=D64)
    k = torch.randn(S, nkv, d, dtype=D64)
    v = torch.randn(S, nkv, d, dtype=D64)
    base = O.causal_attention(q, k, v, B, S)
    k2, v2, q2 = k.clone(), v.clone(), q.clone()
    k2[7:] += 5.0
    v2[7:] -= 3.0
    q2[7:] *= 2.0
    pert = O.causal_attention(q2, k2, v2, B, S)
    assert torch.equal(base[:7], pert[:7])
    assert not torch.allclose(base[7:], pert[7:])


def test_silu_matches_library():
    g = torch.randn(100, dtype=D64) * 4
    assert torch.allclose(O.silu(g), F.silu(g), atol=1e-15)


def test_cross_entropy_matches_library():
    T, H, V = 12, 8, 50
    x = torch.randn(T, H, dtype=D64)
    w = torch.randn(V, H, dtype=D64)
    labels = torch.randint(0, V, (T,))
    labels[[2, 5]] = -1
    ref = F.cross_entropy(x @ w.T, labels.long(), ignore_index=-1)
    for s in (1, 3, 7):
        assert abs(O.lmhead_loss_sharded(x, w, labels, s).item() - ref.item()) < 1e-12
    assert abs(O.lmhead_loss_unsharded(x, w, labels).item() - ref.item()) < 1e-12


# ---------------------------------------------------------------------------
# reductions to simpler layers / brute force
# ---------------------------------------------------------------------------


def test_gqa_equals_mha_with_repeated_kv():
    cfg = tiny_cfg(n_q=4, n_kv=2)
    w = f64(synth.layer_weights(cfg, 0))
    x = synth.activation(cfg, "x").to(D64)
    d = cfg.head_dim
    mha = cfg.with_(n_kv=4)
    w2 = dict(w)
    for n in ("wk", "wv"):
        blocks = w[n].reshape(cfg.n_kv, d, cfg.hidden)
        w2[n] = blocks.repeat_interleave(2, dim=0).reshape(4 * d, cfg.hidden)
    assert torch.allclose(O.layer_forward(x, w, cfg), O.layer_forward(x, w2, mha), atol=1e-13)


def test_moe_reductions():
    cfg = tiny_cfg(ffn=0, n_experts=3, top_k=3, expert_ffn=10)
    w = f64(synth.layer_weights(cfg, 0))
    for k in ("wg", "wu", "wd"):
        w[k] = w[k] * 10
    b = torch.randn(cfg.tokens, cfg.hidden, dtype=D64)
    z = torch.randn(cfg.tokens, 3, dtype=D64)
    # k = E: the softmax-weighted dense mixture of every expert
    mix = sum(torch.softmax(z, -1)[:, e:e + 1] * O.swiglu(b, w["wg"][e], w["wu"][e], w["wd"][e])
              for e in range(3))
    assert torch.allclose(O.moe_mlp(b, z, w["wg"], w["wu"], w["wd"], 3), mix, atol=1e-13)
    # E = 1, k = 1: a dense SwiGLU
    one = O.moe_mlp(b, z[:, :1], w["wg"][:1], w["wu"][:1], w["wd"][:1], 1)
    assert torch.allclose(one, O.swiglu(b, w["wg"][0], w["wu"][0], w["wd"][0]), atol=1e-14)
    # grouped evaluation equals a per-token loop with explicit top-k search
    cfg2 = tiny_cfg(ffn=0, n_experts=5, top_k=2, expert_ffn=6)
    w2 = f64(synth.layer_weights(cfg2, 1))
    z2 = torch.randn(cfg2.tokens, 5, dtype=D64)
    z2[0, :] = torch.tensor([1.0, 2.0, 2.0, 0.5, 2.0], dtype=D64)  # ties -> lower indices
    got = O.moe_mlp(b, z2, w2["wg"], w2["wu"], w2["wd"], 2)
    for t in range(cfg2.tokens):
        row = z2[t].tolist()
        chosen = []
        for _ in range(2):
            best = None
            for e in range(5):
                if e in chosen:
                    continue
                if best is None or row[e] > row[best]:
                    best = e
            chosen.append(best)
        ex = [math.exp(row[e] - max(row[e2] for e2 in chosen)) for e in chosen]
        ref = torch.zeros(cfg2.hidden, dtype=D64)
        for e, wt in zip(chosen, ex):
            hid = []
            for f in range(6):
                gg = sum(b[t, i].item() * w2["wg"][e, f, i].item() for i in range(cfg2.hidden))
                uu = sum(b[t, i].item() * w2["wu"][e, f, i].item() for i in range(cfg2.hidden))
                hid.append(gg / (1 + math.exp(-gg)) * uu)
            for o in range(cfg2.hidden):
                ref[o] += wt / sum(ex) * sum(hid[f] * w2["wd"][e, o, f].item() for f in range(6))
        if t == 0:
            assert chosen == [1, 2]
        assert torch.allclose(got[t], ref, atol=1e-12)


def test_lora_merged_weight_and_zero_b():
    cfg = tiny_cfg(lora_rank=4, lora_alpha=8.0)
    w = f64(synth.layer_weights(cfg, 0))
    lora = f64(synth.lora_weights(cfg, 0, b_zero=False))
    x = synth.activation(cfg, "x").to(D64)
    s = cfg.lora_alpha / cfg.lora_rank
    merged = dict(w)
    for n in "qkvo":
        merged["w" + n] = w["w" + n] + s * lora["b" + n] @ lora["a" + n]
    assert torch.allclose(O.layer_forward(x, w, cfg, lora), O.layer_forward(x, merged, cfg), atol=1e-13)
    lz = f64(synth.lora_weights(cfg, 0, b_zero=True))
    assert torch.equal(O.layer_forward(x, w, cfg, lz), O.layer_forward(x, w, cfg))
    dy = synth.activation(cfg, "dy").to(D64)
    _, grads, _ = O.layer_backward(x, w, dy, cfg, lz)
    for n in "qkvo":
        assert grads["a" + n].abs().max().item() == 0.0
        assert grads["b" + n].abs().max().item() > 0.0


# ---------------------------------------------------------------------------
# stage invariants
# ---------------------------------------------------------------------------


def _tiny_model(cfg):
    layers = [synth.layer_weights(cfg, l, gamma="perturbed") for l in range(2)]
    head = synth.lmhead_weights(cfg)
    ids = synth.token_ids(cfg)
    labels = synth.shifted_labels(ids).reshape(-1)
    return layers, head, ids, labels


def test_recompute_equals_forward_bitwise_and_stage_split_invariance():
    cfg = tiny_cfg(n_q=2, n_kv=1, seq=12)
    layers = [synth.layer_weights(cfg, l, gamma="perturbed") for l in range(3)]
    x = synth.activation(cfg, "x")
    dy = synth.activation(cfg, "dy")
    y, ck = O.stage_forward(x, layers, cfg)
    # recompute from the checkpoints reproduces each layer output exactly
    for i in range(3):
        _, _, y_re = O.layer_backward(ck[i], layers[i], torch.zeros_like(y), cfg)
        nxt = ck[i + 1] if i < 2 else y
        assert torch.equal(y_re, nxt)
    dx, per = O.stage_backward_recompute(ck, layers, dy, cfg)
    # split [0,3) as [0,1) + [1,3)
    y1, ck1 = O.stage_forward(x, layers[:1], cfg)
    y2, ck2 = O.stage_forward(y1, layers[1:], cfg)
    assert torch.equal(y2, y)
    dmid, per2 = O.stage_backward_recompute(ck2, layers[1:], dy, cfg)
    dx2, per1 = O.stage_backward_recompute(ck1, layers[:1], dmid, cfg)
    assert torch.equal(dx2, dx)
    for a, b in zip(per, per1 + per2):
        for n in a:
            assert torch.equal(a[n], b[n])


def test_stagewise_tiny_model_equals_one_graph():
    cfg = synth.config("tiny", seq=16)
    layers, head, ids, labels = _tiny_model(cfg)
    loss_ref, g_ref = O.full_model_fwd_bwd(ids, labels, layers, head, cfg)
    x0 = O.embed(ids, head["embed"].to(D64))
    y, ck = O.stage_forward(x0, layers, cfg)
    loss, dy, dw, dg = O.lmhead_fwd_bwd(y, head["w"], labels, cfg.n_shards, head["gamma_f"], cfg.rms_eps)
    dx0, per = O.stage_backward_recompute(ck, layers, dy, cfg)
    de = O.embed_backward(ids, dx0, cfg.vocab)
    assert abs(loss.item() - loss_ref.item()) < 1e-13
    assert torch.allclose(de, g_ref["embed"], atol=1e-14)
    assert torch.allclose(dw, g_ref["w"], atol=1e-14)
    assert torch.allclose(dg, g_ref["gamma_f"], atol=1e-14)
    for a, b in zip(per, g_ref["layers"]):
        for n in a:
            assert torch.allclose(a[n], b[n], atol=1e-13), n


def test_sharded_lmhead_equals_unsharded_fp32():
    cfg = synth.config("llama3_8b")
    T, H, V = 64, 128, 4000
    x = synth.normal((T, H), 5, "x", dtype=torch.float32)
    w = synth.normal((V, H), 5, "w", 0.02, dtype=torch.float32)
    labels = synth.uniform_int((T,), V, 5, "l")
    l4, dx4, dw4, _ = O.lmhead_fwd_bwd(x, w, labels, 4, dtype=torch.float32)
    l1, dx1, dw1, _ = O.lmhead_fwd_bwd(x, w, labels, 1, dtype=torch.float32)
    lu = O.lmhead_loss_unsharded(x, w, labels)
    assert abs(l4.item() - lu.item()) / abs(lu.item()) < 1e-6
    assert abs(l4.item() - l1.item()) / abs(l1.item()) < 1e-6
    assert ((dx4 - dx1).abs().max() / dx1.abs().max()).item() < 1e-6
    assert ((dw4 - dw1).abs().max() / dw1.abs().max()).item() < 1e-6
    assert cfg.vocab % cfg.n_shards == 0 and O.shard_bounds(cfg.vocab, 4)[1] == (32064, 64128)


def test_fp32_oracle_close_to_fp64_on_tiny_model():
    cfg = synth.config("tiny", seq=32)
    layers, head, ids, labels = _tiny_model(cfg)
    l64, g64 = O.full_model_fwd_bwd(ids, labels, layers, head, cfg, dtype=torch.float64)
    l32, g32 = O.full_model_fwd_bwd(ids, labels, layers, head, cfg, dtype=torch.float32)
    assert abs(l32.item() - l64.item()) / abs(l64.item()) < 1e-5
    for a, b in zip(g32["layers"], g64["layers"]):
        for n in a:
            err = (a[n].double() - b[n]).abs().max() / b[n].abs().max()
            assert err.item() < 1e-5, n


@pytest.mark.parametrize("variant", ["dense", "lora_moe"])
def test_layer_forward_rows_equals_full_forward(variant):
    """The row-sampled layer forward (used for full-size checks) equals the
    full forward at the sampled rows, including rows of the second batch row."""
    kw = dict(n_q=4, n_kv=2)
    if variant == "lora_moe":
        kw.update(lora_rank=3, lora_alpha=6.0, ffn=0, n_experts=4, top_k=2, expert_ffn=12)
    cfg = tiny_cfg(**kw)
    w = f64(synth.layer_weights(cfg, 0, gamma="perturbed"))
    for k in ("wq", "wk", "wv", "wo", "wg", "wu", "wd"):
        w[k] = w[k] * 10
    lora = f64(synth.lora_weights(cfg, 0, b_zero=False)) if cfg.lora_rank else None
    router = synth.router_logits(cfg, 0).to(D64) if cfg.is_moe else None
    x = synth.activation(cfg, "x").to(D64)
    y = O.layer_forward(x, w, cfg, lora, router)
    rows = [0, 3, 7, 8, 15]
    yr = O.layer_forward_rows(x, w, cfg, rows, lora, router)
    assert torch.allclose(yr, y[rows], rtol=1e-12, atol=1e-12)


def test_lmhead_rows_equals_full_gradients():
    """Chunked loss, row-sampled dx and vocabulary-sampled dW equal the full
    autograd LM head (ignored labels included)."""
    g = torch.Generator().manual_seed(3)
    T, H, V = 40, 12, 50
    x = torch.randn(T, H, generator=g, dtype=D64)
    w = torch.randn(V, H, generator=g, dtype=D64) * 0.3
    labels = torch.randint(0, V, (T,), generator=g)
    labels[5] = -1
    loss, dx, dw, _ = O.lmhead_fwd_bwd(x, w, labels, 1)
    rows, vrows = [0, 5, 17, 39], [0, 3, int(labels[2]), 49]
    l2, dxr, dwr = O.lmhead_rows(x, w, labels, rows, vrows, chunk=16)
    assert torch.allclose(l2, loss, rtol=1e-12)
    assert torch.allclose(dxr, dx[rows], rtol=1e-10, atol=1e-14)
    assert torch.allclose(dwr, dw[vrows], rtol=1e-10, atol=1e-14)


def test_mlp_weight_grad_columns_equals_autograd():
    """Column-sampled MLP weight gradients (used at full size) equal the
    autograd gradients of sum(y * dy) at those columns."""
    g = torch.Generator().manual_seed(4)
    T, H, Fd = 20, 8, 12
    b = torch.randn(T, H, generator=g, dtype=D64)
    dy = torch.randn(T, H, generator=g, dtype=D64)
    w = {k: (torch.randn(*sh, generator=g, dtype=D64) * 0.5).requires_grad_(True)
         for k, sh in (("wg", (Fd, H)), ("wu", (Fd, H)), ("wd", (H, Fd)))}
    y = O.swiglu(b, w["wg"], w["wu"], w["wd"])
    gg, gu, gd = torch.autograd.grad((y * dy).sum(), [w["wg"], w["wu"], w["wd"]])
    cols = [0, 5, 11]
    dwd, dwg, dwu = O.mlp_weight_grad_columns(b, dy, {k: v.detach() for k, v in w.items()}, cols)
    assert torch.allclose(dwd, gd[:, cols], rtol=1e-12, atol=1e-12)
    assert torch.allclose(dwg, gg[cols], rtol=1e-12, atol=1e-12)
    assert torch.allclose(dwu, gu[cols], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# the layer's wiring: closed forms with some weights zero, and the layer
# rebuilt from library routines (pre-norm residual layer of the paperlayer.ai
# summary, appendix B.1; the residual sources and norm placement are a reading
# of a component list, so they are fixed here against things the oracle does
# not compute itself)
# ---------------------------------------------------------------------------


def _wiring_case(batch=2, seq=8):
    cfg = tiny_cfg(n_q=4, n_kv=2, batch=batch, seq=seq)
    w = f64(synth.layer_weights(cfg, 0, gamma="perturbed"))
    for k in ("wq", "wk", "wv", "wo", "wg", "wu", "wd"):
        w[k] = w[k] * 10
    x = synth.activation(cfg, "x").to(D64)
    return cfg, w, x


def _lib_swiglu(b, w):
    """SwiGLU MLP from library routines: silu(b Wg^T) * (b Wu^T), then Wd."""
    return F.linear(F.silu(F.linear(b, w["wg"])) * F.linear(b, w["wu"]), w["wd"])


def _lib_norm(x, gamma, cfg):
    return F.rms_norm(x, (x.shape[-1],), gamma, cfg.rms_eps)


def test_layer_wiring_zero_projections_is_identity():
    """Every projection zero: both residual branches vanish, y == x exactly."""
    cfg, w, x = _wiring_case()
    for k in ("wq", "wk", "wv", "wo", "wg", "wu", "wd"):
        w[k] = torch.zeros_like(w[k])
    assert torch.equal(O.layer_forward(x, w, cfg), x)


def test_layer_wiring_zero_wo_is_mlp_of_normed_input():
    """W_o = 0: the attention branch adds nothing, h1 = x, so
    y = x + SwiGLU(RMSNorm(x; gamma2)). Fixes that the MLP reads the second
    norm of the residual stream and that its output is added to x (not to
    the normed input)."""
    cfg, w, x = _wiring_case()
    w["wo"] = torch.zeros_like(w["wo"])
    y, keep = O.layer_forward(x, w, cfg, keep=True)
    assert torch.equal(keep["h1"], x)
    ref = x + _lib_swiglu(_lib_norm(x, w["gamma2"], cfg), w)
    assert torch.allclose(y, ref, rtol=0, atol=1e-13)


def test_layer_wiring_zero_wq_is_running_mean_of_values():
    """W_q = 0: every score is 0, so each query head's output is the running
    mean of its kv head's values over the earlier tokens of its batch row,
    whatever RoPE does to the keys. Then h1 = x + mean(v) W_o^T with v taken
    from RMSNorm(x; gamma1), and y = h1 + SwiGLU(RMSNorm(h1; gamma2)).
    Fixes the first norm's input, the value projection, the GQA head map, the
    per-row restart and the first residual."""
    cfg, w, x = _wiring_case()
    w["wq"] = torch.zeros_like(w["wq"])
    B, S, d = cfg.batch, cfg.seq, cfg.head_dim
    v = F.linear(_lib_norm(x, w["gamma1"], cfg), w["wv"]).reshape(B, S, cfg.n_kv, d)
    mean = torch.cumsum(v, dim=1) / torch.arange(1, S + 1, dtype=D64)[None, :, None, None]
    o = mean.repeat_interleave(cfg.n_q // cfg.n_kv, dim=2).reshape(B * S, cfg.n_q * d)
    h1 = x + F.linear(o, w["wo"])
    y = O.layer_forward(x, w, cfg)
    assert torch.allclose(y, h1 + _lib_swiglu(_lib_norm(h1, w["gamma2"], cfg), w), rtol=0, atol=1e-12)
    w["wd"] = torch.zeros_like(w["wd"])
    assert torch.allclose(O.layer_forward(x, w, cfg), h1, rtol=0, atol=1e-12)


def test_layer_matches_library_composition():
    """The whole layer rebuilt from library routines: torch's rms_norm, RoPE as
    multiplication of the complex pairs (u_i + i u_{i+d/2}) by exp(i theta),
    torch's causal scaled_dot_product_attention with the kv heads repeated per
    query group, silu and linear. Two batch rows, so positions restart."""
    cfg, w, x = _wiring_case()
    B, S, d, nq, nkv = cfg.batch, cfg.seq, cfg.head_dim, cfg.n_q, cfg.n_kv
    half = d // 2
    a = _lib_norm(x, w["gamma1"], cfg)
    th = torch.arange(S, dtype=D64)[:, None] * cfg.rope_base ** (-2.0 * torch.arange(half, dtype=D64) / d)
    rot = torch.polar(torch.ones_like(th), th)                         # [S, d/2]

    def rope_c(u, nh):
        u = u.reshape(B, S, nh, d)
        z = torch.complex(u[..., :half], u[..., half:]) * rot[None, :, None, :]
        return torch.cat([z.real, z.imag], dim=-1).transpose(1, 2)   # [B, nh, S, d]

    q = rope_c(F.linear(a, w["wq"]), nq)
    k = rope_c(F.linear(a, w["wk"]), nkv).repeat_interleave(nq // nkv, dim=1)
    v = F.linear(a, w["wv"]).reshape(B, S, nkv, d).transpose(1, 2).repeat_interleave(nq // nkv, dim=1)
    o = F.scaled_dot_product_attention(q, k, v, is_causal=True).transpose(1, 2).reshape(B * S, nq * d)
    h1 = x + F.linear(o, w["wo"])
    ref = h1 + _lib_swiglu(_lib_norm(h1, w["gamma2"], cfg), w)
    assert torch.allclose(O.layer_forward(x, w, cfg), ref, rtol=0, atol=1e-12)


def test_moe_layer_with_one_expert_equals_dense_layer():
    """A mixture of one expert, top-1 (weight exactly 1), is the dense layer
    with that expert's weights: fixes the MoE layer's residual and norm wiring
    to the dense one pinned above."""
    cfg, w, x = _wiring_case()
    moe = cfg.with_(ffn=0, n_experts=1, top_k=1, expert_ffn=cfg.ffn)
    wm = dict(w)
    for k in ("wg", "wu", "wd"):
        wm[k] = w[k][None]
    router = torch.randn(cfg.tokens, 1, dtype=D64)
    assert torch.allclose(O.layer_forward(x, wm, moe, router=router), O.layer_forward(x, w, cfg),
                          rtol=0, atol=1e-13)


@pytest.mark.parametrize("variant", ["gqa", "qknorm", "lora_moe"])
def test_layer_backward_rows_equals_masked_full_backward(variant):
    """The sparse-upstream-gradient backward used at full size equals the
    complete backward with dy zeroed outside the listed rows, for dx at every
    row and for every trainable gradient; rows after the last listed row of a
    batch row get dx exactly 0 (causality)."""
    kw = dict(n_q=4, n_kv=2)
    if variant == "qknorm":
        kw.update(qk_norm=True)
    if variant == "lora_moe":
        kw.update(lora_rank=3, lora_alpha=6.0, ffn=0, n_experts=4, top_k=2, expert_ffn=12)
    cfg = tiny_cfg(**kw)
    w = f64(synth.layer_weights(cfg, 0, gamma="perturbed"))
    for k in ("wq", "wk", "wv", "wo", "wg", "wu", "wd"):
        w[k] = w[k] * 10
    lora = f64(synth.lora_weights(cfg, 0, b_zero=False)) if cfg.lora_rank else None
    router = synth.router_logits(cfg, 0).to(D64) if cfg.is_moe else None
    x = synth.activation(cfg, "x").to(D64)
    rows = [1, 7, 8, 12]
    dy_rows = synth.normal((len(rows), cfg.hidden), cfg.seed, "dy_rows", 1.0).to(D64)
    dy = torch.zeros_like(x)
    dy[rows] = dy_rows
    dx_ref, g_ref, _ = O.layer_backward(x, w, dy, cfg, lora, router)
    dx, g = O.layer_backward_rows(x, w, rows, dy_rows, cfg, lora, router)
    assert torch.allclose(dx, dx_ref, rtol=1e-12, atol=1e-13)
    assert set(g) == set(g_ref)
    for n in g_ref:
        assert torch.allclose(g[n], g_ref[n], rtol=1e-12, atol=1e-13), n
    assert dx[13:].abs().max().item() == 0.0
    assert dx[:8].abs().min().item() > 0.0
