"""Stage-level parity on the GPU: every output and gradient of the HIP path
compared element by element with the CPU oracle on the same seeded inputs,
plus the invariants the method fixes (recomputation reproduces the forward,
splitting a stage changes nothing)."""
import pytest
import torch

import synth
from oracle import stage as O
from _helpers import GRAD_TOL, LOSS_TOL, ensure_built, max_rel, say, to_f64

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")


@pytest.fixture(scope="module")
def W():
    ensure_built()
    from offloaded_pipeline_stage_amd.worker import Worker
    return Worker


def test_tiny_full_model_fp32_matches_oracle(W):
    """Tiny decoder (2 layers, hidden 256, 4 heads of 64, FFN 688, vocab 4096,
    batch 2 x seq 128, fp32): embedding, fused stage over both layers with the
    LM head, embedding backward -- loss and every gradient."""
    cfg = synth.config("tiny")
    say("tiny full model")
    layers = [synth.layer_weights(cfg, l) for l in range(2)]
    head = synth.lmhead_weights(cfg)
    ids = synth.token_ids(cfg)
    labels = synth.shifted_labels(ids).reshape(-1)
    loss_ref, g_ref = O.full_model_fwd_bwd(ids, labels, layers, head, cfg)

    wk = W(cfg)
    for l in range(2):
        wk.add_layer(l, layers[l])
    wk.add_lmhead(head["w"], head["gamma_f"])
    ctx = wk.ctx
    T, H = cfg.tokens, cfg.hidden
    ids_d = ids.reshape(-1).to(DEV)
    lab_d = labels.to(DEV)
    table = head["embed"].to(DEV)
    x0 = torch.empty(T, H, device=DEV)
    y = torch.empty(T, H, device=DEV)
    dy = torch.empty(T, H, device=DEV)
    dx0 = torch.empty(T, H, device=DEV)
    loss = torch.zeros(1, device=DEV)
    dtable = torch.empty(cfg.vocab, H, device=DEV)
    ws = wk.ctx.workspace(B_OP_FUSED(), cfg.batch, cfg.seq, 2)
    wsh = wk.ctx.workspace(B_OP_LMHEAD(), cfg.batch, cfg.seq)
    ctx.embed_fwd(ids_d, table, x0)
    wk.fused_stage(0, 2, x0, lab_d, ws, wsh, y, dy, dx0, loss)
    ctx.embed_bwd(ids_d, dx0, dtable)
    ctx.sync()
    tol = GRAD_TOL["f32"]
    assert abs(loss.item() - loss_ref.item()) / abs(loss_ref.item()) < LOSS_TOL["f32"]
    assert max_rel(dtable, g_ref["embed"]) < tol
    assert max_rel(wk.head["dw"][0], g_ref["w"]) < tol
    assert max_rel(wk.head["dgamma_f"], g_ref["gamma_f"]) < tol
    for l in range(2):
        got = wk.unpack_grads(wk.layers[l]["g"])
        for n, r in g_ref["layers"][l].items():
            e = max_rel(got[n], r)
            assert e < tol, (l, n, e)


def B_OP_FUSED():
    from offloaded_pipeline_stage_amd import binding
    return binding.RP_OP_FUSED


def B_OP_LMHEAD():
    from offloaded_pipeline_stage_amd import binding
    return binding.RP_OP_LMHEAD


def _layer_case(name, seq, n_layers, gamma="perturbed", **over):
    cfg = synth.config(name, seq=seq, **over)
    layers = [synth.layer_weights(cfg, l, gamma=gamma) for l in range(n_layers)]
    x = synth.activation(cfg, "x")
    dy = synth.activation(cfg, "dy")
    return cfg, layers, x, dy


@pytest.mark.parametrize("name,seq,batch,qkn", [("qwen3_1p7b", 320, 1, False), ("llama3_8b", 200, 2, False),
                                                ("qwen3_1p7b", 257, 2, True)])
def test_bf16_layer_fwd_bwd_matches_oracle(W, name, seq, batch, qkn):
    """One bf16 decoder layer at the workload's real widths (Qwen3-1.7B or
    Llama-3.1-8B shapes) on a short ragged sequence: forward output, dx and
    every weight gradient against the fp64 oracle on the same bf16 inputs.
    qkn: with Qwen3's per-head QK-norm (gains perturbed, so their gradients
    carry signal)."""
    say("bf16 layer", name, seq, batch, "qk-norm" if qkn else "")
    cfg, layers, x, dy = _layer_case(name, seq, 1, batch=batch, qk_norm=qkn)
    wk = W(cfg)
    wk.add_layer(0, layers[0])
    T, H = cfg.tokens, cfg.hidden
    y = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    dx = torch.empty_like(y)
    ws = wk.ctx.workspace(B_OP_FUSED(), cfg.batch, cfg.seq, 1)
    from offloaded_pipeline_stage_amd import binding as Bd
    wk.ctx.stage_fwd(0, 1, cfg.batch, cfg.seq, x.to(DEV), y, ws, flags=Bd.RP_KEEP_ACTS)
    wk.ctx.stage_bwd_recompute(0, 1, cfg.batch, cfg.seq, dy.to(DEV), dx, ws, flags=Bd.RP_USE_KEPT_ACTS)
    wk.ctx.sync()
    y_ref, _ = O.stage_forward(x, layers, cfg)
    dx_ref, g_ref, _ = O.layer_backward(x, layers[0], dy, cfg)
    tol = GRAD_TOL["bf16"]
    assert max_rel(y, y_ref) < tol
    assert max_rel(dx, dx_ref) < tol
    got = wk.unpack_grads(wk.layers[0]["g"])
    for n, r in g_ref.items():
        e = max_rel(got[n], r)
        assert e < tol, (n, e)


@pytest.mark.parametrize("seq,vocab,shards", [(320, 8192, 4), (200, 6176, 4), (100, 4096, 2), (256, 2048, 1)])
def test_bf16_lmhead_sharded_matches_oracle(W, seq, vocab, shards):
    """LM head + CE with vocabulary shards at hidden 4096 (vocab reduced),
    bf16: loss, dx and every shard's weight gradient, at token counts and
    shard widths that leave ragged tiles (320 tokens; 1544-row shards; 100
    tokens, not a multiple of 8), and with a single shard."""
    say("bf16 lm head", seq, vocab, shards)
    cfg = synth.config("llama3_8b", seq=seq, vocab=vocab, n_shards=shards)
    x = synth.activation(cfg, "x")
    w = synth.lmhead_weights(cfg)["w"]
    labels = synth.uniform_labels(cfg)
    labels[7] = -1
    labels[0] = vocab - 1  # the last column of the last shard
    wk = W(cfg)
    wk.add_lmhead(w)
    T, H = cfg.tokens, cfg.hidden
    dx = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    loss = torch.zeros(1, device=DEV)
    ws = wk.ctx.workspace(B_OP_LMHEAD(), cfg.batch, cfg.seq)
    wk.ctx.lmhead_ce_fwd_bwd(cfg.batch, cfg.seq, x.to(DEV), labels.to(DEV), loss, dx, ws)
    wk.ctx.sync()
    l_ref, dx_ref, dw_ref, _ = O.lmhead_fwd_bwd(x, w, labels, shards)
    assert abs(loss.item() - l_ref.item()) / abs(l_ref.item()) < LOSS_TOL["bf16"]
    assert max_rel(dx, dx_ref) < GRAD_TOL["bf16"]
    dw = torch.cat([d.cpu() for d in wk.head["dw"]], dim=0)
    assert max_rel(dw, dw_ref) < GRAD_TOL["bf16"]


@pytest.mark.parametrize("vocab,shards", [(4093, 3), (1000, 1)])
def test_f32_lmhead_ragged_shards_matches_oracle(W, vocab, shards):
    """fp32 LM head + CE whose shard widths are not multiples of 4 (4093 rows
    in shards of 1365/1364/1364, or one shard of 1000), so the cross-entropy
    kernels run their unaligned paths next to the vector ones: loss, dx and
    every shard's weight gradient against the oracle."""
    say("f32 lm head ragged", vocab, shards)
    cfg = synth.config("tiny", vocab=vocab, n_shards=shards, final_norm=False, embedding=False)
    x = synth.activation(cfg, "x")
    w = synth.lmhead_weights(cfg)["w"]
    labels = synth.uniform_labels(cfg)
    labels[3] = -1
    labels[cfg.tokens - 1] = vocab - 1
    wk = W(cfg)
    wk.add_lmhead(w)
    T, H = cfg.tokens, cfg.hidden
    dx = torch.empty(T, H, dtype=torch.float32, device=DEV)
    loss = torch.zeros(1, device=DEV)
    ws = wk.ctx.workspace(B_OP_LMHEAD(), cfg.batch, cfg.seq)
    wk.ctx.lmhead_ce_fwd_bwd(cfg.batch, cfg.seq, x.to(DEV), labels.to(DEV), loss, dx, ws)
    wk.ctx.sync()
    l_ref, dx_ref, dw_ref, _ = O.lmhead_fwd_bwd(x, w, labels, shards)
    assert abs(loss.item() - l_ref.item()) / abs(l_ref.item()) < LOSS_TOL["f32"]
    assert max_rel(dx, dx_ref) < GRAD_TOL["f32"]
    dw = torch.cat([d.cpu() for d in wk.head["dw"]], dim=0)
    assert max_rel(dw, dw_ref) < GRAD_TOL["f32"]


@pytest.mark.parametrize("qkn", [False, True])
def test_recompute_equals_kept_and_split_invariance_bf16(W, qkn):
    """Two bf16 layers: (a) backward from kept activations (fused B_1) and
    backward with recomputation from checkpoints give bit-identical dx and
    gradients; (b) running [0,2) as one stage or as [0,1) + [1,2) gives
    bit-identical outputs and gradients. qkn: with QK-norm."""
    say("recompute/split invariance", "qk-norm" if qkn else "")
    cfg, layers, x, dy = _layer_case("qwen3_1p7b", 136, 2, hidden=1024, n_q=8, n_kv=4, ffn=2048, qk_norm=qkn)
    from offloaded_pipeline_stage_amd import binding as Bd
    wk = W(cfg)
    for l in range(2):
        wk.add_layer(l, layers[l])
    T, H = cfg.tokens, cfg.hidden
    b, s = cfg.batch, cfg.seq
    xd, dyd = x.to(DEV), dy.to(DEV)
    bf = dict(dtype=torch.bfloat16, device=DEV)
    # fused: keep + kept backward
    ws_f = wk.ctx.workspace(Bd.RP_OP_FUSED, b, s, 2)
    y1, dx1 = torch.empty(T, H, **bf), torch.empty(T, H, **bf)
    wk.ctx.stage_fwd(0, 2, b, s, xd, y1, ws_f, flags=Bd.RP_KEEP_ACTS)
    wk.ctx.stage_bwd_recompute(0, 2, b, s, dyd, dx1, ws_f, flags=Bd.RP_USE_KEPT_ACTS)
    wk.ctx.sync()
    g1 = [wk.layers[l]["g"].clone() for l in range(2)]
    # plain forward with host checkpoints, then backward recomputing from them
    ws_fw = wk.ctx.workspace(Bd.RP_OP_STAGE_FWD, b, s, 2)
    ws_bw = wk.ctx.workspace(Bd.RP_OP_STAGE_BWD, b, s, 2)
    ck = [torch.empty(T, H, dtype=torch.bfloat16).pin_memory() for _ in range(2)]
    y2, dx2 = torch.empty(T, H, **bf), torch.empty(T, H, **bf)
    wk.ctx.stage_fwd(0, 2, b, s, xd, y2, ws_fw, ckpt_host=ck)
    wk.ctx.stage_bwd_recompute(0, 2, b, s, dyd, dx2, ws_bw, ckpt=ck)
    wk.ctx.sync()
    g2 = [wk.layers[l]["g"].clone() for l in range(2)]
    assert torch.equal(y1, y2)
    assert torch.equal(ck[0], x)
    assert torch.equal(dx1, dx2)
    for a, c in zip(g1, g2):
        assert torch.equal(a, c)
    # split [0,1) + [1,2), checkpoints on the device
    ws1 = wk.ctx.workspace(Bd.RP_OP_STAGE_FWD, b, s, 1)
    wsb = wk.ctx.workspace(Bd.RP_OP_STAGE_BWD, b, s, 1)
    mid, y3 = torch.empty(T, H, **bf), torch.empty(T, H, **bf)
    wk.ctx.stage_fwd(0, 1, b, s, xd, mid, ws1)
    wk.ctx.stage_fwd(1, 2, b, s, mid, y3, ws1)
    dmid, dx3 = torch.empty(T, H, **bf), torch.empty(T, H, **bf)
    wk.ctx.stage_bwd_recompute(1, 2, b, s, dyd, dmid, wsb, ckpt=[mid], flags=Bd.RP_CKPT_DEVICE)
    wk.ctx.stage_bwd_recompute(0, 1, b, s, dmid, dx3, wsb, ckpt=[xd], flags=Bd.RP_CKPT_DEVICE)
    wk.ctx.sync()
    assert torch.equal(y3, y1)
    assert torch.equal(dx3, dx1)
    for l in range(2):
        assert torch.equal(wk.layers[l]["g"], g1[l])
    # and the two-layer stage agrees with the oracle
    y_ref, ck_ref = O.stage_forward(x, layers, cfg)
    dx_ref, _ = O.stage_backward_recompute(ck_ref, layers, dy, cfg)
    assert max_rel(y1, y_ref) < GRAD_TOL["bf16"]
    assert max_rel(dx1, dx_ref) < GRAD_TOL["bf16"]


@pytest.mark.parametrize("b_zero", [False, True])
def test_bf16_lora_layer_matches_oracle(W, b_zero):
    """LoRA r16 alpha32 on q, k, v, o over a frozen bf16 layer (Qwen3-235B
    attention widths: 64 query / 4 kv heads, hidden 4096; dense MLP here, the
    MoE MLP has its own test), ragged sequence: output, dx and the eight
    adapter gradients against the oracle. B = 0 (the initialisation) must give
    the base output and dA exactly zero."""
    say("bf16 lora layer", b_zero)
    cfg = synth.config("qwen3_235b_moe", seq=200, n_experts=0, top_k=0, expert_ffn=0, ffn=1536)
    lw = synth.layer_weights(cfg, 0, gamma="perturbed")
    lora = synth.lora_weights(cfg, 0, b_zero=b_zero)
    x = synth.activation(cfg, "x")
    dy = synth.activation(cfg, "dy")
    wk = W(cfg)
    wk.add_layer(0, lw, lora=lora)
    T, H = cfg.tokens, cfg.hidden
    y = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    dx = torch.empty_like(y)
    from offloaded_pipeline_stage_amd import binding as Bd
    ws = wk.ctx.workspace(Bd.RP_OP_FUSED, cfg.batch, cfg.seq, 1)
    wk.ctx.stage_fwd(0, 1, cfg.batch, cfg.seq, x.to(DEV), y, ws, flags=Bd.RP_KEEP_ACTS)
    wk.ctx.stage_bwd_recompute(0, 1, cfg.batch, cfg.seq, dy.to(DEV), dx, ws, flags=Bd.RP_USE_KEPT_ACTS)
    wk.ctx.sync()
    y_ref, _ = O.stage_forward(x, [lw], cfg, loras=[lora])
    dx_ref, g_ref, _ = O.layer_backward(x, lw, dy, cfg, lora)
    tol = GRAD_TOL["bf16"]
    assert max_rel(y, y_ref) < tol
    assert max_rel(dx, dx_ref) < tol
    got = wk.unpack_lora_grads(wk.layers[0]["lora_g"])
    for n, r in g_ref.items():
        if b_zero and n.startswith("a"):
            assert torch.count_nonzero(got[n]).item() == 0, n
            continue
        e = max_rel(got[n], r)
        assert e < tol, (n, e)
    if b_zero:
        # B = 0: the adapters change nothing, so y equals the base layer's output
        base_cfg = cfg.with_(lora_rank=0, lora_alpha=0.0)
        wb = W(base_cfg)
        wb.add_layer(0, lw)
        yb = torch.empty_like(y)
        wsb = wb.ctx.workspace(Bd.RP_OP_STAGE_FWD, cfg.batch, cfg.seq, 1)
        wb.ctx.stage_fwd(0, 1, cfg.batch, cfg.seq, x.to(DEV), yb, wsb)
        wb.ctx.sync()
        assert torch.equal(y, yb)


@pytest.mark.parametrize("experts,top_k,seq", [(128, 8, 256), (8, 2, 1100)])
def test_bf16_moe_lora_layer_matches_oracle(W, experts, top_k, seq):
    """MoE LoRA layer (Qwen3-235B-A22B widths: hidden 4096, 64/4 heads, expert
    FFN 1536, LoRA r16 on q/k/v/o, frozen base and experts): top-k routing on
    fp32 logits, grouped expert products, weighted combine; output, dx and the
    adapter gradients against the oracle. The 8-expert case gives each expert
    more than one 256-row tile (full and partial tiles)."""
    say("bf16 moe lora layer", experts, top_k, seq)
    cfg = synth.config("qwen3_235b_moe", seq=seq, n_experts=experts, top_k=top_k)
    lw = synth.layer_weights(cfg, 0, gamma="perturbed")
    lora = synth.lora_weights(cfg, 0, b_zero=False)
    router = synth.router_logits(cfg, 0)
    x = synth.activation(cfg, "x")
    dy = synth.activation(cfg, "dy")
    wk = W(cfg)
    wk.add_layer(0, lw, lora=lora)
    T, H = cfg.tokens, cfg.hidden
    y = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    dx = torch.empty_like(y)
    rd = router.to(DEV)
    from offloaded_pipeline_stage_amd import binding as Bd
    ws = wk.ctx.workspace(Bd.RP_OP_FUSED, cfg.batch, cfg.seq, 1)
    wk.ctx.stage_fwd(0, 1, cfg.batch, cfg.seq, x.to(DEV), y, ws, router=[rd], flags=Bd.RP_KEEP_ACTS)
    wk.ctx.stage_bwd_recompute(0, 1, cfg.batch, cfg.seq, dy.to(DEV), dx, ws, flags=Bd.RP_USE_KEPT_ACTS)
    # the recompute path (router needed again) gives the same bits
    ck = [torch.empty(T, H, dtype=torch.bfloat16).pin_memory()]
    y2, dx2 = torch.empty_like(y), torch.empty_like(y)
    wsf = wk.ctx.workspace(Bd.RP_OP_STAGE_FWD, cfg.batch, cfg.seq, 1)
    wsb = wk.ctx.workspace(Bd.RP_OP_STAGE_BWD, cfg.batch, cfg.seq, 1)
    wk.ctx.sync()
    g_kept = wk.layers[0]["lora_g"].clone()
    wk.ctx.stage_fwd(0, 1, cfg.batch, cfg.seq, x.to(DEV), y2, wsf, ckpt_host=ck, router=[rd])
    wk.ctx.stage_bwd_recompute(0, 1, cfg.batch, cfg.seq, dy.to(DEV), dx2, wsb, ckpt=ck, router=[rd])
    wk.ctx.sync()
    assert torch.equal(y, y2) and torch.equal(dx, dx2)
    assert torch.equal(g_kept, wk.layers[0]["lora_g"])
    y_ref, _ = O.stage_forward(x, [lw], cfg, loras=[lora], routers=[router])
    dx_ref, g_ref, _ = O.layer_backward(x, lw, dy, cfg, lora, router)
    tol = GRAD_TOL["bf16"]
    assert max_rel(y, y_ref) < tol
    assert max_rel(dx, dx_ref) < tol
    got = wk.unpack_lora_grads(wk.layers[0]["lora_g"])
    for n, r in g_ref.items():
        e = max_rel(got[n], r)
        assert e < tol, (n, e)


def test_bf16_layer_odd_head_count_fused_rope(W):
    """The RoPE epilogue of the QKV product on a packed width that 256-column
    tiles do not divide (3 query heads + 1 kv head: 5 heads of 128, the last
    tile half past the end) at a token count that takes the 256 x 256 tiles:
    sampled output rows against the oracle, and the recomputed backward of
    the fused stage equal to the kept one."""
    cfg = synth.StageConfig(name="odd", hidden=384, n_q=3, n_kv=1, head_dim=128, ffn=512, batch=2, seq=10240,
                            dtype="bf16", seed=1234)
    say("bf16 odd head count", cfg.tokens)
    lw = synth.layer_weights(cfg, 0, gamma="perturbed")
    x = synth.activation(cfg, "x")
    dy = synth.activation(cfg, "dy")
    wk = W(cfg)
    wk.add_layer(0, lw)
    ctx = wk.ctx
    T, H, b, s = cfg.tokens, cfg.hidden, cfg.batch, cfg.seq
    xd, dyd = x.to(DEV), dy.to(DEV)
    y, dx, dx2 = (torch.empty(T, H, dtype=torch.bfloat16, device=DEV) for _ in range(3))
    ws = ctx.workspace(B_OP_FUSED(), b, s, 1)
    ctx.stage_fwd(0, 1, b, s, xd, y, ws, flags=1)
    ctx.stage_bwd_recompute(0, 1, b, s, dyd, dx, ws, flags=2)
    ctx.sync()
    g_kept = wk.layers[0]["g"].clone()
    ws_b = ctx.workspace(1, b, s, 1)
    ctx.stage_bwd_recompute(0, 1, b, s, dyd, dx2, ws_b, ckpt=[xd], flags=4)
    ctx.sync()
    assert torch.equal(dx, dx2) and torch.equal(g_kept, wk.layers[0]["g"])
    rows = [0, 1, 255, 256, s - 1, s, s + 300, T - 1]
    ref = O.layer_forward_rows(x.double(), {k: v.double() for k, v in lw.items()}, cfg, rows)
    assert max_rel(y.cpu()[rows], ref) < GRAD_TOL["bf16"]
