"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times, on outputs the oracle can compute one by one (sampled token
rows, sampled weight-gradient rows and columns, the exact LM-head loss) and on
properties that hold at any size (recomputation reproduces the forward bit for
bit, splitting a stage changes nothing, B = 0 adapters get exactly zero dA).

The Qwen3-1.7B-shaped stage is small enough for the complete fp64 oracle, and
the Llama-3.1-8B-shaped layer for the complete fp32 oracle: every output and
gradient is compared element by element there. For the larger layers the
upstream gradient is made zero outside sampled rows; the exact oracle of that
case still gives dx at every row and every weight gradient in full."""
import pytest
import torch

import synth
from oracle import stage as O
from _helpers import GRAD_TOL, LOSS_TOL, ensure_built, max_rel, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")
TOL = GRAD_TOL["bf16"]


@pytest.fixture(scope="module")
def env():
    B = ensure_built()
    from offloaded_pipeline_stage_amd.worker import Worker
    return B, Worker


def sample_rows(T, n=10, seed=0):
    g = torch.Generator().manual_seed(seed)
    rows = {0, 1, T // 2, T - 2, T - 1}
    rows |= set(torch.randint(0, T, (n,), generator=g).tolist())
    return sorted(rows)


def rel_rows(got, ref):
    """max |got - ref| / max |ref| over the sampled rows."""
    return max_rel(got, ref)


def f64(d):
    return {k: v.to(torch.float64) for k, v in d.items()}


def mlp_input(x, w, cfg):
    """b = RMSNorm2(h1) of the layer for every row (the full attention forward)."""
    return O.attention_block(x, w, cfg)[-1]


def test_qwen3_1p7b_stage_full_streamed(env):
    """Qwen3-1.7B-shaped stage at full size (1 x 4096 tokens): weights of five
    layers in pinned host memory streamed through rp_weight_stream_submit;
    forward stage of layers 0-3 with host checkpoints, fused stage of layer 4
    (forward keeping its internals, then backward), gradients downloaded to
    pinned host memory. Everything against the complete fp64 oracle."""
    B, Worker = env
    cfg = synth.config("qwen3_1p7b")
    T, H, b, s = cfg.tokens, cfg.hidden, cfg.batch, cfg.seq
    say("qwen3_1p7b full: inputs")
    layers = [synth.layer_weights(cfg, l, gamma="perturbed") for l in range(5)]
    x = synth.activation(cfg, "x")
    dy = synth.activation(cfg, "dy")
    wk = Worker(cfg)
    host = [wk.pack_layer(layers[l], pinned=True) for l in range(5)]
    for l in range(5):
        wk.add_layer(l, resident=False)
    ctx = wk.ctx
    bf = dict(dtype=torch.bfloat16, device=DEV)
    x_host, dy_host = x.pin_memory(), dy.pin_memory()
    x_d, dy_d = torch.empty(T, H, **bf), torch.empty(T, H, **bf)
    say("qwen3_1p7b full: forward stage [0, 4)")
    t0 = ctx.act_copy(B.RP_H2D, x_d, x_host)
    ctx.weight_stream_submit([(B.RP_PARAM_H2D, B.RP_TGT_LAYER, l, 0, wk.w_bytes, host[l]) for l in range(4)],
                             n_windows=1, max_chunk=16 << 20, gate_ticket=t0)
    ck = [torch.empty(T, H, dtype=torch.bfloat16).pin_memory() for _ in range(4)]
    y4 = torch.empty(T, H, **bf)
    ws_f = ctx.workspace(B.RP_OP_STAGE_FWD, b, s, 4)
    ctx.stage_fwd(0, 4, b, s, x_d, y4, ws_f, ckpt_host=ck)
    say("qwen3_1p7b full: fused stage [4, 5)")
    t1 = ctx.act_copy(B.RP_H2D, dy_d, dy_host)
    ctx.weight_stream_submit([(B.RP_PARAM_H2D, B.RP_TGT_LAYER, 4, 0, wk.w_bytes, host[4])], n_windows=1,
                             max_chunk=16 << 20, gate_ticket=t1)
    y5, dx4 = torch.empty(T, H, **bf), torch.empty(T, H, **bf)
    ws = ctx.workspace(B.RP_OP_FUSED, b, s, 1)
    ctx.stage_fwd(4, 5, b, s, y4, y5, ws, flags=B.RP_KEEP_ACTS)
    ctx.stage_bwd_recompute(4, 5, b, s, dy_d, dx4, ws, flags=B.RP_USE_KEPT_ACTS)
    gh = torch.empty(wk.g_bytes, dtype=torch.uint8).pin_memory()
    ctx.weight_stream_submit([(B.RP_GRAD_D2H, B.RP_TGT_LAYER, 4, 0, wk.g_bytes, gh)], n_windows=1)
    ctx.sync()
    assert torch.equal(ck[0], x)
    say("qwen3_1p7b full: oracle")
    y4_ref, ck_ref = O.stage_forward(x, layers[:4], cfg)
    for i in range(1, 4):
        assert max_rel(ck[i], ck_ref[i]) < TOL, i
    assert max_rel(y4, y4_ref) < TOL
    dx_ref, g_ref, y5_ref = O.layer_backward(y4_ref, layers[4], dy, cfg)
    assert max_rel(y5, y5_ref) < TOL
    assert max_rel(dx4, dx_ref) < TOL
    got = wk.unpack_grads(gh)
    for n, r in g_ref.items():
        e = max_rel(got[n], r)
        assert e < TOL, (n, e)


def test_llama3_8b_layer_full(env):
    """Llama-3.1-8B-shaped layer at full size (1 x 8192 tokens), the calls the
    benchmark times: forward with a host checkpoint, then recompute + backward
    from that checkpoint. Sampled output rows against the fp64 oracle; y, dx
    and all nine weight gradients, every element, against the complete fp32
    oracle; the fused path (kept internals) gives the same bits as the
    recompute path."""
    B, Worker = env
    cfg = synth.config("llama3_8b")
    T, H, b, s = cfg.tokens, cfg.hidden, cfg.batch, cfg.seq
    say("llama3_8b layer full: run")
    lw = synth.layer_weights(cfg, 0, gamma="perturbed")
    x = synth.activation(cfg, "x")
    dy = synth.activation(cfg, "dy")
    wk = Worker(cfg)
    wk.add_layer(0, lw)
    ctx = wk.ctx
    bf = dict(dtype=torch.bfloat16, device=DEV)
    xd, dyd = x.to(DEV), dy.to(DEV)
    ck = [torch.empty(T, H, dtype=torch.bfloat16).pin_memory()]
    y, dx = torch.empty(T, H, **bf), torch.empty(T, H, **bf)
    ws_f = ctx.workspace(B.RP_OP_STAGE_FWD, b, s, 1)
    ws_b = ctx.workspace(B.RP_OP_STAGE_BWD, b, s, 1)
    ctx.stage_fwd(0, 1, b, s, xd, y, ws_f, ckpt_host=ck)
    ctx.stage_bwd_recompute(0, 1, b, s, dyd, dx, ws_b, ckpt=ck)
    ctx.sync()
    g_rc = wk.layers[0]["g"].clone()
    del ws_f, ws_b
    torch.cuda.empty_cache()
    say("llama3_8b layer full: fused path")
    y2, dx2 = torch.empty(T, H, **bf), torch.empty(T, H, **bf)
    ws = ctx.workspace(B.RP_OP_FUSED, b, s, 1)
    ctx.stage_fwd(0, 1, b, s, xd, y2, ws, flags=B.RP_KEEP_ACTS)
    ctx.stage_bwd_recompute(0, 1, b, s, dyd, dx2, ws, flags=B.RP_USE_KEPT_ACTS)
    ctx.sync()
    assert torch.equal(y, y2) and torch.equal(dx, dx2)
    assert torch.equal(g_rc, wk.layers[0]["g"])
    del ws
    torch.cuda.empty_cache()
    say("llama3_8b layer full: oracle rows")
    w64 = f64(lw)
    x64 = x.double()
    rows = sample_rows(T)
    y_ref = O.layer_forward_rows(x64, w64, cfg, rows)
    assert rel_rows(y.cpu()[rows], y_ref) < TOL
    say("llama3_8b layer full: complete fp32 oracle")
    got = {k: v.cpu() for k, v in wk.unpack_grads(wk.layers[0]["g"]).items()}
    y, dx = y.cpu(), dx.cpu()
    del wk, ctx
    torch.cuda.empty_cache()
    # the whole layer, fwd and bwd, in fp32 (the workload's gradient precision;
    # fp64 would need twice the host memory for the 32 T x T score matrices)
    dx_ref, g_ref, y_ref = O.layer_backward(x, lw, dy, cfg, dtype=torch.float32)
    for what, a, r in (("y", y, y_ref), ("dx", dx, dx_ref)):
        e = max_rel(a, r)
        say(f"llama3_8b complete {what}: max rel {e:.2e}")
        assert e < TOL, (what, e)
    for n, r in g_ref.items():
        e = max_rel(got[n], r)
        say(f"llama3_8b complete {n}: max rel {e:.2e}")
        assert e < TOL, (n, e)


def test_llama3_8b_lmhead_full(env):
    """LM head at full size: 8192 x 4096 activations, 128256 x 4096 weights in
    4 vocabulary shards, uniform labels. The mean cross-entropy exactly (fp64
    over every row), dx at sampled rows and dW at sampled vocabulary rows
    (every shard) against the oracle."""
    B, Worker = env
    cfg = synth.config("llama3_8b")
    T, H = cfg.tokens, cfg.hidden
    say("llama3_8b lm head full: run")
    x = synth.activation(cfg, "x")
    w = synth.lmhead_weights(cfg)["w"]
    labels = synth.uniform_labels(cfg)
    wk = Worker(cfg)
    wk.add_lmhead(w)
    dx = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    loss = torch.zeros(1, dtype=torch.float32, device=DEV)
    ws = wk.ctx.workspace(B.RP_OP_LMHEAD, cfg.batch, cfg.seq)
    wk.ctx.lmhead_ce_fwd_bwd(cfg.batch, cfg.seq, x.to(DEV), labels.to(DEV), loss, dx, ws)
    wk.ctx.sync()
    del ws
    torch.cuda.empty_cache()
    say("llama3_8b lm head full: oracle")
    rows = sample_rows(T)
    vrows = sorted(set(sample_rows(cfg.vocab, n=12, seed=2)) | {int(labels[5]), 32063, 32064, 96191, 96192})
    l_ref, dx_ref, dw_ref = O.lmhead_rows(x.double(), w.double(), labels, rows, vrows)
    assert abs(loss.item() - l_ref.item()) / abs(l_ref.item()) < LOSS_TOL["bf16"]
    assert max_rel(dx.cpu()[rows], dx_ref) < TOL
    dw = torch.cat([d.cpu() for d in wk.head["dw"]], dim=0)
    assert max_rel(dw[vrows], dw_ref) < TOL


def test_qwen3_32b_stage_full(env):
    """Qwen3-32B-shaped stage at full size (1 x 16384 tokens, hidden 5120,
    64/8 heads, FFN 25600): forward stage of layers 0-1, then the fused stage
    of layer 2 on its own input. Checks: the layer-1 input checkpoint (layer 0's
    output) at sampled rows; running [0, 2) as one stage or as [0, 1) + [1, 2)
    gives the same bits; the fused layer's sampled output rows and sampled MLP
    weight gradients; its kept and recomputed backward give the same bits."""
    B, Worker = env
    cfg = synth.config("qwen3_32b")
    T, H, b, s = cfg.tokens, cfg.hidden, cfg.batch, cfg.seq
    say("qwen3_32b full: forward stage")
    layers = [synth.layer_weights(cfg, l, gamma="perturbed") for l in range(3)]
    x = synth.activation(cfg, "x")
    x2 = synth.activation(cfg, "x2")
    dy = synth.activation(cfg, "dy")
    wk = Worker(cfg)
    for l in range(3):
        wk.add_layer(l, layers[l])
    ctx = wk.ctx
    bf = dict(dtype=torch.bfloat16, device=DEV)
    xd = x.to(DEV)
    ck = [torch.empty(T, H, dtype=torch.bfloat16).pin_memory() for _ in range(2)]
    y2 = torch.empty(T, H, **bf)
    ws_f = ctx.workspace(B.RP_OP_STAGE_FWD, b, s, 2)
    ctx.stage_fwd(0, 2, b, s, xd, y2, ws_f, ckpt_host=ck)
    mid, y2b = torch.empty(T, H, **bf), torch.empty(T, H, **bf)
    ctx.stage_fwd(0, 1, b, s, xd, mid, ws_f)
    ctx.stage_fwd(1, 2, b, s, mid, y2b, ws_f)
    ctx.sync()
    assert torch.equal(y2, y2b)
    assert torch.equal(ck[1], mid.cpu())
    del ws_f
    torch.cuda.empty_cache()
    say("qwen3_32b full: fused stage")
    x2d, dyd = x2.to(DEV), dy.to(DEV)
    y3, dx3 = torch.empty(T, H, **bf), torch.empty(T, H, **bf)
    ws = ctx.workspace(B.RP_OP_FUSED, b, s, 1)
    ctx.stage_fwd(2, 3, b, s, x2d, y3, ws, flags=B.RP_KEEP_ACTS)
    ctx.stage_bwd_recompute(2, 3, b, s, dyd, dx3, ws, flags=B.RP_USE_KEPT_ACTS)
    ctx.sync()
    g_kept = wk.layers[2]["g"].clone()
    del ws
    torch.cuda.empty_cache()
    dx3b = torch.empty(T, H, **bf)
    ws_b = ctx.workspace(B.RP_OP_STAGE_BWD, b, s, 1)
    ctx.stage_bwd_recompute(2, 3, b, s, dyd, dx3b, ws_b, ckpt=[x2d], flags=B.RP_CKPT_DEVICE)
    ctx.sync()
    assert torch.equal(dx3, dx3b)
    assert torch.equal(g_kept, wk.layers[2]["g"])
    del ws_b
    torch.cuda.empty_cache()
    say("qwen3_32b full: oracle rows")
    rows = sample_rows(T, n=6)
    l0 = f64(layers[0])
    ref = O.layer_forward_rows(x.double(), l0, cfg, rows)
    assert rel_rows(ck[1][rows], ref) < TOL
    l2 = f64(layers[2])
    ref3 = O.layer_forward_rows(x2.double(), l2, cfg, rows)
    assert rel_rows(y3.cpu()[rows], ref3) < TOL
    say("qwen3_32b full: oracle MLP gradients")
    bmat = mlp_input(x2.double(), l2, cfg)
    cols = sample_rows(cfg.ffn, n=8, seed=3)
    dwd, dwg, dwu = O.mlp_weight_grad_columns(bmat, dy.double(), l2, cols)
    got = wk.unpack_grads(wk.layers[2]["g"])
    assert max_rel(got["wd"][:, cols], dwd) < TOL
    assert max_rel(got["wg"][cols], dwg) < TOL
    assert max_rel(got["wu"][cols], dwu) < TOL


def test_qwen3_235b_moe_lora_stage_full(env):
    """Qwen3-235B-A22B-shaped MoE LoRA stage at full size (1 x 32768 tokens,
    128 experts top-8, expert FFN 1536, LoRA r16 alpha32 initialised B = 0,
    frozen base): forward keeping its internals, then backward. Sampled output
    rows against the oracle (routing on the same fp32 logits); dA exactly zero
    (B = 0); the kept and recomputed backward give the same bits."""
    B, Worker = env
    cfg = synth.config("qwen3_235b_moe")
    T, H, b, s = cfg.tokens, cfg.hidden, cfg.batch, cfg.seq
    say("qwen3_235b full: run")
    lw = synth.layer_weights(cfg, 0, gamma="perturbed")
    lora = synth.lora_weights(cfg, 0, b_zero=True)
    router = synth.router_logits(cfg, 0)
    x = synth.activation(cfg, "x")
    dy = synth.activation(cfg, "dy")
    wk = Worker(cfg)
    wk.add_layer(0, lw, lora=lora)
    ctx = wk.ctx
    bf = dict(dtype=torch.bfloat16, device=DEV)
    xd, dyd, rd = x.to(DEV), dy.to(DEV), router.to(DEV)
    y, dx = torch.empty(T, H, **bf), torch.empty(T, H, **bf)
    ws = ctx.workspace(B.RP_OP_FUSED, b, s, 1)
    ctx.stage_fwd(0, 1, b, s, xd, y, ws, router=[rd], flags=B.RP_KEEP_ACTS)
    ctx.stage_bwd_recompute(0, 1, b, s, dyd, dx, ws, flags=B.RP_USE_KEPT_ACTS)
    ctx.sync()
    g_kept = wk.layers[0]["lora_g"].clone()
    del ws
    torch.cuda.empty_cache()
    got = wk.unpack_lora_grads(wk.layers[0]["lora_g"])
    for n in ("aq", "ak", "av", "ao"):
        assert torch.count_nonzero(got[n]).item() == 0, n
    for n in ("bq", "bk", "bv", "bo"):
        assert torch.isfinite(got[n]).all() and torch.count_nonzero(got[n]).item() > 0, n
    say("qwen3_235b full: recompute path")
    dx2 = torch.empty(T, H, **bf)
    ws_b = ctx.workspace(B.RP_OP_STAGE_BWD, b, s, 1)
    ctx.stage_bwd_recompute(0, 1, b, s, dyd, dx2, ws_b, ckpt=[xd], router=[rd], flags=B.RP_CKPT_DEVICE)
    ctx.sync()
    assert torch.equal(dx, dx2)
    assert torch.equal(g_kept, wk.layers[0]["lora_g"])
    del ws_b
    torch.cuda.empty_cache()
    say("qwen3_235b full: oracle rows")
    rows = sample_rows(T, n=6)
    ref = O.layer_forward_rows(x.double(), f64(lw), cfg, rows, f64(lora), router.double())
    assert rel_rows(y.cpu()[rows], ref) < TOL


# ---------------------------------------------------------------------------
# complete gradients at full size: an upstream gradient that is zero outside
# a set of sampled token rows. Every kernel still runs over every row and
# tile at the benchmark's launch configuration; the exact oracle
# (layer_backward_rows) gives dx at every row and every weight gradient in
# full, so both are compared element by element.
# ---------------------------------------------------------------------------


def sparse_dy(cfg, n=16, seed=7):
    """dy with N(0, 1) rows at the sampled positions (tile edges, the first
    and last rows, random rows) and zeros elsewhere."""
    T, H = cfg.tokens, cfg.hidden
    rows = set(sample_rows(T, n=n, seed=seed)) | {127, 128, 255, 256, T - 129, T - 128}
    rows = sorted(r for r in rows if 0 <= r < T)
    dy_rows = synth.normal((len(rows), H), cfg.seed, "dy_rows", 1.0, dtype=torch.bfloat16)
    dy = torch.zeros(T, H, dtype=torch.bfloat16)
    dy[rows] = dy_rows
    return rows, dy_rows, dy


def check_grads(got, ref, what):
    for n, r in ref.items():
        e = max_rel(got[n], r)
        say(f"{what} {n}: max rel {e:.2e}")
        assert e < TOL, (what, n, e)


def test_llama3_8b_layer_full_grads_sparse_dy(env):
    """Llama-3.1-8B-shaped layer at 1 x 8192 tokens, the benchmark's calls
    (forward with a host checkpoint, recompute + backward from it): dx at all
    8192 rows and all nine weight gradients against the exact oracle."""
    B, Worker = env
    cfg = synth.config("llama3_8b")
    T, H, b, s = cfg.tokens, cfg.hidden, cfg.batch, cfg.seq
    say("llama3_8b sparse-dy: run")
    lw = synth.layer_weights(cfg, 0, gamma="perturbed")
    x = synth.activation(cfg, "x")
    rows, dy_rows, dy = sparse_dy(cfg)
    wk = Worker(cfg)
    wk.add_layer(0, lw)
    ctx = wk.ctx
    bf = dict(dtype=torch.bfloat16, device=DEV)
    xd, dyd = x.to(DEV), dy.to(DEV)
    ck = [torch.empty(T, H, dtype=torch.bfloat16).pin_memory()]
    y, dx = torch.empty(T, H, **bf), torch.empty(T, H, **bf)
    ws_f = ctx.workspace(B.RP_OP_STAGE_FWD, b, s, 1)
    ws_b = ctx.workspace(B.RP_OP_STAGE_BWD, b, s, 1)
    ctx.stage_fwd(0, 1, b, s, xd, y, ws_f, ckpt_host=ck)
    ctx.stage_bwd_recompute(0, 1, b, s, dyd, dx, ws_b, ckpt=ck)
    ctx.sync()
    got = {k: v.cpu() for k, v in wk.unpack_grads(wk.layers[0]["g"]).items()}
    dx = dx.cpu()
    del ws_f, ws_b, wk, ctx
    torch.cuda.empty_cache()
    say("llama3_8b sparse-dy: oracle")
    dx_ref, g_ref = O.layer_backward_rows(x.double(), f64(lw), rows, dy_rows.double(), cfg)
    e = max_rel(dx, dx_ref)
    say(f"llama3_8b sparse-dy dx: max rel {e:.2e}")
    assert e < TOL
    check_grads(got, g_ref, "llama3_8b sparse-dy")


def test_qwen3_32b_layer_full_grads_sparse_dy(env):
    """Qwen3-32B-shaped fused stage at 1 x 16384 tokens (64/8 heads, FFN
    25600): forward keeping its internals, then backward. dx at all 16384 rows
    and all nine weight gradients against the exact oracle."""
    B, Worker = env
    cfg = synth.config("qwen3_32b")
    T, H, b, s = cfg.tokens, cfg.hidden, cfg.batch, cfg.seq
    say("qwen3_32b sparse-dy: run")
    lw = synth.layer_weights(cfg, 2, gamma="perturbed")
    x = synth.activation(cfg, "x2")
    rows, dy_rows, dy = sparse_dy(cfg)
    wk = Worker(cfg)
    wk.add_layer(2, lw)
    ctx = wk.ctx
    bf = dict(dtype=torch.bfloat16, device=DEV)
    xd, dyd = x.to(DEV), dy.to(DEV)
    y, dx = torch.empty(T, H, **bf), torch.empty(T, H, **bf)
    ws = ctx.workspace(B.RP_OP_FUSED, b, s, 1)
    ctx.stage_fwd(2, 3, b, s, xd, y, ws, flags=B.RP_KEEP_ACTS)
    ctx.stage_bwd_recompute(2, 3, b, s, dyd, dx, ws, flags=B.RP_USE_KEPT_ACTS)
    ctx.sync()
    got = {k: v.cpu() for k, v in wk.unpack_grads(wk.layers[2]["g"]).items()}
    dx = dx.cpu()
    del ws, wk, ctx
    torch.cuda.empty_cache()
    say("qwen3_32b sparse-dy: oracle")
    dx_ref, g_ref = O.layer_backward_rows(x.double(), f64(lw), rows, dy_rows.double(), cfg)
    e = max_rel(dx, dx_ref)
    say(f"qwen3_32b sparse-dy dx: max rel {e:.2e}")
    assert e < TOL
    check_grads(got, g_ref, "qwen3_32b sparse-dy")


def test_qwen3_235b_moe_lora_full_grads_sparse_dy(env):
    """Qwen3-235B-A22B-shaped MoE LoRA stage at 1 x 32768 tokens with
    adapters B ~ N(0, 0.02) (so every adapter gradient carries signal):
    fused forward + backward, dx at all 32768 rows and all eight adapter
    gradients against the exact oracle (routing on the same fp32 logits)."""
    B, Worker = env
    cfg = synth.config("qwen3_235b_moe")
    T, H, b, s = cfg.tokens, cfg.hidden, cfg.batch, cfg.seq
    say("qwen3_235b sparse-dy: run")
    lw = synth.layer_weights(cfg, 0, gamma="perturbed")
    lora = synth.lora_weights(cfg, 0, b_zero=False)
    router = synth.router_logits(cfg, 0)
    x = synth.activation(cfg, "x")
    rows, dy_rows, dy = sparse_dy(cfg)
    wk = Worker(cfg)
    wk.add_layer(0, lw, lora=lora)
    ctx = wk.ctx
    bf = dict(dtype=torch.bfloat16, device=DEV)
    xd, dyd, rd = x.to(DEV), dy.to(DEV), router.to(DEV)
    y, dx = torch.empty(T, H, **bf), torch.empty(T, H, **bf)
    ws = ctx.workspace(B.RP_OP_FUSED, b, s, 1)
    ctx.stage_fwd(0, 1, b, s, xd, y, ws, router=[rd], flags=B.RP_KEEP_ACTS)
    ctx.stage_bwd_recompute(0, 1, b, s, dyd, dx, ws, flags=B.RP_USE_KEPT_ACTS)
    ctx.sync()
    got = {k: v.cpu() for k, v in wk.unpack_lora_grads(wk.layers[0]["lora_g"]).items()}
    dx = dx.cpu()
    del ws, wk, ctx
    torch.cuda.empty_cache()
    say("qwen3_235b sparse-dy: oracle")
    # the kernels take the adapters rounded to bf16 once per call; so does the oracle
    lora_b = {k: v.to(torch.bfloat16).double() for k, v in lora.items()}
    dx_ref, g_ref = O.layer_backward_rows(x.double(), f64(lw), rows, dy_rows.double(), cfg, lora_b,
                                          router.double())
    e = max_rel(dx, dx_ref)
    say(f"qwen3_235b sparse-dy dx: max rel {e:.2e}")
    assert e < TOL
    check_grads(got, g_ref, "qwen3_235b sparse-dy")
