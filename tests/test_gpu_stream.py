"""Weight streaming and the ABI's error paths on the GPU: weights uploaded
from pinned host memory through gated transfer windows give bit-identical
results to resident weights; gradients downloaded to pinned host memory equal
the device copies; bad arguments are rejected before anything is enqueued."""
import pytest
import torch

import synth
from _helpers import ensure_built, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")


@pytest.fixture(scope="module")
def env():
    B = ensure_built()
    from offloaded_pipeline_stage_amd.worker import Worker
    return B, Worker


def _small_cfg():
    return synth.config("qwen3_1p7b", seq=128, hidden=512, n_q=4, n_kv=2, ffn=1024)


def test_streamed_weights_and_grad_download_bit_identical(env):
    B, Worker = env
    say("weight streaming")
    cfg = _small_cfg()
    layers = [synth.layer_weights(cfg, l, gamma="perturbed") for l in range(2)]
    x = synth.activation(cfg, "x")
    dy = synth.activation(cfg, "dy")
    T, H, b, s = cfg.tokens, cfg.hidden, cfg.batch, cfg.seq
    bf = dict(dtype=torch.bfloat16, device=DEV)

    def run(wk, xd, dyd):
        ws = wk.ctx.workspace(B.RP_OP_FUSED, b, s, 2)
        y, dx = torch.empty(T, H, **bf), torch.empty(T, H, **bf)
        wk.ctx.stage_fwd(0, 2, b, s, xd, y, ws, flags=B.RP_KEEP_ACTS)
        wk.ctx.stage_bwd_recompute(0, 2, b, s, dyd, dx, ws, flags=B.RP_USE_KEPT_ACTS)
        return y, dx

    ref = Worker(cfg)
    for l in range(2):
        ref.add_layer(l, layers[l])
    y_ref, dx_ref = run(ref, x.to(DEV), dy.to(DEV))
    ref.ctx.sync()

    wk = Worker(cfg)
    host = [wk.pack_layer(layers[l], pinned=True) for l in range(2)]
    for l in range(2):
        wk.add_layer(l, resident=False)
    # activation uploads first; parameter window w is gated behind activation
    # ticket t0 + w (window 0 behind x, window 1 behind dy, window 2 behind a
    # third copy)
    x_host, dy_host = x.pin_memory(), dy.pin_memory()
    x_dev, dy_dev = torch.empty(T, H, **bf), torch.empty(T, H, **bf)
    t0 = wk.ctx.act_copy(B.RP_H2D, x_dev, x_host)
    items = [(B.RP_PARAM_H2D, B.RP_TGT_LAYER, l, 0, wk.w_bytes, host[l]) for l in range(2)]
    wk.ctx.weight_stream_submit(items, n_windows=3, max_chunk=1 << 20, gate_ticket=t0)
    wk.ctx.act_copy(B.RP_H2D, dy_dev, dy_host)
    mark_h = torch.zeros(256, dtype=torch.uint8).pin_memory()
    mark_d = torch.empty(256, dtype=torch.uint8, device=DEV)
    wk.ctx.act_copy(B.RP_H2D, mark_d, mark_h)
    y, dx = run(wk, x_dev, dy_dev)
    gh = [torch.empty(wk.g_bytes, dtype=torch.uint8).pin_memory() for _ in range(2)]
    wk.ctx.weight_stream_submit([(B.RP_GRAD_D2H, B.RP_TGT_LAYER, l, 0, wk.g_bytes, gh[l]) for l in range(2)],
                                n_windows=2)
    wk.ctx.sync()
    assert torch.equal(y, y_ref) and torch.equal(dx, dx_ref)
    for l in range(2):
        assert torch.equal(wk.layers[l]["w"].cpu(), host[l])
        assert torch.equal(gh[l], wk.layers[l]["g"].cpu())
        assert torch.equal(gh[l], ref.layers[l]["g"].cpu())


def test_grad_download_chunked_and_unaligned_paths(env):
    """Gradient downloads (by DMA) of an aligned block in chunks over three
    windows and of a range at a host address 8 bytes past a boundary with a
    ragged size: both must reproduce the device bytes exactly, and leave the
    host bytes around them untouched."""
    B, Worker = env
    say("download paths")
    cfg = _small_cfg()
    wk = Worker(cfg)
    wk.add_layer(0, synth.layer_weights(cfg, 0))
    g = wk.layers[0]["g"].view(torch.uint8)
    gb = wk.g_bytes
    gen = torch.Generator().manual_seed(7)
    g[:gb].copy_(torch.randint(0, 256, (gb,), dtype=torch.uint8, generator=gen).to(DEV))
    torch.cuda.synchronize()
    h_al = torch.zeros(gb, dtype=torch.uint8).pin_memory()
    h_mis = torch.zeros(gb + 64, dtype=torch.uint8).pin_memory()
    off, nb = 4096, 123457  # device offset and a size that is not a multiple of 16
    wk.ctx.weight_stream_submit([(B.RP_GRAD_D2H, B.RP_TGT_LAYER, 0, 0, gb, h_al)], n_windows=3, max_chunk=1 << 16)
    wk.ctx.weight_stream_submit([(B.RP_GRAD_D2H, B.RP_TGT_LAYER, 0, off, nb, h_mis.data_ptr() + 8)],
                                n_windows=2, max_chunk=1 << 14)
    wk.ctx.sync()
    dev = g[:gb].cpu()
    assert torch.equal(h_al, dev)
    assert torch.equal(h_mis[8:8 + nb], dev[off:off + nb])
    assert not h_mis[:8].any() and not h_mis[8 + nb:].any()


def test_bf16_grad_download_rounds_to_nearest_even(env):
    """RP_GRAD_D2H_BF16 (the pages' low-precision gradients on the link): an
    fp32 gradient block downloaded in chunks over three windows, and a range
    inside it, arrive as the fp32 values rounded to nearest even (torch's
    rounding) -- ties, tiny values, infinities and NaN included -- and the host
    bytes around the range stay untouched. Misaligned ranges are rejected."""
    B, Worker = env
    say("bf16 gradient download")
    cfg = _small_cfg()
    wk = Worker(cfg)
    wk.add_layer(0, synth.layer_weights(cfg, 0))
    gb = wk.g_bytes
    n = gb // 4
    gen = torch.Generator().manual_seed(11)
    vals = torch.randn(n, generator=gen) * 3
    specials = torch.tensor([1.00390625, 1.01171875, -1.00390625, 1e-30, -3e-35, float("inf"), float("-inf"),
                             65504.0, 3.3895314e38, 0.0, -0.0])
    vals[:specials.numel()] = specials
    g = wk.layers[0]["g"].view(torch.float32)
    g[:n].copy_(vals.to(DEV))
    torch.cuda.synchronize()
    h = torch.zeros(n, dtype=torch.bfloat16).pin_memory()
    off, nb = 4096, 32 * 1000
    h2 = torch.zeros(nb // 4 + 64, dtype=torch.bfloat16).pin_memory()
    wk.ctx.weight_stream_submit([(B.RP_GRAD_D2H_BF16, B.RP_TGT_LAYER, 0, 0, gb, h)], n_windows=3, max_chunk=1 << 16)
    wk.ctx.weight_stream_submit([(B.RP_GRAD_D2H_BF16, B.RP_TGT_LAYER, 0, off, nb, h2.data_ptr() + 64)],
                                n_windows=2, max_chunk=1 << 12)
    wk.ctx.sync()
    ref = vals.to(torch.bfloat16)
    assert torch.equal(h.view(torch.int16), ref.view(torch.int16))
    seg = h2[32:32 + nb // 4]
    assert torch.equal(seg.view(torch.int16), ref[off // 4:off // 4 + nb // 4].view(torch.int16))
    assert not h2[:32].view(torch.int16).any() and not h2[32 + nb // 4:].view(torch.int16).any()
    nan = torch.tensor([float("nan")])
    g[:1].copy_(nan.to(DEV))
    torch.cuda.synchronize()
    wk.ctx.weight_stream_submit([(B.RP_GRAD_D2H_BF16, B.RP_TGT_LAYER, 0, 0, 32, h)])
    wk.ctx.sync()
    assert torch.isnan(h[:1].float()).all()
    with pytest.raises(B.RPError):
        wk.ctx.weight_stream_submit([(B.RP_GRAD_D2H_BF16, B.RP_TGT_LAYER, 0, 16, 64, h)])


def test_deferred_window_waits_for_its_ticket(env):
    B, Worker = env
    say("deferred window")
    cfg = _small_cfg()
    wk = Worker(cfg)
    wk.add_layer(0, resident=False)
    host = wk.pack_layer(synth.layer_weights(cfg, 0), pinned=True)
    # gate on a ticket that has not been issued yet: the stage call refuses
    wk.ctx.weight_stream_submit([(B.RP_PARAM_H2D, B.RP_TGT_LAYER, 0, 0, wk.w_bytes, host)], gate_ticket=5)
    T, H = cfg.tokens, cfg.hidden
    x = torch.zeros(T, H, dtype=torch.bfloat16, device=DEV)
    y = torch.empty_like(x)
    ws = wk.ctx.workspace(B.RP_OP_STAGE_FWD, cfg.batch, cfg.seq, 1)
    with pytest.raises(B.RPError) as e:
        wk.ctx.stage_fwd(0, 1, cfg.batch, cfg.seq, x, y, ws)
    assert e.value.status == B.RP_ERR_STATE
    # issuing tickets 0..5 releases the window
    hx = torch.zeros(16, dtype=torch.uint8).pin_memory()
    dx = torch.zeros(16, dtype=torch.uint8, device=DEV)
    for _ in range(6):
        wk.ctx.act_copy(B.RP_H2D, dx, hx)
    wk.ctx.stage_fwd(0, 1, cfg.batch, cfg.seq, x, y, ws)
    wk.ctx.sync()
    assert torch.equal(wk.layers[0]["w"].cpu(), host)


def test_activation_download_unaligned_and_ragged(env):
    """Activation downloads (by DMA) into pinned host memory at an address 8
    bytes past a boundary with a size that is not a multiple of 16, and into
    an aligned buffer: the host bytes equal the device bytes, the bytes
    around them stay untouched, and the download's ticket orders a later
    upload of the same host bytes."""
    B, Worker = env
    say("activation download paths")
    cfg = _small_cfg()
    wk = Worker(cfg)
    n = 200001
    gen = torch.Generator().manual_seed(11)
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, generator=gen).to(DEV)
    back = torch.empty(n, dtype=torch.uint8, device=DEV)
    torch.cuda.synchronize()
    host = torch.full((n + 64,), 0xA5, dtype=torch.uint8).pin_memory()
    al = torch.zeros(n, dtype=torch.uint8).pin_memory()
    t0 = wk.ctx.act_copy(B.RP_D2H, host[8:8 + n], src)
    t1 = wk.ctx.act_copy(B.RP_D2H, al, src)
    wk.ctx.act_wait(B.RP_ON_ACT_H2D, t1)
    wk.ctx.act_copy(B.RP_H2D, back, al)
    wk.ctx.sync()
    ref = src.cpu()
    assert t1 == t0 + 1
    assert torch.equal(host[8:8 + n], ref)
    assert torch.all(host[:8] == 0xA5) and torch.all(host[8 + n:] == 0xA5)
    assert torch.equal(al, ref)
    assert torch.equal(back.cpu(), ref)


def test_error_paths(env):
    B, Worker = env
    say("error paths")
    cfg = _small_cfg()
    wk = Worker(cfg)
    wk.add_layer(0, synth.layer_weights(cfg, 0))
    T, H, b, s = cfg.tokens, cfg.hidden, cfg.batch, cfg.seq
    x = torch.zeros(T, H, dtype=torch.bfloat16, device=DEV)
    y = torch.empty_like(x)
    small = torch.empty(1024, dtype=torch.uint8, device=DEV)
    with pytest.raises(B.RPError) as e:
        wk.ctx.stage_fwd(0, 1, b, s, x, y, small)
    assert e.value.status == B.RP_ERR_WORKSPACE
    ws = wk.ctx.workspace(B.RP_OP_FUSED, b, s, 1)
    with pytest.raises(B.RPError) as e:
        wk.ctx.stage_bwd_recompute(0, 1, b, s, x, y, ws, flags=B.RP_USE_KEPT_ACTS)
    assert e.value.status == B.RP_ERR_STATE
    pageable = torch.zeros(T, H, dtype=torch.bfloat16)
    with pytest.raises(B.RPError) as e:
        wk.ctx.act_copy(B.RP_D2H, pageable, x)
    assert e.value.status == B.RP_ERR_NOT_PINNED
    with pytest.raises(B.RPError) as e:
        wk.ctx.stage_fwd(0, 2, b, s, x, y, ws)  # layer 1 not bound
    assert e.value.status == B.RP_ERR_INVALID
    with pytest.raises(B.RPError) as e:
        wk.ctx.stage_fwd(0, 1, b, s, x, x, ws)  # output aliases input
    assert e.value.status == B.RP_ERR_INVALID
    wk.ctx.sync()


@pytest.mark.parametrize("side", [False, True])
def test_calls_ordered_after_torch_stream(env, side):
    """torch writes a stage call's input late on its current stream (a bounded
    sleep kernel ahead of the write), and the call follows with no
    synchronisation in between: it must read the written values. On the
    default stream the library's blocking streams give the order (and torch's
    next default-stream write waits for the call's reads); on another stream
    the binding's event does."""
    B, Worker = env
    say("stream order", "side stream" if side else "default stream")
    cfg = _small_cfg()
    wk = Worker(cfg)
    wk.add_layer(0, synth.layer_weights(cfg, 0, gamma="perturbed"))
    ctx = wk.ctx
    T, H, b, s = cfg.tokens, cfg.hidden, cfg.batch, cfg.seq
    x_val = synth.activation(cfg, "x").to(DEV)
    ws = ctx.workspace(B.RP_OP_STAGE_FWD, b, s, 1)
    y_ref = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    torch.cuda.synchronize()
    ctx.stage_fwd(0, 1, b, s, x_val, y_ref, ws)
    ctx.sync()
    x = torch.zeros_like(x_val)
    y = torch.zeros_like(y_ref)
    torch.cuda.synchronize()
    st = torch.cuda.Stream() if side else torch.cuda.default_stream()
    with torch.cuda.stream(st):
        torch.cuda._sleep(50_000_000)  # tens of milliseconds
        x.copy_(x_val)
        ctx.stage_fwd(0, 1, b, s, x, y, ws)
        if not side:
            x.zero_()  # waits for the call's reads of x
    ctx.sync()
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
