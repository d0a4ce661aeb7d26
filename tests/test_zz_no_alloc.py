"""rp_op_attn_bwd_noalloc, the attention backward for callers that cannot
allocate device memory, against rp_op_attn_bwd (workspace from the caller):
two calls in a row on one context, the second on a smaller input, each
bit-identical to the workspace path. Sizes beyond the fixed scratch are
rejected before anything is enqueued."""
import pytest
import torch

import synth
from _helpers import ensure_built, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    return ensure_built()


def _case(B, ctx, cfg, batch, seq, tag):
    nq, nkv, d = cfg.n_q, cfg.n_kv, cfg.head_dim
    T, W = batch * seq, (nq + 2 * nkv) * d
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    dev = torch.device("cuda")
    qkv = synth.normal((T, W), 9, f"na_qkv_{tag}", dtype=dt).to(dev)
    dout = synth.normal((T, nq * d), 9, f"na_do_{tag}", dtype=dt).to(dev)
    o = torch.empty(T, nq * d, dtype=dt, device=dev)
    lse = torch.empty(nq, T, dtype=torch.float32, device=dev)
    ctx.op_attn_fwd(batch, seq, qkv, o, lse)
    ref = torch.full((T, W), float("nan"), dtype=dt, device=dev)
    ws = ctx.workspace(B.RP_OP_STAGE_BWD, batch, seq, 1)
    ctx.op_attn_bwd(batch, seq, qkv, o, dout, lse, ref, ws)
    got = torch.full((T, W), float("nan"), dtype=dt, device=dev)
    ctx.op_attn_bwd_noalloc(batch, seq, qkv, o, dout, lse, got)
    ctx.sync()
    return got, ref


@pytest.mark.parametrize("dtype,d,nq,nkv", [("bf16", 128, 8, 2), ("f32", 64, 4, 2)])
def test_attn_bwd_noalloc_matches_workspace_path(B, dtype, d, nq, nkv):
    cfg = synth.StageConfig(name="na", hidden=max(256, nq * d), n_q=nq, n_kv=nkv, head_dim=d, ffn=512,
                            batch=1, seq=64, dtype=dtype)
    ctx = B.Context(cfg)
    for batch, seq in ((2, 700), (1, 300)):
        say("attn bwd noalloc", dtype, d, nq, nkv, batch, seq)
        got, ref = _case(B, ctx, cfg, batch, seq, f"{dtype}{batch}x{seq}")
        assert torch.isfinite(ref.float()).all()
        assert torch.equal(got, ref)
    # beyond the fixed scratch: rejected on the host, nothing enqueued
    big_seq = (1 << 21) // nq + 1
    dummy = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(B.RPError) as e:
        ctx.op_attn_bwd_noalloc(1, big_seq, dummy, dummy, dummy, dummy, dummy)
    assert e.value.status == B.RP_ERR_UNSUPPORTED
    ctx.sync()
    ctx.close()
