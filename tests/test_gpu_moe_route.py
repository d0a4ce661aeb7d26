"""MoE routing on the GPU through rp_op_moe_route, its integer outputs bit
for bit: the selected experts (value descending, equal logits lower index
first), the per-expert counts and first rows, and the grouped order (a stable
counting sort of the (token, slot) pairs by expert) with its inverse. The
top-k routing is the MoE layer of the paperlayer.ai summary, appendix C.2.
Logits are quantised to a few values so that ties at the top-k boundary are
common; the weights (a float softmax) are compared within fp32 rounding."""
import numpy as np
import pytest
import torch

import synth
from oracle import stage as O
from _helpers import ensure_built, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")


@pytest.fixture(scope="module")
def B():
    return ensure_built()


def grouped_order(idx: torch.Tensor, E: int):
    """Stable sort of the flattened (token, slot) pairs by expert: counts,
    first rows, the token of each grouped row and the grouped row of each pair."""
    flat = idx.reshape(-1).numpy()
    k = idx.shape[1]
    order = np.argsort(flat, kind="stable")
    cnt = np.bincount(flat, minlength=E)
    off = np.concatenate([[0], np.cumsum(cnt)])
    inv = np.empty_like(order)
    inv[order] = np.arange(order.size)
    return (torch.from_numpy(cnt.astype(np.int32)), torch.from_numpy(off.astype(np.int32)),
            torch.from_numpy((order // k).astype(np.int32)), torch.from_numpy(inv.astype(np.int32)), order)


def route_on_gpu(B, E, k, T, logits):
    cfg = synth.StageConfig(name="route", hidden=256, n_q=2, n_kv=1, head_dim=128, ffn=0, batch=1, seq=T,
                            dtype="bf16", n_experts=E, top_k=k, expert_ffn=64)
    ctx = B.Context(cfg)
    i32 = dict(dtype=torch.int32, device=DEV)
    f32 = dict(dtype=torch.float32, device=DEV)
    out = dict(idx=torch.full((T, k), -7, **i32), wgt=torch.full((T, k), float("nan"), **f32),
               cnt=torch.full((E,), -7, **i32), off=torch.full((E + 1,), -7, **i32),
               perm_row=torch.full((T * k,), -7, **i32), perm_w=torch.full((T * k,), float("nan"), **f32),
               inv=torch.full((T * k,), -7, **i32))
    ws = ctx.workspace(B.RP_OP_MOE_ROUTE, 1, T)
    ctx.op_moe_route(1, T, logits.to(DEV), out["idx"], out["wgt"], out["cnt"], out["off"], out["perm_row"],
                     out["perm_w"], out["inv"], ws)
    ctx.sync()
    res = {n: t.cpu() for n, t in out.items()}
    ctx.close()
    return res


def tied_logits(T, E, seed):
    """N(0, 4) rounded to integers, then quartered: steps of 1/4, a few dozen
    distinct values per row, so the k-th and (k+1)-th largest often tie; plus
    rows that are all equal and a row with more tied leaders than k."""
    z = torch.round(synth.normal((T, E), seed, "tied", 2.0)) / 4.0
    z[0] = 0.0                     # all equal: experts 0 .. k-1
    z[1] = 1.0
    z[2, :] = -1.0
    z[2, E - 1] = 3.0
    z[2, E // 2:E // 2 + 20] = 2.0  # more tied leaders than k
    return z


CASES = [
    # experts, top_k, tokens, logits
    (128, 8, 32768, "tied"),       # the 235B-A22B-shaped stage's routing, full token count
    (128, 8, 32768, "workload"),   # its N(0, 1) logits
    (8, 2, 1100, "tied"),          # small, ragged against the kernels' tiles
    (256, 16, 300, "tied"),        # the largest expert count and top-k the kernels take
    (3, 3, 5, "tied"),             # k = E: every expert, weights a full softmax
]


@pytest.mark.parametrize("E,k,T,kind", CASES)
def test_moe_route_bit_exact(B, E, k, T, kind):
    say("moe route", E, k, T, kind)
    if kind == "tied":
        logits = tied_logits(T, E, 100 + E + k)
    else:
        cfg = synth.config("qwen3_235b_moe")
        assert (cfg.n_experts, cfg.top_k, cfg.tokens) == (E, k, T)
        logits = synth.router_logits(cfg, 0)
    got = route_on_gpu(B, E, k, T, logits)
    idx_ref, w_ref = O.topk_route(logits.double(), k)
    n_ties = int((logits.double().gather(1, idx_ref[:, -1:]) == logits.double()).sum() - T)
    say(f"  rows x candidates tied with the k-th value beyond itself: {n_ties}")
    if kind == "tied":
        assert n_ties > T // 10
    assert torch.equal(got["idx"], idx_ref.to(torch.int32))
    cnt, off, perm_row, inv, order = grouped_order(idx_ref, E)
    assert torch.equal(got["cnt"], cnt)
    assert torch.equal(got["off"], off)
    assert torch.equal(got["perm_row"], perm_row)
    assert torch.equal(got["inv"], inv)
    # the weights: fp32 softmax of the selected logits vs fp64
    assert (got["wgt"].double() - w_ref).abs().max().item() < 1e-6
    assert torch.equal(got["perm_w"], got["wgt"].reshape(-1)[torch.from_numpy(order)])
    # tied selections get equal weights, bit for bit
    sel = logits.gather(1, idx_ref)
    same = sel[:, :, None] == sel[:, None, :]
    wg = got["wgt"]
    assert torch.equal((wg[:, :, None] == wg[:, None, :]) | ~same, torch.ones_like(same))
