"""C-ABI checks that need no GPU: the library loads, exports every function
include/rp.h declares, and its pure host functions (block layout, transfer
planner) agree with the oracle bit for bit."""
import os
import random
import re
import subprocess

import pytest

import synth
from oracle import sched as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rp.h")


@pytest.fixture(scope="module")
def B():
    from offloaded_pipeline_stage_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from offloaded_pipeline_stage_amd import build
        build.build(verbose=False)
    binding.lib()
    return binding


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rp_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_stage_calls():
    fns = header_functions()
    for need in ("rp_stage_fwd", "rp_stage_bwd_recompute", "rp_lmhead_ce_fwd_bwd", "rp_weight_stream_submit"):
        assert need in fns


def test_library_exports_every_declared_function(B):
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (rp_[a-z0-9_]+)\b", out))
    missing = [f for f in header_functions() if f not in exported]
    assert not missing, missing
    # the binding declares exactly the header's functions
    assert sorted(B.EXPORTS) == header_functions()


def test_status_strings(B):
    lib = B.lib()
    assert lib.rp_status_string(B.RP_OK) == b"RP_OK"
    assert lib.rp_status_string(B.RP_ERR_NOT_PINNED) == b"RP_ERR_NOT_PINNED"
    assert lib.rp_version().startswith(b"roundpipe")


@pytest.mark.parametrize("name", ["tiny", "qwen3_1p7b", "llama3_8b", "qwen3_32b"])
def test_block_layout_is_aligned_and_disjoint(B, name):
    cfg = synth.config(name)
    H, Q, KV, F = cfg.hidden, cfg.q_dim, cfg.kv_dim, cfg.ffn
    es = 2 if cfg.dtype == "bf16" else 4
    expect = {B.RP_T_GAMMA1: H, B.RP_T_WQKV: (Q + 2 * KV) * H, B.RP_T_WO: H * Q, B.RP_T_GAMMA2: H,
              B.RP_T_WGU: 2 * F * H, B.RP_T_WD: H * F}
    for block, size in ((B.RP_BLOCK_WEIGHT, es), (B.RP_BLOCK_GRAD, 4)):
        spans = []
        for tid, n in expect.items():
            off, nb, tot = B.block_layout(cfg, block, tid)
            assert off % 256 == 0 and nb == n * size
            spans.append((off, off + nb))
        spans.sort()
        assert all(a[1] <= b[0] for a, b in zip(spans, spans[1:]))
        assert tot >= spans[-1][1] and tot % 256 == 0
    # the paper-scale sizes: Llama-3.1-8B layer = 218.1M parameters
    if name == "llama3_8b":
        n = sum(expect.values())
        assert n == 218_112_000


def test_planner_matches_oracle_bit_for_bit(B):
    rng = random.Random(99)
    for _ in range(300):
        n = rng.randint(0, 9)
        sizes = [rng.choice([rng.randint(1, 5000), rng.randint(1, 10 ** 9)]) for _ in range(n)]
        nw = rng.randint(1, 6)
        cap = rng.choice([0, 0, rng.randint(1000, 10 ** 8)])
        align = rng.choice([1, 256, 4096])
        got = B.xfer_plan(sizes, nw, cap, align)
        chunks = S.split_items(sizes, nw, align=align, max_chunk=cap)
        win = S.lpt_assign([c[2] for c in chunks], nw)
        expect = [(c[0], c[1], c[2], w) for c, w in zip(chunks, win)]
        assert got == expect


def test_planner_layer_blocks_into_windows(B):
    # an 8B-shaped layer block + the 4 LM-head shards over 4 windows: LPT keeps
    # the windows within Graham's bound of the even split
    cfg = synth.config("llama3_8b")
    sizes = [B.block_bytes(cfg, B.RP_BLOCK_WEIGHT)] + [32064 * 4096 * 2] * 4
    plan = B.xfer_plan(sizes, 4)
    load = [0] * 4
    for _, _, nb, w in plan:
        load[w] += nb
    assert sum(load) == sum(sizes)
    assert max(load) <= (4 / 3) * (sum(sizes) / 4) + max(nb for _, _, nb, _ in plan)


@pytest.mark.skipif(__import__("torch").cuda.is_available(), reason="checks the no-GPU error path")
def test_ctx_create_without_gpu_fails_cleanly(B):
    import ctypes as C
    cfg = B.make_cfg(synth.config("tiny"))
    h = C.c_void_p()
    st = B.lib().rp_ctx_create(0, C.byref(cfg), None, C.byref(h))
    assert st in (B.RP_ERR_HIP, B.RP_ERR_INVALID)
    assert not h.value


def test_microbatch_window_gates():
    """Window j of a stage's transfers is gated on the last activation upload
    of micro-batch j + 1 (the last micro-batch for the final window), with
    tickets numbered in the order the stage issues its copies."""
    from offloaded_pipeline_stage_amd.microbatch import MicrobatchPass
    # forward stage, M = 3: up x0 (t0), [fwd 0], up x1 (t0+1), down y0 (t0+2),
    # [fwd 1], up x2 (t0+3), down y1 (t0+4), [fwd 2], down y2 (t0+5)
    fwd = [("h2d", 0), ("compute", 0), ("h2d", 1), ("d2h", 0), ("compute", 1), ("h2d", 2), ("d2h", 1),
           ("compute", 2), ("d2h", 2)]
    ops = [(k, None, None, j) if k != "compute" else (k, j) for k, j in fwd]
    assert MicrobatchPass.window_gates(ops, 10, 3) == [11, 13, 13]
    # backward stage, M = 2: two uploads (checkpoint, dy) per micro-batch
    bwd = [("h2d", 0), ("h2d", 0), ("compute", 0), ("h2d", 1), ("h2d", 1), ("d2h", 0), ("compute", 1),
           ("d2h", 1)]
    ops = [(k, None, None, j) if k != "compute" else (k, j) for k, j in bwd]
    assert MicrobatchPass.window_gates(ops, 0, 2) == [3, 3]
    # one micro-batch: the single window follows its upload
    assert MicrobatchPass.window_gates([("h2d", None, None, 0), ("compute", 0), ("d2h", None, None, 0)], 5, 1) == [5]


def test_partition_matches_oracle_greedy_and_exhaustive(B):
    """rp_partition (section 4.4) against the oracle: the same partition as the
    oracle's statement of the greedy, and the optimum of an exhaustive search
    over every contiguous partition (integer and real-valued times)."""
    rng = random.Random(4321)
    n_ok = 0
    for it in range(300):
        L = rng.randint(1, 7)
        if it % 2:
            f = [rng.randint(1, 9) for _ in range(L)]
            b = [max(1, 3 * x + rng.randint(-2, 2)) for x in f]
            h = rng.randint(1, 25)
        else:
            f = [rng.uniform(0.5, 9.0) for _ in range(L)]
            b = [3.0 * x + rng.uniform(-1.0, 1.0) for x in f]
            h = rng.uniform(1.0, 25.0)
        mf = [rng.randint(1, 5) for _ in range(L)]
        mb = [rng.randint(1, 8) for _ in range(L)]
        mh = rng.randint(1, 8)
        cap = rng.randint(8, 30)
        M, N = rng.randint(1, 16), rng.randint(1, 8)
        e = S.partition_exhaustive(f, b, h, mf, mb, mh, cap, M, N)
        g = S.partition_greedy(f, b, h, mf, mb, mh, cap, M, N)
        if e is None:
            with pytest.raises(B.RPError):
                B.partition(f, b, h, mf, mb, mh, cap, M, N)
            continue
        n_ok += 1
        got = B.partition(f, b, h, mf, mb, mh, cap, M, N)
        assert got == (g[0], tuple(g[1]), g[2], tuple(g[3]))
        assert abs(got[0] - e[0]) <= 1e-9 * e[0]
    assert n_ok > 200


def test_partition_fills_fused_stage_and_rejects_bad_input(B):
    # eight equal layers, LM head = one backward: B_1 holds two layers
    assert B.partition([1.0] * 8, [3.0] * 8, 3.0, [1.0] * 8, [1.0] * 8, 1.0, 100.0, 16, 4) == \
        ((16 * 4 + 12) * 9.0, (6,), 2, (3, 3))
    # one GPU and room for everything: a single fused stage (no recomputation)
    assert B.partition([1.0] * 4, [3.0] * 4, 2.0, [1.0] * 4, [1.0] * 4, 1.0, 100.0, 4, 1) == \
        (4 * 14.0, (), 4, ())
    with pytest.raises(B.RPError):  # the LM head alone exceeds the memory cap
        B.partition([1.0], [3.0], 2.0, [1.0], [1.0], 50.0, 10.0, 1, 1)
    with pytest.raises(B.RPError):  # negative time
        B.partition([-1.0], [3.0], 2.0, [1.0], [1.0], 1.0, 10.0, 1, 1)


def test_model_partition_stages_cover_every_layer_once():
    """The whole-model driver's stage list (section 3.2): forward stages front
    to back over [0, L - b1), the fused stage B_1 over the last b1 layers,
    backward stages back to front over [0, L - b1); malformed partitions are
    refused."""
    from offloaded_pipeline_stage_amd.model import Partition
    st = Partition((2, 1), 3, (1, 2)).stages(6)
    assert st == [("F", 0, 2), ("F", 2, 3), ("B1", 3, 6), ("B", 2, 3), ("B", 0, 2)]
    assert Partition.fused(4).stages(4) == [("B1", 0, 4)]
    assert Partition.one_layer_per_stage(3).stages(3) == [("F", 0, 1), ("F", 1, 2), ("B1", 2, 3), ("B", 1, 2),
                                                          ("B", 0, 1)]
    for bad in (Partition((2,), 3, (1, 2)), Partition((3,), 3, (2,)), Partition((6,), 0, (6,))):
        with pytest.raises(ValueError):
            bad.stages(6)
