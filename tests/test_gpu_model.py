"""A whole model through RoundPipe's stage structure on one GPU (pages:
section 3.2 stage structure, section 4.4 profiling and partitioning): every
partition -- one fused stage, one layer per stage, hand-picked splits and the
partitioner's own choice from profiled layer times -- gives bit-identical loss
and gradients, and they match the oracle's end-to-end fp64 model."""
import pytest
import torch

import synth
from _helpers import GRAD_TOL, LOSS_TOL, ensure_built, max_rel, say
from oracle import stage as O

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")
N_LAYERS = 6


def _collect(m):
    out = {"loss": m.loss.clone(), "dtable": m.dtable.clone(), "dw": [t.clone() for t in m.wk.head["dw"]],
           "dgamma_f": m.wk.head["dgamma_f"].clone()}
    for l in range(m.L):
        out[f"layer{l}"] = {k: v.clone() for k, v in m.layer_grads(l).items()}
    return out


def _same(a, b):
    if isinstance(a, torch.Tensor):
        return torch.equal(a, b)
    if isinstance(a, dict):
        return a.keys() == b.keys() and all(_same(a[k], b[k]) for k in a)
    return len(a) == len(b) and all(_same(x, y) for x, y in zip(a, b))


def test_partitions_bit_identical_and_match_oracle():
    ensure_built()
    from offloaded_pipeline_stage_amd.model import Partition, RoundPipeModel
    cfg = synth.config("tiny")
    layers = [synth.layer_weights(cfg, l, gamma="perturbed") for l in range(N_LAYERS)]
    head = synth.lmhead_weights(cfg)
    ids = synth.token_ids(cfg)
    labels = synth.shifted_labels(ids).reshape(-1)
    m = RoundPipeModel(cfg, layers, head)
    ids_d = ids.reshape(-1).to(torch.int32).to(DEV)
    lab_d = labels.to(torch.int32).to(DEV)

    f, bw, h = m.profile(ids_d, lab_d)
    say("profiled ms", [round(x, 3) for x in f], [round(x, 3) for x in bw], round(h, 3))
    assert all(x > 0 for x in f + bw) and h >= 0
    _, planned = m.plan(f, bw, h, n_micro=8, n_gpus=4, mem_cap=1e15)
    say("planned", planned)
    parts = [Partition.fused(N_LAYERS), Partition.one_layer_per_stage(N_LAYERS),
             Partition((2, 2), 2, (3, 1)), Partition((1, 3), 2, (1, 1, 2)), planned]
    results = []
    for p in parts:
        say("partition", p)
        for rep in range(2):
            m.step(ids_d, lab_d, part=p)
            m.ctx.sync()
            results.append((p, rep, _collect(m)))
    ref = results[0][2]
    for p, rep, r in results[1:]:
        for k in ref:
            assert _same(r[k], ref[k]), f"partition {p} pass {rep}: {k} differs from the fused stage"

    loss_ref, g_ref = O.full_model_fwd_bwd(ids, labels, layers, head, cfg)
    tol = GRAD_TOL["f32"]
    assert abs(ref["loss"].item() - loss_ref.item()) / abs(loss_ref.item()) < LOSS_TOL["f32"]
    assert max_rel(ref["dtable"], g_ref["embed"]) < tol
    assert max_rel(ref["dw"][0], g_ref["w"]) < tol
    assert max_rel(ref["dgamma_f"], g_ref["gamma_f"]) < tol
    for l in range(N_LAYERS):
        for n, r in g_ref["layers"][l].items():
            e = max_rel(ref[f"layer{l}"][n], r)
            assert e < tol, (l, n, e)
    m.close()
