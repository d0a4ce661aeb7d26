"""Training iterations end to end on one GPU worker with the host optimizer
(RoundPipe paper, sections 2.1.2 and 4.3): every iteration uploads the
layers' master copy from pinned host memory through the transfer engine,
runs forward and backward, downloads the gradients into the master gradient
buffers, and queues an asynchronous Adam step, with the per-layer protocol
ordering the two. Checked: the weights each iteration uploaded are exactly
the staleness-1 sequence (iteration i sees step i - 2's weights), the
optimizer's fp32 copy equals a sequential replay of Adam on the downloaded
gradients bit for bit, and each iteration's gradients match the fp64 oracle
model at the weights that iteration saw."""
import numpy as np
import pytest
import torch

import synth
from _helpers import GRAD_TOL, ensure_built, max_rel, say
from oracle import optim as OO
from oracle import stage as O

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")
N_ITER, N_LAYERS = 5, 2


def test_staleness1_training_with_streamed_master_copy():
    B = ensure_built()
    from offloaded_pipeline_stage_amd.model import RoundPipeModel
    from offloaded_pipeline_stage_amd.optimizer import AdamParams, OptimizerWorker
    say("training loop", N_ITER, "iterations")
    cfg = synth.config("tiny")
    layers = [synth.layer_weights(cfg, l, gamma="perturbed") for l in range(N_LAYERS)]
    head = synth.lmhead_weights(cfg)
    ids = synth.token_ids(cfg)
    labels = synth.shifted_labels(ids).reshape(-1)
    m = RoundPipeModel(cfg, layers, head)
    wk, ctx = m.wk, m.ctx
    ids_d, lab_d = ids.reshape(-1).to(torch.int32).to(DEV), labels.to(torch.int32).to(DEV)
    master_w = [wk.pack_layer(layers[l], pinned=True) for l in range(N_LAYERS)]
    master_g = [torch.zeros(wk.g_bytes, dtype=torch.uint8).pin_memory() for _ in range(N_LAYERS)]
    opt = OptimizerWorker(N_LAYERS, torch.float32, n_threads=4, timeout_ms=60000)
    for l in range(N_LAYERS):
        opt.bind_blocks(cfg, l, master_w[l], master_g[l])
    hp = AdamParams(lr=2e-3, beta1=0.9, beta2=0.99, eps=1e-8)
    seen, grads = [], []
    for i in range(N_ITER):
        for l in range(N_LAYERS):
            opt.wait(B.RP_OPT_PCP_DONE, l, i - 2)
        ctx.weight_stream_submit([(B.RP_PARAM_H2D, B.RP_TGT_LAYER, l, 0, wk.w_bytes, master_w[l])
                                  for l in range(N_LAYERS)], n_windows=2)
        ctx.sync()
        # the protocol keeps P-cp out of the master copy until this signal
        seen.append([master_w[l].clone() for l in range(N_LAYERS)])
        for l in range(N_LAYERS):
            assert torch.equal(wk.layers[l]["w"].cpu(), seen[-1][l]), f"iteration {i}: layer {l} upload"
            opt.signal(B.RP_OPT_PARAMS_UPLOADED, l, i)
        m.step(ids_d, lab_d)
        ctx.sync()
        for l in range(N_LAYERS):
            opt.wait(B.RP_OPT_GCP_DONE, l, i - 1)
        ctx.weight_stream_submit([(B.RP_GRAD_D2H, B.RP_TGT_LAYER, l, 0, wk.g_bytes, master_g[l])
                                  for l in range(N_LAYERS)], n_windows=2)
        ctx.sync()
        grads.append([master_g[l].clone() for l in range(N_LAYERS)])
        for l in range(N_LAYERS):
            opt.signal(B.RP_OPT_GRADS_DOWNLOADED, l, i)
        opt.step(i, hp)
    opt.signal(B.RP_OPT_PARAMS_UPLOADED, -1, N_ITER)
    opt.sync()

    # the trainable tensors of a block, flattened in block order (fp32 model:
    # the weight and gradient blocks share the layout)
    def flat(block):
        d = wk.unpack_grads(block)
        return np.concatenate([d[n].reshape(-1).numpy() for n in O.trainable_names(cfg)])

    def as_layers(blocks):
        return [{n: t.clone() for n, t in wk.unpack_grads(b).items()} for b in blocks]

    for l in range(N_LAYERS):
        w = flat(master_w[l] if N_ITER == 0 else seen[0][l]).astype(np.float32)
        mom, vel = np.zeros_like(w), np.zeros_like(w)
        produced = [w.copy()]
        for i in range(N_ITER):
            assert np.array_equal(flat(seen[i][l]), produced[max(i - 1, 0)]), f"layer {l}: iteration {i} weights"
            w, mom, vel = OO.adam_step_f32(w, mom, vel, flat(grads[i][l]), i + 1, lr=hp.lr, beta1=hp.beta1,
                                           beta2=hp.beta2, eps=hp.eps)
            produced.append(w.copy())
        # the optimizer reads its tensors in block order as well
        assert np.array_equal(opt.read(l, 0).numpy(), w), f"layer {l}: optimizer copy"
    assert not torch.equal(seen[2][0], seen[0][0]), "the weights never changed"

    tol = GRAD_TOL["f32"]
    for i in range(N_ITER):
        _, g_ref = O.full_model_fwd_bwd(ids, labels, as_layers(seen[i]), head, cfg)
        for l in range(N_LAYERS):
            got = wk.unpack_grads(grads[i][l])
            for n, r in g_ref["layers"][l].items():
                e = max_rel(got[n], r)
                assert e < tol, (i, l, n, e)
    opt.close()
    m.close()
