"""Shared helpers of the GPU parity tests (no stage arithmetic here)."""
import os
import sys

import torch

# parity tolerances: bf16 storage with fp32 accumulation vs the fp64 oracle,
# and the fp32 tiny decoder
LOSS_TOL = {"bf16": 1e-3, "f32": 1e-4}
GRAD_TOL = {"bf16": 2e-2, "f32": 1e-4}


def max_rel(got, ref) -> float:
    """max |got - ref| / max |ref| over the tensor."""
    g = got.detach().double().cpu()
    r = ref.detach().double().cpu()
    den = r.abs().max().item()
    return (g - r).abs().max().item() / (den if den > 0 else 1.0)


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def ensure_built():
    from offloaded_pipeline_stage_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        raise RuntimeError("librp.so is not built; run python -m offloaded_pipeline_stage_amd.build first")
    binding.lib()
    return binding


def to_f64(d):
    return {k: v.to(torch.float64) for k, v in d.items()}
