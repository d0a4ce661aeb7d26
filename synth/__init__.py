"""Seeded synthetic inputs for offloaded pipeline stages.

This module is shared by the CPU oracle and the HIP path. It holds the
workload shapes and the seeded random draws only: no stage arithmetic
(no norm, projection, attention, loss or gradient) lives here.

Every tensor is drawn from its own torch CPU generator, seeded from
(config seed, tensor name) through SHA-256, so a tensor's bytes do not depend
on which other tensors were drawn or in what order. Normal draws are made in
fp32 and then rounded to the workload's storage dtype (round to nearest even
for bf16); both sides of a parity comparison consume the identical bytes.

Workload shapes follow the five stage workloads of the RoundPipe evaluation
models (RoundPipe paper, section 5.1 "Workloads": Qwen3-1.7B, Llama-3.1-8B,
Qwen3-32B, Qwen3-235B-A22B), each cut down to the per-worker stage that one
GPU executes, plus a tiny full decoder used as the exact fp32 reference.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field, replace
from typing import Dict

import torch

__all__ = [
    "StageConfig", "CONFIGS", "config", "tensor_seed", "normal", "uniform_int",
    "layer_weights", "lora_weights", "lmhead_weights", "activation",
    "token_ids", "shifted_labels", "uniform_labels", "router_logits",
    "storage_dtype",
]


@dataclass(frozen=True)
class StageConfig:
    name: str
    hidden: int
    n_q: int
    n_kv: int
    head_dim: int
    ffn: int                   # dense SwiGLU width (0 for MoE layers)
    batch: int
    seq: int
    dtype: str                 # "f32" or "bf16": weights and activations
    vocab: int = 0             # LM-head vocabulary (0: no LM head in this workload)
    n_shards: int = 1          # LM-head vocabulary shards
    n_experts: int = 0         # 0: dense MLP
    top_k: int = 0
    expert_ffn: int = 0
    lora_rank: int = 0         # 0: no adapters (full fine-tune)
    lora_alpha: float = 0.0
    rms_eps: float = 1e-6
    rope_base: float = 10000.0
    fwd_layers: int = 1        # layers run by the forward stage call
    bwd_layers: int = 1        # layers run by the recompute+backward call
    final_norm: bool = False   # LM head preceded by a final RMSNorm
    qk_norm: bool = False      # per-head RMSNorm of q and k before RoPE (Qwen3-style)
    embedding: bool = False    # full model: token embedding in front
    weight_std: float = 0.02
    seed: int = 1000

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    @property
    def q_dim(self) -> int:
        return self.n_q * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv * self.head_dim

    @property
    def is_moe(self) -> bool:
        return self.n_experts > 0

    def with_(self, **kw) -> "StageConfig":
        return replace(self, **kw)


CONFIGS: Dict[str, StageConfig] = {
    # Tiny decoder, fp32 everywhere: 2 layers, untied LM head, embedding.
    "tiny": StageConfig(
        name="tiny", hidden=256, n_q=4, n_kv=4, head_dim=64, ffn=688,
        batch=2, seq=128, dtype="f32", vocab=4096, n_shards=1,
        fwd_layers=2, bwd_layers=2, final_norm=True, embedding=True, seed=1001),
    # Qwen3-1.7B-shaped stage: 4 layers forward, 1 layer fused recompute+bwd.
    "qwen3_1p7b": StageConfig(
        name="qwen3_1p7b", hidden=2048, n_q=16, n_kv=8, head_dim=128, ffn=6144,
        batch=1, seq=4096, dtype="bf16", fwd_layers=4, bwd_layers=1, seed=1002),
    # Llama-3.1-8B-shaped stage: 1 layer fused recompute+bwd plus the LM head
    # (4096 x 128256, 4 vocabulary shards of 32064 rows).
    "llama3_8b": StageConfig(
        name="llama3_8b", hidden=4096, n_q=32, n_kv=8, head_dim=128, ffn=14336,
        batch=1, seq=8192, dtype="bf16", vocab=128256, n_shards=4,
        fwd_layers=1, bwd_layers=1, seed=1003),
    # Qwen3-32B-shaped full fine-tune stage: 2 layers forward + 1 fused.
    "qwen3_32b": StageConfig(
        name="qwen3_32b", hidden=5120, n_q=64, n_kv=8, head_dim=128, ffn=25600,
        batch=1, seq=16384, dtype="bf16", fwd_layers=2, bwd_layers=1, seed=1004),
    # Qwen3-235B-A22B-shaped MoE LoRA stage: 128 experts, top-8, LoRA r16.
    "qwen3_235b_moe": StageConfig(
        name="qwen3_235b_moe", hidden=4096, n_q=64, n_kv=4, head_dim=128, ffn=0,
        batch=1, seq=32768, dtype="bf16", n_experts=128, top_k=8,
        expert_ffn=1536, lora_rank=16, lora_alpha=32.0,
        fwd_layers=1, bwd_layers=1, seed=1005),
}


def config(name: str, **overrides) -> StageConfig:
    cfg = CONFIGS[name]
    return cfg.with_(**overrides) if overrides else cfg


def storage_dtype(cfg: StageConfig) -> torch.dtype:
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def tensor_seed(seed: int, name: str) -> int:
    """63-bit generator seed for one named tensor of one workload."""
    h = hashlib.sha256(f"{seed}/{name}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(seed: int, name: str) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(tensor_seed(seed, name))
    return g


def normal(shape, seed: int, name: str, std: float = 1.0, mean: float = 0.0,
           dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """N(mean, std^2) draws in fp32, rounded once to ``dtype``."""
    t = torch.randn(tuple(shape), generator=_gen(seed, name), dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t.to(dtype)


def uniform_int(shape, high: int, seed: int, name: str) -> torch.Tensor:
    """Integers uniform over [0, high), int32."""
    return torch.randint(0, high, tuple(shape), generator=_gen(seed, name),
                         dtype=torch.int64).to(torch.int32)


def layer_weights(cfg: StageConfig, layer: int, gamma: str = "ones",
                  seed: int | None = None) -> Dict[str, torch.Tensor]:
    """One decoder layer's weights, [out, in] row-major (y = x W^T).

    gamma="ones" gives unit RMSNorm gains; gamma="perturbed" gives 1 + N(0, std^2)
    so that gain gradients are exercised with non-trivial values.
    """
    s = cfg.seed if seed is None else seed
    dt = storage_dtype(cfg)
    H, std = cfg.hidden, cfg.weight_std
    p = f"layer{layer}/"

    def gam(n, size=H):
        if gamma == "ones":
            return torch.ones(size, dtype=torch.float32).to(dt)
        return normal((size,), s, p + n, std=std, mean=1.0, dtype=dt)

    w = {
        "gamma1": gam("gamma1"),
        "wq": normal((cfg.q_dim, H), s, p + "wq", std, dtype=dt),
        "wk": normal((cfg.kv_dim, H), s, p + "wk", std, dtype=dt),
        "wv": normal((cfg.kv_dim, H), s, p + "wv", std, dtype=dt),
        "wo": normal((H, cfg.q_dim), s, p + "wo", std, dtype=dt),
        "gamma2": gam("gamma2"),
    }
    if cfg.is_moe:
        E, Fe = cfg.n_experts, cfg.expert_ffn
        w["wg"] = normal((E, Fe, H), s, p + "experts/wg", std, dtype=dt)
        w["wu"] = normal((E, Fe, H), s, p + "experts/wu", std, dtype=dt)
        w["wd"] = normal((E, H, Fe), s, p + "experts/wd", std, dtype=dt)
    else:
        F = cfg.ffn
        w["wg"] = normal((F, H), s, p + "wg", std, dtype=dt)
        w["wu"] = normal((F, H), s, p + "wu", std, dtype=dt)
        w["wd"] = normal((H, F), s, p + "wd", std, dtype=dt)
    if cfg.qk_norm:
        w["qnorm"] = gam("qnorm", cfg.head_dim)
        w["knorm"] = gam("knorm", cfg.head_dim)
    return w


def lora_weights(cfg: StageConfig, layer: int, b_zero: bool = True,
                 seed: int | None = None) -> Dict[str, torch.Tensor]:
    """fp32 LoRA adapters on q, k, v, o: A [r, in] ~ N(0, std^2), B [out, r].

    B is zero at initialisation (b_zero=True); b_zero=False draws B ~ N(0, std^2)
    so that the adapter path carries signal in both directions.
    """
    s = cfg.seed if seed is None else seed
    r, H, std = cfg.lora_rank, cfg.hidden, cfg.weight_std
    p = f"layer{layer}/lora/"
    dims = {"q": (cfg.q_dim, H), "k": (cfg.kv_dim, H), "v": (cfg.kv_dim, H),
            "o": (H, cfg.q_dim)}
    out = {}
    for n, (o, i) in dims.items():
        out["a" + n] = normal((r, i), s, p + "a" + n, std)
        out["b" + n] = (torch.zeros(o, r) if b_zero
                        else normal((o, r), s, p + "b" + n, std))
    return out


def lmhead_weights(cfg: StageConfig, seed: int | None = None) -> Dict[str, torch.Tensor]:
    s = cfg.seed if seed is None else seed
    dt = storage_dtype(cfg)
    out = {"w": normal((cfg.vocab, cfg.hidden), s, "lmhead/w", cfg.weight_std, dtype=dt)}
    if cfg.final_norm:
        out["gamma_f"] = torch.ones(cfg.hidden, dtype=torch.float32).to(dt)
    if cfg.embedding:
        out["embed"] = normal((cfg.vocab, cfg.hidden), s, "embed", cfg.weight_std, dtype=dt)
    return out


def activation(cfg: StageConfig, name: str, seed: int | None = None,
               tokens: int | None = None) -> torch.Tensor:
    """[tokens, hidden] N(0, 1) activation (stage input x or upstream grad dy)."""
    s = cfg.seed if seed is None else seed
    T = cfg.tokens if tokens is None else tokens
    return normal((T, cfg.hidden), s, "act/" + name, 1.0, dtype=storage_dtype(cfg))


def token_ids(cfg: StageConfig, seed: int | None = None) -> torch.Tensor:
    s = cfg.seed if seed is None else seed
    return uniform_int((cfg.batch, cfg.seq), cfg.vocab, s, "ids")


def shifted_labels(ids: torch.Tensor) -> torch.Tensor:
    """label[b, t] = ids[b, t + 1]; the last position of every row is -1 (ignored)."""
    lab = torch.full_like(ids, -1)
    lab[:, :-1] = ids[:, 1:]
    return lab


def uniform_labels(cfg: StageConfig, seed: int | None = None) -> torch.Tensor:
    s = cfg.seed if seed is None else seed
    return uniform_int((cfg.tokens,), cfg.vocab, s, "labels")


def router_logits(cfg: StageConfig, layer: int, seed: int | None = None,
                  tokens: int | None = None) -> torch.Tensor:
    """fp32 router logits [tokens, n_experts] ~ N(0, 1)."""
    s = cfg.seed if seed is None else seed
    T = cfg.tokens if tokens is None else tokens
    return normal((T, cfg.n_experts), s, f"layer{layer}/router", 1.0)
