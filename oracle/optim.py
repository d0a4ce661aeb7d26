"""Host optimizer semantics, stated plainly -- TEST INFRASTRUCTURE ONLY.

* Adam (Kingma and Ba, "Adam: A Method for Stochastic Optimization") with
  decoupled weight decay (Loshchilov and Hutter, "Decoupled Weight Decay
  Regularization"), as the optimizer of the mixed-precision training the
  RoundPipe paper builds on (section 2.1.2; section 4.3.1 names the fp32
  optimizer copy of the weights);
* staleness-1 asynchronous updates (section 2.1.2): iteration i computes its
  gradients on the weights produced by step i - 2, i.e. after iteration
  i - 2's gradients were applied (the initial weights for i < 2).

Precision follows the paper's three copies (section 4.3.1): the optimizer
copy and moments are fp32, the master copy the GPU reads is rounded to the
master dtype. `adam_step_f32` takes every operation as one fp32 rounding in
the order written, with 1 - beta and the bias corrections 1 - beta^s formed in
double and rounded once; `adam_step_f64` is the same formula in fp64.
"""
from __future__ import annotations

from typing import Callable, List

import numpy as np


def adam_step_f32(w, m, v, g, s: int, lr, beta1, beta2, eps, weight_decay=0.0, grad_scale=1.0):
    """One Adam step (s = 1-based step count) on float32 arrays; returns the
    new (w, m, v). Hyper-parameters are taken as float32 values."""
    f = np.float32
    b1, b2, lr, eps, wd, gs = f(beta1), f(beta2), f(lr), f(eps), f(weight_decay), f(grad_scale)
    c1, c2 = f(1.0 - float(b1)), f(1.0 - float(b2))
    bc1, bc2 = f(1.0 - float(b1) ** s), f(1.0 - float(b2) ** s)
    g = gs * g
    m = b1 * m + c1 * g
    v = b2 * v + c2 * (g * g)
    upd = (m / bc1) / (np.sqrt(v / bc2) + eps)
    if wd != 0:
        upd = upd + wd * w
    return w - lr * upd, m, v


def adam_step_f64(w, m, v, g, s: int, lr, beta1, beta2, eps, weight_decay=0.0, grad_scale=1.0):
    g = grad_scale * g
    m = beta1 * m + (1 - beta1) * g
    v = beta2 * v + (1 - beta2) * g * g
    upd = (m / (1 - beta1 ** s)) / (np.sqrt(v / (1 - beta2 ** s)) + eps) + weight_decay * w
    return w - lr * upd, m, v


def to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bfloat16 (ties to even), returned as float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32)


def staleness1_run(w0: np.ndarray, grad_of: Callable[[int, np.ndarray], np.ndarray], n_iter: int,
                   hp: dict, master=to_bf16):
    """Train n_iter iterations with staleness-1 updates. grad_of(i, w_seen)
    gives iteration i's gradient from the master weights it saw. Returns
    (the master weights each iteration saw, final fp32 weights)."""
    w = w0.astype(np.float32)
    m = np.zeros_like(w)
    v = np.zeros_like(w)
    produced: List[np.ndarray] = [master(w)]  # produced[k]: master after k steps
    seen = []
    for i in range(n_iter):
        w_seen = produced[max(i - 1, 0)]
        seen.append(w_seen)
        g = grad_of(i, w_seen).astype(np.float32)
        w, m, v = adam_step_f32(w, m, v, g, i + 1, **hp)
        produced.append(master(w))
    return seen, w
