"""fp64 CPU oracle for one optimizer step: Muon on the weight matrices,
AdamW on the embedding and the lm_head.

TEST INFRASTRUCTURE ONLY.  Imported by the test-suite; the GPU path never
calls it and shares no code with it (numpy and ``gpt_inputs`` only).

What the pages fix ("Introducing nanochat", GitHub discussion #1):
  * the pretraining log and the paragraph after it: Muon optimises the
    matrices (every Wq, Wk, Wv, Wo, W1, W2, grouped by shape, each matrix on
    its own), AdamW the embedding and the unembedding, and there are no other
    trainable parameters; the AdamW learning rates are scaled by
    1/sqrt(d/768);
  * the report card's base-model section: embedding lr 0.2, unembedding lr
    0.004, matrix lr 0.02, weight decay 0, gradient clipping at norm 1.0.

The pages name Muon without its algorithm.  This module follows the
published description (K. Jordan et al., "Muon: An optimizer for hidden
layers in neural networks", 2024): SGD momentum with Nesterov's look-ahead,
then the update is replaced by an approximate orthogonalisation of itself --
normalise by the Frobenius norm, then iterate the quintic Newton-Schulz map
X <- a X + (b A + c A^2) X, A = X X^T, on the wide orientation of the
matrix, five times, with (a, b, c) = (3.4445, -4.7750, 2.0315) -- and scaled
by sqrt(max(1, rows/cols)).  Momentum is kept in the interpolating form
buf <- mu buf + (1 - mu) g, u = (1 - mu) g + mu buf; it differs from the
original buf <- mu buf + g, u = g + mu buf by the factor (1 - mu) only, which
the normalisation removes.

AdamW is Adam's bias-corrected moments (Kingma and Ba, 2015) with the weight
decay decoupled from the gradient (Loshchilov and Hutter, 2019):
  m <- b1 m + (1 - b1) g,  v <- b2 v + (1 - b2) g^2,
  p <- p (1 - lr wd) - lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps).
Muon takes the same decoupled decay: p <- p (1 - lr wd) - lr s O.

Gradient clipping (the report card's grad_clip) scales every gradient by
min(1, clip / (||g|| + 1e-6)), ||g|| the 2-norm over all parameters, before
either update; clip <= 0 disables it.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Tuple

import numpy as np

import gpt_inputs as gi

NS_COEFFS = (3.4445, -4.7750, 2.0315)
NS_EPS = 1e-7
CLIP_EPS = 1e-6


@dataclasses.dataclass
class OptimParams:
    lr_matrix: float = 0.02
    momentum: float = 0.95
    nesterov: bool = True
    ns_steps: int = 5
    lr_embedding: float = 0.2
    lr_unembedding: float = 0.004
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0
    grad_clip: float = 1.0
    step: int = 1          # AdamW step count t (1 on the first step)


def newton_schulz(G: np.ndarray, steps: int, coeffs=NS_COEFFS, eps: float = NS_EPS) -> np.ndarray:
    """Approximate orthogonalisation of G: the quintic Newton-Schulz
    iteration on G / (||G||_F + eps), run on the wide orientation."""
    a, b, c = coeffs
    X = np.asarray(G, dtype=np.float64) / (np.linalg.norm(G) + eps)
    tall = X.shape[0] > X.shape[1]
    if tall:
        X = X.T
    for _ in range(steps):
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    return X.T if tall else X


def muon_scale(rows: int, cols: int) -> float:
    return math.sqrt(max(1.0, rows / cols))


def muon_update(p: np.ndarray, g: np.ndarray, buf: np.ndarray, hp: OptimParams) -> Tuple[np.ndarray, np.ndarray]:
    """(new p, new momentum buffer) of one matrix."""
    mu = hp.momentum
    buf = mu * buf + (1.0 - mu) * g
    u = (1.0 - mu) * g + mu * buf if hp.nesterov else buf
    O = newton_schulz(u, hp.ns_steps)
    lr = hp.lr_matrix
    p = p * (1.0 - lr * hp.weight_decay) - lr * muon_scale(*p.shape) * O
    return p, buf


def adamw_update(p: np.ndarray, g: np.ndarray, m: np.ndarray, v: np.ndarray, lr: float,
                 hp: OptimParams) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(new p, new m, new v) of one tensor at step hp.step."""
    t = hp.step
    m = hp.beta1 * m + (1.0 - hp.beta1) * g
    v = hp.beta2 * v + (1.0 - hp.beta2) * g * g
    mhat = m / (1.0 - hp.beta1 ** t)
    vhat = v / (1.0 - hp.beta2 ** t)
    p = p * (1.0 - lr * hp.weight_decay) - lr * mhat / (np.sqrt(vhat) + hp.eps)
    return p, m, v


def global_norm(grads: Dict[str, np.ndarray]) -> float:
    return math.sqrt(sum(float(np.sum(np.square(g, dtype=np.float64))) for g in grads.values()))


def clip_coefficient(norm: float, clip: float) -> float:
    if clip <= 0:
        return 1.0
    return min(1.0, clip / (norm + CLIP_EPS))


def is_matrix_param(name: str) -> bool:
    """Muon's parameters: every per-layer projection; AdamW's: E and U."""
    return name not in ("E", "U")


def init_state(s: gi.GPTShape) -> Dict[str, Dict[str, np.ndarray]]:
    """Zero optimizer state: Muon momentum per matrix, AdamW (m, v) per tensor."""
    st = {}
    for name, shp in gi.param_shapes(s):
        if is_matrix_param(name):
            st[name] = {"buf": np.zeros(shp)}
        else:
            st[name] = {"m": np.zeros(shp), "v": np.zeros(shp)}
    return st


def optim_step(s: gi.GPTShape, master: Dict[str, np.ndarray], grads: Dict[str, np.ndarray],
               state: Dict[str, Dict[str, np.ndarray]], hp: OptimParams):
    """One optimizer step over every parameter.  Returns (new master weights,
    new state, global gradient norm before clipping); the inputs are not
    modified."""
    norm = global_norm(grads)
    cf = clip_coefficient(norm, hp.grad_clip)
    new_p, new_st = {}, {}
    for name, p in master.items():
        g = grads[name] * cf
        if is_matrix_param(name):
            new_p[name], buf = muon_update(p, g, state[name]["buf"], hp)
            new_st[name] = {"buf": buf}
        else:
            lr = hp.lr_embedding if name == "E" else hp.lr_unembedding
            new_p[name], m, v = adamw_update(p, g, state[name]["m"], state[name]["v"], lr, hp)
            new_st[name] = {"m": m, "v": v}
    return new_p, new_st, norm
