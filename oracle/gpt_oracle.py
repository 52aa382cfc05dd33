"""fp64 CPU oracle for one forward+backward step of the GPT decoder.

TEST INFRASTRUCTURE ONLY.  This module is imported by the test-suite, by the
smoke check and by the benchmark's CPU-baseline leg; the GPU path never calls
it, and it shares no code with the GPU path (it imports only numpy and the
seeded workload module ``gpt_inputs``).

What it computes is the plain definition of the network the nanochat pages
describe, evaluated in float64 with hand-derived adjoints:

  * "Introducing nanochat" (GitHub discussion #1), pretraining log and the
    paragraph after it: untied token embedding and lm_head, per layer separate
    Q, K, V, O projections [d, d] and an MLP of width 4d ([4d, d] up,
    [d, 4d] down), no biases and no norm gains ("no other trainable
    parameters"), so the parameter count is 2*V*d + L*(4d^2 + 8d^2).
  * nanochat User Guide, section 10 "How It Works", base model paragraph:
    rotary position embeddings, QK-norm, ReLU^2 MLP, untied weights,
    sliding-window attention pattern.
  * "supa beginna nanochat" (discussion #677), troubleshooting: the loss is
    PyTorch-style mean cross-entropy over the target positions; rows are
    drawn as T+1 ids and split into inputs and shifted targets.

Grouped-query attention (nanochat User Guide, section 10, base model
paragraph, lists Group-Query Attention among the architecture's features):
with n_kv_head = Hkv < H, Wk and Wv are [Hkv*Dh, d], and query head h attends
with the keys and values of head h // (H / Hkv).  The backward sums the key
and value gradients of the H/Hkv query heads that share a key/value head.
Hkv = H is plain multi-head attention.

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):
  pre-norm blocks plus a final norm before lm_head, no norm after the
  embedding; RMSNorm eps = cfg.norm_eps for every norm; RoPE half-split pairs
  with theta_i = base**(-2i/Dh) rotating by +t*theta_i, applied before the
  per-head QK RMSNorm; attention scale 1/sqrt(Dh); a window of W keys means
  0 <= i-j <= W-1; layer l uses pattern[l % len] with the last layer full.

FP8 configuration (precision "fp8"): the "FP8 matrix products" of the d24
speedrun ("supa beginna nanochat" discussion #677) and of the
alpha-nanochat-d24 model card are an encoding of the four linear layers'
operands, so the oracle takes that encoding as a step of the method
(``Fp8Operands``): forward operands (weights and activations) are encoded in
OCP E4M3 and gradient operands in E5M2, each tensor with its own current
per-tensor scale (``fp8_codec.quantize_tensor``); the products of the decoded
operands are then exact (fp64), and gradients pass the encoding unchanged
(straight-through).  The fused QKV weight [d + 2 Hkv Dh, d] and its output
gradient [BT, d + 2 Hkv Dh] are one tensor each.  Everything else stays exact.

Memory plan: the residual stream h is checkpointed (fp64) at each layer input;
the backward recomputes the layer's internals from it.  Attention is done one
batch row at a time, cross-entropy in chunks of rows, so neither the full
[B, H, T, T] probabilities nor the full [B*T, V] logits exist at once.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Tuple

import numpy as np

import gpt_inputs as gi

from . import fp8_codec

# ---------------------------------------------------------------------------
# Elementary operations (each one a plain definition)
# ---------------------------------------------------------------------------


def rmsnorm(x: np.ndarray, eps: float) -> Tuple[np.ndarray, np.ndarray]:
    """Parameter-free RMSNorm over the last axis: y = x / sqrt(mean(x^2) + eps).

    Returns (y, r) with r = 1/sqrt(mean(x^2)+eps) (shape x.shape[:-1] + (1,)).
    """
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x * r, r


def rmsnorm_bwd(dy: np.ndarray, y: np.ndarray, r: np.ndarray) -> np.ndarray:
    """Adjoint of rmsnorm.  With y = x*r and dr/dx_j = -r^3 x_j / D:

    dx_j = r*dy_j - r^3 x_j/D * sum_i dy_i x_i = r * (dy_j - y_j * mean(dy*y)).
    """
    return r * (dy - y * np.mean(dy * y, axis=-1, keepdims=True))


def rope_tables(seq_len: int, head_dim: int, base: float) -> Tuple[np.ndarray, np.ndarray]:
    """cos/sin of t*theta_i, theta_i = base**(-2i/Dh), i < Dh/2; shape [T, Dh/2]."""
    half = head_dim // 2
    theta = base ** (-2.0 * np.arange(half, dtype=np.float64) / head_dim)
    ang = np.arange(seq_len, dtype=np.float64)[:, None] * theta[None, :]
    return np.cos(ang), np.sin(ang)


def rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate half-split pairs (x[i], x[i+Dh/2]) by +t*theta_i.

    x: [B, T, H, Dh]; cos/sin: [T, Dh/2].
    """
    half = x.shape[-1] // 2
    c = cos[None, :, None, :]
    s = sin[None, :, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def rope_bwd(dy: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Adjoint of rope: the transposed (inverse) rotation."""
    half = dy.shape[-1] // 2
    c = cos[None, :, None, :]
    s = sin[None, :, None, :]
    d1, d2 = dy[..., :half], dy[..., half:]
    return np.concatenate([d1 * c + d2 * s, -d1 * s + d2 * c], axis=-1)


def attention_mask(seq_len: int, window: int) -> np.ndarray:
    """allowed[i, j] = 0 <= i - j <= window - 1 (causal, W most recent keys)."""
    i = np.arange(seq_len)[:, None]
    j = np.arange(seq_len)[None, :]
    return (j <= i) & (i - j < window)


def attention_probs(q: np.ndarray, k: np.ndarray, window: int) -> np.ndarray:
    """Softmax probabilities for one batch row.  q, k: [H, T, Dh] -> P [H, T, T]."""
    dh = q.shape[-1]
    s = np.matmul(q, np.swapaxes(k, -1, -2)) / math.sqrt(dh)
    allowed = attention_mask(q.shape[-2], window)
    s = np.where(allowed[None], s, -np.inf)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    return p / p.sum(axis=-1, keepdims=True)


def attention_fwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, window: int) -> np.ndarray:
    """o_i = sum_j softmax_j(q_i.k_j/sqrt(Dh) | mask) v_j.  q,k,v: [H, T, Dh]."""
    return np.matmul(attention_probs(q, k, window), v)


def attention_bwd(do: np.ndarray, q: np.ndarray, k: np.ndarray, v: np.ndarray,
                  window: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Adjoint of attention_fwd for one batch row -> (dq, dk, dv), [H, T, Dh].

    dv = P^T do;  dP = do v^T;  dS = P * (dP - rowsum(P*dP));
    dq = dS k / sqrt(Dh);  dk = dS^T q / sqrt(Dh).
    """
    dh = q.shape[-1]
    p = attention_probs(q, k, window)
    dv = np.matmul(np.swapaxes(p, -1, -2), do)
    dp = np.matmul(do, np.swapaxes(v, -1, -2))
    ds = p * (dp - np.sum(p * dp, axis=-1, keepdims=True))
    dq = np.matmul(ds, k) / math.sqrt(dh)
    dk = np.matmul(np.swapaxes(ds, -1, -2), q) / math.sqrt(dh)
    return dq, dk, dv


def expand_kv(x: np.ndarray, n_head: int) -> np.ndarray:
    """[Hkv, T, Dh] -> [H, T, Dh]: query head h reads key/value head
    h // (H / Hkv) (grouped-query attention)."""
    return np.repeat(x, n_head // x.shape[0], axis=0)


def reduce_kv(dx: np.ndarray, kv_heads: int) -> np.ndarray:
    """Adjoint of expand_kv: [H, T, Dh] -> [Hkv, T, Dh], the sum over the
    query heads of each group."""
    H, T, Dh = dx.shape
    return dx.reshape(kv_heads, H // kv_heads, T, Dh).sum(axis=1)


def logsumexp_rows(z: np.ndarray) -> np.ndarray:
    m = z.max(axis=-1, keepdims=True)
    return (m + np.log(np.sum(np.exp(z - m), axis=-1, keepdims=True)))[..., 0]


# ---------------------------------------------------------------------------
# The network
# ---------------------------------------------------------------------------


# ---------------------------------------------------------------------------
# Operands of the linear layers (QKV, O, W1, W2)
# ---------------------------------------------------------------------------


class LinearOperands:
    """Exact operands: the linear layers multiply the values themselves.

    ``what`` names the operand: activations "n1" (attention input norm),
    "o" (attention output), "n2" (MLP input norm), "g" (relu(u)^2);
    gradients "dh2" (residual gradient into W2), "du" (into W1), "dh1"
    (into Wo); ``grad_fused`` is the fused QKV output gradient."""

    def weights(self, s: gi.GPTShape, W: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
        return W

    def act(self, x: np.ndarray, what: str = "") -> np.ndarray:
        return x

    def grad(self, g: np.ndarray, what: str = "") -> np.ndarray:
        return g

    def grad_fused(self, *parts: np.ndarray) -> Tuple[np.ndarray, ...]:
        """Gradient operands of column blocks that form one tensor."""
        return parts


def fp8_value(x: np.ndarray, fmt: str) -> np.ndarray:
    """The value an fp8-encoded tensor stands for: decode(code) / scale."""
    codes, scale = fp8_codec.quantize_tensor(x, fmt)
    return fp8_codec.decode(codes, fmt) / scale


class Fp8Operands(LinearOperands):
    """FP8 configuration: E4M3 weights and activations, E5M2 gradients, one
    current scale per tensor (the fused QKV weight is one tensor)."""

    def weights(self, s, W):
        out = dict(W)
        d = s.d_model
        for l in range(s.depth):
            qkv = fp8_value(np.concatenate([W[f"L{l}.Wq"], W[f"L{l}.Wk"], W[f"L{l}.Wv"]]), "e4m3")
            dkv = W[f"L{l}.Wk"].shape[0]
            out[f"L{l}.Wq"], out[f"L{l}.Wk"], out[f"L{l}.Wv"] = qkv[:d], qkv[d:d + dkv], qkv[d + dkv:]
            for w in ("Wo", "W1", "W2"):
                out[f"L{l}.{w}"] = fp8_value(W[f"L{l}.{w}"], "e4m3")
        return out

    def act(self, x, what=""):
        return fp8_value(x, "e4m3")

    def grad(self, g, what=""):
        return fp8_value(g, "e5m2")

    def grad_fused(self, *parts):
        q = self.grad(np.concatenate(parts, axis=1))
        cuts = np.cumsum([p.shape[1] for p in parts])[:-1]
        return tuple(np.split(q, cuts, axis=1))


def operands_for(s: gi.GPTShape) -> LinearOperands:
    return Fp8Operands() if s.precision == "fp8" else LinearOperands()


class _Layer:
    """Forward internals of one block, recomputed from its input h.  W holds
    the linear weights as the operands encoder ``enc`` presents them."""

    def __init__(self, s: gi.GPTShape, W: Dict[str, np.ndarray], l: int,
                 h: np.ndarray, cos: np.ndarray, sin: np.ndarray, window: int,
                 enc: LinearOperands):
        B, T, H, Dh, eps = s.batch, s.seq_len, s.n_head, s.head_dim, s.norm_eps
        Hkv = s.kv_heads
        self.h_in = h
        self.a, self.r1 = rmsnorm(h, eps)                          # [BT, d]
        self.aq = enc.act(self.a, "n1")
        q = (self.aq @ W[f"L{l}.Wq"].T).reshape(B, T, H, Dh)
        k = (self.aq @ W[f"L{l}.Wk"].T).reshape(B, T, Hkv, Dh)
        self.v = (self.aq @ W[f"L{l}.Wv"].T).reshape(B, T, Hkv, Dh)
        self.qr, self.kr = rope(q, cos, sin), rope(k, cos, sin)
        self.qn, self.rq = rmsnorm(self.qr, eps)                   # QK-norm
        self.kn, self.rk = rmsnorm(self.kr, eps)
        o = np.empty((B, T, H, Dh))
        for b in range(B):  # one batch row at a time: P is [H, T, T]
            qb = self.qn[b].transpose(1, 0, 2)
            kb = expand_kv(self.kn[b].transpose(1, 0, 2), H)
            vb = expand_kv(self.v[b].transpose(1, 0, 2), H)
            o[b] = attention_fwd(qb, kb, vb, window).transpose(1, 0, 2)
        self.o = o.reshape(B * T, H * Dh)
        self.oq = enc.act(self.o, "o")
        self.h_mid = h + self.oq @ W[f"L{l}.Wo"].T
        self.m, self.r2 = rmsnorm(self.h_mid, eps)
        self.mq = enc.act(self.m, "n2")
        self.u = self.mq @ W[f"L{l}.W1"].T
        self.g = np.maximum(self.u, 0.0) ** 2
        self.gq = enc.act(self.g, "g")
        self.h_out = self.h_mid + self.gq @ W[f"L{l}.W2"].T


def param_count(s: gi.GPTShape) -> int:
    return int(sum(r * c for _, (r, c) in gi.param_shapes(s)))


def _embed(W, X):
    return W["E"][X.reshape(-1)]


def forward(s: gi.GPTShape, W: Dict[str, np.ndarray], X: np.ndarray,
            keep_layers: bool = False, enc: Optional[LinearOperands] = None):
    """Forward pass -> (final residual h [BT, d], list of layer inputs, layers).

    ``layers`` (the full internals) is only kept when keep_layers is set.
    ``enc`` defaults to the workload's own operand encoding.
    """
    enc = enc or operands_for(s)
    return _forward(s, enc.weights(s, W), X, keep_layers, enc)


def _forward(s, W, X, keep_layers, enc):
    cos, sin = rope_tables(s.seq_len, s.head_dim, s.rope_base)
    wins = gi.layer_windows(s)
    h = _embed(W, X)
    h_ins, layers = [], []
    for l in range(s.depth):
        h_ins.append(h)
        lay = _Layer(s, W, l, h, cos, sin, wins[l], enc)
        h = lay.h_out
        if keep_layers:
            layers.append(lay)
        del lay
    return h, h_ins, layers


def logits(s: gi.GPTShape, W: Dict[str, np.ndarray], X: np.ndarray) -> np.ndarray:
    """z = N(h_L) U^T, [B, T, V] (small configs only)."""
    h, _, _ = forward(s, W, X)
    n, _ = rmsnorm(h, s.norm_eps)
    return (n @ W["U"].T).reshape(s.batch, s.seq_len, s.vocab)


def _xent(s, W, h, Y, chunk_rows: int, want_grads: bool):
    """Mean cross-entropy of z = N(h) U^T against Y, done in row chunks.

    Returns (loss, dn [BT, d] or None, dU or None, per-row loss, lse).
    dz = (softmax(z) - onehot(Y)) / BT.
    """
    BT = h.shape[0]
    n, r = rmsnorm(h, s.norm_eps)
    y = Y.reshape(-1)
    U = W["U"]
    row_loss = np.empty(BT)
    lse_all = np.empty(BT)
    dn = np.empty_like(n) if want_grads else None
    dU = np.zeros_like(U) if want_grads else None
    for a in range(0, BT, chunk_rows):
        b = min(BT, a + chunk_rows)
        z = n[a:b] @ U.T
        lse = logsumexp_rows(z)
        lse_all[a:b] = lse
        row_loss[a:b] = lse - z[np.arange(b - a), y[a:b]]
        if want_grads:
            dz = np.exp(z - lse[:, None])
            dz[np.arange(b - a), y[a:b]] -= 1.0
            dz /= BT
            dn[a:b] = dz @ U
            dU += dz.T @ n[a:b]
    loss = float(np.sum(row_loss) / BT)
    if not want_grads:
        return loss, None, None, row_loss, lse_all
    dh = rmsnorm_bwd(dn, n, r)
    return loss, dh, dU, row_loss, lse_all


def loss_only(s: gi.GPTShape, W: Dict[str, np.ndarray], X: np.ndarray,
              Y: np.ndarray, chunk_rows: int = 1024, enc: Optional[LinearOperands] = None) -> float:
    h, _, _ = forward(s, W, X, enc=enc)
    return _xent(s, W, h, Y, chunk_rows, want_grads=False)[0]


def forward_backward(s: gi.GPTShape, W: Dict[str, np.ndarray], X: np.ndarray,
                     Y: np.ndarray, chunk_rows: int = 1024,
                     want_grads: bool = True, enc: Optional[LinearOperands] = None):
    """One training step of the definition: returns (loss, grads dict).

    Gradients are of the mean loss, one fp64 array per parameter tensor in
    the same [rows, cols] shape as the weight.  ``enc`` defaults to the
    workload's own operand encoding (fp8 for precision "fp8"); the gradient
    of an encoded weight is taken as the gradient of the weight.
    """
    B, T, H, Dh, d = s.batch, s.seq_len, s.n_head, s.head_dim, s.d_model
    enc = enc or operands_for(s)
    Wl = enc.weights(s, W)
    h, h_ins, _ = _forward(s, Wl, X, False, enc)
    loss, dh, dU, _, _ = _xent(s, W, h, Y, chunk_rows, want_grads)
    if not want_grads:
        return loss, {}
    del h
    cos, sin = rope_tables(T, Dh, s.rope_base)
    wins = gi.layer_windows(s)
    grads: Dict[str, np.ndarray] = {"U": dU}
    for l in reversed(range(s.depth)):
        L = _Layer(s, Wl, l, h_ins[l], cos, sin, wins[l], enc)
        h_ins[l] = None
        # MLP: h_out = h_mid + g W2^T, g = relu(u)^2, u = m W1^T, m = N(h_mid)
        dhq = enc.grad(dh, "dh2")
        grads[f"L{l}.W2"] = dhq.T @ L.gq
        dg = dhq @ Wl[f"L{l}.W2"]
        du = dg * 2.0 * np.maximum(L.u, 0.0)
        duq = enc.grad(du, "du")
        grads[f"L{l}.W1"] = duq.T @ L.mq
        dm = duq @ Wl[f"L{l}.W1"]
        dh = dh + rmsnorm_bwd(dm, L.m, L.r2)
        # attention: h_mid = h_in + o Wo^T
        dhq = enc.grad(dh, "dh1")
        grads[f"L{l}.Wo"] = dhq.T @ L.oq
        do = (dhq @ Wl[f"L{l}.Wo"]).reshape(B, T, H, Dh)
        Hkv = s.kv_heads
        dqn = np.empty_like(do)
        dkn = np.empty((B, T, Hkv, Dh))
        dv = np.empty((B, T, Hkv, Dh))
        for b in range(B):
            qb = L.qn[b].transpose(1, 0, 2)
            kb = expand_kv(L.kn[b].transpose(1, 0, 2), H)
            vb = expand_kv(L.v[b].transpose(1, 0, 2), H)
            dq_, dk_, dv_ = attention_bwd(do[b].transpose(1, 0, 2), qb, kb, vb, wins[l])
            dqn[b] = dq_.transpose(1, 0, 2)
            dkn[b] = reduce_kv(dk_, Hkv).transpose(1, 0, 2)
            dv[b] = reduce_kv(dv_, Hkv).transpose(1, 0, 2)
        dq = rope_bwd(rmsnorm_bwd(dqn, L.qn, L.rq), cos, sin).reshape(B * T, d)
        dk = rope_bwd(rmsnorm_bwd(dkn, L.kn, L.rk), cos, sin).reshape(B * T, Hkv * Dh)
        dv = dv.reshape(B * T, Hkv * Dh)
        dq, dk, dv = enc.grad_fused(dq, dk, dv)   # the fused projection's output gradient
        grads[f"L{l}.Wq"] = dq.T @ L.aq
        grads[f"L{l}.Wk"] = dk.T @ L.aq
        grads[f"L{l}.Wv"] = dv.T @ L.aq
        da = dq @ Wl[f"L{l}.Wq"] + dk @ Wl[f"L{l}.Wk"] + dv @ Wl[f"L{l}.Wv"]
        dh = dh + rmsnorm_bwd(da, L.a, L.r1)
        del L
    dE = np.zeros((s.vocab, d))
    np.add.at(dE, X.reshape(-1), dh)
    grads["E"] = dE
    return loss, grads

