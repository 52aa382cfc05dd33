"""FLOP accounting and peak figures used to report tokens/s, MFU and rooflines.

Model FLOPs per token follow the convention of the pages' training log
("Introducing nanochat", pretraining log, "Estimated FLOPs per token"):
6 x (every matrix parameter except the token embedding, lm_head included)
plus 12 x H x Dh x T_eff per layer for attention, with T_eff = T for full
layers; sliding-window layers count T_eff = W (a reading: the pages are
silent on windowed layers).  The algorithmic variant counts only the
(query, key) pairs the causal / window mask leaves visible.
"""
from __future__ import annotations

# MI355X dense peaks (AMD public specification), FLOP/s and byte/s.
PEAK_BF16 = 2.5166e15
PEAK_FP8 = 5.0332e15
PEAK_FP32_MFMA = 157.3e12
PEAK_HBM = 8.0e12


def _windows(s):
    out = []
    for l in range(s.depth):
        c = s.window_pattern[l % len(s.window_pattern)]
        if l == s.depth - 1 or c == "L":
            out.append(s.seq_len)
        else:
            out.append(min(s.window, s.seq_len))
    return out


def scaling_params(s) -> int:
    """Matrix parameters except the token embedding: per layer Wq, Wo [d, d],
    Wk, Wv [Hkv*Dh, d] (d x d without grouped-query attention), W1, W2; plus
    the lm_head."""
    d, f, v, L = s.d_model, s.mlp_hidden, s.vocab, s.depth
    dkv = getattr(s, "kv_heads", s.n_head) * s.head_dim
    return L * (2 * d * d + 2 * dkv * d + 2 * d * f) + v * d


def flops_per_token(s) -> int:
    """Conventional model FLOPs per token (the pages' estimate)."""
    attn = sum(12 * s.n_head * s.head_dim * w for w in _windows(s))
    return 6 * scaling_params(s) + attn


def visible_pairs(T: int, W: int) -> float:
    if W >= T:
        return T * (T + 1) / 2.0
    return W * (W + 1) / 2.0 + (T - W) * W


def algorithmic_flops_per_token(s) -> float:
    """Matrix FLOPs plus attention over visible (query, key) pairs only."""
    attn = sum(12 * s.n_head * s.head_dim * visible_pairs(s.seq_len, w) / s.seq_len for w in _windows(s))
    return 6.0 * scaling_params(s) + attn


def mfu(tokens_per_s: float, s, peak: float = PEAK_BF16) -> float:
    return tokens_per_s * flops_per_token(s) / peak
