"""Seeded synthetic workloads for the GPT training step.

This module is shared by the GPU path's tests/bench and by the CPU oracle.  It
holds workload definitions (shapes, layer pattern, dtype policy) and the seeded
random draws (weights, token ids).  It contains none of the method's
arithmetic: no norm, projection, attention or loss is computed here.

Recipe (stated once, used everywhere):
  * weights: numpy ``Generator(PCG64(weight_seed))``; tensors are drawn in
    parameter-layout order (E, then per layer Wq, Wk, Wv, Wo, W1, W2, then U)
    as fp64 standard normals times ``init_std`` (0.02), converted to fp32 with
    round-to-nearest-even, then (bf16 configs) to bf16 with round-to-nearest-
    even on the fp32 bit pattern.  Shapes are [out, in] like a linear layer.
  * tokens: ``Generator(PCG64(token_seed))`` draws B rows of T+1 ids; the
    inputs are ids[:, :T] and the next-token targets ids[:, 1:].
    'uniform' ids come from ``integers(0, V)``; 'zipf' ids use p(k) ~ k**-s
    for ranks k = 1..V (id = k-1) sampled by inverse CDF on an fp64 CDF with
    ``searchsorted(cdf, u, side='right')``.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Tuple

import numpy as np

__all__ = [
    "GPTShape", "PRESETS", "preset", "param_shapes", "layer_windows",
    "make_weights", "make_tokens", "bf16_bits_from_f32", "bf16_bits_to_f64",
    "zipf_probabilities", "weights_f64", "grad_sample_indices", "grad_full_rows",
]


@dataclasses.dataclass(frozen=True)
class GPTShape:
    """Shape and policy of one workload (one forward+backward step)."""
    name: str
    depth: int
    d_model: int
    n_head: int
    head_dim: int
    mlp_hidden: int
    vocab: int
    seq_len: int
    batch: int
    window: int = 0            # keys per sliding window (incl. self); 0 = none
    window_pattern: str = "L"  # cycled over layers, last layer forced to 'L'
    rope_base: float = 10000.0
    norm_eps: float = 1e-6
    precision: str = "bf16"    # 'fp32' | 'bf16' | 'fp8'
    token_dist: str = "uniform"  # 'uniform' | 'zipf'
    zipf_s: float = 1.1
    init_std: float = 0.02
    weight_seed: int = 0
    token_seed: int = 1
    n_kv_head: int = 0         # key/value heads (grouped-query attention); 0 = n_head

    @property
    def bt(self) -> int:
        return self.batch * self.seq_len

    @property
    def kv_heads(self) -> int:
        """Key/value heads: n_kv_head, or n_head when it is 0 (plain
        multi-head attention).  Query head h reads key/value head
        h // (n_head // kv_heads)."""
        return self.n_kv_head or self.n_head

    @property
    def param_dtype(self) -> str:
        return "fp32" if self.precision == "fp32" else "bf16"

    def replace(self, **kw) -> "GPTShape":
        return dataclasses.replace(self, **kw)


PRESETS: Dict[str, GPTShape] = {
    "tiny": GPTShape("tiny", depth=2, d_model=64, n_head=2, head_dim=32,
                     mlp_hidden=256, vocab=2048, seq_len=128, batch=1,
                     precision="fp32", token_dist="uniform"),
    "d12": GPTShape("d12", depth=12, d_model=768, n_head=6, head_dim=128,
                    mlp_hidden=3072, vocab=32768, seq_len=2048, batch=8,
                    precision="bf16", token_dist="uniform"),
    "d20": GPTShape("d20", depth=20, d_model=1280, n_head=10, head_dim=128,
                    mlp_hidden=5120, vocab=65536, seq_len=2048, batch=16,
                    precision="bf16", token_dist="zipf"),
    "d24": GPTShape("d24", depth=24, d_model=1536, n_head=12, head_dim=128,
                    mlp_hidden=6144, vocab=32768, seq_len=2048, batch=8,
                    window=1024, window_pattern="SSSL",
                    precision="bf16", token_dist="zipf"),
    "d24-fp8": GPTShape("d24-fp8", depth=24, d_model=1536, n_head=12,
                        head_dim=128, mlp_hidden=6144, vocab=32768,
                        seq_len=2048, batch=8, window=1024,
                        window_pattern="SSSL", precision="fp8",
                        token_dist="zipf"),
}


def preset(name: str, **overrides) -> GPTShape:
    return PRESETS[name].replace(**overrides) if overrides else PRESETS[name]


def layer_windows(s: GPTShape) -> List[int]:
    """Per-layer key window (number of most recent keys incl. self).

    Layer l takes ``window_pattern[l % len]``; the last layer is always 'L'.
    'L' means full causal context, returned as ``seq_len``.
    """
    out = []
    for l in range(s.depth):
        c = s.window_pattern[l % len(s.window_pattern)]
        if l == s.depth - 1:
            c = "L"
        if c == "L":
            out.append(s.seq_len)
        elif c == "S":
            if s.window <= 0:
                raise ValueError("pattern has 'S' but window <= 0")
            out.append(min(s.window, s.seq_len))
        else:
            raise ValueError(f"bad window pattern char {c!r}")
    return out


def param_shapes(s: GPTShape) -> List[Tuple[str, Tuple[int, int]]]:
    """(name, [rows, cols]) in parameter-layout order."""
    d, f, v = s.d_model, s.mlp_hidden, s.vocab
    dkv = s.kv_heads * s.head_dim
    out = [("E", (v, d))]
    for l in range(s.depth):
        out += [(f"L{l}.Wq", (d, d)), (f"L{l}.Wk", (dkv, d)),
                (f"L{l}.Wv", (dkv, d)), (f"L{l}.Wo", (d, d)),
                (f"L{l}.W1", (f, d)), (f"L{l}.W2", (d, f))]
    out.append(("U", (v, d)))
    return out


def bf16_bits_from_f32(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern (uint16), round-to-nearest-even, NaN kept."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x32)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """bf16 bit pattern (uint16) -> exact fp64 value."""
    u = (np.asarray(b, dtype=np.uint32) << 16).astype(np.uint32)
    return u.view(np.float32).astype(np.float64)


def make_weights(s: GPTShape, zero_lm_head: bool = False) -> Dict[str, np.ndarray]:
    """Seeded weights.  fp32 configs: float32 arrays; otherwise uint16 bf16 bits.

    Draw order is the layout order of ``param_shapes`` so that every tensor's
    values depend only on the seed and the shapes before it.
    """
    rng = np.random.Generator(np.random.PCG64(s.weight_seed))
    out = {}
    for name, shp in param_shapes(s):
        x = (rng.standard_normal(shp) * s.init_std).astype(np.float32)
        if name == "U" and zero_lm_head:
            x[...] = 0.0
        out[name] = x if s.param_dtype == "fp32" else bf16_bits_from_f32(x)
    return out


def weights_f64(s: GPTShape, w: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    """The exact fp64 values of the weight bytes ``make_weights`` produced."""
    if s.param_dtype == "fp32":
        return {k: v.astype(np.float64) for k, v in w.items()}
    return {k: bf16_bits_to_f64(v) for k, v in w.items()}


def zipf_probabilities(vocab: int, s: float) -> np.ndarray:
    k = np.arange(1, vocab + 1, dtype=np.float64)
    p = k ** (-s)
    return p / p.sum()


def make_tokens(s: GPTShape) -> Tuple[np.ndarray, np.ndarray]:
    """(inputs, targets), both int32 [B, T]; rows of T+1 ids split by one."""
    rng = np.random.Generator(np.random.PCG64(s.token_seed))
    n = (s.batch, s.seq_len + 1)
    if s.token_dist == "uniform":
        ids = rng.integers(0, s.vocab, size=n)
    elif s.token_dist == "zipf":
        cdf = np.cumsum(zipf_probabilities(s.vocab, s.zipf_s))
        u = rng.random(n)
        ids = np.searchsorted(cdf, u, side="right")
        ids = np.minimum(ids, s.vocab - 1)
    else:
        raise ValueError(s.token_dist)
    ids = ids.astype(np.int32)
    return np.ascontiguousarray(ids[:, :-1]), np.ascontiguousarray(ids[:, 1:])


def grad_full_rows(s: GPTShape, X: np.ndarray, seed: int = 4321) -> Dict[str, np.ndarray]:
    """Seeded row indices (sorted, int64) of three gradients whose rows the
    full-size checks compare whole: 256 embedding rows among the ids the
    batch X uses, 64 rows of layer 0's Wq and 64 of the last layer's W1."""
    rng = np.random.Generator(np.random.PCG64(seed))
    seen = np.unique(X)
    out = {"E": np.sort(rng.choice(seen, size=min(256, seen.size), replace=False)).astype(np.int64)}
    for name in ("L0.Wq", f"L{s.depth - 1}.W1"):
        r = dict(param_shapes(s))[name][0]
        out[name] = np.sort(rng.choice(r, size=min(64, r), replace=False)).astype(np.int64)
    return out


def grad_sample_indices(s: GPTShape, n_per_tensor: int, seed: int = 1234) -> Dict[str, np.ndarray]:
    """Seeded flat indices (sorted, int64) at which full-size gradients are sampled."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {}
    for name, (r, c) in param_shapes(s):
        k = min(n_per_tensor, r * c)
        out[name] = np.sort(rng.choice(r * c, size=k, replace=False)).astype(np.int64)
    return out
