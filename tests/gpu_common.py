"""Helpers shared by the GPU tests: workloads, parity metrics, oracle calls."""
import sys

import numpy as np

import gpt_inputs as gi


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def cosine(a: np.ndarray, b: np.ndarray) -> float:
    a = a.reshape(-1).astype(np.float64)
    b = b.reshape(-1).astype(np.float64)
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 or nb == 0:
        return 1.0 if na == nb else 0.0
    return float(a @ b / (na * nb))


# Tolerances: bf16 step within 1e-2 relative loss and per-tensor gradient
# cosine >= 0.999; fp32 step within 1e-5 relative loss.  The fp32 gradient
# bar (cosine >= 0.99999, max error <= 1e-3 of the tensor's largest entry)
# follows from fp32 accumulation over at most a few thousand terms.
TOL = {
    "fp32": dict(loss_rel=1e-5, cos=0.99999, maxrel=1e-3),
    "bf16": dict(loss_rel=1e-2, cos=0.999, maxrel=None),
    "fp8": dict(loss_rel=3e-2, cos=0.99, maxrel=None),
}

# Step workloads small enough for the oracle to finish in seconds.  They keep
# the real head dims and span several GEMM / attention tiles with ragged
# tails (rows, vocab and sequence not multiples of the tiles), plus
# sliding-window layers.
SMALL = {
    "tiny": gi.preset("tiny"),
    "fp32_win": gi.GPTShape("fp32_win", depth=3, d_model=128, n_head=2, head_dim=64, mlp_hidden=256,
                            vocab=520, seq_len=150, batch=2, window=40, window_pattern="SSL",
                            precision="fp32", token_dist="uniform"),
    "bf16_mid": gi.GPTShape("bf16_mid", depth=2, d_model=256, n_head=2, head_dim=128, mlp_hidden=1024,
                            vocab=1000, seq_len=200, batch=2, window=64, window_pattern="SL",
                            precision="bf16", token_dist="zipf"),
    "d12_short": gi.preset("d12", seq_len=256, batch=1),
    "d24_short": gi.preset("d24", seq_len=384, batch=1, window=128),
    # fp8 linear layers (B*T a multiple of 64)
    "fp8_mid": gi.GPTShape("fp8_mid", depth=2, d_model=256, n_head=2, head_dim=128, mlp_hidden=1024,
                           vocab=1000, seq_len=224, batch=2, window=64, window_pattern="SL",
                           precision="fp8", token_dist="zipf"),
    "d24_fp8_short": gi.preset("d24-fp8", seq_len=384, batch=1, window=128),
    # grouped-query attention: query heads sharing key/value heads
    "gqa_fp32": gi.GPTShape("gqa_fp32", depth=2, d_model=128, n_head=4, head_dim=32, mlp_hidden=256,
                            vocab=520, seq_len=150, batch=2, window=40, window_pattern="SL",
                            precision="fp32", token_dist="uniform", n_kv_head=2),
    "gqa_bf16": gi.GPTShape("gqa_bf16", depth=2, d_model=512, n_head=4, head_dim=128, mlp_hidden=1024,
                            vocab=1000, seq_len=200, batch=2, window=64, window_pattern="SL",
                            precision="bf16", token_dist="zipf", n_kv_head=1),
    "d24_gqa_short": gi.preset("d24", seq_len=384, batch=1, window=128, n_kv_head=4),
    # sequences of 192 tokens, three rows: the 256- and 128-row tiles of the
    # QKV product (with the rotary epilogue) straddle sequence boundaries and
    # end past the last row
    "bf16_t192": gi.GPTShape("bf16_t192", depth=2, d_model=1536, n_head=12, head_dim=128, mlp_hidden=2048,
                             vocab=1000, seq_len=192, batch=3, window=64, window_pattern="SL",
                             precision="bf16", token_dist="zipf"),
    "gqa_t192": gi.GPTShape("gqa_t192", depth=2, d_model=512, n_head=4, head_dim=128, mlp_hidden=1024,
                            vocab=1000, seq_len=192, batch=3, window=64, window_pattern="SL",
                            precision="bf16", token_dist="zipf", n_kv_head=2),
    # skewed ids over many positions: the embedding gradient's long runs
    # (ids with more than 256 rows, summed in 128-row segments) at a size the
    # oracle compares whole
    "zipf_long_runs": gi.GPTShape("zipf_long_runs", depth=1, d_model=256, n_head=2, head_dim=128, mlp_hidden=512,
                                  vocab=1000, seq_len=2048, batch=2, window=0, window_pattern="L",
                                  precision="bf16", token_dist="zipf"),
    "gqa_fp8": gi.GPTShape("gqa_fp8", depth=2, d_model=256, n_head=2, head_dim=128, mlp_hidden=1024,
                           vocab=1000, seq_len=224, batch=2, window=64, window_pattern="SL",
                           precision="fp8", token_dist="zipf", n_kv_head=1),
}


def oracle_step(s):
    from oracle import gpt_oracle as O
    W8 = gi.make_weights(s)
    W = gi.weights_f64(s, W8)
    X, Y = gi.make_tokens(s)
    loss, G = O.forward_backward(s, W, X, Y)
    return W8, X, Y, loss, G
