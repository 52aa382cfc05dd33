"""GPU parity of KV-cache inference (``gpt_prefill`` / ``gpt_decode``)
against the fp64 oracle's logits.

Prefill n tokens, then decode the following tokens of the same seeded
sequence one position at a time (teacher forcing); every returned logit
row must match the oracle's logits at that position (the oracle runs the
plain full-sequence forward).  The bar: per (row, position) cosine >= 0.9995
and max |error| <= 0.05 -- the bf16 step's forward reaches the same per-row
log-sum-exp to 3e-2 -- with the argmax agreeing wherever the oracle's top
two logits are more than 0.1 apart.
"""
import ctypes

import numpy as np
import pytest

import gpt_inputs as gi
from tests.gpu_common import SMALL, cosine, log

pytestmark = pytest.mark.gpu

INFER = {
    "bf16_mid": SMALL["bf16_mid"],
    # several 256-key attention splits: full layer sees up to 600 keys, the
    # windowed layer 300
    "infer_mid": gi.GPTShape("infer_mid", depth=2, d_model=256, n_head=2, head_dim=128, mlp_hidden=1024,
                             vocab=1000, seq_len=600, batch=3, window=300, window_pattern="SL",
                             precision="bf16", token_dist="zipf"),
    "dh64": gi.GPTShape("dh64", depth=3, d_model=192, n_head=3, head_dim=64, mlp_hidden=768, vocab=520,
                        seq_len=320, batch=5, window=100, window_pattern="SSL", precision="bf16",
                        token_dist="uniform"),
    # grouped-query attention: 4 query heads share 2 key/value heads
    "gqa_dh64": gi.GPTShape("gqa_dh64", depth=2, d_model=256, n_head=4, head_dim=64, mlp_hidden=512, vocab=520,
                            seq_len=300, batch=3, window=90, window_pattern="SL", precision="bf16",
                            token_dist="uniform", n_kv_head=2),
}


def _check_logits(z, ref, where):
    assert np.all(np.isfinite(z)), where
    for b in range(ref.shape[0]):
        c = cosine(z[b], ref[b])
        err = np.max(np.abs(z[b] - ref[b]))
        assert c >= 0.9995 and err <= 0.05, (where, b, c, err)
        top2 = np.sort(ref[b])[-2:]
        if top2[1] - top2[0] > 0.1:
            assert np.argmax(z[b]) == np.argmax(ref[b]), (where, b)


@pytest.mark.parametrize("name", list(INFER))
def test_prefill_then_decode_matches_oracle(name):
    import decoder_only_transformer_fwd_amd as G
    from oracle import gpt_oracle as O
    s = INFER[name]
    W8 = gi.make_weights(s)
    X, _ = gi.make_tokens(s)
    ref = O.logits(s, gi.weights_f64(s, W8), X)   # [B, T, V]
    n0 = s.seq_len // 3 + 1
    log(f"inference parity: {name}, prefill {n0}, decode to {s.seq_len - 1}")
    sess = G.Session(s, W8)
    sess.infer_init()
    z = sess.prefill(X[:, :n0]).cpu().numpy()
    _check_logits(z, ref[:, n0 - 1], f"prefill {n0}")
    for pos in range(n0, s.seq_len):
        z = sess.decode(X[:, pos], pos).cpu().numpy()
        _check_logits(z, ref[:, pos], f"decode {pos}")
    sess.close()


def test_prefill_and_decode_paths_agree():
    """Logits at position p from a prefill of p+1 tokens and from a prefill
    of p tokens plus one decode step."""
    import decoder_only_transformer_fwd_amd as G
    s = INFER["infer_mid"]
    W8 = gi.make_weights(s)
    X, _ = gi.make_tokens(s)
    log("prefill vs decode: infer_mid")
    sess = G.Session(s, W8)
    sess.infer_init()
    for p in (1, 255, 256, 511):
        a = sess.prefill(X[:, :p + 1]).cpu().numpy()
        sess.prefill(X[:, :p])
        b = sess.decode(X[:, p], p).cpu().numpy()
        for r in range(s.batch):
            assert cosine(a[r], b[r]) >= 0.9999 and np.max(np.abs(a[r] - b[r])) <= 0.03, (p, r)
    sess.close()


def test_full_size_decode_matches_oracle_row():
    """d24 (B 8, the benchmark's launch configuration): prefill 1024 tokens,
    decode 8; row 0 against the oracle's logits of that row."""
    import decoder_only_transformer_fwd_amd as G
    from oracle import gpt_oracle as O
    s = gi.preset("d24")
    n0, steps = 1024, 8
    W8 = gi.make_weights(s)
    X, _ = gi.make_tokens(s)
    log("inference at d24: prefill 1024, decode 8")
    sess = G.Session(s, W8)
    sess.infer_init()
    zs = [sess.prefill(X[:, :n0]).cpu().numpy()]
    for pos in range(n0, n0 + steps):
        zs.append(sess.decode(X[:, pos], pos).cpu().numpy())
    sess.close()
    s1 = s.replace(batch=1, seq_len=n0 + steps)
    ref = O.logits(s1, gi.weights_f64(s, W8), X[:1, :n0 + steps])[0]
    for k, z in enumerate(zs):
        _check_logits(z[:1], ref[None, n0 - 1 + k], f"position {n0 - 1 + k}")


def test_inference_errors():
    import decoder_only_transformer_fwd_amd as G
    s = INFER["bf16_mid"]
    W8 = gi.make_weights(s)
    X, _ = gi.make_tokens(s)
    log("inference argument checks: bf16_mid")
    sess = G.Session(s, W8)
    sess.infer_init()
    t = sess.torch
    tok = t.from_numpy(np.ascontiguousarray(X)).to(sess.device)
    lib = G._lib
    kv, lg = sess.kv.data_ptr(), sess.logits.data_ptr()
    assert lib.gpt_prefill(sess.handle, tok.data_ptr(), s.seq_len + 1, kv, lg) == G.GPT_EINVAL
    assert lib.gpt_prefill(sess.handle, tok.data_ptr(), 0, kv, lg) == G.GPT_EINVAL
    assert lib.gpt_decode(sess.handle, tok.data_ptr(), s.seq_len, kv, lg) == G.GPT_EINVAL
    assert lib.gpt_decode(sess.handle, tok.data_ptr(), 0, kv, lg) == G.GPT_EINVAL
    bad = tok[:, 0].clone()
    bad[1] = s.vocab
    sess.prefill(X[:, :10])
    assert lib.gpt_decode(sess.handle, bad.data_ptr(), 10, kv, lg) == G.GPT_ETOKEN
    sess.close()
    # fp32 models are trained, not served
    s32 = SMALL["tiny"]
    sess = G.Session(s32, gi.make_weights(s32))
    nb = G.gpt_kv_cache_bytes(sess.cfg)
    kv32 = t.empty(nb, dtype=t.uint8, device=sess.device)
    lg32 = t.empty((s32.batch, s32.vocab), dtype=t.float32, device=sess.device)
    tk = t.zeros((s32.batch, 4), dtype=t.int32, device=sess.device)
    assert lib.gpt_prefill(sess.handle, tk.data_ptr(), 4, kv32.data_ptr(), lg32.data_ptr()) == G.GPT_EINVAL
    sess.close()


def test_graph_replays_match_eager_steps():
    """Decoding steps replay one captured HIP graph; profiled steps run
    eagerly.  Every replay, with eager work and synchronisation in between,
    must give the eager step's logits bit for bit."""
    import decoder_only_transformer_fwd_amd as G
    s = INFER["infer_mid"]
    W8 = gi.make_weights(s)
    X, _ = gi.make_tokens(s)
    n0, steps = 250, 12
    log("decode graph vs eager: infer_mid")
    sess = G.Session(s, W8)
    sess.infer_init()
    t = sess.torch
    sess.profile(True)
    sess.prefill(X[:, :n0])
    eager = [sess.decode(X[:, p], p).clone() for p in range(n0, n0 + steps)]
    sess.profile(False)
    sess.prefill(X[:, :n0])
    for k, p in enumerate(range(n0, n0 + steps)):
        z = sess.decode(X[:, p], p)
        assert bool((z == eager[k]).all()), p
        junk = t.randn(1000, device=sess.device).sum()   # eager work between replays
        t.cuda.synchronize()
        del junk
    sess.close()


def test_fp8_model_serves_with_its_bf16_weights():
    """An FP8-configured model prefills and decodes with bf16 products on its
    bf16 weights: the same logits, bit for bit, as the bf16-configured model
    with the same weights."""
    import decoder_only_transformer_fwd_amd as G
    s8 = SMALL["fp8_mid"]
    sb = s8.replace(precision="bf16")
    W8 = gi.make_weights(s8)
    X, _ = gi.make_tokens(s8)
    log("fp8 model inference vs bf16 model: fp8_mid")
    out = []
    for s in (s8, sb):
        sess = G.Session(s, W8)
        sess.infer_init()
        zs = [sess.prefill(X[:, :100]).clone()]
        for p in range(100, 104):
            zs.append(sess.decode(X[:, p], p).clone())
        out.append(zs)
        sess.close()
    for a, b in zip(*out):
        assert bool((a == b).all())
