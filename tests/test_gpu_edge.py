"""GPU parity of the training step at the degenerate ends of the
configuration space, against the fp64 oracle: one-token sequences, a
one-key attention window, a window wider than the sequence, the smallest
vocabulary, one layer, head_dim 64 in bf16."""
import numpy as np
import pytest

import gpt_inputs as gi
from tests.gpu_common import TOL, cosine, log

pytestmark = pytest.mark.gpu

EDGE = {
    # every sequence is a single token: attention sees only itself
    "t1": gi.GPTShape("t1", depth=1, d_model=128, n_head=1, head_dim=128, mlp_hidden=256, vocab=64,
                      seq_len=1, batch=5, precision="bf16", token_dist="uniform"),
    # a one-key window on the first layer (self only), full causal on the last
    "w1": gi.GPTShape("w1", depth=2, d_model=128, n_head=2, head_dim=64, mlp_hidden=256, vocab=200,
                      seq_len=130, batch=2, window=1, window_pattern="SL", precision="bf16",
                      token_dist="zipf"),
    # window wider than the sequence (clipped to it), the smallest vocabulary
    "wide_v8": gi.GPTShape("wide_v8", depth=2, d_model=192, n_head=3, head_dim=64, mlp_hidden=320, vocab=8,
                           seq_len=70, batch=3, window=500, window_pattern="S", precision="bf16",
                           token_dist="uniform"),
    "fp32_t1": gi.GPTShape("fp32_t1", depth=2, d_model=64, n_head=2, head_dim=32, mlp_hidden=128, vocab=96,
                           seq_len=1, batch=7, precision="fp32", token_dist="uniform"),
}


@pytest.mark.parametrize("name", list(EDGE))
def test_degenerate_shapes_match_oracle(name):
    import decoder_only_transformer_fwd_amd as G
    from oracle import gpt_oracle as O
    s = EDGE[name]
    W8 = gi.make_weights(s)
    X, Y = gi.make_tokens(s)
    loss_ref, G_ref = O.forward_backward(s, gi.weights_f64(s, W8), X, Y)
    log(f"edge parity: {name} {s}")
    sess = G.Session(s, W8)
    sess.set_tokens(X, Y)
    loss = sess.step()
    Gg = sess.grads_numpy()
    tol = TOL[s.precision]
    rel = abs(loss - loss_ref) / abs(loss_ref)
    log(f"  loss gpu={loss:.8f} oracle={loss_ref:.8f} rel={rel:.2e}")
    assert rel <= tol["loss_rel"]
    # With one visible key the softmax has no derivative, so the oracle's Wq
    # and Wk gradients are exactly zero.  The GPU forms them from dP - D with
    # D = rowsum(dO * O): in bf16, P enters the P V product rounded to bf16
    # while its row sum stays fp32, so O differs from v by up to 2^-9
    # relative, and dP - D leaves noise of that order (bar 2^-8 of the
    # largest gradient entry); in fp32 only summation-order noise.
    scale = max(np.max(np.abs(g)) for g in G_ref.values())
    for n, g_ref in G_ref.items():
        if not np.any(g_ref):
            noise = np.max(np.abs(Gg[n])) / scale
            log(f"  {n}: oracle zero, gpu max |g| / scale = {noise:.1e}")
            assert noise <= (1e-6 if s.precision == "fp32" else 2.0 ** -8), (n, noise)
            continue
        c = cosine(Gg[n], g_ref)
        assert c >= tol["cos"], (n, c)
        if tol["maxrel"] is not None:
            assert np.max(np.abs(Gg[n] - g_ref)) / np.max(np.abs(g_ref)) <= tol["maxrel"], n
    sess.close()
