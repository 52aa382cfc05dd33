"""Pins for the oracle's FP8 configuration (encoded linear-layer operands).

An independent model written with torch on the CPU in float64 and
differentiated by autograd, where every encoding point of the recipe is an
autograd function -- forward operands: encode+decode on the way forward and
pass-through on the way back; gradient operands: identity forward, encode the
incoming gradient on the way back -- must reproduce the oracle's loss and its
hand-derived gradients.  This pins where the encodings sit (which operands,
forward or backward, the fused QKV tensor) and that the oracle's adjoints use
the encoded operands.  The encoder itself is pinned by the codec tests, and
the exact network (all encodings off) by the finite-difference tests.
"""
import math

import numpy as np
import pytest

import gpt_inputs as gi
from oracle import gpt_oracle as O

torch = pytest.importorskip("torch")

SHAPE = gi.GPTShape("fp8_pin", depth=2, d_model=64, n_head=2, head_dim=32, mlp_hidden=256, vocab=128,
                    seq_len=32, batch=2, window=8, window_pattern="SL", precision="fp8", token_dist="uniform")


class _EncFwd(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, fmt):
        return torch.from_numpy(O.fp8_value(x.detach().numpy(), fmt))

    @staticmethod
    def backward(ctx, g):
        return g, None


class _EncGrad(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x):
        return x.clone()

    @staticmethod
    def backward(ctx, g):
        return torch.from_numpy(O.fp8_value(g.detach().numpy(), "e5m2"))


def _torch_step(s, W, X, Y, fp8: bool):
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in W.items()}
    fwd = (lambda x: _EncFwd.apply(x, "e4m3")) if fp8 else (lambda x: x)
    bwd = _EncGrad.apply if fp8 else (lambda x: x)

    def lin(x, w):   # y = enc(x) enc(w)^T, gradient of y encoded
        return bwd(fwd(x) @ fwd(w).T)

    def norm(x):
        return x / torch.sqrt((x * x).mean(-1, keepdim=True) + s.norm_eps)

    B, T, H, Dh, d = s.batch, s.seq_len, s.n_head, s.head_dim, s.d_model
    half = Dh // 2
    inv = s.rope_base ** (-torch.arange(half, dtype=torch.float64) * 2.0 / Dh)
    ang = torch.arange(T, dtype=torch.float64)[:, None] * inv[None]
    c, sn = torch.cos(ang)[None, :, None], torch.sin(ang)[None, :, None]
    i = torch.arange(T)[:, None]
    j = torch.arange(T)[None]
    h = t["E"][torch.from_numpy(X.reshape(-1)).long()]
    for l, win in enumerate(gi.layer_windows(s)):
        a = norm(h)
        wqkv = torch.cat([t[f"L{l}.Wq"], t[f"L{l}.Wk"], t[f"L{l}.Wv"]])
        qkv = lin(a, wqkv)
        q, k, v = (qkv[:, n * d:(n + 1) * d].reshape(B, T, H, Dh) for n in range(3))

        def rot(x):
            x1, x2 = x[..., :half], x[..., half:]
            return torch.cat([x1 * c - x2 * sn, x1 * sn + x2 * c], -1)

        q, k = norm(rot(q)), norm(rot(k))
        sc = torch.einsum("bihd,bjhd->bhij", q, k) / math.sqrt(Dh)
        sc = sc.masked_fill(~((j <= i) & (i - j < win)), float("-inf"))
        o = torch.einsum("bhij,bjhd->bihd", torch.softmax(sc, -1), v).reshape(B * T, d)
        h = h + lin(o, t[f"L{l}.Wo"])
        u = lin(norm(h), t[f"L{l}.W1"])
        h = h + lin(torch.relu(u) ** 2, t[f"L{l}.W2"])
    z = norm(h) @ t["U"].T
    loss = torch.nn.functional.cross_entropy(z, torch.from_numpy(Y.reshape(-1)).long())
    loss.backward()
    return float(loss.detach()), {k: v.grad.detach().numpy() for k, v in t.items()}


@pytest.fixture(scope="module")
def case():
    s = SHAPE
    W = gi.weights_f64(s, gi.make_weights(s))
    X, Y = gi.make_tokens(s)
    return s, W, X, Y


def test_fp8_oracle_matches_autograd_with_encodings(case):
    s, W, X, Y = case
    loss, G = O.forward_backward(s, W, X, Y)          # precision "fp8": encoded operands
    loss_t, G_t = _torch_step(s, W, X, Y, fp8=True)
    assert abs(loss - loss_t) <= 1e-12 * abs(loss)
    for n, g in G.items():
        np.testing.assert_allclose(g, G_t[n], rtol=1e-9, atol=1e-12 * np.max(np.abs(G_t[n])), err_msg=n)


def test_exact_oracle_matches_autograd(case):
    s, W, X, Y = case
    loss, G = O.forward_backward(s, W, X, Y, enc=O.LinearOperands())
    loss_t, G_t = _torch_step(s, W, X, Y, fp8=False)
    assert abs(loss - loss_t) <= 1e-12 * abs(loss)
    for n, g in G.items():
        np.testing.assert_allclose(g, G_t[n], rtol=1e-9, atol=1e-12 * np.max(np.abs(G_t[n])), err_msg=n)


def test_fp8_encoding_changes_the_step_but_slightly(case):
    """The encodings move the loss by well under 1 % and leave every gradient
    pointing the same way (cosine > 0.95) on this small model."""
    s, W, X, Y = case
    l8, G8 = O.forward_backward(s, W, X, Y)
    l, G = O.forward_backward(s, W, X, Y, enc=O.LinearOperands())
    assert l8 != l and abs(l8 - l) < 1e-2 * l
    for n in G:
        a, b = G8[n].reshape(-1), G[n].reshape(-1)
        if np.any(b):
            assert a @ b / (np.linalg.norm(a) * np.linalg.norm(b)) > 0.95, n


def test_fp8_weight_operands_are_representable(case):
    """Each encoded weight is code/scale for one scale per tensor: multiplied
    by its scale it lands exactly on E4M3 values, and the largest magnitude
    maps to 448.  The fused QKV weight shares one scale."""
    from oracle import fp8_codec as F
    s, W, _, _ = case
    Wl = O.Fp8Operands().weights(s, W)
    _, vals = F.finite_table("e4m3")
    for l in range(s.depth):
        for group in (("Wq", "Wk", "Wv"), ("Wo",), ("W1",), ("W2",)):
            orig = np.concatenate([W[f"L{l}.{g}"] for g in group])
            enc = np.concatenate([Wl[f"L{l}.{g}"] for g in group])
            scale = 448.0 / np.max(np.abs(orig))
            y = np.abs(enc) * scale
            assert np.max(y) == pytest.approx(448.0, rel=1e-12)
            nearest = vals[np.abs(y.reshape(-1, 1) - vals[None]).argmin(1)]
            np.testing.assert_allclose(y.reshape(-1), nearest, rtol=1e-12, atol=1e-12)
