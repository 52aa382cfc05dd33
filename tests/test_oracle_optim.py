"""Pins for the optimizer oracle (Muon + AdamW), against closed forms and
independent evaluations rather than against itself."""
import math

import numpy as np
import pytest

import gpt_inputs as gi
from oracle import optim_oracle as OO


def _svd_orthogonalise(G, steps=5, coeffs=OO.NS_COEFFS, eps=OO.NS_EPS):
    """The Newton-Schulz map acts on singular values only: for
    G = U diag(s) V^T it returns U diag(phi(s / (||G||_F + eps))) V^T with
    phi the scalar quintic a x + b x^3 + c x^5 applied `steps` times."""
    a, b, c = coeffs
    U, s, Vt = np.linalg.svd(G, full_matrices=False)
    x = s / (np.linalg.norm(G) + eps)
    for _ in range(steps):
        x = a * x + b * x ** 3 + c * x ** 5
    return (U * x) @ Vt


@pytest.mark.parametrize("shape", [(6, 6), (9, 4), (4, 9), (32, 128)])
def test_newton_schulz_acts_on_singular_values(shape):
    rng = np.random.default_rng(sum(shape))
    G = rng.standard_normal(shape) + 3.0 * np.outer(rng.standard_normal(shape[0]), rng.standard_normal(shape[1]))
    np.testing.assert_allclose(OO.newton_schulz(G, 5), _svd_orthogonalise(G), rtol=0, atol=1e-11)
    # a different number of steps is a different map
    assert not np.allclose(OO.newton_schulz(G, 4), _svd_orthogonalise(G))


def test_newton_schulz_pushes_singular_values_towards_one():
    rng = np.random.default_rng(7)
    G = rng.standard_normal((48, 96))
    s = np.linalg.svd(OO.newton_schulz(G, 5), compute_uv=False)
    assert s.min() > 0.5 and s.max() < 1.25


def _muon_original(p, grads, hp):
    """Muon as first published: buf <- mu buf + g, u = g + mu buf (Nesterov),
    orthogonalised through the SVD, scaled by sqrt(max(1, rows/cols))."""
    buf = np.zeros_like(p)
    for g in grads:
        buf = hp.momentum * buf + g
        u = g + hp.momentum * buf if hp.nesterov else buf
        p = p * (1 - hp.lr_matrix * hp.weight_decay) - hp.lr_matrix * math.sqrt(max(1, p.shape[0] / p.shape[1])) \
            * _svd_orthogonalise(u)
    return p


@pytest.mark.parametrize("shape,nesterov", [((24, 24), True), ((40, 10), True), ((10, 40), False)])
def test_muon_matches_the_original_momentum_form(shape, nesterov):
    rng = np.random.default_rng(3)
    hp = OO.OptimParams(lr_matrix=0.05, momentum=0.9, nesterov=nesterov, weight_decay=0.1)
    p0 = rng.standard_normal(shape) * 0.1
    grads = [rng.standard_normal(shape) * 10.0 ** k for k in (0, 1, -1)]
    p, buf = p0, np.zeros(shape)
    for g in grads:
        p, buf = OO.muon_update(p, g, buf, hp)
    # the two momentum forms differ by a factor the normalisation removes (up
    # to its epsilon)
    np.testing.assert_allclose(p, _muon_original(p0, grads, hp), rtol=0, atol=1e-8)


def test_adamw_constant_gradient_takes_sign_steps():
    """With a constant gradient the bias-corrected moments are exactly g and
    g^2, so every step moves each weight by lr * g / (|g| + eps)."""
    rng = np.random.default_rng(5)
    hp = OO.OptimParams(beta1=0.8, beta2=0.95, eps=1e-10, weight_decay=0.0)
    p = rng.standard_normal((5, 7))
    g = rng.standard_normal((5, 7))
    m = np.zeros_like(p)
    v = np.zeros_like(p)
    lr = 0.01
    for t in range(1, 6):
        hp.step = t
        p_new, m, v = OO.adamw_update(p, g, m, v, lr, hp)
        np.testing.assert_allclose(p - p_new, lr * g / (np.abs(g) + hp.eps), rtol=1e-12, atol=1e-15)
        p = p_new


def test_adamw_decoupled_weight_decay():
    """A zero gradient leaves only the decay: p <- p (1 - lr wd)."""
    hp = OO.OptimParams(weight_decay=0.2, step=3)
    p = np.array([[1.0, -2.0]])
    p_new, _, _ = OO.adamw_update(p, np.zeros_like(p), np.zeros_like(p), np.zeros_like(p), 0.5, hp)
    np.testing.assert_allclose(p_new, p * 0.9, rtol=1e-15)


def test_clip_coefficient():
    grads = {"E": np.array([[3.0, 0.0]]), "U": np.array([[0.0, 4.0]])}
    n = OO.global_norm(grads)
    assert n == 5.0
    assert OO.clip_coefficient(n, 1.0) == 1.0 / (5.0 + 1e-6)
    assert OO.clip_coefficient(n, 10.0) == 1.0
    assert OO.clip_coefficient(n, 0.0) == 1.0


def test_optim_step_routes_parameters():
    """First step, no decay: each E / U entry moves by its own AdamW lr (the
    sign step), and each matrix moves by lr * s times a matrix whose singular
    values the Newton-Schulz map has pushed towards one."""
    s = gi.preset("tiny")
    rng = np.random.default_rng(11)
    master = {n: rng.standard_normal(shp) * 0.02 for n, shp in gi.param_shapes(s)}
    # magnitudes bounded away from zero, so that |g| >> eps everywhere
    grads = {n: rng.choice([-1.0, 1.0], size=shp) * rng.uniform(0.5, 1.0, size=shp) * 1e-4
             for n, shp in gi.param_shapes(s)}
    hp = OO.OptimParams(lr_matrix=0.02, lr_embedding=0.2, lr_unembedding=0.004, weight_decay=0.0,
                        grad_clip=1.0, eps=1e-12)
    new, st, norm = OO.optim_step(s, master, grads, OO.init_state(s), hp)
    assert norm < 1.0
    np.testing.assert_allclose(np.abs(master["E"] - new["E"]), 0.2, rtol=1e-6)
    np.testing.assert_allclose(np.abs(master["U"] - new["U"]), 0.004, rtol=1e-6)
    for n, p in master.items():
        if n in ("E", "U"):
            continue
        step = (p - new[n]) / (0.02 * OO.muon_scale(*p.shape))
        sv = np.linalg.svd(step, compute_uv=False)
        # (a square Gaussian matrix keeps a few tiny singular values that
        # five steps do not lift all the way)
        assert np.median(sv) > 0.65 and sv.max() < 1.25, n
        np.testing.assert_allclose(st[n]["buf"], 0.05 * grads[n], rtol=1e-12)
