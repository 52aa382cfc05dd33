"""GPU parity of the optimizer step (Muon + AdamW, ``gpt_optim_step``)
against the fp64 optimizer oracle.

Inputs are seeded synthetic gradients in the parameter layout, scaled so
that their global norm exceeds the clip (clipping active).  Muon's
orthogonalisation runs in bf16, as the published method does: each matrix's
update (new master minus old) must match the oracle's to cosine >= 0.999 with
a norm within 1 % (five bf16 Newton-Schulz iterations reproduce the fp64
map to about 1e-4 in cosine).  AdamW is elementwise fp32: each entry's
update within 1e-4 of its learning rate.  The bf16 weight buffer must hold
the masters rounded to nearest even, bit for bit.
"""
import ctypes

import numpy as np
import pytest

import gpt_inputs as gi
from tests.gpu_common import SMALL, cosine, log

pytestmark = pytest.mark.gpu

HP = dict(matrix_lr=0.02, momentum=0.95, nesterov=1, ns_steps=5, embedding_lr=0.2, unembedding_lr=0.004,
          beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1, grad_clip=1.0)


def _oracle_hp(step, **over):
    from oracle import optim_oracle as OO
    kw = {**HP, **over}
    return OO.OptimParams(lr_matrix=kw["matrix_lr"], momentum=kw["momentum"], nesterov=bool(kw["nesterov"]),
                          ns_steps=kw["ns_steps"], lr_embedding=kw["embedding_lr"],
                          lr_unembedding=kw["unembedding_lr"], beta1=kw["beta1"], beta2=kw["beta2"],
                          eps=kw["eps"], weight_decay=kw["weight_decay"], grad_clip=kw["grad_clip"], step=step)


def _gpu_hp(step, **over):
    import decoder_only_transformer_fwd_amd as G
    return G.optim_params(**{**HP, **over}, step=step)


def synthetic_grads(s, seed, scale=1e-3):
    """Seeded gradients per tensor: Gaussian plus a rank-one part (gradients
    of linear layers are far from isotropic)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {}
    for name, (r, c) in gi.param_shapes(s):
        g = rng.standard_normal((r, c)) + 2.0 * np.outer(rng.standard_normal(r), rng.standard_normal(c)) / np.sqrt(c)
        out[name] = (g * scale).astype(np.float32)
    return out


def _set_grads(sess, grads):
    t = sess.torch
    host = np.zeros(sess.total, dtype=np.float32)
    for name, off, r, c in sess.layout:
        host[off:off + r * c] = grads[name].reshape(-1)
    sess.grads.copy_(t.from_numpy(host).to(sess.device))


def _check_bf16_weights(sess, master):
    """The bf16 weight buffer holds the fp32 masters rounded to nearest even."""
    t = sess.torch
    if sess.shape.precision == "fp32":
        return
    flat = np.zeros(sess.total, dtype=np.float32)
    for name, off, r, c in sess.layout:
        flat[off:off + r * c] = master[name].reshape(-1)
    want = t.from_numpy(flat).to(sess.device).to(t.bfloat16)
    for name, off, r, c in sess.layout:
        got = sess.weights[off:off + r * c]
        assert bool((got.view(t.int16) == want[off:off + r * c].view(t.int16)).all()), name


def _compare(name, d_gpu, d_ref, is_matrix, lr):
    if is_matrix:
        c = cosine(d_gpu, d_ref)
        nr = np.linalg.norm(d_gpu) / np.linalg.norm(d_ref)
        assert c >= 0.999 and abs(nr - 1) <= 0.01, (name, c, nr)
        return c
    err = np.max(np.abs(d_gpu - d_ref))
    assert err <= 1e-4 * lr, (name, err)
    return 1.0


@pytest.mark.parametrize("name", ["tiny", "bf16_mid", "gqa_bf16"])
def test_optimizer_steps_match_oracle(name):
    import decoder_only_transformer_fwd_amd as G
    from oracle import optim_oracle as OO
    s = SMALL[name]
    W8 = gi.make_weights(s)
    master_ref = gi.weights_f64(s, W8)
    state_ref = OO.init_state(s)
    log(f"optimizer parity: {name}")
    sess = G.Session(s, W8)
    sess.optim_init()
    m0 = sess.master_numpy()
    for k in master_ref:
        assert np.array_equal(m0[k].astype(np.float64), master_ref[k]), k
    for step in (1, 2, 3):
        grads = synthetic_grads(s, seed=100 + step, scale=3e-2)
        _set_grads(sess, grads)
        norm = sess.optim_step(_gpu_hp(step), want_norm=True)
        new_ref, state_ref, norm_ref = OO.optim_step(s, master_ref, {k: v.astype(np.float64) for k, v in grads.items()},
                                                     state_ref, _oracle_hp(step))
        assert norm_ref > HP["grad_clip"]   # clipping is active
        assert abs(norm - norm_ref) / norm_ref < 1e-5
        master = sess.master_numpy()
        worst = 2.0
        for k in master_ref:
            is_m = OO.is_matrix_param(k)
            lr = HP["matrix_lr"] if is_m else HP["embedding_lr"] if k == "E" else HP["unembedding_lr"]
            worst = min(worst, _compare(k, master[k] - m0[k], new_ref[k] - master_ref[k], is_m, lr))
        log(f"  step {step}: grad norm gpu={norm:.6f} oracle={norm_ref:.6f}, worst matrix-update cosine {worst:.6f}")
        _check_bf16_weights(sess, master)
        # continue from the GPU's own masters, so that each step is compared
        # on the same starting point
        master_ref = {k: v.astype(np.float64) for k, v in master.items()}
        m0 = master
    sess.close()


def test_orthogonalisation_alone_at_full_size():
    """d24 shapes, momentum off, no decay, no clipping, lr 1: each sampled
    matrix's update is -sqrt(max(1, rows/cols)) * NS(g)."""
    import decoder_only_transformer_fwd_amd as G
    from oracle import optim_oracle as OO
    s = gi.preset("d24")
    W8 = gi.make_weights(s)
    log("orthogonalisation at d24 shapes")
    sess = G.Session(s, W8)
    sess.optim_init()
    m0 = sess.master_numpy()
    grads = synthetic_grads(s, seed=7)
    _set_grads(sess, grads)
    hp = dict(matrix_lr=1.0, momentum=0.0, nesterov=0, weight_decay=0.0, grad_clip=0.0)
    sess.optim_step(_gpu_hp(1, **hp))
    master = sess.master_numpy()
    for k in ["L0.Wq", "L5.Wv", "L23.Wo", "L0.W1", "L11.W1", "L0.W2", "L23.W2"]:
        d_gpu = master[k].astype(np.float64) - m0[k]
        r, c = grads[k].shape
        d_ref = -OO.muon_scale(r, c) * OO.newton_schulz(grads[k].astype(np.float64), 5)
        cs = cosine(d_gpu, d_ref)
        nr = np.linalg.norm(d_gpu) / np.linalg.norm(d_ref)
        log(f"  {k}: cosine {cs:.6f} norm ratio {nr:.5f}")
        assert cs >= 0.999 and abs(nr - 1) <= 0.01, (k, cs, nr)
    sess.close()


def test_full_size_step_adamw_samples_and_determinism():
    """d24: AdamW entries sampled against the oracle; two runs from the same
    start give bit-identical masters."""
    import decoder_only_transformer_fwd_amd as G
    from oracle import optim_oracle as OO
    s = gi.preset("d24")
    W8 = gi.make_weights(s)
    log("optimizer at d24: AdamW samples, determinism")
    grads = synthetic_grads(s, seed=9)
    outs = []
    for _ in range(2):
        sess = G.Session(s, W8)
        sess.optim_init()
        _set_grads(sess, grads)
        norm = sess.optim_step(_gpu_hp(1), want_norm=True)
        outs.append((norm, sess.master_numpy()))
        sess.close()
    norm, master = outs[0]
    assert outs[1][0] == norm
    for k in master:
        assert np.array_equal(master[k], outs[1][1][k]), k
    g64 = {k: v.astype(np.float64) for k, v in grads.items()}
    norm_ref = OO.global_norm(g64)
    assert abs(norm - norm_ref) / norm_ref < 1e-5
    cf = OO.clip_coefficient(norm_ref, HP["grad_clip"])
    hp = _oracle_hp(1)
    W = gi.weights_f64(s, W8)
    rng = np.random.default_rng(3)
    for k, lr in (("E", HP["embedding_lr"]), ("U", HP["unembedding_lr"])):
        rows = rng.choice(W[k].shape[0], size=64, replace=False)
        p_ref, _, _ = OO.adamw_update(W[k][rows], g64[k][rows] * cf, np.zeros_like(W[k][rows]),
                                      np.zeros_like(W[k][rows]), lr, hp)
        err = np.max(np.abs((master[k][rows] - W[k][rows]) - (p_ref - W[k][rows])))
        assert err <= 1e-4 * lr, (k, err)


def test_training_steps_reduce_the_loss():
    """Forward+backward then an optimizer step, repeated on one batch: the
    loss falls."""
    import decoder_only_transformer_fwd_amd as G
    s = SMALL["bf16_mid"]
    W8 = gi.make_weights(s)
    X, Y = gi.make_tokens(s)
    log("training loop: bf16_mid")
    sess = G.Session(s, W8)
    sess.set_tokens(X, Y)
    sess.optim_init()
    losses = []
    for step in range(1, 7):
        losses.append(sess.step())
        sess.optim_step(_gpu_hp(step, weight_decay=0.0))
    losses.append(sess.step())
    log("  losses " + " ".join(f"{x:.4f}" for x in losses))
    assert all(b < a for a, b in zip(losses, losses[1:]))
    assert losses[-1] < losses[0] - 0.5
    sess.close()


def test_bad_optimizer_arguments_are_rejected():
    import decoder_only_transformer_fwd_amd as G
    s = SMALL["tiny"]
    W8 = gi.make_weights(s)
    log("optimizer argument checks: tiny")
    sess = G.Session(s, W8)
    t = sess.torch
    nb = G.gpt_optim_state_bytes(sess.cfg)
    state = t.empty(nb, dtype=t.uint8, device=sess.device)
    hp = _gpu_hp(1)
    # a state that was never prepared
    rc = G._lib.gpt_optim_step(sess.handle, state.data_ptr(), sess.grads.data_ptr(), ctypes.byref(hp), None)
    assert rc == G.GPT_EINVAL
    # too small a state
    assert G._lib.gpt_optim_init(sess.handle, state.data_ptr(), nb - 256) == G.GPT_ESPACE
    G.gpt_optim_init(sess.handle, state.data_ptr(), nb)
    w0 = sess.weights.clone()
    for bad in (dict(momentum=1.0), dict(beta2=1.0), dict(eps=0.0), dict(ns_steps=0), dict(matrix_lr=float("nan")),
                dict(nesterov=2)):
        hpb = _gpu_hp(1, **bad)
        rc = G._lib.gpt_optim_step(sess.handle, state.data_ptr(), sess.grads.data_ptr(), ctypes.byref(hpb), None)
        assert rc == G.GPT_EINVAL, bad
    hpb = _gpu_hp(0)
    assert G._lib.gpt_optim_step(sess.handle, state.data_ptr(), sess.grads.data_ptr(), ctypes.byref(hpb),
                                 None) == G.GPT_EINVAL
    t.cuda.synchronize()
    assert bool((sess.weights == w0).all())   # nothing was enqueued
    sess.close()
