"""Gradient accumulation over micro-batches (``gpt_step_accum``) on the GPU.

The mean loss of a batch of B rows is the mean of the mean losses of k
micro-batches of B/k rows, so its gradient is the sum of the micro-batch
gradients, each scaled by 1/k (nanochat's training loop: gradient
accumulation over micro-steps).

* Against the oracle: two micro-batches at grad_scale 1/2 accumulate the
  gradient the fp64 oracle computes for the whole batch (fp32 and bf16), or,
  for the fp8 recipe, whose per-tensor scales are taken per call, the mean of
  the oracle's micro-batch gradients; both to the step's tolerances.
* Exactness at full size, in the configuration the benchmark times: the same
  micro-batch twice at grad_scale 1/2 (store, then accumulate) reproduces a
  plain step bit for bit.  Halving is exact in binary floating point, every
  kernel is deterministic, and each accumulated element is one rounded sum of
  two equal halves.
* A positive power-of-two grad_scale scales every gradient exactly; bad
  arguments are rejected before any work is enqueued.
"""
import ctypes

import numpy as np
import pytest

import gpt_inputs as gi
from tests.gpu_common import SMALL, TOL, cosine, log

pytestmark = pytest.mark.gpu


def _split_rows(X, Y, k):
    b = X.shape[0] // k
    return [(X[i * b:(i + 1) * b], Y[i * b:(i + 1) * b]) for i in range(k)]


ACCUM_CASES = {
    "fp32_win": SMALL["fp32_win"],                       # batch 2 -> 2 x 1
    "bf16_mid_b4": SMALL["bf16_mid"].replace(batch=4),   # batch 4 -> 2 x 2
    "fp8_mid_b4": SMALL["fp8_mid"].replace(batch=4),     # batch 4 -> 2 x 2
}


@pytest.mark.parametrize("name", list(ACCUM_CASES))
def test_accumulated_micro_batches_match_oracle(name):
    import decoder_only_transformer_fwd_amd as G
    from oracle import gpt_oracle as O
    s = ACCUM_CASES[name]
    k = 2
    sm = s.replace(batch=s.batch // k)
    W8 = gi.make_weights(s)
    W = gi.weights_f64(s, W8)
    X, Y = gi.make_tokens(s)
    parts = _split_rows(X, Y, k)
    if s.precision == "fp8":
        # the recipe scales each call's tensors by their own amax: the
        # reference is the mean of the oracle's micro-batch results
        refs = [O.forward_backward(sm, W, x, y) for x, y in parts]
        loss_ref = float(np.mean([r[0] for r in refs]))
        G_ref = {n: sum(r[1][n] for r in refs) / k for n in refs[0][1]}
    else:
        loss_ref, G_ref = O.forward_backward(s, W, X, Y)
    log(f"accumulation parity: {name} ({k} micro-batches of {sm.batch})")
    sess = G.Session(sm, W8)
    losses = []
    for i, (x, y) in enumerate(parts):
        sess.set_tokens(x, y)
        losses.append(sess.step_accum(1.0 / k, accumulate=i > 0))
    loss = float(np.mean(losses))
    Gg = sess.grads_numpy()
    tol = TOL[s.precision]
    rel = abs(loss - loss_ref) / abs(loss_ref)
    log(f"  mean micro loss gpu={loss:.8f} oracle={loss_ref:.8f} rel={rel:.2e}")
    assert rel <= tol["loss_rel"]
    worst = (2.0, None)
    for n, g_ref in G_ref.items():
        if not np.any(g_ref):
            continue
        c = cosine(Gg[n], g_ref)
        worst = min(worst, (c, n))
        assert c >= tol["cos"], (n, c)
        if tol["maxrel"] is not None:
            err = np.max(np.abs(Gg[n] - g_ref)) / np.max(np.abs(g_ref))
            assert err <= tol["maxrel"], (n, err)
    log(f"  worst grad cosine {worst[0]:.7f} ({worst[1]})")
    # rows of E that no token of either micro-batch uses stay exactly zero
    unseen = np.setdiff1d(np.arange(s.vocab), np.unique(X))
    assert np.all(Gg["E"][unseen] == 0.0)
    sess.close()


@pytest.mark.parametrize("name", ["d12", "d24", "d24-fp8"])
def test_two_half_steps_equal_one_step_bitwise(name):
    import decoder_only_transformer_fwd_amd as G
    s = gi.preset(name)
    W8 = gi.make_weights(s)
    X, Y = gi.make_tokens(s)
    log(f"accumulation exactness: {name}")
    sess = G.Session(s, W8)
    sess.set_tokens(X, Y)
    loss = sess.step()
    g1 = sess.grads.clone()
    # fill with garbage first: the storing call must overwrite every element
    sess.grads.fill_(float("nan"))
    l_a = sess.step_accum(0.5, accumulate=False)
    l_b = sess.step_accum(0.5, accumulate=True)
    assert l_a == loss and l_b == loss
    diff = int((sess.grads != g1).sum().item())
    log(f"  elements that differ: {diff} of {g1.numel()}")
    assert diff == 0
    sess.close()


def test_grad_scale_is_exact_for_powers_of_two():
    import decoder_only_transformer_fwd_amd as G
    s = SMALL["bf16_mid"]
    W8 = gi.make_weights(s)
    X, Y = gi.make_tokens(s)
    log("grad_scale: bf16_mid")
    sess = G.Session(s, W8)
    sess.set_tokens(X, Y)
    sess.step()
    g1 = sess.grads.clone()
    for scale in (0.25, 4.0, 0.0):
        sess.step_accum(scale, accumulate=False)
        assert bool((sess.grads == g1 * scale).all()), scale
    # a negative scale is checked only up to rounding: negating the logit
    # gradient was measured not to negate every gradient bit for bit
    sess.step_accum(-1.0, accumulate=False)
    c = cosine(-sess.grads.cpu().numpy(), g1.cpu().numpy())
    log(f"  grad_scale -1: cosine {c:.9f}")
    assert c >= 0.9999
    # accumulating a zero-scaled step leaves the buffer as it was
    sess.step()
    sess.step_accum(0.0, accumulate=True)
    assert bool((sess.grads == g1).all())
    sess.close()


def test_bad_accumulation_arguments_are_rejected():
    import decoder_only_transformer_fwd_amd as G
    s = SMALL["tiny"]
    W8 = gi.make_weights(s)
    X, Y = gi.make_tokens(s)
    log("accumulation argument checks: tiny")
    sess = G.Session(s, W8)
    sess.set_tokens(X, Y)
    sess.step()
    g1 = sess.grads.clone()
    loss = ctypes.c_float()
    for scale, acc in ((float("nan"), 0), (float("inf"), 1), (1.0, 2), (1.0, -1)):
        rc = G._lib.gpt_step_accum(sess.handle, sess.tokens.data_ptr(), sess.targets.data_ptr(),
                                   sess.grads.data_ptr(), scale, acc, ctypes.byref(loss))
        assert rc == G.GPT_EINVAL, (scale, acc, rc)
    # nothing was enqueued: the gradients are untouched
    assert bool((sess.grads == g1).all())
    sess.close()


@pytest.mark.parametrize("name", ["bf16_mid", "fp8_mid"])
def test_micro_batch_graph_matches_eager_steps(name):
    """gpt_step_micro (n micro-batches replayed as one captured graph) gives
    the gradients and losses of n gpt_step_accum calls bit for bit, on every
    replay, with eager work and synchronisation between replays; with
    profiling on it runs eagerly, every product in order, and agrees with
    in-order steps.  (fp8: the call quantises
    the unchanged weights once, the separate calls once each, to the same
    codes.)"""
    import decoder_only_transformer_fwd_amd as G
    s6 = SMALL[name].replace(batch=6)
    s = s6.replace(batch=2)
    n = 3
    W8 = gi.make_weights(s6)
    X, Y = gi.make_tokens(s6)
    Xm = X.reshape(n, s.batch, s.seq_len)
    Ym = Y.reshape(n, s.batch, s.seq_len)
    log(f"micro-batch graph vs eager: {name}, 3 x 2 rows")
    sess = G.Session(s, W8)
    t = sess.torch
    ref_losses = []
    for i in range(n):
        sess.set_tokens(Xm[i], Ym[i])
        ref_losses.append(sess.step_accum(1.0 / n, accumulate=i > 0))
    ref = sess.grads.clone()
    Xd = t.from_numpy(np.ascontiguousarray(Xm)).to(sess.device)
    Yd = t.from_numpy(np.ascontiguousarray(Ym)).to(sess.device)
    for rep in range(3):
        sess.grads.fill_(float("nan"))
        losses = sess.step_micro(Xd, Yd, 1.0 / n, accumulate=False)
        assert losses == ref_losses, (rep, losses, ref_losses)
        assert bool((sess.grads == ref).all()), rep
        junk = t.randn(4096, device=sess.device).cumsum(0)   # eager work between replays
        t.cuda.synchronize()
        del junk
    # accumulating onto what the buffer holds: the same bits as the eager
    # accumulating steps
    for i in range(n):
        sess.set_tokens(Xm[i], Ym[i])
        sess.step_accum(1.0 / n, accumulate=True)
    ref2 = sess.grads.clone()
    sess.grads.copy_(ref)
    sess.step_micro(Xd, Yd, 1.0 / n, accumulate=True)
    assert bool((sess.grads == ref2).all())
    # profiled, the micro-batches run eagerly with every product in order on
    # one stream: the same bits as in-order accumulating steps
    sess.overlap(False)
    for i in range(n):
        sess.set_tokens(Xm[i], Ym[i])
        sess.step_accum(1.0 / n, accumulate=i > 0)
    ref_ordered = sess.grads.clone()
    sess.overlap(True)
    sess.profile(True)
    losses = sess.step_micro(Xd, Yd, 1.0 / n, accumulate=False)
    sess.profile(False)
    assert losses == ref_losses and bool((sess.grads == ref_ordered).all())
    # an out-of-range id in the last micro-batch is reported
    Yb = Yd.clone()
    Yb[n - 1, 0, 3] = s.vocab
    rc = G._lib.gpt_step_micro(sess.handle, Xd.data_ptr(), Yb.data_ptr(), n, sess.grads.data_ptr(), 1.0 / n, 0,
                               (ctypes.c_float * n)())
    assert rc == G.GPT_ETOKEN
    sess.close()
