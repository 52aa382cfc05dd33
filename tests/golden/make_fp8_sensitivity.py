"""How well-conditioned the FP8 configuration's step is, measured on the oracle alone.

Two fp64 evaluations of the same fp8 recipe are compared: the oracle's own
(operands encoded from their exact values) and one whose operands are first
rounded to bf16 (RNE) and then encoded, as an implementation that keeps its
activations and gradients in bf16 does.  Both are faithful evaluations of the
recipe; where they disagree, the encoding has amplified a bf16-level
difference (a value that lands on the other side of an fp8 rounding
boundary moves by a whole fp8 step).  The per-tensor gradient cosine between
the two is stored, and the GPU parity tests derive the fp8 gradient bar for
each tensor from it.  Only ``oracle/``, ``gpt_inputs`` and the test-suite's
workload table are used.

Usage:  python tests/golden/make_fp8_sensitivity.py fp8_mid d24_fp8_short d24-fp8
(d24-fp8 reuses the stored oracle_d24-fp8.npz and compares sampled values.)
"""
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import gpt_inputs as gi  # noqa: E402
from oracle import gpt_oracle as O  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "fp8_sensitivity.json")


class Fp8OperandsFromBf16(O.Fp8Operands):
    """The fp8 encoding applied to operands rounded to bf16 first."""

    @staticmethod
    def _bf16(x):
        return gi.bf16_bits_to_f64(gi.bf16_bits_from_f32(np.asarray(x, dtype=np.float32))).reshape(x.shape)

    def act(self, x):
        return super().act(self._bf16(x))

    def grad(self, g):
        return super().grad(self._bf16(g))


def _cos(a, b):
    a, b = a.reshape(-1), b.reshape(-1)
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    return 1.0 if na == nb == 0 else float(a @ b / (na * nb))


def run(name: str) -> dict:
    from tests.gpu_common import SMALL
    t0 = time.time()
    full = name in gi.PRESETS and name not in SMALL
    s = gi.preset(name) if full else SMALL[name]
    W = gi.weights_f64(s, gi.make_weights(s))
    X, Y = gi.make_tokens(s)
    loss_b, Gb = O.forward_backward(s, W, X, Y, enc=Fp8OperandsFromBf16())
    if full:
        ref = np.load(os.path.join(os.path.dirname(OUT), f"oracle_{name}.npz"), allow_pickle=False)
        idx = gi.grad_sample_indices(s, int(ref["n_samples"]))
        cos = {str(n): _cos(Gb[str(n)].reshape(-1)[idx[str(n)]], ref["samples"][k])
               for k, n in enumerate(ref["names"])}
        loss = float(ref["loss"])
    else:
        loss, G = O.forward_backward(s, W, X, Y)
        cos = {n: _cos(Gb[n], G[n]) for n in G if np.any(G[n])}
    worst = min(cos.items(), key=lambda kv: kv[1])
    print(f"{name}: loss {loss:.9f} vs {loss_b:.9f}; worst cosine {worst[1]:.5f} ({worst[0]}); "
          f"{time.time() - t0:.0f}s", flush=True)
    return {"loss": loss, "loss_bf16_operands": loss_b, "cosine": cos}


if __name__ == "__main__":
    data = json.load(open(OUT)) if os.path.exists(OUT) else {}
    for n in sys.argv[1:]:
        data[n] = run(n)
        with open(OUT, "w") as f:
            json.dump(data, f, indent=1, sort_keys=True)
