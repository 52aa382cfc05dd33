"""Write the oracle's full-size results used by the GPU parity tests.

For each full workload (d12, d20, d24, and d24-fp8, whose linear-layer
operands the oracle encodes in fp8 as that workload's method does) this runs
the fp64 oracle once on the seeded inputs and stores:
the loss, the L2 norm of every gradient tensor, the gradient values at
seeded sample positions (``gpt_inputs.grad_sample_indices``, 2048 per
tensor), and complete rows of three gradients (``gpt_inputs.grad_full_rows``):
the embedding rows of 256 seeded ids among those the batch uses, 64 seeded
rows of layer 0's Wq and 64 of the last layer's W1, each row whole, so that
the tests can compare them element by element.
Only ``oracle/`` and ``gpt_inputs`` are used.

Usage:  python tests/golden/make_full_size_golden.py d12 d20 d24 d24-fp8
"""
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import gpt_inputs as gi  # noqa: E402
from oracle import gpt_oracle as O  # noqa: E402

N_SAMPLES = 2048
OUT = os.path.dirname(os.path.abspath(__file__))


def run(name: str) -> None:
    s = gi.preset(name)
    t0 = time.time()
    W = gi.weights_f64(s, gi.make_weights(s))
    X, Y = gi.make_tokens(s)
    loss, G = O.forward_backward(s, W, X, Y)
    dt = time.time() - t0
    idx = gi.grad_sample_indices(s, N_SAMPLES)
    names = [n for n, _ in gi.param_shapes(s)]
    samples = np.stack([G[n].reshape(-1)[idx[n]] for n in names])
    norms = np.array([np.linalg.norm(G[n]) for n in names])
    rows = gi.grad_full_rows(s, X)
    full = {f"rows_{n}": G[n][r].astype(np.float32) for n, r in rows.items()}
    path = os.path.join(OUT, f"oracle_{name}.npz")
    np.savez_compressed(path, loss=np.float64(loss), names=np.array(names), norms=norms,
                        samples=samples.astype(np.float64), n_samples=N_SAMPLES, seconds=dt,
                        row_names=np.array(list(rows)), **full)
    print(f"{name}: loss {loss:.9f}  oracle {dt:.1f}s -> {path}", flush=True)


if __name__ == "__main__":
    for n in sys.argv[1:] or ["d12", "d20", "d24"]:
        run(n)
