"""Benchmark: tokens/s and MFU of one GPT forward+backward training step on
one MI355X, through the C ABI (``gpt_step``).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config d24] [--grad-accum N]

A step is one ``gpt_step`` call on one batch of seeded synthetic tokens with
seeded random weights (inputs resident in HBM before the timed region); the
timed region is K steps bracketed by device synchronisation.  With
``--grad-accum N`` a step is one ``gpt_step_micro`` call over N different
micro-batches of the workload's batch size (one captured graph),
accumulating the gradient of their mean loss (N times the tokens per step); with ``--optimizer`` each step
ends with a Muon + AdamW update of the weights (``gpt_optim_step``).  The JSON line
also carries the roofline of the dominant kernel (HIP-event timing of every
launch site inside the timed region) and the CPU oracle's throughput on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import gpt_inputs as gi  # noqa: E402

METRIC = "training tokens/sec + MFU, d20/d24 GPT fwd+bwd step on 1×MI355X"


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def cpu_baseline(s, budget_rows: int = 1) -> dict:
    """Time the fp64 oracle on one batch row (T tokens) of the workload."""
    from oracle import gpt_oracle as O
    try:
        import threadpoolctl
        cores = max(int(i.get("num_threads", 1)) for i in threadpoolctl.threadpool_info()) or os.cpu_count()
    except Exception:
        cores = os.cpu_count()
    sample = s.replace(batch=budget_rows)
    W = gi.weights_f64(sample, gi.make_weights(sample))
    X, Y = gi.make_tokens(sample)
    # the same forward+backward, repeated until about 10 s of CPU work
    t0 = time.perf_counter()
    reps = 0
    while True:
        O.forward_backward(sample, W, X, Y)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0:
            break
    what = "one forward+backward" if reps == 1 else f"{reps} forward+backward passes"
    return {"value": reps * sample.bt / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{what} of the full {s.name} model on {budget_rows} of its {s.batch} "
                      f"rows ({sample.bt} tokens each), fp64 numpy, {dt:.1f} s"}


def decode_bytes(s, pos: int) -> float:
    """HBM bytes one decode step must move at position pos: every weight
    matrix and the lm_head once (bf16), the batch's embedding rows, and each
    layer's visible cached keys and values plus the new ones."""
    d, f, dkv = s.d_model, s.mlp_hidden, s.kv_heads * s.head_dim
    weights = 2.0 * (s.depth * (2 * d * d + 2 * dkv * d + 2 * d * f) + s.vocab * d) + 2.0 * s.batch * d
    kv = 0.0
    for w in gi.layer_windows(s):
        vis = min(pos + 1, w)
        kv += 2.0 * 2.0 * s.batch * s.kv_heads * s.head_dim * (vis + 1)
    logits = 4.0 * s.batch * s.vocab
    return weights + kv + logits


def bench_decode(args, s) -> int:
    import torch
    import decoder_only_transformer_fwd_amd as G
    from decoder_only_transformer_fwd_amd import metrics as Mx
    P, K, Wm = args.prompt, args.steps, args.warmup
    if P + Wm + K > s.seq_len:
        log(f"--prompt + --warmup + --steps must be <= seq_len ({s.seq_len})")
        return 2
    log(f"bench decode: {s}, prompt {P}, {K} timed steps")
    W8 = gi.make_weights(s)
    sess = G.Session(s, W8)
    del W8
    sess.infer_init()
    X, _ = gi.make_tokens(s)
    prompt = torch.from_numpy(np.ascontiguousarray(X[:, :P])).to(sess.device)
    toks = [torch.from_numpy(np.ascontiguousarray(X[:, p])).to(sess.device) for p in range(P, P + Wm + K)]
    sess.prefill(prompt)   # warm-up of the prefill path
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    sess.prefill(prompt)
    torch.cuda.synchronize()
    t_prefill = time.perf_counter() - t0
    # timed: each step replays the captured graph of the decoding step
    for i in range(Wm):
        sess.decode(toks[i], P + i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(Wm, Wm + K):
        sess.decode(toks[i], P + i)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms = dt / K * 1e3
    byts = sum(decode_bytes(s, P + i) for i in range(Wm, Wm + K)) / K
    # per-launch timing: the same steps again, run eagerly with HIP events
    sess.prefill(prompt)
    for i in range(Wm):
        sess.decode(toks[i], P + i)
    sess.profile(True)
    for i in range(Wm, Wm + K):
        sess.decode(toks[i], P + i)
    sites = sess.profile_sites()
    sess.profile(False)
    kernel_ms = sum(x["total_ms"] for x in sites) / K
    if args.sites:
        for x in sorted(sites, key=lambda x: -x["total_ms"]):
            log(f"  {x['name']:28s} {x['launches']:6d} launches {x['total_ms'] / K:9.4f} ms/step")
    out = {
        "metric": "decode tokens/s (KV-cache, one token per row per step)",
        "value": s.batch * K / dt,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights, seeded token ids)",
        "config": {"workload": s.name, "depth": s.depth, "d_model": s.d_model, "n_head": s.n_head,
                   "n_kv_head": s.kv_heads,
                   "head_dim": s.head_dim, "mlp_hidden": s.mlp_hidden, "vocab": s.vocab, "batch": s.batch,
                   "prompt": P, "window": s.window, "window_pattern": s.window_pattern},
        "prefill": {"tokens_per_s": s.batch * P / t_prefill, "ms": t_prefill * 1e3},
        "roofline": {"bound": "hbm", "achieved": byts / (ms * 1e-3) / 1e9, "peak": Mx.PEAK_HBM / 1e9,
                     "unit": "GB/s", "frac": byts / (ms * 1e-3) / Mx.PEAK_HBM, "traffic": None,
                     "kernel": "whole decode step (graph replay, wall time)", "bytes_per_step": byts,
                     "kernel_ms_per_step_eager": kernel_ms},
        "cpu_baseline": None,
    }
    sess.close()
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="d24", choices=sorted(gi.PRESETS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sites", action="store_true", help="print per-site timings to stderr")
    ap.add_argument("--grad-accum", type=int, default=1,
                    help="micro-batches accumulated per step (gpt_step_accum)")
    ap.add_argument("--optimizer", action="store_true",
                    help="end every step with a Muon + AdamW update (gpt_optim_step)")
    ap.add_argument("--decode", action="store_true",
                    help="KV-cache inference instead of training: prefill --prompt tokens per row, "
                         "then time --steps decode steps (one token per row each)")
    ap.add_argument("--prompt", type=int, default=1024)
    ap.add_argument("--no-overlap", action="store_true",
                    help="run the weight-gradient products in order on the step's stream "
                         "(gpt_overlap_enable(m, 0)) instead of on the handle's second stream")
    ap.add_argument("--no-rope-epilogue", action="store_true",
                    help="run the rotary step and QK norm as a separate pass after the QKV product "
                         "(gpt_rope_epilogue_enable(m, 0)) instead of in its epilogue")
    args = ap.parse_args()
    if args.gpus != 1:
        log("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)")
        return 2

    import torch
    import decoder_only_transformer_fwd_amd as G
    from decoder_only_transformer_fwd_amd import metrics as Mx

    s = gi.preset(args.config)
    if args.decode:
        return bench_decode(args, s)
    n_acc = args.grad_accum
    if n_acc < 1:
        log("--grad-accum must be at least 1")
        return 2
    log(f"bench: {s}" + (f", {n_acc} micro-batches per step" if n_acc > 1 else ""))
    W8 = gi.make_weights(s)
    sess = G.Session(s, W8)
    del W8
    if args.no_overlap:
        sess.overlap(False)
    if args.no_rope_epilogue:
        sess.rope_epilogue(False)
    if n_acc == 1:
        X, Y = gi.make_tokens(s)
        sess.set_tokens(X, Y)

        def step():
            return sess.step()
    else:
        # N micro-batches drawn as one batch of N*B rows, all resident on the
        # device before timing; one gpt_step_micro call (one graph replay)
        # per step
        X, Y = gi.make_tokens(s.replace(batch=s.batch * n_acc))
        Xd = torch.from_numpy(np.ascontiguousarray(X.reshape(n_acc, s.batch, s.seq_len))).to(sess.device)
        Yd = torch.from_numpy(np.ascontiguousarray(Y.reshape(n_acc, s.batch, s.seq_len))).to(sess.device)

        def step():
            losses = G.gpt_step_micro(sess.handle, Xd.data_ptr(), Yd.data_ptr(), n_acc, sess.grads.data_ptr(),
                                      1.0 / n_acc, False)
            return float(np.mean(losses))
    if args.optimizer:
        # the report card's learning rates, AdamW's scaled by 1/sqrt(d/768)
        sc = (s.d_model / 768) ** -0.5
        hp = G.optim_params(matrix_lr=0.02, momentum=0.95, nesterov=1, ns_steps=5, embedding_lr=0.2 * sc,
                            unembedding_lr=0.004 * sc, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0,
                            grad_clip=1.0, step=1)
        sess.optim_init()
        fwd_bwd = step

        def step():
            loss = fwd_bwd()
            sess.optim_step(hp)
            hp.step += 1
            return loss
    for _ in range(args.warmup):
        step()
    # `value` comes from K steps run exactly as a user runs them.  The
    # per-launch figures (roofline, --sites) come from K more steps with a
    # HIP event pair recorded on the step's stream around every launch site:
    # the event packets add ~5 % of idle time between launches, so they stay
    # out of the first timing.  A step of several micro-batches replays a
    # captured graph, which runs eagerly when profiled; one profiled step
    # suffices there.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    loss = 0.0
    for _ in range(args.steps):
        loss = step()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    site_steps = 1 if n_acc > 1 else args.steps
    sess.profile(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(site_steps):
        step()
    torch.cuda.synchronize()
    dt_prof = time.perf_counter() - t1
    sites = sess.profile_sites()
    sess.profile(False)

    tok_s = s.bt * n_acc * args.steps / dt
    peak = Mx.PEAK_FP32_MFMA if s.precision == "fp32" else Mx.PEAK_BF16
    mfu = tok_s * Mx.flops_per_token(s) / peak
    total_site_ms = sum(x["total_ms"] for x in sites)
    if args.sites:
        for x in sorted(sites, key=lambda x: -x["total_ms"]):
            per = x["total_ms"] / max(1, x["launches"])
            rate = x["work"] / max(1, x["launches"]) / (per * 1e-3) if per > 0 else 0.0
            unit = "TFLOP/s" if x["work_kind"] == "flops" else "GB/s"
            scale = 1e12 if unit == "TFLOP/s" else 1e9
            log(f"  {x['name']:28s} {x['launches']:6d} launches {x['total_ms'] / site_steps:9.3f} ms/step "
                f"{100 * x['total_ms'] / total_site_ms:5.1f}%  {rate / scale:9.1f} {unit}")
    # Roofline of the dominant kernel: sites launching the same kernel
    # (template instantiation) are aggregated, as a profiler's per-kernel
    # statistics are.
    kernels = {}
    for x in sites:
        k = kernels.setdefault(x["kernel"], {"kernel": x["kernel"], "sites": [], "launches": 0, "total_ms": 0.0,
                                             "work": 0.0, "work_kind": x["work_kind"]})
        k["sites"].append(x["name"])
        k["launches"] += x["launches"]
        k["total_ms"] += x["total_ms"]
        k["work"] += x["work"]
    dom = max(kernels.values(), key=lambda k: k["total_ms"])
    avg_s = dom["total_ms"] / dom["launches"] * 1e-3
    work_per_launch = dom["work"] / dom["launches"]
    if dom["work_kind"] == "flops":
        # a product is priced at the MFMA peak of its own operand type
        kpeak = (Mx.PEAK_FP32_MFMA if s.precision == "fp32" else
                 Mx.PEAK_FP8 if "fp8" in dom["kernel"] else Mx.PEAK_BF16)
        roof = {"bound": "mfma", "achieved": work_per_launch / avg_s / 1e12, "peak": kpeak / 1e12,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": work_per_launch / avg_s / 1e9, "peak": Mx.PEAK_HBM / 1e9, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    # HBM bytes per launch of this kernel from the committed rocprofv3
    # FETCH_SIZE / WRITE_SIZE summary, if it was taken from the current
    # kernel sources
    from decoder_only_transformer_fwd_amd import profiling as Pf
    tr = Pf.traffic_lookup(os.path.join(ROOT, "profiles", f"gpt_step_{s.name}_{s.precision}_traffic.md"),
                           dom["kernel"])
    roof["traffic"] = None if tr is None else tr[0] + tr[1]
    if tr is not None:
        roof["traffic_read"], roof["traffic_written"] = tr
    roof["kernel"] = dom["kernel"]
    roof["sites"] = dom["sites"]
    roof["avg_launch_us"] = avg_s * 1e6
    roof["share_of_step"] = dom["total_ms"] / total_site_ms
    if args.sites:
        log("per kernel:")
        for k in sorted(kernels.values(), key=lambda k: -k["total_ms"])[:12]:
            log(f"  {k['total_ms'] / site_steps:9.3f} ms/step {k['launches'] // site_steps:5d}/step "
                f"avg {k['total_ms'] / k['launches'] * 1e3:9.1f} us  {k['kernel']}  [{', '.join(k['sites'])}]")

    extra = {}
    if s.precision == "fp8":
        f8 = [x for x in sites if "fp8" in x["kernel"] and x["work_kind"] == "flops"]
        f8_ms = sum(x["total_ms"] for x in f8)
        f8_rate = sum(x["work"] for x in f8) / (f8_ms * 1e-3) if f8_ms > 0 else 0.0
        extra["fp8_gemm"] = {"tflops": f8_rate / 1e12, "frac_of_fp8_peak": f8_rate / Mx.PEAK_FP8,
                             "share_of_step": f8_ms / total_site_ms}
    dtype = {"fp32": "f32", "bf16": "bf16", "fp8": "fp8+bf16"}[s.precision]
    out = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dt / args.steps * 1e3,
        "ms_per_step_profiled": dt_prof / site_steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded N(0,0.02) weights, seeded token ids)",
        "config": {"workload": s.name, "depth": s.depth, "d_model": s.d_model, "n_head": s.n_head,
                   "n_kv_head": s.kv_heads,
                   "head_dim": s.head_dim, "mlp_hidden": s.mlp_hidden, "vocab": s.vocab,
                   "seq_len": s.seq_len, "batch": s.batch, "grad_accum": n_acc, "tokens_per_step": s.bt * n_acc,
                   "optimizer": "muon+adamw" if args.optimizer else None,
                   "window": s.window, "window_pattern": s.window_pattern, "token_dist": s.token_dist,
                   "precision": s.precision, "overlapped_weight_gradients": not args.no_overlap,
                   "rope_in_qkv_epilogue": not args.no_rope_epilogue and s.precision == "bf16" and
                   s.head_dim == 128 and s.seq_len % 64 == 0},
        "mfu": mfu,
        "mfu_peak_tflops": peak / 1e12,
        "model_flops_per_token": Mx.flops_per_token(s),
        "loss": loss,
        "roofline": roof,
        **extra,
    }
    if not args.no_cpu_baseline:
        sess.close()
        del sess
        torch.cuda.empty_cache()
        log("cpu baseline: timing the oracle on one batch row")
        out["cpu_baseline"] = cpu_baseline(s)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
