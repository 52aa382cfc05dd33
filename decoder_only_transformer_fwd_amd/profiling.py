"""Helpers for rocprofv3 measurements of the GPT step.

    python -m decoder_only_transformer_fwd_amd.profiling copy --mib 1024
        one plain device-to-device copy of a known size, repeated 3 times
        (run under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE to calibrate the
        counters: bytes moved / counter reading);

    python -m decoder_only_transformer_fwd_amd.profiling stats STATS_CSV --title T --command C [--note N]
        markdown table of a `rocprofv3 --kernel-trace --stats` kernel summary;

    python -m decoder_only_transformer_fwd_amd.profiling traffic --fetch F.csv --write W.csv
            --copy-fetch CF.csv --copy-write CW.csv --copy-mib 1024 --command C
        per-kernel HBM bytes per dispatch from two --pmc passes, each scaled by
        the same counter's reading for the plain copy;

    python -m decoder_only_transformer_fwd_amd.profiling report B1.json B2.json ... --command C
        one table row per bench.py JSON line.

The kernel names in rocprofv3's CSV output are the mangled template names;
GEMM instantiations are decoded into their tile parameters.
"""
from __future__ import annotations

import argparse
import csv
import re
import sys
from collections import defaultdict

_GARBLED = re.compile(r"gemm_kernel<[^>]*?>?, (\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (true|false), (true|false), (\d+)")
# tiles with the ping-pong schedule, by (BM, BN, waves M, waves N, row bytes,
# stages); the library's bf16 plan launches the 8-wave, 64-byte, 4-stage tile
# only with the ping-pong schedule
_PP = {(256, 256, 2, 4, 64, 4), (256, 256, 2, 4, 64, 5), (256, 128, 4, 2, 128, 3), (256, 256, 4, 2, 64, 4)}


def _demangle(names):
    """c++filt over the names (the __bf16 type's mangling spelled as a vendor type)."""
    import subprocess
    try:
        r = subprocess.run(["c++filt"], input="\n".join(n.replace("DF16b", "u6__bf16") for n in names),
                           capture_output=True, text=True, check=True)
        out = r.stdout.split("\n")
        return out[:len(names)]
    except (OSError, subprocess.CalledProcessError):
        return list(names)


def decode(name: str, demangled: str = None) -> str:
    """The kernel's label in the form the step's profiler uses, e.g.
    gemm_kernel<bf16, 128, 128, 2, 2, 128, 2, true, false, 1> or
    attn_fwd_kernel<bf16, 128>."""
    dm = demangled if demangled is not None else _demangle([name])[0]
    dm = dm.replace("__bf16", "bf16").replace("gk::", "").replace("unsigned char", "u8")
    dm = re.sub(r"^void ", "", dm)
    dm = re.sub(r"\((GemmArgs|AttnArgs|[^()]*)\)$", "", dm)
    if "gemm_kernel<" in dm:
        m = re.match(r"gemm_kernel<(bf16|float|u8), (Mfma<\w+>|MfmaF8<(\d), (\d)>), (\d+), (\d+), (\d+), (\d+), "
                     r"(\d+), (\d+), (true|false), (true|false), (\d+), \w+, (true|false), (true|false)>$", dm)
        batched = False
        if m:
            ty, _, fb, fa, bm, bn, wgm, wgn, rb, ns, akc, bkc, epi, pp, bt = m.groups()
            batched = bt == "true"
            if ty == "u8":
                fmt = {"0": "e4m3", "1": "e5m2"}
                ty = f"fp8 {fmt[fa]} x {fmt[fb]}"   # the MFMA takes the B operand first
            pp = pp == "true"
        else:   # the profiler's demangler garbles some instantiations; keep the numbers
            g = _GARBLED.search(dm)
            if not g:
                return dm
            bm, bn, wgm, wgn, rb, ns, akc, bkc, epi = g.groups()
            ty = "bf16"
            key = tuple(int(x) for x in (bm, bn, wgm, wgn, rb, ns))
            pp = key in _PP
            # the last template argument (the batched flag) survives the garbling
            batched = dm.endswith(", true>")
        return (f"gemm_kernel<{ty}, {bm}, {bn}, {wgm}, {wgn}, {rb}, {ns}, {akc}, {bkc}, {epi}"
                f"{', ping-pong' if pp else ''}{', batched' if batched else ''}>")
    return dm


def _decode_all(names):
    return {n: decode(n, d) for n, d in zip(names, _demangle(names))}


def stats_md(path: str, title: str, command: str, note: str = "") -> str:
    rows = list(csv.DictReader(open(path)))
    labels = _decode_all([r["Name"] for r in rows])
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    out = [f"# {title}", "", "Command (from the repository root, on one MI355X):", "", "```", command, "```", ""]
    if note:
        out += [note, ""]
    out += [f"Total kernel time {total / 1e6:.1f} ms over all traced calls.", "",
            "| kernel | calls | avg (us) | total % |", "|---|---:|---:|---:|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        out.append(f"| {labels[r['Name']]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{100 * float(r['TotalDurationNs']) / total:.2f} |")
    return "\n".join(out) + "\n"


def _per_dispatch(path: str, counter: str):
    """{dispatch id: (kernel name, summed counter value)} from a --pmc CSV."""
    acc = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        d = r["Dispatch_Id"]
        name, v = acc.get(d, (r["Kernel_Name"], 0.0))
        acc[d] = (name, v + float(r["Counter_Value"]))
    return acc


def _copy_factor(path: str, counter: str, nbytes: float) -> float:
    """Bytes per counter unit, from the largest dispatch of the copy run."""
    vals = [v for _, v in _per_dispatch(path, counter).values()]
    return nbytes / max(vals)


def _avg_ns(stats: str):
    """{raw kernel name: average duration in ns} from a --stats CSV."""
    if not stats:
        return {}
    return {r["Name"]: float(r["AverageNs"]) for r in csv.DictReader(open(stats))}


def traffic_md(fetch: str, write: str, copy_fetch: str, copy_write: str, copy_mib: float, command: str,
               top: int = 25, stats: str = None) -> str:
    nbytes = copy_mib * 2 ** 20
    ff = _copy_factor(copy_fetch, "FETCH_SIZE", nbytes)
    fw = _copy_factor(copy_write, "WRITE_SIZE", nbytes)
    agg = defaultdict(lambda: [0, 0.0, 0.0])
    for _, (name, v) in _per_dispatch(fetch, "FETCH_SIZE").items():
        agg[name][0] += 1
        agg[name][1] += v * ff
    for _, (name, v) in _per_dispatch(write, "WRITE_SIZE").items():
        agg[name][2] += v * fw
    out = ["# HBM traffic per dispatch (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
           "Commands (from the repository root, on one MI355X), one counter per pass:", "", "```", command, "```", "",
           f"Calibration: a plain {copy_mib:.0f} MiB device copy reads and writes {nbytes:.0f} bytes; "
           f"bytes per counter unit: FETCH_SIZE x {ff:.1f}, WRITE_SIZE x {fw:.1f}.", "",
           "| kernel | dispatches | read MB / dispatch | written MB / dispatch | HBM GB/s |",
           "|---|---:|---:|---:|---:|"]
    if stats:
        out[-3:-3] = ["", "HBM GB/s: the measured bytes per dispatch over the kernel's average duration in the "
                          "workload's kernel trace (`--kernel-trace --stats`, its own run)."]
    labels = _decode_all(list(agg))
    dur = _avg_ns(stats)
    for name, (n, rd, wr) in sorted(agg.items(), key=lambda kv: -(kv[1][1] + kv[1][2]))[:top]:
        rate = f"{(rd + wr) / n / dur[name]:.0f}" if name in dur else "-"
        out.append(f"| {labels[name]} | {n} | {rd / n / 1e6:.2f} | {wr / max(n, 1) / 1e6:.2f} | {rate} |")
    out += ["", f"Kernel sources: {source_digest()}"]
    return "\n".join(out) + "\n"


N_SIMD = 1024    # 256 CUs x 4 SIMDs
N_XCD = 8


def mfma_md(pmc: str, stats: str, command: str, note: str = "", top: int = 30) -> str:
    """Per-kernel MFMA utilisation from GRBM_GUI_ACTIVE and
    SQ_VALU_MFMA_BUSY_CYCLES: busy = MFMA-busy SIMD cycles / (1024 SIMDs x
    GRBM_GUI_ACTIVE / 8 XCDs)."""
    gui = _per_dispatch(pmc, "GRBM_GUI_ACTIVE")
    busy = _per_dispatch(pmc, "SQ_VALU_MFMA_BUSY_CYCLES")
    agg = defaultdict(lambda: [0, 0.0, 0.0])
    for d, (name, g) in gui.items():
        agg[name][0] += 1
        agg[name][1] += g / N_XCD
        agg[name][2] += busy.get(d, (name, 0.0))[1]
    dur = _avg_ns(stats)
    out = ["# MFMA utilisation per kernel (rocprofv3 GRBM_GUI_ACTIVE, SQ_VALU_MFMA_BUSY_CYCLES)", "",
           "Command (from the repository root, on one MI355X):", "", "```", command, "```", ""]
    if note:
        out += [note, ""]
    out += ["MFMA busy: MFMA-busy SIMD cycles divided by (1024 SIMDs x GRBM_GUI_ACTIVE / 8), the "
            "graphics engine's active cycles per XCD during the dispatch.  GRBM_GUI_ACTIVE also counts "
            "each dispatch's start-up and drain (for the short kernels of this run it exceeds duration x "
            "2.4 GHz), so the fraction is a lower bound, loosest for short dispatches.  The profiler "
            "serialises dispatches in a counter run, so clocks and durations there differ from the "
            "back-to-back step.", "",
            "| kernel | dispatches | avg duration (us) | GRBM_GUI_ACTIVE / 8 per dispatch | MFMA busy |",
            "|---|---:|---:|---:|---:|"]
    labels = _decode_all(list(agg))
    for name, (n, cyc, b) in sorted(agg.items(), key=lambda kv: -kv[1][1])[:top]:
        c = cyc / n
        du = f"{dur[name] / 1e3:.1f}" if name in dur else "-"
        out.append(f"| {labels[name]} | {n} | {du} | {c:.3g} | {100 * b / n / N_SIMD / c:.0f} % |")
    return "\n".join(out) + "\n"


def report_md(paths, command: str, note: str = "") -> str:
    """One row per bench JSON line (a file each): throughput, MFU, the
    dominant kernel's roofline and the oracle's CPU rate."""
    import json
    out = ["# Training step per workload: throughput, MFU, roofline, CPU oracle", "",
           "Command (from the repository root, on one MI355X), once per workload W:", "", "```", command, "```", ""]
    if note:
        out += [note, ""]
    out += ["| workload | precision | tokens / step | ms / step | tokens/s | MFU | dominant kernel (sites) | "
            "bound | achieved | peak | frac | HBM traffic MB / launch | share of step | CPU oracle tokens/s (cores) |",
            "|---|---|---:|---:|---:|---:|---|---|---:|---:|---:|---:|---:|---:|"]
    for p in paths:
        r = json.loads(open(p).read().strip().splitlines()[-1])
        c, f = r["config"], r["roofline"]
        cb = r.get("cpu_baseline")
        cpu = f"{cb['value']:.1f} ({cb['cores']})" if cb else "-"
        tr = f"{f['traffic'] / 1e6:.1f}" if f.get("traffic") else "-"
        sites = ", ".join(f.get("sites", []))
        out.append(f"| {c['workload']} | {c['precision']} | {c['tokens_per_step']} | {r['ms_per_step']:.2f} | "
                   f"{r['value']:.0f} | {100 * r['mfu']:.1f} % | {f['kernel']} ({sites}) | {f['bound']} | "
                   f"{f['achieved']:.1f} {f['unit']} | {f['peak']:.1f} | {f['frac']:.3f} | {tr} | "
                   f"{100 * f.get('share_of_step', 0):.1f} % | {cpu} |")
    samples = []
    for p in paths:
        r = json.loads(open(p).read().strip().splitlines()[-1])
        if r.get("cpu_baseline"):
            samples.append(f"{r['config']['workload']}: {r['cpu_baseline']['sample']}")
    if samples:
        out += ["", "CPU oracle samples:", ""] + [f"- {x}" for x in samples]
    return "\n".join(out) + "\n"


# sources of the optimizer's and the decoder's own kernels and launch code,
# which the training step does not run
_NOT_STEP = {"optim.hip", "infer.hip", "optim_host.cpp", "infer_host.cpp"}


def source_digest() -> str:
    """sha256 over the sources of the step's kernels and their launches, to
    tell whether a traffic measurement of the step still describes the
    current kernels."""
    import hashlib
    import os
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(here)):
        if f.endswith((".hip", ".h", ".cpp")) and f not in _NOT_STEP:
            h.update(f.encode())
            h.update(open(os.path.join(here, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_lookup(md_path: str, label: str):
    """(read, written) bytes per dispatch of `label` from a traffic summary,
    or None when the summary is missing, does not list the kernel, or was
    taken from different kernel sources."""
    import os
    if not os.path.exists(md_path):
        return None
    text = open(md_path).read()
    m = re.search(r"Kernel sources: (\w+)", text)
    if not m or m.group(1) != source_digest():
        return None
    for line in text.splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) in (4, 5) and cells[0] == label:
            return float(cells[2]) * 1e6, float(cells[3]) * 1e6
    return None


def _copy(mib: float) -> None:
    import torch
    n = int(mib * 2 ** 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {n * 4} bytes x 3", flush=True)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=float, default=1024)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--title", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--note", default="")
    t = sub.add_parser("traffic")
    for k in ("fetch", "write", "copy-fetch", "copy-write", "command"):
        t.add_argument("--" + k, required=True)
    t.add_argument("--copy-mib", type=float, default=1024)
    t.add_argument("--stats", default=None)
    u = sub.add_parser("mfma")
    for k in ("pmc", "stats", "command"):
        u.add_argument("--" + k, required=True)
    u.add_argument("--note", default="")
    r = sub.add_parser("report")
    r.add_argument("json", nargs="+")
    r.add_argument("--command", required=True)
    r.add_argument("--note", default="")
    a = ap.parse_args(argv)
    if a.cmd == "copy":
        _copy(a.mib)
    elif a.cmd == "stats":
        sys.stdout.write(stats_md(a.csv, a.title, a.command, a.note))
    elif a.cmd == "report":
        sys.stdout.write(report_md(a.json, a.command, a.note))
    elif a.cmd == "mfma":
        sys.stdout.write(mfma_md(a.pmc, a.stats, a.command, a.note))
    else:
        sys.stdout.write(traffic_md(a.fetch, a.write, a.copy_fetch, a.copy_write, a.copy_mib, a.command,
                                    stats=a.stats))
    return 0


if __name__ == "__main__":
    sys.exit(main())
