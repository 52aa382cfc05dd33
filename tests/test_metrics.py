"""The FLOP convention used for MFU reproduces the pages' printed estimates."""
import json
import os

import gpt_inputs as gi

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _page(key):
    with open(os.path.join(GOLDEN, "page_values.json")) as f:
        return json.load(f)[key]


def test_flops_per_token_matches_d20_log():
    from decoder_only_transformer_fwd_amd import metrics as M
    for key in ("d20_flops_per_token_T2048", "d20_flops_per_token_T1024"):
        pv = _page(key)
        s = gi.preset("d20", seq_len=pv["config"]["seq_len"])
        assert abs(M.flops_per_token(s) - pv["value"]) <= pv["rel_tol"] * pv["value"]


def test_algorithmic_flops_count_visible_pairs():
    from decoder_only_transformer_fwd_amd import metrics as M
    assert M.visible_pairs(4, 4) == 10 and M.visible_pairs(5, 2) == 3 + 3 * 2
    s = gi.preset("d24")
    # windowed layers: algorithmic < conventional; no window: ratio (T+1)/(2T)
    assert M.algorithmic_flops_per_token(s) < M.flops_per_token(s)
    t = gi.preset("d12")
    attn_conv = M.flops_per_token(t) - 6 * M.scaling_params(t)
    attn_alg = M.algorithmic_flops_per_token(t) - 6 * M.scaling_params(t)
    assert abs(attn_alg / attn_conv - (t.seq_len + 1) / (2 * t.seq_len)) < 1e-12


def test_profiler_kernel_names_decode_to_step_labels():
    from decoder_only_transformer_fwd_amd import profiling as Pf
    base = "void gk::gemm_kernel<__bf16, gk::Mfma<__bf16>, 256, 256, 2, 4, 64, 4, true, false, 8, __bf16, true, {}>" \
           "(gk::GemmArgs)"
    assert Pf.decode("k", base.format("false")) == "gemm_kernel<bf16, 256, 256, 2, 4, 64, 4, true, false, 8, ping-pong>"
    assert Pf.decode("k", base.format("true")) == \
        "gemm_kernel<bf16, 256, 256, 2, 4, 64, 4, true, false, 8, ping-pong, batched>"
    garbled = "void gk::gemm_kernel<bool _Accum, gk, Mfma<bool _Accum>, 256, 256, 2, 4, 64, 4, true, true, 8, " \
              "bool _Accum, bool, E, {}>(gk::GemmArgs)"
    assert Pf.decode("k", garbled.format("false")) == \
        "gemm_kernel<bf16, 256, 256, 2, 4, 64, 4, true, true, 8, ping-pong>"
    assert Pf.decode("k", garbled.format("true")) == \
        "gemm_kernel<bf16, 256, 256, 2, 4, 64, 4, true, true, 8, ping-pong, batched>"


def test_traffic_summary_lookup(tmp_path):
    from decoder_only_transformer_fwd_amd import profiling as Pf
    p = tmp_path / "t.md"
    row = "| gemm_kernel<bf16, 1> | 4 | 1.50 | 0.25 | 900 |"
    p.write_text(f"| kernel | dispatches | read | written | GB/s |\n|---|---:|---:|---:|---:|\n{row}\n\n"
                 f"Kernel sources: {Pf.source_digest()}\n")
    assert Pf.traffic_lookup(str(p), "gemm_kernel<bf16, 1>") == (1.5e6, 0.25e6)
    assert Pf.traffic_lookup(str(p), "other") is None
    p.write_text(p.read_text().replace(Pf.source_digest(), "0" * 16))   # other kernel sources: stale
    assert Pf.traffic_lookup(str(p), "gemm_kernel<bf16, 1>") is None


def test_head_tile_decodes_as_ping_pong():
    from decoder_only_transformer_fwd_amd import profiling as Pf
    name = "void gk::gemm_kernel<__bf16, gk::Mfma<__bf16>, 256, 256, 4, 2, 64, 4, true, true, 13, __bf16, true, false>" \
           "(gk::GemmArgs)"
    assert Pf.decode("k", name) == "gemm_kernel<bf16, 256, 256, 4, 2, 64, 4, true, true, 13, ping-pong>"


def test_traffic_summary_scales_counters_by_the_copy(tmp_path):
    """Per-dispatch bytes = counter reading x (bytes the plain copy moved / its
    reading), summed over the counter's instances, averaged over dispatches."""
    from decoder_only_transformer_fwd_amd import profiling as Pf

    def pmc(path, counter, rows):
        with open(path, "w") as f:
            f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
            for d, k, v in rows:
                f.write(f"{d},{k},{counter},{v}\n")
    mib = 2.0
    nbytes = mib * 2 ** 20
    pmc(tmp_path / "cf.csv", "FETCH_SIZE", [(1, "copy", nbytes / 2048 / 2), (1, "copy", nbytes / 2048 / 2)])
    pmc(tmp_path / "cw.csv", "WRITE_SIZE", [(1, "copy", nbytes / 1024)])
    # kernel k: two dispatches, fetch readings 10 + 30 (two instances each), write 5 and 15
    pmc(tmp_path / "f.csv", "FETCH_SIZE", [(7, "k", 4), (7, "k", 6), (8, "k", 10), (8, "k", 20)])
    pmc(tmp_path / "w.csv", "WRITE_SIZE", [(7, "k", 5), (8, "k", 15)])
    md = Pf.traffic_md(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(tmp_path / "cf.csv"),
                       str(tmp_path / "cw.csv"), mib, "cmd")
    row = [ln for ln in md.splitlines() if ln.startswith("| k |")][0]
    cells = [c.strip() for c in row.strip("|").split("|")]
    assert cells[1] == "2"
    assert abs(float(cells[2]) - (40 / 2) * 2048 / 1e6) < 1e-2    # MB read per dispatch
    assert abs(float(cells[3]) - (20 / 2) * 1024 / 1e6) < 1e-2    # MB written per dispatch


def test_report_renders_one_row_per_bench_line(tmp_path):
    import json
    from decoder_only_transformer_fwd_amd import profiling as Pf
    line = {"value": 1234.5, "ms_per_step": 13.27, "mfu": 0.25,
            "config": {"workload": "w1", "precision": "bf16", "tokens_per_step": 16384},
            "roofline": {"kernel": "gemm_kernel<bf16, 1>", "sites": ["a", "b"], "bound": "mfma", "achieved": 900.0,
                         "unit": "TFLOP/s", "peak": 2516.6, "frac": 0.3576, "traffic": 5.0e8, "share_of_step": 0.2},
            "cpu_baseline": {"value": 51.0, "cores": 16, "sample": "one pass"}}
    p = tmp_path / "b.json"
    p.write_text("log line\n" + json.dumps(line) + "\n")
    md = Pf.report_md([str(p)], "python3 -u bench.py --config W")
    row = [ln for ln in md.splitlines() if ln.startswith("| w1 |")][0]
    assert "| 13.27 | 1234 | 25.0 % |" in row and "(a, b)" in row and "0.358" in row and "| 500.0 |" in row
    assert "51.0 (16)" in row and "- w1: one pass" in md
