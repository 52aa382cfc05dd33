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
