"""Host-side checks of the C ABI: the library loads, exports every declared
entry point, and validates configurations without touching a GPU."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import gpt_inputs as gi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gpt.h")


@pytest.fixture(scope="module")
def M():
    import decoder_only_transformer_fwd_amd as M
    return M


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(gpt_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_step_entry_points():
    fns = declared_functions()
    for f in ("gpt_create", "gpt_step", "gpt_destroy", "gpt_workspace_bytes", "gpt_param_layout"):
        assert f in fns


def test_library_exports_every_declared_symbol(M):
    lib = ctypes.CDLL(M.LIB_PATH)
    for f in declared_functions():
        assert hasattr(lib, f), f
    assert sorted(M.EXPORTED) == declared_functions()


@pytest.mark.parametrize("name", ["tiny", "d12", "d20", "d24"])
def test_param_layout_matches_workload_shapes(M, name):
    s = gi.preset(name)
    layout, total = M.gpt_param_layout(M.make_config(s))
    want = gi.param_shapes(s)
    assert [(n, (r, c)) for n, _, r, c in layout] == want
    prev_end = 0
    for n, off, r, c in layout:
        assert off % 128 == 0 and off >= prev_end
        prev_end = off + r * c
    assert total >= prev_end
    # Wq, Wk, Wv of a layer are adjacent: one [3d, d] operand
    offs = {n: o for n, o, _, _ in layout}
    d = s.d_model
    for l in range(s.depth):
        assert offs[f"L{l}.Wk"] == offs[f"L{l}.Wq"] + d * d
        assert offs[f"L{l}.Wv"] == offs[f"L{l}.Wq"] + 2 * d * d


def test_d20_parameter_total(M):
    layout, _ = M.gpt_param_layout(M.make_config(gi.preset("d20")))
    assert sum(r * c for _, _, r, c in layout) == 560_988_160


@pytest.mark.parametrize("name", ["tiny", "d12", "d20", "d24", "d24-fp8"])
def test_workspace_bytes_is_sane(M, name):
    s = gi.preset(name)
    b = M.gpt_workspace_bytes(M.make_config(s))
    assert b % 256 == 0
    # at least the saved activations: per layer qkv + u + g in the parameter type
    es = 4 if s.precision == "fp32" else 2
    assert b > s.depth * s.bt * (3 * s.d_model + 2 * s.mlp_hidden) * es
    assert b < 200 * 2 ** 30


BAD = [
    dict(head_dim=48, d_model=96, n_head=2),     # unsupported head_dim
    dict(n_head=3),                              # d != H * Dh
    dict(vocab=1001),                            # vocab not a multiple of 8
    dict(batch=20, seq_len=2048),                # B*T too large
    dict(window_pattern="SX"),                   # bad pattern char
    dict(window=0, window_pattern="SL"),         # S layer without a window
    dict(mlp_hidden=100),                        # F not a multiple of 64
    dict(depth=0),
    dict(precision="fp8", seq_len=100, batch=1),  # fp8 needs B*T % 64 == 0
    dict(precision="fp8", head_dim=32, d_model=64, n_head=2),  # fp8 attention is bf16: Dh 64/128
    dict(n_head=4, d_model=128, n_kv_head=3),    # key/value heads must divide the query heads
    dict(n_kv_head=4),                           # more key/value heads than query heads
    dict(norm_eps=0.0),                          # the norms need eps > 0
    dict(norm_eps=-1e-6),
    dict(rope_base=0.0),
]


@pytest.mark.parametrize("bad", BAD)
def test_bad_configs_are_rejected(M, bad):
    s = gi.preset("tiny").replace(**bad)
    with pytest.raises(M.GPTError) as e:
        M.gpt_workspace_bytes(M.make_config(s))
    assert e.value.code == M.GPT_EINVAL
    assert M.gpt_create_rc(M.make_config(s, weights=256, workspace=512, workspace_bytes=1 << 40)) == M.GPT_EINVAL


def test_create_argument_errors(M):
    s = gi.preset("tiny")
    need = M.gpt_workspace_bytes(M.make_config(s))
    assert M.gpt_create_rc(M.make_config(s)) == M.GPT_ENULL
    assert M.gpt_create_rc(M.make_config(s, weights=0x1000, workspace=0x1010, workspace_bytes=need)) == M.GPT_EALIGN
    assert M.gpt_create_rc(M.make_config(s, weights=0x1000, workspace=0x2000, workspace_bytes=need - 256)) == M.GPT_ESPACE


def test_gemm_argument_errors(M):
    with pytest.raises(M.GPTError):
        M.gpt_gemm(1, 0, 100, 64, 64, 256, 256, 256)   # M not a multiple of 8
    with pytest.raises(M.GPTError):
        M.gpt_gemm(1, 3, 64, 64, 64, 256, 256, 256)    # bad layout
    with pytest.raises(M.GPTError):
        M.gpt_gemm(1, 0, 64, 64, 64, 0, 256, 256)      # NULL operand


def test_fp8_argument_errors(M):
    with pytest.raises(M.GPTError):
        M.gpt_fp8_quantize(2, 256, 64, 64, 256, 256, 256)      # bad format
    with pytest.raises(M.GPTError):
        M.gpt_fp8_quantize(0, 256, 64, 100, 256, 256, 256)     # cols not a multiple of 64
    with pytest.raises(M.GPTError):
        M.gpt_fp8_quantize(0, 0, 64, 64, 256, 256, 256)        # NULL input
    with pytest.raises(M.GPTError):
        M.gpt_gemm_fp8(0, 64, 64, 40, 256, 256, 256, 256, 256)  # K not a multiple of 16
    with pytest.raises(M.GPTError):
        M.gpt_gemm_fp8(3, 64, 64, 64, 256, 256, 256, 256, 256)  # bad format


def test_fp8_workspace_holds_the_codes(M):
    s = gi.preset("d24")
    b16 = M.gpt_workspace_bytes(M.make_config(s))
    b8 = M.gpt_workspace_bytes(M.make_config(s.replace(precision="fp8")))
    d, F, L, BT = s.d_model, s.mlp_hidden, s.depth, s.bt
    # saved transposed activation codes + two copies of every weight's codes
    assert b8 - b16 >= L * (3 * d * BT + F * BT + 2 * (4 * d * d + 2 * F * d))


def test_strerror(M):
    assert M.gpt_strerror(M.GPT_ETOKEN) == "token id out of range"
    assert M.gpt_strerror(12345) == "unknown error"


@pytest.mark.parametrize("name", ["tiny", "d24"])
def test_kv_cache_and_optimizer_state_sizes(M, name):
    """The KV cache is K and V of every layer, bf16 [B, H, T, Dh]; the
    optimizer state holds at least the fp32 masters (bf16 parameters), one
    fp32 momentum per matrix entry and two AdamW moments per E / U entry."""
    s = gi.preset(name)
    cfg = M.make_config(s)
    assert M.gpt_kv_cache_bytes(cfg) == 2 * s.depth * s.batch * s.n_head * s.seq_len * s.head_dim * 2
    layout, total = M.gpt_param_layout(cfg)
    n_mat = sum(r * c for n, _, r, c in layout if n not in ("E", "U"))
    n_emb = sum(r * c for n, _, r, c in layout if n in ("E", "U"))
    need = 4 * (n_mat + 2 * n_emb) + (4 * total if s.precision != "fp32" else 0)
    got = M.gpt_optim_state_bytes(cfg)
    assert got >= need
    # plus the Newton-Schulz buffers of the largest shape group (bf16: two
    # copies of the group's matrices and two of its Gram matrices)
    d, f = s.d_model, s.mlp_hidden
    groups = [(4 * s.depth, d, d), (s.depth, f, d), (s.depth, d, f)]
    ns = max(2 * 2 * n * r * c + 2 * 2 * n * min(r, c) ** 2 for n, r, c in groups)
    assert got >= need + ns
    assert got <= need + ns + 64 * 2 ** 20   # tables, partials and padding are small


def test_optimizer_and_inference_argument_errors(M):
    lib = M._lib
    assert lib.gpt_optim_init(None, None, 0) == M.GPT_ENULL
    assert lib.gpt_optim_step(None, None, None, None, None) == M.GPT_ENULL
    assert lib.gpt_prefill(None, None, 1, None, None) == M.GPT_ENULL
    assert lib.gpt_decode(None, None, 1, None, None) == M.GPT_ENULL
    losses = (ctypes.c_float * 1)()
    assert lib.gpt_step_micro(None, None, None, 1, None, 1.0, 0, losses) == M.GPT_ENULL
    b = ctypes.c_size_t()
    assert lib.gpt_kv_cache_bytes(None, ctypes.byref(b)) == M.GPT_ENULL
    assert lib.gpt_optim_state_bytes(M.make_config(gi.preset("tiny")), None) == M.GPT_ENULL


def test_library_rope_table_matches_pinned_schedule(M):
    """The table the library uploads (computed on the host) against the
    hard-coded rotary angles of the oracle's pin."""
    from tests.test_oracle import ROPE_PINS
    s = gi.preset("d24").replace(seq_len=1001)
    c, sn = M.gpt_rope_table(M.make_config(s))
    assert c.shape == (1001, 64)
    for i, t, ang in ROPE_PINS:
        assert abs(float(c[t, i]) - math.cos(ang)) < 2e-7, (i, t)
        assert abs(float(sn[t, i]) - math.sin(ang)) < 2e-7, (i, t)


def test_noalloc_rejects_partials_beyond_its_scratch(M):
    """Host-side checks of gpt_gemm_noalloc: sizes past the scratch limit are
    refused before anything reaches the GPU."""
    lim = M.NOALLOC_SCRATCH_BYTES // 4
    # 2048 x 2048 x 8 splits = 32 Mi partial sums > 16 Mi
    with pytest.raises(M.GPTError) as e:
        M.gpt_gemm_noalloc(1, 2, 2048, 2048, 16384, 256, 256, 256, splits=8)
    assert e.value.code == M.GPT_EINVAL and "scratch" in str(e.value)
    assert 2048 * 2048 * 8 > lim
    with pytest.raises(M.GPTError):
        M.gpt_gemm_noalloc(1, 0, 64, 64, 64, 256, 256, 256, splits=2)   # KK layout is not split
    with pytest.raises(M.GPTError):
        M.gpt_gemm_noalloc(1, 2, 64, 64, 64, 0, 256, 256, splits=2)     # NULL operand


@pytest.mark.parametrize("kv", [1, 2, 4])
def test_grouped_query_layout(M, kv):
    """Wk and Wv are [Hkv*Dh, d] and the fused QKV block stays contiguous."""
    s = gi.preset("d24").replace(n_kv_head=kv)
    layout, total = M.gpt_param_layout(M.make_config(s))
    assert [(n, (r, c)) for n, _, r, c in layout] == gi.param_shapes(s)
    offs = {n: o for n, o, _, _ in layout}
    d, dkv = s.d_model, kv * s.head_dim
    for l in range(s.depth):
        assert offs[f"L{l}.Wk"] == offs[f"L{l}.Wq"] + d * d
        assert offs[f"L{l}.Wv"] == offs[f"L{l}.Wq"] + d * d + dkv * d
    assert M.gpt_kv_cache_bytes(M.make_config(s)) == 2 * s.depth * s.batch * kv * s.seq_len * s.head_dim * 2
    # fewer key/value heads need less workspace
    assert M.gpt_workspace_bytes(M.make_config(s)) < M.gpt_workspace_bytes(M.make_config(gi.preset("d24")))
