"""GPU parity of the MFMA GEMM kernel (all three operand layouts, every tile
shape, split-K) against fp64 products of the same rounded inputs."""
import numpy as np
import pytest

import gpt_inputs as gi
from tests.gpu_common import log

pytestmark = pytest.mark.gpu

LAYOUT_KK, LAYOUT_KN, LAYOUT_MN = 0, 1, 2
# 256x256, 256x128, 128x128 (4 waves); 256x256, 256x128 (8 waves); ping-pong 256x256 (4, 5 stages), 256x128
TILES_BF16 = [0, 1, 2, 4, 5, 10, 11, 12]
TILES_F32 = [2, 3]          # 128x128, 64x64


def _operands(dtype, layout, M, N, K, seed):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((M, K)).astype(np.float32)
    b = rng.standard_normal((N, K)).astype(np.float32)
    if dtype == 1:
        a64 = gi.bf16_bits_to_f64(gi.bf16_bits_from_f32(a))
        b64 = gi.bf16_bits_to_f64(gi.bf16_bits_from_f32(b))
    else:
        a64, b64 = a.astype(np.float64), b.astype(np.float64)
    ref = a64 @ b64.T
    # storage layouts
    a_st = a64 if layout in (LAYOUT_KK, LAYOUT_KN) else a64.T
    b_st = b64 if layout == LAYOUT_KK else b64.T
    return np.ascontiguousarray(a_st), np.ascontiguousarray(b_st), ref


def _dev(x, dtype):
    import torch
    t = torch.from_numpy(x.astype(np.float32)).cuda()
    return t.to(torch.bfloat16) if dtype == 1 else t


def run_gemm(dtype, layout, M, N, K, tile, splits=1, seed=0):
    import torch
    import decoder_only_transformer_fwd_amd as G
    a, b, ref = _operands(dtype, layout, M, N, K, seed)
    A, B = _dev(a, dtype), _dev(b, dtype)
    C = torch.full((M, N), float("nan"), device="cuda", dtype=torch.float32)
    ws = torch.empty(max(1, splits * M * N), device="cuda", dtype=torch.float32)
    log(f"gemm dtype={dtype} layout={layout} M={M} N={N} K={K} tile={tile} splits={splits}")
    G.gpt_gemm(dtype, layout, M, N, K, A.data_ptr(), B.data_ptr(), C.data_ptr(), ws.data_ptr(), splits, tile,
               torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    c = C.cpu().numpy().astype(np.float64)
    return c, ref


def _check(c, ref, K):
    assert np.all(np.isfinite(c)), "unwritten or non-finite outputs"
    err = np.max(np.abs(c - ref))
    scale = np.sqrt(K) * 1.0
    assert err <= 2e-5 * scale * 4, (err, scale)


@pytest.mark.parametrize("layout", [LAYOUT_KK, LAYOUT_KN, LAYOUT_MN])
@pytest.mark.parametrize("tile", TILES_BF16)
def test_gemm_bf16_ragged(layout, tile):
    c, ref = run_gemm(1, layout, 264, 200, 328, tile)
    _check(c, ref, 328)


@pytest.mark.parametrize("layout", [LAYOUT_KK, LAYOUT_KN, LAYOUT_MN])
@pytest.mark.parametrize("tile", TILES_F32)
def test_gemm_f32_ragged(layout, tile):
    c, ref = run_gemm(0, layout, 136, 72, 200, tile)
    _check(c, ref, 200)


@pytest.mark.parametrize("layout", [LAYOUT_KN, LAYOUT_MN])
@pytest.mark.parametrize("tile", [2, 10])
def test_gemm_split_k(layout, tile):
    c, ref = run_gemm(1, layout, 256, 192, 2048, tile, splits=5)
    _check(c, ref, 2048)


@pytest.mark.parametrize("tile", [0, 4, 6, 7, 8, 9, 10, 11, 12])
def test_gemm_bf16_multi_tile(tile):
    c, ref = run_gemm(1, LAYOUT_KK, 1024, 768, 512, tile, seed=3)
    _check(c, ref, 512)


@pytest.mark.parametrize("layout", [LAYOUT_KN, LAYOUT_MN])
@pytest.mark.parametrize("tile", [10, 11, 12])
def test_gemm_bf16_ping_pong_multi_tile(layout, tile):
    c, ref = run_gemm(1, layout, 768, 1024, 640, tile, seed=4)
    _check(c, ref, 640)


@pytest.mark.parametrize("tile", [6, 7, 8, 9, 10, 11, 12])
def test_gemm_bf16_deep_pipeline_ragged(tile):
    # K not a multiple of the 32- or 64-element step, fewer steps than stages
    layouts = [LAYOUT_KK, LAYOUT_KN, LAYOUT_MN] if tile >= 10 else [LAYOUT_KK]
    for layout in layouts:
        for K in (40, 328):
            c, ref = run_gemm(1, layout, 264, 200, K, tile)
            _check(c, ref, K)
