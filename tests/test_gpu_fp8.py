"""GPU checks of the fp8 building blocks through the C ABI.

The quantiser must reproduce the oracle's OCP codec bit for bit, with the
scale and the products x * s rounded in fp32 on both sides (the precision in
which the quantiser takes its rounding decisions).  The fp8 product must
match the exact fp64 product of the decoded codes, rescaled by
1 / (s_a s_b), to within fp32 accumulation error.
"""
import numpy as np
import pytest

import gpt_inputs as gi
from oracle import fp8_codec as F
from tests.gpu_common import log

pytestmark = pytest.mark.gpu

FMT = {0: "e4m3", 1: "e5m2"}


def _dev_bf16(torch, x64):
    bits = gi.bf16_bits_from_f32(np.asarray(x64, dtype=np.float32))
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).cuda()
    return t, gi.bf16_bits_to_f64(bits)


def _quantize(torch, G, fmt, xt, R, C, transposed=True):
    q = torch.empty((R, C), dtype=torch.uint8, device="cuda")
    qT = torch.empty((C, R), dtype=torch.uint8, device="cuda") if transposed else None
    amax = torch.full((64,), 12345, dtype=torch.int32, device="cuda")   # scratch, overwritten
    scale = torch.zeros(1, dtype=torch.float32, device="cuda")
    G.gpt_fp8_quantize(fmt, xt.data_ptr(), R, C, amax.data_ptr(), scale.data_ptr(), q.data_ptr(),
                       qT.data_ptr() if transposed else 0, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return q, qT, scale


def _wide_range(rng, shape, scale):
    """Normals times 10^U(-5, 0): values over many binades, incl. fp8 subnormals."""
    x = rng.standard_normal(shape) * scale * 10.0 ** rng.uniform(-5, 0, shape)
    x.flat[::97] = 0.0
    x.flat[1::101] = -0.0
    return x


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("R,C", [(64, 64), (200, 192), (448, 1536), (1000, 320)])
def test_quantize_is_bit_exact(fmt, R, C):
    import torch
    import decoder_only_transformer_fwd_amd as G
    rng = np.random.default_rng(1000 * R + C + fmt)
    x = _wide_range(rng, (R, C), 0.5)
    x[R // 2, C // 3] = -3.75   # the amax, negative
    xt, xb = _dev_bf16(torch, x)
    log(f"quantize fmt={FMT[fmt]} R={R} C={C}")
    q, qT, scale = _quantize(torch, G, fmt, xt, R, C)
    want, s = F.quantize_tensor(xb, FMT[fmt], dtype=np.float32)
    assert np.float32(scale.item()) == np.float32(s)
    got = q.cpu().numpy()
    bad = np.argwhere(got != want)
    assert bad.size == 0, (len(bad), bad[:5], got[tuple(bad[0])], want[tuple(bad[0])], xb[tuple(bad[0])])
    np.testing.assert_array_equal(qT.cpu().numpy(), want.T)


@pytest.mark.parametrize("fmt", [0, 1])
def test_quantize_all_zero_tensor(fmt):
    import torch
    import decoder_only_transformer_fwd_amd as G
    x = np.zeros((64, 128))
    x[:, ::2] = -0.0
    xt, xb = _dev_bf16(torch, x)
    q, qT, scale = _quantize(torch, G, fmt, xt, 64, 128, transposed=False)
    want, s = F.quantize_tensor(xb, FMT[fmt], dtype=np.float32)
    assert s == 1.0 and scale.item() == 1.0
    np.testing.assert_array_equal(q.cpu().numpy(), want)


def _codes(rng, fmt, shape, sigma):
    """Codes of quantised normals (the oracle's encoder), and their values."""
    c = F.encode(rng.standard_normal(shape) * sigma, fmt)
    return c, F.decode(c, fmt)


@pytest.mark.parametrize("fmt_a,M,N,K,splits", [
    (0, 256, 128, 256, 1),
    (0, 200, 136, 272, 1),      # ragged in M, N and K
    (1, 384, 1536, 1536, 1),
    (1, 520, 264, 4096, 3),     # split K, ragged tiles
    (1, 512, 512, 16384, 4),    # weight-gradient depth
])
def test_fp8_gemm_matches_exact_products(fmt_a, M, N, K, splits):
    import torch
    import decoder_only_transformer_fwd_amd as G
    rng = np.random.default_rng(M * 7 + N * 3 + K + fmt_a)
    ca, va = _codes(rng, FMT[fmt_a], (M, K), 100.0 if fmt_a == 0 else 3000.0)
    cb, vb = _codes(rng, "e4m3", (N, K), 60.0)
    sa, sb = np.float32(3.5), np.float32(0.1875)
    want = (va @ vb.T) / (float(sa) * float(sb))
    bound = (np.abs(va) @ np.abs(vb).T) / (float(sa) * float(sb))
    log(f"fp8 gemm fmt_a={FMT[fmt_a]} M={M} N={N} K={K} splits={splits}")
    A = torch.from_numpy(ca).cuda()
    B = torch.from_numpy(cb).cuda()
    scales = torch.tensor([sa, sb], dtype=torch.float32, device="cuda")
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(splits * M * N if splits > 1 else 1, dtype=torch.float32, device="cuda")
    G.gpt_gemm_fp8(fmt_a, M, N, K, A.data_ptr(), B.data_ptr(), scales.data_ptr(), scales.data_ptr() + 4,
                   C.data_ptr(), ws.data_ptr() if splits > 1 else 0, splits, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = C.cpu().numpy().astype(np.float64)
    err = np.abs(got - want)
    worst = float(np.max(err / (bound + 1e-30)))
    log(f"  max |err| / sum|a||b| = {worst:.2e}")
    assert np.all(np.isfinite(got))
    assert worst <= 2e-5
