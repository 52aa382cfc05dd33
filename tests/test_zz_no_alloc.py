"""gpt_gemm_noalloc (split-K partials in the library's own scratch array)
against gpt_gemm (partials in a caller workspace): the same kernels, so the
outputs must agree bit for bit.  Two calls in a row, the second smaller, so
the second reads nothing the first left behind."""
import numpy as np
import pytest

from tests.gpu_common import log

pytestmark = pytest.mark.gpu

LAYOUT_KN, LAYOUT_MN = 1, 2


def _pair(dtype, layout, M, N, K, splits, seed):
    import torch
    import decoder_only_transformer_fwd_amd as G
    rng = np.random.default_rng(seed)
    ar = (K, M) if layout == LAYOUT_MN else (M, K)
    tdt = torch.bfloat16 if dtype == 1 else torch.float32
    A = torch.from_numpy(rng.standard_normal(ar).astype(np.float32)).cuda().to(tdt)
    B = torch.from_numpy(rng.standard_normal((K, N)).astype(np.float32)).cuda().to(tdt)
    st = torch.cuda.current_stream().cuda_stream
    C1 = torch.full((M, N), float("nan"), device="cuda")
    C2 = torch.full((M, N), float("nan"), device="cuda")
    ws = torch.empty(splits * M * N, device="cuda")
    log(f"noalloc gemm dtype={dtype} layout={layout} M={M} N={N} K={K} splits={splits}")
    G.gpt_gemm(dtype, layout, M, N, K, A.data_ptr(), B.data_ptr(), C1.data_ptr(), ws.data_ptr(), splits, -1, st)
    G.gpt_gemm_noalloc(dtype, layout, M, N, K, A.data_ptr(), B.data_ptr(), C2.data_ptr(), splits, -1, st)
    torch.cuda.synchronize()
    c1, c2 = C1.cpu().numpy(), C2.cpu().numpy()
    assert np.all(np.isfinite(c2))
    assert np.array_equal(c1, c2)
    # and against the plain product (rounded operands, fp64)
    ref = A.float().cpu().numpy().astype(np.float64)
    ref = (ref.T if layout == LAYOUT_MN else ref) @ B.float().cpu().numpy().astype(np.float64)
    assert np.max(np.abs(c2 - ref)) <= 1e-4 * np.sqrt(K)


@pytest.mark.parametrize("dtype", [1, 0])
def test_noalloc_matches_workspace_entry_point(dtype):
    # a weight-gradient shaped product split 4 ways, then a smaller one split 3 ways
    _pair(dtype, LAYOUT_MN, 1536, 1536, 8192, 4, seed=1)
    _pair(dtype, LAYOUT_KN, 256, 520, 3000, 3, seed=2)
    # no split (the scratch is not touched)
    _pair(dtype, LAYOUT_MN, 128, 64, 512, 1, seed=3)
