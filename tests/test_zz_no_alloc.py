"""sf_gemm_noalloc (no workspace, static device scratch) gives the same bits
as sf_gemm with a caller workspace, on two calls in a row with the second
smaller, across the three layouts and with and without split-K; sizes whose
partial sums exceed the static scratch are refused before any device work."""

import numpy as np
import pytest
import torch

from layer_sliding_offloaded_amd import runtime as rt
from layer_sliding_offloaded_amd import sf
from tests.gpu.helpers import say

pytestmark = pytest.mark.gpu


def _operands(layout, M, N, K, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    a_shape = (K, M) if layout == 2 else (M, K)
    b_shape = (N, K) if layout == 0 else (K, N)
    A = torch.randn(a_shape, generator=g, device="cuda").to(torch.bfloat16)
    B = torch.randn(b_shape, generator=g, device="cuda").to(torch.bfloat16)
    return A, B, a_shape[1], b_shape[1]


def _with_workspace(layout, out_f32, M, N, K, A, lda, B, ldb):
    C = torch.empty((M, N), device="cuda", dtype=torch.float32 if out_f32 else torch.bfloat16)
    wsb = sf.sf_gemm_workspace_bytes(M, N, K)
    ws = rt.device_bytes(max(wsb, 256))
    sf.sf_gemm(sf.SF_BF16, layout, out_f32, M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, C.data_ptr(), N,
               rt.stream_handle(), ws.data_ptr(), wsb)
    return C


def _noalloc(layout, out_f32, M, N, K, A, lda, B, ldb):
    C = torch.full((M, N), float("nan"), device="cuda", dtype=torch.float32 if out_f32 else torch.bfloat16)
    sf.sf_gemm_noalloc(sf.SF_BF16, layout, out_f32, M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, C.data_ptr(), N,
                       rt.stream_handle())
    return C


# (layout, out_f32, first (M, N, K), second smaller (M, N, K))
CASES = [
    (1, 0, (1024, 1024, 8192), (512, 256, 4096)),   # NN: long-K split, then a small-grid split
    (2, 1, (256, 512, 8192), (128, 256, 4096)),     # TN, fp32 out: split both times
    (0, 0, (2048, 512, 2048), (256, 128, 1024)),    # NT
    (0, 0, (4096, 4096, 1024), (64, 64, 64)),       # NT, large grid: no split
]


@pytest.mark.parametrize("layout,out_f32,first,second", CASES)
def test_noalloc_matches_workspace_gemm(layout, out_f32, first, second):
    say("gemm-noalloc", layout, out_f32, first, second)
    ops = [_operands(layout, *shape, seed) for shape, seed in ((first, 1), (second, 2))]
    # two calls in a row: the second (smaller) finds the first's partial sums in the scratch
    got = [_noalloc(layout, out_f32, *shape, A, lda, B, ldb) for shape, (A, B, lda, ldb) in zip((first, second), ops)]
    ref = [_with_workspace(layout, out_f32, *shape, A, lda, B, ldb)
           for shape, (A, B, lda, ldb) in zip((first, second), ops)]
    torch.cuda.synchronize()
    for shape, g, r in zip((first, second), got, ref):
        say("shape", shape, "split-K bytes", sf.sf_gemm_workspace_bytes(*shape))
        assert torch.equal(g.view(torch.int16) if not out_f32 else g.view(torch.int32),
                           r.view(torch.int16) if not out_f32 else r.view(torch.int32)), shape
    if layout == 1:
        assert sf.sf_gemm_workspace_bytes(*first) > 0 and sf.sf_gemm_workspace_bytes(*second) > 0


def test_noalloc_refuses_partials_beyond_the_scratch():
    # [T, H] from K = 32768 over 152 tiles of 256 x 256: two k-ranges of fp32
    # partial sums, 2 * 2048 * 4864 * 4 bytes > 64 MiB
    M, N, K = 2048, 4864, 32768
    need = sf.sf_gemm_workspace_bytes(M, N, K)
    say("gemm-noalloc-refuse", need)
    assert need > sf.GEMM_STATIC_SCRATCH_BYTES
    # full-size operands, so that even a launch would stay in bounds
    A = torch.zeros((M, K), device="cuda", dtype=torch.bfloat16)
    B = torch.zeros((K, N), device="cuda", dtype=torch.bfloat16)
    C = torch.full((M, N), 7.0, device="cuda", dtype=torch.bfloat16)
    with pytest.raises(sf.SfError) as ei:
        sf.sf_gemm_noalloc(sf.SF_BF16, 1, 0, M, N, K, A.data_ptr(), K, B.data_ptr(), N, C.data_ptr(), N,
                           rt.stream_handle())
    assert ei.value.code == sf.SF_ERR_POOL
    torch.cuda.synchronize()
    assert torch.all(C == 7.0)
