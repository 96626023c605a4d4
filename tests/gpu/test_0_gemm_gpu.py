"""Parity of the MFMA GEMM (sf_gemm) in its three operand layouts against a
float64 matmul of the same stored operands, at sizes spanning several tiles
with ragged tails in every dimension."""

import numpy as np
import pytest
import torch

from layer_sliding_offloaded_amd import runtime as rt
from layer_sliding_offloaded_amd import sf
from tests.gpu.helpers import rel, say

pytestmark = pytest.mark.gpu

# the last two have few output tiles and a long K: split-K applies when a workspace is given
SHAPES = [(128, 256, 64), (200, 688, 256), (1000, 520, 1376), (37, 8, 8), (4096, 1024, 520), (300, 3072, 2048),
          (512, 1024, 32000), (1024, 1024, 2600),
          # >= 256 tiles of 256 x 256: the large-grid kernels, ragged in M, N and K (K % 32 = 8)
          (4104, 4112, 1000),
          # large grids with fewer k-steps than one pass of the NT kernel's 12-step loop body:
          # two 32-k steps, the second and the only 64-k B line partly past K; 7 steps, 4 lines
          (4104, 4104, 40), (2056, 8200, 200)]


@pytest.mark.parametrize("layout", [0, 1, 2], ids=["NT", "NN", "TN"])
@pytest.mark.parametrize("dtype", [sf.SF_F32, sf.SF_BF16, sf.SF_F16], ids=["f32", "bf16", "f16"])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_parity(layout, dtype, M, N, K):
    say("gemm", layout, dtype, M, N, K)
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    tdt = {sf.SF_F32: torch.float32, sf.SF_BF16: torch.bfloat16, sf.SF_F16: torch.float16}[dtype]
    a_shape = (K, M) if layout == 2 else (M, K)
    b_shape = (N, K) if layout == 0 else (K, N)
    if a_shape[1] % 8:
        # out of contract (A's contiguous dimension: M for TN, K otherwise):
        # refused on the host before any device work
        dA = torch.zeros(a_shape, dtype=tdt, device="cuda")
        dB = torch.zeros(b_shape, dtype=tdt, device="cuda")
        C = torch.zeros((M, N), dtype=torch.float32, device="cuda")
        with pytest.raises(sf.SfError) as e:
            sf.sf_gemm(dtype, layout, 1, M, N, K, dA.data_ptr(), a_shape[1], dB.data_ptr(), b_shape[1],
                       C.data_ptr(), N, rt.stream_handle(), None, 0)
        assert e.value.code == sf.SF_ERR_UNSUPPORTED
        return
    A = torch.from_numpy(rng.standard_normal(a_shape, dtype=np.float32)).to(tdt)
    B = torch.from_numpy(rng.standard_normal(b_shape, dtype=np.float32)).to(tdt)
    a64 = A.double().numpy()
    b64 = B.double().numpy()
    ref = (a64.T if layout == 2 else a64) @ (b64.T if layout == 0 else b64)
    dA, dB = A.cuda(), B.cuda()
    wsb = sf.sf_gemm_workspace_bytes(M, N, K)
    ws = rt.empty(max(wsb, 16), dtype=torch.uint8)
    out = {}
    for split in (False, True):
        for out_f32 in (1, 0):
            C = torch.full((M, N), float("nan"), dtype=torch.float32 if out_f32 else tdt, device="cuda")
            sf.sf_gemm(dtype, layout, out_f32, M, N, K, dA.data_ptr(), a_shape[1], dB.data_ptr(), b_shape[1],
                       C.data_ptr(), N, rt.stream_handle(), ws.data_ptr() if split else None, wsb if split else 0)
            torch.cuda.synchronize()
            out[split, out_f32] = C.double().cpu().numpy()
        # fp32 accumulation over K terms: relative error ~ sqrt(K) 2^-24 (1e-5 at K = 32000)
        tol = 1e-5
        assert rel(out[split, 1], ref) <= tol, (split, rel(out[split, 1], ref))
        # storage-dtype output: one more rounding of the fp32 result (bf16:
        # 2^-9, fp16: 2^-12 relative at most)
        tol_s = {sf.SF_F32: 1e-5, sf.SF_BF16: 4e-3, sf.SF_F16: 5e-4}[dtype]
        assert rel(out[split, 0], ref) <= tol_s
