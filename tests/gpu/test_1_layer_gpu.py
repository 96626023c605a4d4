"""Parity of one decoder layer's forward and backward (HIP path via the C ABI)
against the fp64 oracle, element by element on the same seeded inputs.

Tolerances (relative L2 per tensor): 1e-4 for fp32 storage, 2e-2 for bf16
storage; also on the residual-free deltas y - x and dx - dy.  fp16 storage
gets the same multiple of its unit roundoff as bf16: 2e-2 is 5.1 x 2^-8, so
5.1 x 2^-11 = 2.5e-3.
"""

import numpy as np
import pytest
import torch

import seeded_inputs as si
from tests.gpu.helpers import LayerRun, check_errors, layer_errors, make_layer_case, say

pytestmark = pytest.mark.gpu

W = si.WORKLOADS
BASE = W["layer-h256-fp32"]

GQA128 = dict(hidden=512, n_heads=4, n_kv_heads=2, head_dim=128, ffn=1376)
F16_TOL = 2.5e-3
# name: (workload, tolerance, input scale)
CASES = {
    # the fp32 single-layer workload at its full size
    "fp32-h256-b1-s128": (BASE, 1e-4, 1.0),
    # ragged: T = 200 (not a multiple of any tile), seq 100 (ragged attention tiles), F = 688
    "fp32-h256-b2-s100": (BASE.with_(batch=2, seq=100), 1e-4, 1.0),
    "fp32-gqa-d128-s72": (BASE.with_(batch=1, seq=72, **GQA128), 1e-4, 1.0),
    "bf16-h256-b2-s160": (BASE.with_(dtype="bf16", batch=2, seq=160), 2e-2, 0.05),
    "bf16-h256-b2-s160-x1": (BASE.with_(dtype="bf16", batch=2, seq=160), 2e-2, 1.0),
    "bf16-gqa-d128-b2-s200": (BASE.with_(dtype="bf16", batch=2, seq=200, **GQA128), 2e-2, 0.05),
    "bf16-mqa-d64-s130": (BASE.with_(dtype="bf16", hidden=512, n_heads=8, n_kv_heads=1, head_dim=64, ffn=1024,
                                     batch=1, seq=130), 2e-2, 0.05),
    "bf16-seq1": (BASE.with_(dtype="bf16", batch=3, seq=1), 2e-2, 0.05),
    # attention tile edges: one key tile exactly, a second tile of one row, tile-aligned rows
    "bf16-s64": (BASE.with_(dtype="bf16", batch=2, seq=64), 2e-2, 0.05),
    "bf16-gqa-d128-s65": (BASE.with_(dtype="bf16", batch=1, seq=65, **GQA128), 2e-2, 0.05),
    "bf16-s128": (BASE.with_(dtype="bf16", batch=2, seq=128), 2e-2, 0.05),
    # one layer of the 4-layer h1024 stack at its full size (T = 2048), standard inputs
    "bf16-stack4-h1024-full": (W["stack4-h1024-bf16"], 2e-2, 1.0),
    # fp16 storage: the same kernels with IEEE half operands
    "f16-h256-b2-s160": (BASE.with_(dtype="f16", batch=2, seq=160), F16_TOL, 0.05),
    "f16-h256-b2-s160-x1": (BASE.with_(dtype="f16", batch=2, seq=160), F16_TOL, 1.0),
    "f16-gqa-d128-b2-s200": (BASE.with_(dtype="f16", batch=2, seq=200, **GQA128), F16_TOL, 0.05),
    "f16-s65-seq-edge": (BASE.with_(dtype="f16", batch=2, seq=65), F16_TOL, 0.05),
    "f16-seq1": (BASE.with_(dtype="f16", batch=3, seq=1), F16_TOL, 0.05),
    "f16-stack4-h1024-full": (W["stack4-h1024-bf16"].with_(dtype="f16"), F16_TOL, 1.0),
    # wide rows (one block of four waves per row for the RMSNorm forward and
    # backward): hidden 4096 and 6144 in 16-bit storage, 2048 in fp32
    "bf16-h4096-wide-rows": (BASE.with_(dtype="bf16", hidden=4096, n_heads=32, n_kv_heads=8, head_dim=128,
                                        ffn=1024, batch=1, seq=64), 2e-2, 0.05),
    "f16-h6144-wide-rows": (BASE.with_(dtype="f16", hidden=6144, n_heads=48, n_kv_heads=8, head_dim=128, ffn=512,
                                       batch=1, seq=40), F16_TOL, 0.05),
    "fp32-h2048-wide-rows": (BASE.with_(hidden=2048, n_heads=16, n_kv_heads=16, head_dim=128, ffn=1024, batch=2,
                                        seq=24), 1e-4, 1.0),
}


@pytest.mark.parametrize("name", list(CASES))
def test_layer_parity(name):
    w, tol, scale = CASES[name]
    say(name, w, "input scale", scale)
    p, x, dy = make_layer_case(w, scale=scale)
    r = LayerRun(w, p, x, dy)
    r.fwd()
    r.bwd()
    y, dx, g = r.results()
    r.close()
    errs = layer_errors(w, p, x, dy, y, dx, g)
    print({k: f"{v:.2e}" for k, v in errs.items()})
    bad = check_errors(errs, tol)
    assert not bad, bad


def test_layer_backward_is_deterministic():
    w = BASE.with_(dtype="bf16", batch=2, seq=256)
    say("determinism", w)
    p, x, dy = make_layer_case(w)
    r = LayerRun(w, p, x, dy)
    r.fwd()
    r.bwd()
    y1, dx1, g1 = r.results()
    r.fwd()
    r.bwd()
    y2, dx2, g2 = r.results()
    r.close()
    assert np.array_equal(y1, y2) and np.array_equal(dx1, dx2)
    for k in g1:
        assert np.array_equal(g1[k], g2[k]), k


def test_causal_prefix_property():
    """Upstream gradient only at positions <= s0: every dx row after s0 is exactly 0."""
    w = BASE.with_(dtype="bf16", batch=2, seq=192)
    say("causal-prefix", w)
    p, x, dy = make_layer_case(w)
    s0 = 70
    dy = dy.copy()
    dy[:, s0 + 1:] = 0.0
    r = LayerRun(w, p, x, dy)
    r.fwd()
    r.bwd()
    _, dx, _ = r.results()
    r.close()
    assert np.all(dx[:, s0 + 1:] == 0.0)
    assert np.all(np.any(dx[:, :s0 + 1] != 0.0, axis=-1))
