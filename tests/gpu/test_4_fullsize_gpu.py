"""Parity of one decoder layer at the full sizes of the larger workloads (the
1.3B- and 6.7B-shaped layers, T = 8192, and the 123B-shaped GQA slice,
hidden 12288, seq 4096; the 6.7B- and 123B-shaped layers also in fp16
storage), in the
same launch configuration the engine uses.

The fp64 oracle cannot run a whole layer at these sizes, so two exact
reductions are used:

* prefix: the upstream gradient is nonzero only at the first P positions of
  sequence 0.  By causality every output the backward produces then depends
  on that prefix alone -- the oracle runs the layer on x[0, :P] -- and every
  other dx row must be exactly zero.  The weight gradients are sums over
  those P rows only.
* late rows: the forward output at a few late positions of the last sequence
  (up to S - 1, so every key tile is crossed) is computed one row at a time
  by ``oracle.layer_fwd_rows``.
"""

import numpy as np
import pytest

import oracle
import seeded_inputs as si
from tests.gpu.helpers import LayerRun, check_errors, f64, oracle_shape, rel, say

pytestmark = pytest.mark.gpu

# name: (workload, prefix P, tolerance, storage unit roundoff of the deltas' floor)
F16_TOL = 2.5e-3  # the bf16 bound's multiple of the unit roundoff (5.1 x 2^-11)
CASES = {
    "llama1.3b-bf16": (si.WORKLOADS["llama1.3b-bf16"], 160, 2e-2, 2.0 ** -8),
    "llama6.7b-bf16": (si.WORKLOADS["llama6.7b-bf16"], 160, 2e-2, 2.0 ** -8),
    "slice123b-gqa-bf16": (si.WORKLOADS["slice123b-gqa-bf16"], 96, 2e-2, 2.0 ** -8),
    "llama6.7b-f16": (si.WORKLOADS["llama6.7b-bf16"].with_(dtype="f16"), 160, F16_TOL, 2.0 ** -11),
    "slice123b-gqa-f16": (si.WORKLOADS["slice123b-gqa-bf16"].with_(dtype="f16"), 96, F16_TOL, 2.0 ** -11),
}


@pytest.mark.parametrize("name", list(CASES))
def test_full_size_layer(name):
    w, P, tol, u = CASES[name]
    say("full-size layer", name, "prefix", P)
    p = si.layer_params(w, 0, gains="random")
    x = si.layer_input(w)
    dy = si.upstream_grad(w)
    dy_m = np.zeros_like(dy)
    dy_m[0, :P] = dy[0, :P]
    r = LayerRun(w, p, x, dy_m)
    r.fwd()
    r.bwd()
    y, dx, g = r.results()
    r.close()
    del r

    # exact zeros outside the prefix
    assert np.all(dx[0, P:] == 0.0)
    assert np.all(dx[1:] == 0.0)

    p64 = f64(p)
    del p
    sh = oracle_shape(w.with_(batch=1, seq=P))
    x0 = x[0:1, :P].astype(np.float64)
    yo, cache = oracle.layer_fwd(p64, x0, sh)
    dxo, go = oracle.layer_bwd(p64, cache, dy_m[0:1, :P].astype(np.float64), sh)
    errs = {"y": rel(y[0:1, :P], yo), "y-x": rel(y[0:1, :P] - x0, yo - x0), "dx": rel(dx[0:1, :P], dxo),
            "dx-dy": rel(dx[0:1, :P] - dy_m[0:1, :P], dxo - dy_m[0:1, :P])}
    errs["floor:y-x"] = u * np.linalg.norm(yo) / np.linalg.norm(yo - x0)
    errs["floor:dx-dy"] = u * np.linalg.norm(dxo) / np.linalg.norm(dxo - dy_m[0:1, :P])
    for k in go:
        errs["d" + k] = rel(g[k], go[k])
    del go, cache
    # late rows of the last sequence, forward only
    S = w.seq
    rows = np.array(sorted({S // 3, (2 * S) // 3, S - 65, S - 1}))
    xl = x[w.batch - 1].astype(np.float64)
    yl = oracle.layer_fwd_rows(p64, xl, rows, oracle_shape(w))
    errs["y_late"] = rel(y[w.batch - 1, rows], yl)
    errs["y-x_late"] = rel(y[w.batch - 1, rows] - xl[rows], yl - xl[rows])
    errs["floor:y-x_late"] = u * np.linalg.norm(yl) / np.linalg.norm(yl - xl[rows])
    print({k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    bad = check_errors(errs, tol)
    assert not bad, bad
