"""The sliding step at the full size of the 123B-shaped slice, in the
configuration bench.py times (8 layers of hidden 12288, 96 query / 8 KV heads
of 128, ffn 28672, T = 4096; window 2, two pinned gradient slots, no
optimizer, steps pipelined, the turnaround layers kept in their units).
After three back-to-back steps the two slots hold the fp32 weight gradients
of the last two layers of the backward (layers 1 and 0), which must equal,
bit for bit, those of the same kernels run layer by layer with every weight
resident (sf_layer_fwd / sf_layer_bwd).  Those gradients depend on every
layer's forward (the page order of the forward, the preloaded and kept
layers) and on the input gradient each later layer's backward passes down,
so a wrong buffer anywhere in the step changes them.  The resident layer at
this size is checked against the oracle by the full-size layer tests (exact
causal-prefix and late-row reductions), so this carries that parity to the
benchmarked step."""

import pytest
import torch

import seeded_inputs as si
from layer_sliding_offloaded_amd import runtime as rt
from layer_sliding_offloaded_amd import sf
from tests.gpu.helpers import say

pytestmark = pytest.mark.gpu


def test_sliding_step_full_size_matches_resident_bitwise():
    w = si.WORKLOADS["slice123b-gqa-bf16"]
    nl, steps = w.n_layers, 3
    say("sliding step full size", w.name, "layers", nl, "window", w.window, "steps", steps)
    slots = 2
    torch._C._host_emptyCache()  # pinned blocks cached by earlier tests
    eng = rt.Engine(w, lambda l: si.layer_params(w, l), None, window=w.window, n_grad_slots=slots, adam=False,
                    chunk=2048, pipeline=True, keep_turnaround=True, draw_threads=4)
    L = eng.layout
    x = rt.to_storage_tensor(si.layer_input(w), w).cuda()
    dy = rt.to_storage_tensor(si.upstream_grad(w), w).cuda()

    say("resident reference")
    c = rt.Context(w, 2048)
    s = rt.stream_handle()
    dws = [eng.h_params[l].cuda() for l in range(nl)]
    xs = [x] + [rt.empty(w.tokens, w.hidden, dtype=rt.storage_dtype(w)) for _ in range(nl)]
    saved = [rt.device_bytes(L.saved_bytes) for _ in range(nl)]
    for l in range(nl):
        sf.sf_layer_fwd(c.ctx, dws[l].data_ptr(), xs[l].data_ptr(), xs[l + 1].data_ptr(), saved[l].data_ptr(), s)
    dbuf = dy.clone()
    ref = [None] * nl
    for l in reversed(range(nl)):
        g = rt.empty(L.grad_bytes // 4, dtype=torch.float32)
        sf.sf_layer_bwd(c.ctx, dws[l].data_ptr(), xs[l].data_ptr(), saved[l].data_ptr(), dbuf.data_ptr(),
                        dbuf.data_ptr(), g.data_ptr(), s)
        ref[l] = g
    torch.cuda.synchronize()
    c.close()
    del dws, xs, saved, dbuf

    say("engine steps")
    for t in range(steps):
        eng.step(x, dy)
    agg = eng.sync()
    torch.cuda.synchronize()
    assert agg["d2h_bytes"] > 0 and agg["h2d_bytes"] > 0
    # compared as raw 32-bit words, tensor by tensor (the padding between
    # tensors is not part of the result); each slot must hold one of the last
    # two layers' gradients exactly, and the two slots different layers
    def same(got, want):
        return all(torch.equal(got[o:o + n], want[o:o + n])
                   for o, n in ((L.grad_off[k] // 4, L.grad_bytes_t[k] // 4) for k in range(9)))

    held = []
    for sl in range(slots):
        got = eng.h_slots[sl][:L.grad_bytes].cuda().view(torch.int32)
        held.append([l for l in (0, 1) if same(got, ref[l].view(torch.int32))])
        del got
    say("slots hold layers", held)
    assert sorted(h[0] for h in held if len(h) == 1) == [0, 1], held
    eng.close()
    del eng, ref, x, dy
    torch.cuda.empty_cache()
    torch._C._host_emptyCache()
