"""Step-level parity of the sliding engine with the fp64 oracle.

The engine's whole training iteration -- embedding, every decoder layer with
its weights streamed in, the fused LinearCrossEntropy head, the backward with
each layer's fp32 gradients streamed out, host Adam -- against
``oracle.stack_step`` and ``oracle.adam_step`` on the same seeded inputs, at
the shape of the 4-layer hidden-1024 stack (16 heads x 64, ffn 2816, vocab
32000, batch 4 x seq 512; window 2), which is the benchmarked stack.

The pages' engine overlaps the host update of L_i with the device's work on
L_{i-1} (es "Resumen tecnico" §2A "Actualizacion Asincrona"), which the
pipelined schedule carries across the step boundary, and moves activations
through host memory (de §2B "Sliding Activation Checkpointing"); both are
scheduling, so every mode must reach the oracle's numbers.

Gradients are read from the engine's pinned gradient slots: the backward
hands the slots out in turn (layer n_layers-1 first), so with
k * n_layers slots step s's gradients of layer i stay in slot
(s-1) * n_layers + n_layers-1-i for k steps.

Tolerances: rel-L2 per tensor <= 2e-2 for bf16 gradients and the loss; post-
step weights <= 1e-3 relative.  Adam's update is invariant to the gradient's
scale, which is why the gradients are compared directly.  In fp32 storage,
where the gradients are exact to ~1e-6, the update itself (w_t - w_0) is held
to 1e-3 against the oracle's, which fixes the tensors Adam is applied to, its
step numbers and its order.
"""

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from layer_sliding_offloaded_amd import runtime as rt
from layer_sliding_offloaded_amd import sf
from tests.gpu.helpers import f64, oracle_shape, oracle_trajectory, rel, say, stack_inputs

pytestmark = pytest.mark.gpu

C2 = si.WORKLOADS["stack4-h1024-bf16"]
STEPS = 3
HP = si.ADAM
BF16_TOL = 2e-2
W_TOL = 1e-3


@pytest.fixture(scope="module")
def c2_case():
    layers, head, ids = stack_inputs(C2)
    traj = oracle_trajectory(C2, layers, head, ids, STEPS, HP, oracle.round_bf16)
    return layers, head, ids, traj


def _slot_grads(eng, slot, shapes):
    return rt.unpack_grads(eng.layout, eng.h_slots[slot].numpy().view(np.float32), shapes)


def _head_grads_device(eng):
    """dgf and dW_lm as the engine left them in d_head_grads [dE | dgf | dWlm]."""
    V, H = eng.w.vocab, eng.w.hidden
    hg = eng.d_head_grads.cpu().numpy()
    return hg[V * H:V * H + H], hg[V * H + H:].reshape(V, H)


def _check_grads(errs, got, ref, tag, tol):
    for k in ref:
        errs[f"{tag}.d{k}"] = (rel(got[k], ref[k]), tol)


def _fail(errs):
    bad = {k: f"{v:.3e} > {t:g}" for k, (v, t) in errs.items() if not v <= t}
    say("errors", {k: f"{v:.2e}" for k, (v, _) in errs.items()})
    assert not bad, bad


def test_engine_c2_gradients_match_oracle_adam_off(c2_case):
    """Adam off: loss, every layer's nine gradients, the dense embedding
    gradient, the final gain's and the LM head's gradients of one engine
    step against the oracle, tensor by tensor."""
    layers, head, ids, traj = c2_case
    w = C2
    nl = w.n_layers
    say("engine-c2-adam-off", w)
    eng = rt.Engine(w, layers, head, window=2, n_grad_slots=nl, adam=False, chunk=2048)
    loss, _ = eng.step(torch.from_numpy(ids.reshape(-1)).cuda())
    eng.sync()
    torch.cuda.synchronize()
    ref = traj[0]
    shapes = {k: v.shape for k, v in layers[0].items()}
    errs = {"loss": (abs(loss - ref["loss"]) / ref["loss"], BF16_TOL)}
    for i in range(nl):
        _check_grads(errs, _slot_grads(eng, nl - 1 - i, shapes), ref["layers"][i], f"L{i}", BF16_TOL)
    V, H = w.vocab, w.hidden
    hg = eng.d_head_grads.cpu().numpy()
    errs["dE"] = (rel(hg[:V * H].reshape(V, H), ref["head"]["E"]), BF16_TOL)
    errs["dgf"] = (rel(hg[V * H:V * H + H], ref["head"]["gf"]), BF16_TOL)
    errs["dWlm"] = (rel(hg[V * H + H:].reshape(V, H), ref["head"]["Wlm"]), BF16_TOL)
    eng.close()
    _fail(errs)


def test_engine_c2_keep_turnaround_pipelined_matches_oracle(c2_case):
    """Without Adam, with the parameters fixed between steps: the layers that
    end the backward in their units open the next forward without an upload,
    and steps return while the last gradient copies still run.  Two such
    steps give the same gradients, bit for bit, as one plain step, the
    oracle's gradients within the bf16 tolerance, and move W layers' worth
    of parameters less over the host link in the second step."""
    layers, head, ids, traj = c2_case
    w = C2
    nl = w.n_layers
    say("engine-c2-keep-turnaround", w)
    d_ids = torch.from_numpy(ids.reshape(-1)).cuda()
    ref = rt.Engine(w, layers, head, window=2, n_grad_slots=nl, adam=False, chunk=2048)
    loss0, st0 = ref.step(d_ids)
    ref.sync()
    ref_slots = [t.numpy().copy() for t in ref.h_slots]
    ref.close()
    eng = rt.Engine(w, layers, head, window=2, n_grad_slots=nl, adam=False, chunk=2048, pipeline=True,
                    keep_turnaround=True)
    losses = [eng.step(d_ids)[0] for _ in range(2)]
    agg = eng.sync()
    torch.cuda.synchronize()
    assert losses == [loss0, loss0]
    for k in range(nl):
        assert np.array_equal(eng.h_slots[k].numpy(), ref_slots[k]), k
    assert agg["h2d_bytes"] == 2 * st0["h2d_bytes"] - 2 * eng.layout.param_bytes
    assert agg["d2h_bytes"] == 2 * st0["d2h_bytes"]
    shapes = {k: v.shape for k, v in layers[0].items()}
    errs = {"loss": (abs(losses[-1] - traj[0]["loss"]) / traj[0]["loss"], BF16_TOL)}
    for i in range(nl):
        _check_grads(errs, _slot_grads(eng, nl - 1 - i, shapes), traj[0]["layers"][i], f"L{i}", BF16_TOL)
    eng.close()
    _fail(errs)


@pytest.mark.parametrize("mode", ["sync", "pipeline", "ckpt", "pipeline-ckpt"])
def test_engine_c2_steps_match_oracle(c2_case, mode):
    """Three Adam steps of the engine at the C2 shape against the oracle's
    three-step trajectory: every step's loss and layer gradients, the last
    step's head gradients, and the weights after the last step.  Pipelined,
    the three steps run back to back with host Adam of one step overlapping
    the next step's device work."""
    layers, head, ids, traj = c2_case
    w = C2
    nl = w.n_layers
    pipe, ck = "pipeline" in mode, "ckpt" in mode
    say("engine-c2-steps", mode, w)
    eng = rt.Engine(w, layers, head, window=2, n_grad_slots=STEPS * nl, adam=True, chunk=2048, adam_hp=HP,
                    ckpt=ck, pipeline=pipe)
    L = eng.layout
    d_ids = torch.from_numpy(ids.reshape(-1)).cuda()
    nh = eng.h_head_master.size
    h0 = eng.h_head_master.copy()
    losses = []
    for t in range(STEPS):
        loss, _ = eng.step(d_ids)
        losses.append(loss)
        if not pipe:
            eng.sync()
    eng.sync()
    torch.cuda.synchronize()
    shapes = {k: v.shape for k, v in layers[0].items()}
    errs = {}
    for t in range(STEPS):
        ref = traj[t]
        errs[f"s{t + 1}.loss"] = (abs(losses[t] - ref["loss"]) / ref["loss"], BF16_TOL)
        for i in range(nl):
            slot = t * nl + nl - 1 - i
            _check_grads(errs, _slot_grads(eng, slot, shapes), ref["layers"][i], f"s{t + 1}.L{i}", BF16_TOL)
    last = traj[-1]
    dgf, dwlm = _head_grads_device(eng)
    errs[f"s{STEPS}.dgf"] = (rel(dgf, last["head"]["gf"]), BF16_TOL)
    errs[f"s{STEPS}.dWlm"] = (rel(dwlm, last["head"]["Wlm"]), BF16_TOL)
    for i in range(nl):
        got = eng.h_master[i].astype(np.float64)
        want = rt.master_from_params(L, last["master_layers"][i]).astype(np.float64)
        errs[f"L{i}.w"] = (rel(got, want), W_TOL)
        # the bf16 parameters the next step reads are the rounded masters
        bits = eng.h_params[i].numpy().view(np.uint16)
        for k, name in enumerate(sf.TENSOR_NAMES):
            o, n, po = L.grad_off[k] // 4, L.grad_bytes_t[k] // 4, L.off[k] // 2
            assert np.array_equal(bits[po:po + n], si.f32_to_bf16_bits(eng.h_master[i][o:o + n])), (i, name)
    # head: device Adam state (fp32 masters [E | gf | Wlm])
    torch.cuda.synchronize()
    hm = eng.d_head_state[:nh].cpu().numpy().astype(np.float64)
    V, H = w.vocab, w.hidden
    for name, lo, hi in (("E", 0, V * H), ("gf", V * H, V * H + H), ("Wlm", V * H + H, nh)):
        want = last["master_head"][name].reshape(-1)
        errs[f"head.{name}.w"] = (rel(hm[lo:hi], want), W_TOL)
    eng.close()
    _fail(errs)
    # Embedding rows with a zero gradient keep their weights exactly: ids
    # absent from the batch, and ids seen only at a sequence's last position
    # (it has no target, and causal attention lets x0 there reach only that
    # position's output).  Every other row moves.
    moved = np.zeros(V, dtype=bool)
    moved[ids[:, :-1].reshape(-1)] = True
    E1 = hm[:V * H].reshape(V, H)
    E0 = h0[:V * H].reshape(V, H)
    assert np.array_equal(E1[~moved], E0[~moved])
    assert np.all(np.any(E1[moved] != E0[moved], axis=1))


F32_TOL = 1e-4


@pytest.mark.parametrize("n_layers", [1, 3])
def test_engine_fp32_matches_oracle(n_layers):
    """fp32 storage end to end through sf_slide_step (the layer-h256-fp32
    shape: hidden 256, 4 heads x 64, ffn 688, batch 1 x seq 128), one and
    three layers with window 2, no head (x and dy in), two Adam steps: every
    layer's gradients of both steps, the last layer's output and the input
    gradient at 1e-4, and the update w_2 - w_0 of every layer at 1e-3 against
    the oracle's two-step trajectory (fp32 parameters between the steps); the
    fp32 parameters the engine streams (a separate buffer from the master)
    are the master's copy."""
    w = si.WORKLOADS["layer-h256-fp32"].with_(n_layers=n_layers)
    say("engine-fp32", n_layers, w)
    layers = [si.layer_params(w, l, gains="random") for l in range(n_layers)]
    x = si.layer_input(w)
    dy = si.upstream_grad(w)
    eng = rt.Engine(w, layers, None, window=2, n_grad_slots=2 * n_layers, adam=True, adam_hp=HP)
    L = eng.layout
    d_x = rt.to_storage_tensor(x, w).cuda()
    d_dy = rt.to_storage_tensor(dy, w).cuda()
    for _ in range(2):
        eng.step(d_x, d_dy)
    eng.sync()
    torch.cuda.synchronize()
    sh = oracle_shape(w)
    rnd32 = lambda a: np.asarray(a, dtype=np.float32).astype(np.float64)
    cur = [f64(p) for p in layers]
    master = [f64(p) for p in layers]
    states = [{k: (np.zeros_like(v), np.zeros_like(v)) for k, v in p.items()} for p in cur]
    grads, outs = [], []
    for t in (1, 2):
        xs, caches = [x.astype(np.float64)], []
        for p in cur:
            y, c = oracle.layer_fwd(p, xs[-1], sh)
            xs.append(y)
            caches.append(c)
        d = dy.astype(np.float64)
        lg = [None] * n_layers
        for i in reversed(range(n_layers)):
            d, lg[i] = oracle.layer_bwd(cur[i], caches[i], d, sh)
        grads.append(lg)
        outs.append((xs[-1], d))
        for i in range(n_layers):
            master[i] = oracle.model.adam_all(master[i], lg[i], states[i], t, HP["lr"], HP["b1"], HP["b2"], HP["eps"])
            cur[i] = {k: rnd32(v) for k, v in master[i].items()}
    errs = {}
    shapes = {k: v.shape for k, v in layers[0].items()}
    n = w.tokens * w.hidden * 4
    base = eng.act.data_ptr()
    oy = sf.sf_engine_layer_input(eng.eng, n_layers) - base
    od = sf.sf_engine_dx0(eng.eng) - base
    yo, do = outs[-1]
    yL = eng.act[oy:oy + n].cpu().numpy().view(np.float32).reshape(yo.shape)
    dx0 = eng.act[od:od + n].cpu().numpy().view(np.float32).reshape(do.shape)
    errs["y"] = (rel(yL, yo), F32_TOL)
    errs["dx"] = (rel(dx0, do), F32_TOL)
    errs["dx-dy"] = (rel(dx0 - dy, do - dy), F32_TOL)
    for t in range(2):
        for i in range(n_layers):
            g = _slot_grads(eng, t * n_layers + n_layers - 1 - i, shapes)
            _check_grads(errs, g, grads[t][i], f"s{t + 1}.L{i}", F32_TOL)
    for i in range(n_layers):
        w0 = rt.master_from_params(L, layers[i]).astype(np.float64)
        want = rt.master_from_params(L, master[i]).astype(np.float64)
        got = eng.h_master[i].astype(np.float64)
        errs[f"L{i}.w"] = (rel(got, want), W_TOL)
        errs[f"L{i}.w2-w0"] = (rel(got - w0, want - w0), W_TOL)
        # the fp32 parameter buffer the engine streams holds the master's values
        prm = eng.h_params[i].numpy().view(np.float32)
        for k in range(9):
            o, cnt, po = L.grad_off[k] // 4, L.grad_bytes_t[k] // 4, L.off[k] // 4
            assert np.array_equal(prm[po:po + cnt], eng.h_master[i][o:o + cnt]), (i, k)
    eng.close()
    _fail(errs)
