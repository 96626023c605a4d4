"""fp16 storage with dynamic loss scaling, against the oracle.

The pages name FP16 beside BF16 as the format the FP32 masters are converted
into through the shared CPU buffers (de §2B "Gemeinsame Puffer auf der CPU",
es §2B, fr §2B).  fp16's range needs loss scaling (oracle/loss_scale.py): the
backward starts from the loss gradient times S, Adam takes g / S, a tensor
group is updated only if its gradients and all computed before it in the
backward are finite, and S halves after a non-finite step and doubles after
a window of finite ones.

Tolerances: fp16 gradients of a step taken at the oracle's own weights (the
first step) 2.5e-3 (the bf16 bound's multiple of the unit roundoff, 5.1 x
2^-11); later steps of a trajectory, whose weights differ from the oracle's
by the roundings of the fp16 parameters in between, at the 16-bit bound of
2e-2; weights after Adam 1e-3.
"""

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from layer_sliding_offloaded_amd import runtime as rt
from layer_sliding_offloaded_amd import sf
from tests.gpu.helpers import oracle_trajectory, oracle_trajectory_skips, rel, say, stack_inputs

pytestmark = pytest.mark.gpu

C2F = si.WORKLOADS["stack4-h1024-bf16"].with_(dtype="f16")
HP = si.ADAM
F16_TOL = 2.5e-3
TRAJ_TOL = 2e-2
W_TOL = 1e-3
STEPS = 3


def _fail(errs):
    bad = {k: f"{v:.3e} > {t:g}" for k, (v, t) in errs.items() if not v <= t}
    say("errors", {k: f"{v:.2e}" for k, (v, _) in errs.items()})
    assert not bad, bad


def _f16_bits(a):
    return np.asarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("scale", [1.0, 1.0 / 4096])
def test_adam_f16_host_device_bitwise_and_oracle(scale):
    """fp16 copies and a gradient scale: the host (F16C) and device Adam give
    the same bits; with g given times 4096 and grad_scale 1/4096 the update
    equals the oracle's on g."""
    say("adam-f16", scale)
    rng = np.random.default_rng(4)
    n = 1_000_003
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    hp_, hm, hv = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    dp, dm, dv = (torch.from_numpy(a.copy()).cuda() for a in (p0, hm, hv))
    out = rt.empty(n, dtype=torch.float16)
    hb = np.zeros(n, np.uint16)
    p64, m64, v64 = p0.astype(np.float64), np.zeros(n), np.zeros(n)
    for t in (1, 2, 3):
        g = (rng.standard_normal(n) * 10.0 ** rng.uniform(-5, 0, n)).astype(np.float32)
        gs = (g / np.float32(scale)).astype(np.float32)   # the scaled gradient (exact: power of two)
        dg = torch.from_numpy(gs).cuda()
        sf.sf_adam_device_ex(sf.SF_F16, dp.data_ptr(), dm.data_ptr(), dv.data_ptr(), dg.data_ptr(), out.data_ptr(),
                             n, t, HP["lr"], HP["b1"], HP["b2"], HP["eps"], scale, rt.stream_handle())
        sf.sf_adam_host_ex(sf.SF_F16, hp_.ctypes.data, hm.ctypes.data, hv.ctypes.data, gs.ctypes.data, hb.ctypes.data,
                           n, t, HP["lr"], HP["b1"], HP["b2"], HP["eps"], scale, 4)
        p64, m64, v64 = oracle.adam_step(p64, m64, v64, g.astype(np.float64), t, HP["lr"], HP["b1"], HP["b2"],
                                         HP["eps"])
        torch.cuda.synchronize()
        assert np.array_equal(dp.cpu().numpy(), hp_)
        assert np.array_equal(dm.cpu().numpy(), hm) and np.array_equal(dv.cpu().numpy(), hv)
        assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), hb)
        assert np.array_equal(hb, _f16_bits(hp_))
        assert rel(hp_, p64) <= 1e-6


@pytest.fixture(scope="module")
def c2f_case():
    layers, head, ids = stack_inputs(C2F)
    traj = oracle_trajectory(C2F, layers, head, ids, STEPS, HP, oracle.round_f16)
    return layers, head, ids, traj


@pytest.mark.parametrize("mode", ["sync", "pipeline", "ckpt"])
def test_engine_f16_steps_match_oracle(c2f_case, mode):
    """Three fp16 Adam steps of the 4-layer h1024 stack (vocab 32000, batch
    4 x seq 512) with the default loss scale 65536: every step's loss and
    layer gradients (the slots hold S g), the last step's head gradients and
    every weight after the last step against the oracle's fp16 trajectory;
    the fp16 parameters are the rounded masters; no update skipped and S
    kept."""
    layers, head, ids, traj = c2f_case
    w = C2F
    nl = w.n_layers
    pipe, ck = mode == "pipeline", mode == "ckpt"
    say("engine-f16", mode, w)
    eng = rt.Engine(w, layers, head, window=2, n_grad_slots=STEPS * nl, adam=True, chunk=2048, adam_hp=HP,
                    ckpt=ck, pipeline=pipe)
    L = eng.layout
    d_ids = torch.from_numpy(ids.reshape(-1)).cuda()
    losses, scales, skipped = [], [], []
    for t in range(STEPS):
        loss, st = eng.step(d_ids)
        losses.append(loss)
        scales.append(st["loss_scale"])
        if not pipe:
            st = eng.sync()
        skipped.append(st["skipped"])
    agg = eng.sync()
    torch.cuda.synchronize()
    # a sync's stats carry the last step's scale and skip count
    assert agg["loss_scale"] == 65536.0 and agg["skipped"] == 0, agg
    assert scales == [65536.0] * STEPS, scales
    assert skipped == [0] * STEPS, skipped
    shapes = {k: v.shape for k, v in layers[0].items()}
    S = 65536.0
    errs = {}
    for t in range(STEPS):
        ref = traj[t]
        tol = F16_TOL if t == 0 else TRAJ_TOL
        errs[f"s{t + 1}.loss"] = (abs(losses[t] - ref["loss"]) / ref["loss"], F16_TOL)
        for i in range(nl):
            slot = t * nl + nl - 1 - i
            flat = eng.h_slots[slot].numpy().view(np.float32) / np.float32(S)
            g = rt.unpack_grads(L, flat, shapes)
            for k in g:
                errs[f"s{t + 1}.L{i}.d{k}"] = (rel(g[k], ref["layers"][i][k]), tol)
    V, H = w.vocab, w.hidden
    hg = eng.d_head_grads.cpu().numpy() / S
    errs["s3.dgf"] = (rel(hg[V * H:V * H + H], traj[-1]["head"]["gf"]), TRAJ_TOL)
    errs["s3.dWlm"] = (rel(hg[V * H + H:].reshape(V, H), traj[-1]["head"]["Wlm"]), TRAJ_TOL)
    for i in range(nl):
        got = eng.h_master[i].astype(np.float64)
        want = rt.master_from_params(L, traj[-1]["master_layers"][i]).astype(np.float64)
        errs[f"L{i}.w"] = (rel(got, want), W_TOL)
        bits = eng.h_params[i].numpy().view(np.uint16)
        for k, name in enumerate(sf.TENSOR_NAMES):
            o, n, po = L.grad_off[k] // 4, L.grad_bytes_t[k] // 4, L.off[k] // 2
            assert np.array_equal(bits[po:po + n], _f16_bits(eng.h_master[i][o:o + n])), (i, name)
    nh = eng.h_head_master.size
    hm = eng.d_head_state[:nh].cpu().numpy().astype(np.float64)
    for name, lo, hi in (("E", 0, V * H), ("gf", V * H, V * H + H), ("Wlm", V * H + H, nh)):
        errs[f"head.{name}.w"] = (rel(hm[lo:hi], traj[-1]["master_head"][name].reshape(-1)), W_TOL)
    eng.close()
    _fail(errs)


def test_engine_f16_overflow_skips_whole_steps(c2f_case):
    """An initial loss scale of 2^40 overflows fp16 in the head's gradients:
    every update of the step is skipped (weights, moments, head and
    embedding state keep their bits) and S halves each step.  The first step
    whose head gradients fit may still overflow in a lower layer; its
    updates follow the layer-wise rule (the head and the layers above the
    first non-finite one update, that layer, those below it and the
    embedding do not).  The weights never moved before, so every tensor that
    moves in that step matches the oracle's first step: its gradients
    (slots / S) and its weights after the step."""
    layers, head, ids, traj = c2f_case
    w = C2F
    nl = w.n_layers
    say("engine-f16-overflow", w)
    eng = rt.Engine(w, layers, head, window=2, n_grad_slots=nl, adam=True, chunk=2048, adam_hp=HP,
                    loss_scale=2.0 ** 40)
    L = eng.layout
    d_ids = torch.from_numpy(ids.reshape(-1)).cuda()
    w0 = [m.copy() for m in eng.h_master]
    p0 = [p.numpy().copy() for p in eng.h_params]
    nh = eng.h_head_master.size
    h0 = eng.d_head_state.cpu().numpy().copy()
    E0 = eng.d_E.view(torch.int16).cpu().numpy().copy()
    scale = 2.0 ** 40
    for step in range(1, 41):
        loss, st = eng.step(d_ids)
        say("step", step, "scale", st["loss_scale"], "skipped", st["skipped"])
        assert st["loss_scale"] == scale
        if st["skipped"] < nl + 2:
            break
        for i in range(nl):
            assert np.array_equal(eng.h_master[i], w0[i]) and not eng.h_m[i].any() and not eng.h_v[i].any(), i
            assert np.array_equal(eng.h_params[i].numpy(), p0[i]), i
        torch.cuda.synchronize()
        assert np.array_equal(eng.d_head_state.cpu().numpy(), h0)
        assert np.array_equal(eng.d_E.view(torch.int16).cpu().numpy(), E0)
        scale /= 2.0
    else:
        pytest.fail("the head's gradients never fit fp16")
    assert 2.0 ** 10 <= scale < 2.0 ** 40
    # the first step with updates: which tensors moved follows the rule
    moved = [not np.array_equal(eng.h_master[i], w0[i]) for i in range(nl)]
    n_sk = moved.count(False)
    assert moved == [False] * n_sk + [True] * (nl - n_sk), moved   # a suffix of the backward order skips
    assert st["skipped"] == n_sk + (1 if n_sk else 0), (st, moved)  # + the embedding when any layer skips
    torch.cuda.synchronize()
    hs = eng.d_head_state.cpu().numpy()
    V, H = w.vocab, w.hidden
    assert np.array_equal(hs[:V * H], h0[:V * H]) == (n_sk > 0)
    ref = traj[0]
    shapes = {k: v.shape for k, v in layers[0].items()}
    errs = {"loss": (abs(loss - ref["loss"]) / ref["loss"], F16_TOL)}
    for i in range(nl):
        if not moved[i]:
            assert not eng.h_m[i].any(), i
            continue
        g = rt.unpack_grads(L, eng.h_slots[nl - 1 - i].numpy().view(np.float32) / np.float32(scale), shapes)
        for k in g:
            errs[f"L{i}.d{k}"] = (rel(g[k], ref["layers"][i][k]), F16_TOL)
        want = rt.master_from_params(L, ref["master_layers"][i]).astype(np.float64)
        errs[f"L{i}.w"] = (rel(eng.h_master[i].astype(np.float64), want), W_TOL)
    groups = (("gf", V * H, V * H + H), ("Wlm", V * H + H, nh)) + ((("E", 0, V * H),) if n_sk == 0 else ())
    for name, lo, hi in groups:
        errs[f"head.{name}.w"] = (rel(hs[lo:hi].astype(np.float64), ref["master_head"][name].reshape(-1)), W_TOL)
    eng.close()
    _fail(errs)


@pytest.fixture(scope="module")
def c2f_fault_case(c2f_case):
    """The oracle's two-step trajectory when layer 1 of 4 reports a non-finite
    gradient in every step: oracle.applied_updates decides (layers 3, 2 and
    the LM head update, layers 1, 0 and the embedding do not)."""
    layers, head, ids, _ = c2f_case
    traj = oracle_trajectory_skips(C2F, layers, head, ids, 2, HP, oracle.round_f16,
                                   lambda t: (False, [False, True, False, False]))
    return layers, head, ids, traj


@pytest.mark.parametrize("pipeline", [False, True])
def test_engine_f16_nonfinite_layer_skips_it_and_below(c2f_fault_case, pipeline, monkeypatch):
    """A non-finite gradient reported for layer 1 of 4 (test hook) in every
    step: against the oracle's trajectory under the same skip rule, layers 3
    and 2 and the final gain / LM head are updated (both steps' gradients and
    the weights after the second), layers 1 and 0 and the embedding keep
    their bits and zero moments, and S halves after each step."""
    layers, head, ids, traj = c2f_fault_case
    w = C2F
    nl = w.n_layers
    assert traj[0]["applied"] == (True, [False, False, True, True], False)
    say("engine-f16-layer-fault", pipeline, w)
    monkeypatch.setenv("SF_FAULT_NONFINITE_LAYER", "1")
    eng = rt.Engine(w, layers, head, window=2, n_grad_slots=2 * nl, adam=True, chunk=2048, adam_hp=HP,
                    pipeline=pipeline)
    monkeypatch.delenv("SF_FAULT_NONFINITE_LAYER")
    L = eng.layout
    d_ids = torch.from_numpy(ids.reshape(-1)).cuda()
    w0 = [m.copy() for m in eng.h_master]
    nh = eng.h_head_master.size
    h0 = eng.d_head_state.cpu().numpy().copy()
    E0 = eng.d_E.view(torch.int16).cpu().numpy().copy()
    scales, skipped = [], []
    for _ in range(2):
        loss, st = eng.step(d_ids)
        scales.append(st["loss_scale"])
        if not pipeline:
            skipped.append(st["skipped"])
    eng.sync()
    torch.cuda.synchronize()
    assert scales == [65536.0, 32768.0], scales
    if not pipeline:
        assert skipped == [3, 3], skipped
    shapes = {k: v.shape for k, v in layers[0].items()}
    errs = {}
    for i in range(nl):
        if i <= 1:
            assert np.array_equal(eng.h_master[i], w0[i]) and not eng.h_m[i].any(), i
            continue
        for t in range(2):
            g = rt.unpack_grads(L, eng.h_slots[t * nl + nl - 1 - i].numpy().view(np.float32) / np.float32(scales[t]),
                                shapes)
            for k in g:
                errs[f"s{t + 1}.L{i}.d{k}"] = (rel(g[k], traj[t]["layers"][i][k]), F16_TOL if t == 0 else TRAJ_TOL)
        want = rt.master_from_params(L, traj[-1]["master_layers"][i]).astype(np.float64)
        errs[f"L{i}.w"] = (rel(eng.h_master[i].astype(np.float64), want), W_TOL)
    hs = eng.d_head_state.cpu().numpy()
    V, H = w.vocab, w.hidden
    assert np.array_equal(hs[:V * H], h0[:V * H])             # embedding master untouched
    assert np.array_equal(eng.d_E.view(torch.int16).cpu().numpy(), E0)
    for name, lo, hi in (("gf", V * H, V * H + H), ("Wlm", V * H + H, nh)):
        errs[f"head.{name}.w"] = (rel(hs[lo:hi].astype(np.float64), traj[-1]["master_head"][name].reshape(-1)), W_TOL)
    eng.close()
    _fail(errs)
