"""The sliding engine: one training iteration with a window of resident layers
must equal the plain resident computation bitwise (deterministic kernels,
Adam on this iteration's gradients), and match the oracle's stack step."""

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from layer_sliding_offloaded_amd import runtime as rt
from layer_sliding_offloaded_amd import sf
from tests.gpu.helpers import f64, oracle_shape, rel, say

pytestmark = pytest.mark.gpu

STACK = si.WORKLOADS["layer-h256-fp32"].with_(dtype="bf16", vocab=1000, batch=2, seq=128, n_layers=4)


def make_stack(w, n_layers):
    layers = [si.layer_params(w, l, gains="random") for l in range(n_layers)]
    head = dict(E=si.embedding(w), gf=si.final_gain(w, gains="random"), Wlm=si.lm_head(w))
    return layers, head


def manual_step(w, layers, head, ids, chunk, t, hp, masters, moments, head_state):
    """Resident reference: every layer's weights on the device, the same kernels
    through sf_layer_fwd / sf_head_fwd_bwd / sf_layer_bwd / sf_embed_bwd, then
    sf_adam_host on each tensor.  Updates masters/moments/head_state in place
    and returns (loss, new layer params (bf16 values), new head params)."""
    c = rt.Context(w, chunk)
    L = c.layout
    s = rt.stream_handle()
    dws = [rt.pack_params(L, p, w).cuda() for p in layers]
    dt = rt.storage_dtype(w)
    d_E = rt.to_storage_tensor(head["E"], w).cuda()
    d_gf = rt.to_storage_tensor(head["gf"], w).cuda()
    d_wlm = rt.to_storage_tensor(head["Wlm"], w).cuda()
    d_ids = torch.from_numpy(ids.reshape(-1)).cuda()
    xs = [rt.empty(w.tokens, w.hidden, dtype=dt) for _ in range(len(layers) + 1)]
    saved = [rt.device_bytes(L.saved_bytes) for _ in layers]
    sf.sf_embed_fwd(c.ctx, d_E.data_ptr(), d_ids.data_ptr(), xs[0].data_ptr(), s)
    for i in range(len(layers)):
        sf.sf_layer_fwd(c.ctx, dws[i].data_ptr(), xs[i].data_ptr(), xs[i + 1].data_ptr(), saved[i].data_ptr(), s)
    V, H = w.vocab, w.hidden
    hg = rt.empty(2 * V * H + H, dtype=torch.float32)
    loss = rt.empty(1, dtype=torch.float32)
    dbuf = rt.empty_like(xs[0])
    sf.sf_head_fwd_bwd(c.ctx, d_gf.data_ptr(), d_wlm.data_ptr(), xs[-1].data_ptr(), d_ids.data_ptr(), loss.data_ptr(),
                       dbuf.data_ptr(), hg[V * H:].data_ptr(), hg[V * H + H:].data_ptr(), s)
    grads = []
    for i in reversed(range(len(layers))):
        g = rt.empty(L.grad_bytes // 4, dtype=torch.float32)
        sf.sf_layer_bwd(c.ctx, dws[i].data_ptr(), xs[i].data_ptr(), saved[i].data_ptr(), dbuf.data_ptr(),
                        dbuf.data_ptr(), g.data_ptr(), s)
        grads.insert(0, g)
    sf.sf_embed_bwd(c.ctx, dbuf.data_ptr(), d_ids.data_ptr(), hg.data_ptr(), s)
    torch.cuda.synchronize()
    new_layers = []
    for i in range(len(layers)):
        g = grads[i].cpu().numpy()
        pm, (mm, vm) = masters[i], moments[i]
        out = np.zeros(L.param_bytes // 2, dtype=np.uint16)
        for k in range(9):
            o, n, po = L.grad_off[k] // 4, L.grad_bytes_t[k] // 4, L.off[k] // 2
            sf.sf_adam_host(pm[o:].ctypes.data, mm[o:].ctypes.data, vm[o:].ctypes.data, g[o:].ctypes.data,
                            out[po:].ctypes.data, n, t, hp["lr"], hp["b1"], hp["b2"], hp["eps"], 2)
        new_layers.append(out)
    hgn = hg.cpu().numpy()
    hm, hmm, hvm = head_state
    hout = np.zeros(hm.size, dtype=np.uint16)
    sf.sf_adam_host(hm.ctypes.data, hmm.ctypes.data, hvm.ctypes.data, hgn.ctypes.data, hout.ctypes.data, hm.size, t,
                    hp["lr"], hp["b1"], hp["b2"], hp["eps"], 2)
    lv = loss.item()
    c.close()
    return lv, new_layers, hout, grads, hgn


def engine_head_state(eng):
    """(fp32 master, storage bits) of the engine's embedding/head after a step."""
    if eng.head_adam == "host":
        return eng.h_head_master, eng.h_head_params.view(torch.int16).numpy().view(np.uint16)
    torch.cuda.synchronize()
    nh = eng.h_head_master.size
    master = eng.d_head_state[:nh].cpu().numpy()
    bits = torch.cat([eng.d_E.reshape(-1), eng.d_gf.reshape(-1), eng.d_wlm.reshape(-1)]).view(torch.int16)
    return master, bits.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("window,slots,n_layers,head_adam", [(2, 2, 4, "device"), (2, 2, 4, "host"),
                                                             (3, 3, 5, "device"), (2, 2, 1, "host")])
def test_engine_matches_resident_bitwise(window, slots, n_layers, head_adam):
    w = STACK.with_(n_layers=n_layers)
    say("engine", window, slots, n_layers, head_adam, w)
    layers, head = make_stack(w, n_layers)
    ids = si.token_ids(w)
    hp = si.ADAM
    eng = rt.Engine(w, layers, head, window=window, n_grad_slots=slots, adam=True, chunk=96, adam_hp=hp,
                    head_adam=head_adam)
    L = eng.layout
    masters = [rt.master_from_params(L, p) for p in layers]
    moments = [(np.zeros_like(m), np.zeros_like(m)) for m in masters]
    flat = np.concatenate([head["E"].reshape(-1), head["gf"].reshape(-1), head["Wlm"].reshape(-1)]).astype(np.float32)
    head_state = (flat.copy(), np.zeros_like(flat), np.zeros_like(flat))
    d_ids = torch.from_numpy(ids.reshape(-1)).cuda()
    cur_layers, cur_head = layers, head
    for t in (1, 2):
        loss_e, st = eng.step(d_ids)
        say("step", t, "loss", loss_e, {k: round(v, 3) for k, v in st.items()})
        loss_m, new_layers, hout, _, _ = manual_step(w, cur_layers, cur_head, ids, 96, t, hp, masters, moments,
                                                     head_state)
        assert loss_e == loss_m
        for i in range(n_layers):
            assert np.array_equal(eng.h_master[i], masters[i]), (t, i)
            assert np.array_equal(eng.h_params[i].numpy().view(np.uint16), new_layers[i]), (t, i)
        master, bits = engine_head_state(eng)
        assert np.array_equal(master, head_state[0])
        assert np.array_equal(bits, hout)
        # next step's inputs for the manual path: the bf16 copies Adam wrote
        shapes = {k: v.shape for k, v in layers[0].items()}
        cur_layers = [rt.unpack_params(L, torch.from_numpy(nl.view(np.uint8)), shapes, w) for nl in new_layers]
        hf = si.bf16_bits_to_f32(hout)
        VH = w.vocab * w.hidden
        cur_head = dict(E=hf[:VH].reshape(w.vocab, w.hidden), gf=hf[VH:VH + w.hidden],
                        Wlm=hf[VH + w.hidden:].reshape(w.vocab, w.hidden))
        assert 0.0 <= st["overlap_pct"] <= 100.0 + 1e-6 and st["h2d_bytes"] > 0 and st["d2h_bytes"] > 0
        assert st["busy_ms"] <= st["span_ms"] + 1e-3
        tr = eng.trace()
        kinds = {r[0] for r in tr}
        assert {"compute", "h2d", "d2h", "adam"} <= kinds, kinds
        assert all(r[1] <= r[2] for r in tr)
        # every layer's gradients leave and are updated (in one or more ranges)
        assert {int(r[3]) for r in tr if r[0] == "adam"} == set(range(n_layers))
        d2h = sum(r[3] for r in tr if r[0] == "d2h")
        assert d2h == st["d2h_bytes"]
    eng.close()


@pytest.mark.parametrize("dtype", [sf.SF_BF16, sf.SF_F32])
def test_device_adam_matches_host_bitwise_and_oracle(dtype):
    say("device-adam", dtype)
    rng = np.random.default_rng(3)
    n = 1_000_003
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    hp = si.ADAM
    hp_, hm, hv = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    dp = torch.from_numpy(p0.copy()).cuda()
    dm = torch.zeros(n, device="cuda")
    dv = torch.zeros(n, device="cuda")
    out = rt.empty(n, dtype=torch.bfloat16 if dtype == sf.SF_BF16 else torch.float32)
    hb = np.zeros(n, np.uint16)
    p64, m64, v64 = p0.astype(np.float64), np.zeros(n), np.zeros(n)
    for t in (1, 2, 3):
        g = (rng.standard_normal(n) * 10.0 ** rng.uniform(-5, 0, n)).astype(np.float32)
        dg = torch.from_numpy(g).cuda()
        sf.sf_adam_device(dtype, dp.data_ptr(), dm.data_ptr(), dv.data_ptr(), dg.data_ptr(), out.data_ptr(), n, t,
                          hp["lr"], hp["b1"], hp["b2"], hp["eps"], rt.stream_handle())
        sf.sf_adam_host(hp_.ctypes.data, hm.ctypes.data, hv.ctypes.data, g.ctypes.data,
                        hb.ctypes.data if dtype == sf.SF_BF16 else None, n, t, hp["lr"], hp["b1"], hp["b2"],
                        hp["eps"], 4)
        p64, m64, v64 = oracle.adam_step(p64, m64, v64, g.astype(np.float64), t, hp["lr"], hp["b1"], hp["b2"],
                                         hp["eps"])
        torch.cuda.synchronize()
        assert np.array_equal(dp.cpu().numpy(), hp_)
        assert np.array_equal(dm.cpu().numpy(), hm) and np.array_equal(dv.cpu().numpy(), hv)
        if dtype == sf.SF_BF16:
            assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), hb)
        else:
            assert np.array_equal(out.cpu().numpy(), hp_)
        assert rel(hp_, p64) <= 1e-6


@pytest.mark.parametrize("n,off", [(1, 0), (17, 3), (100_003, 5), (4096, 8)])
def test_host_adam_vector_path_bitwise(n, off):
    """The host Adam's 16-wide streamed path, its unaligned head and its tail
    give the same bits as the device kernel on the same inputs."""
    say("host-adam-vector", n, off)
    rng = np.random.default_rng(11 + n)
    hp = si.ADAM
    p0 = (rng.standard_normal(n + off) * 0.02).astype(np.float32)
    g = (rng.standard_normal(n + off) * 10.0 ** rng.uniform(-5, 0, n + off)).astype(np.float32)
    m0 = (rng.standard_normal(n + off) * 1e-3).astype(np.float32)
    v0 = (rng.random(n + off) * 1e-5).astype(np.float32)
    hp_, hm, hv = p0.copy(), m0.copy(), v0.copy()
    hb = np.zeros(n + off, np.uint16)
    sf.sf_adam_host(hp_[off:].ctypes.data, hm[off:].ctypes.data, hv[off:].ctypes.data, g[off:].ctypes.data,
                    hb[off:].ctypes.data, n, 2, hp["lr"], hp["b1"], hp["b2"], hp["eps"], 3)
    dp, dm, dv = (torch.from_numpy(a[off:].copy()).cuda() for a in (p0, m0, v0))
    dg = torch.from_numpy(g[off:].copy()).cuda()
    out = rt.empty(n, dtype=torch.bfloat16)
    sf.sf_adam_device(sf.SF_BF16, dp.data_ptr(), dm.data_ptr(), dv.data_ptr(), dg.data_ptr(), out.data_ptr(), n, 2,
                      hp["lr"], hp["b1"], hp["b2"], hp["eps"], rt.stream_handle())
    torch.cuda.synchronize()
    assert np.array_equal(dp.cpu().numpy(), hp_[off:])
    assert np.array_equal(dm.cpu().numpy(), hm[off:]) and np.array_equal(dv.cpu().numpy(), hv[off:])
    assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), hb[off:])
    assert np.array_equal(hp_[:off], p0[:off]) and np.all(hb[:off] == 0)


def test_engine_step_matches_oracle():
    w = STACK
    say("engine-vs-oracle", w)
    layers, head = make_stack(w, w.n_layers)
    ids = si.token_ids(w)
    hp = si.ADAM
    eng = rt.Engine(w, layers, head, window=2, n_grad_slots=2, adam=True, chunk=128, adam_hp=hp)
    loss, _ = eng.step(torch.from_numpy(ids.reshape(-1)).cuda())
    sh = oracle_shape(w)
    lo, lg, dE, dgf, dWlm = oracle.stack_step([f64(p) for p in layers], head["E"].astype(np.float64),
                                              head["gf"].astype(np.float64), head["Wlm"].astype(np.float64), ids, sh)
    assert abs(loss - lo) / lo <= 2e-2
    L = eng.layout
    errs = {}
    for i, p in enumerate(layers):
        w0 = rt.master_from_params(L, p).astype(np.float64)
        st = {k: (np.zeros_like(v, dtype=np.float64), np.zeros_like(v, dtype=np.float64)) for k, v in p.items()}
        w1 = oracle.model.adam_all(f64(p), lg[i], st, 1, hp["lr"], hp["b1"], hp["b2"], hp["eps"])
        refd = np.zeros_like(w0)
        for k, name in enumerate(sf.TENSOR_NAMES):
            o, n = L.grad_off[k] // 4, L.grad_bytes_t[k] // 4
            refd[o:o + n] = (w1[name] - f64(p)[name]).reshape(-1)
        got = eng.h_master[i].astype(np.float64)
        errs[f"w{i}"] = rel(got, w0 + refd)
        errs[f"dw{i}"] = rel(got - w0, refd)  # reported: the step itself
    print({k: f"{v:.2e}" for k, v in errs.items()})
    for k, v in errs.items():
        if k.startswith("w"):
            assert v <= 1e-3, (k, v)
    eng.close()


def test_engine_grouped_head_dw_matches_per_chunk():
    """The engine's deferred last LM-head weight-gradient product
    (head_last_dw) with dlogits kept for groups of chunks: 64-row chunks in
    groups of 192 over T = 256 (the deferred group is the last 64 rows).
    One step: the loss, every layer's master and the embedding and final
    gain (none of which reads dW_lm) have the bits of one product per
    chunk, the LM head's master only differs in the order of its fp32 sums."""
    w = STACK
    say("engine-grouped-dw", w)
    layers, head = make_stack(w, w.n_layers)
    d_ids = torch.from_numpy(si.token_ids(w).reshape(-1)).cuda()
    out = []
    for dw_rows in (0, 192):
        eng = rt.Engine(w, layers, head, window=2, n_grad_slots=2, adam=True, chunk=64, adam_hp=si.ADAM,
                        head_dw_rows=dw_rows)
        loss, _ = eng.step(d_ids)
        eng.sync()
        torch.cuda.synchronize()
        nh = eng.h_head_master.size
        out.append((loss, [m.copy() for m in eng.h_master], eng.d_head_state[:nh].cpu().numpy()))
        eng.close()
    (l0, m0, h0), (l1, m1, h1) = out
    V, H = w.vocab, w.hidden
    assert l0 == l1
    assert all(np.array_equal(a, b) for a, b in zip(m0, m1))
    assert np.array_equal(h0[:V * H + H], h1[:V * H + H])
    assert rel(h1[V * H + H:], h0[V * H + H:]) <= 1e-6


def test_engine_without_head_or_adam():
    w = STACK.with_(vocab=0, n_layers=3)
    say("engine-no-head", w)
    layers = [si.layer_params(w, l, gains="random") for l in range(3)]
    x = si.layer_input(w)
    dy = si.upstream_grad(w)
    eng = rt.Engine(w, layers, None, window=2, n_grad_slots=2, adam=False)
    d_x = rt.to_storage_tensor(x, w).cuda()
    d_dy = rt.to_storage_tensor(dy, w).cuda()
    loss, st = eng.step(d_x, d_dy)
    torch.cuda.synchronize()
    # reference through the per-layer ABI
    c = rt.Context(w)
    L = c.layout
    s = rt.stream_handle()
    dws = [rt.pack_params(L, p, w).cuda() for p in layers]
    xs = [d_x] + [rt.empty_like(d_x) for _ in layers]
    saved = [rt.device_bytes(L.saved_bytes) for _ in layers]
    for i in range(3):
        sf.sf_layer_fwd(c.ctx, dws[i].data_ptr(), xs[i].data_ptr(), xs[i + 1].data_ptr(), saved[i].data_ptr(), s)
    d = d_dy.clone()
    g = rt.empty(L.grad_bytes // 4, dtype=torch.float32)
    for i in reversed(range(3)):
        sf.sf_layer_bwd(c.ctx, dws[i].data_ptr(), xs[i].data_ptr(), saved[i].data_ptr(), d.data_ptr(), d.data_ptr(),
                        g.data_ptr(), s)
    # the engine's activation region is eng.act: locate the two outputs in it
    base = eng.act.data_ptr()
    n = w.tokens * w.hidden * 2
    oy = sf.sf_engine_layer_input(eng.eng, 3) - base
    od = sf.sf_engine_dx0(eng.eng) - base
    yL = eng.act[oy:oy + n].view(torch.bfloat16).reshape(d_x.shape)
    dx0 = eng.act[od:od + n].view(torch.bfloat16).reshape(d_x.shape)
    assert torch.equal(yL, xs[3])
    assert torch.equal(dx0, d)
    assert st["h2d_bytes"] == (2 * 3 - 2) * L.param_bytes  # the last window of layers is reused
    c.close()
    eng.close()


@pytest.mark.parametrize("window,n_layers,with_head", [(2, 8, False), (2, 7, True), (3, 10, False)])
def test_engine_keep_turnaround_pages_match_plain_bitwise(window, n_layers, with_head):
    """Without Adam after the first step, the forward runs its layers from
    parameter regions for the first two windows, then alternates gradient
    and parameter regions (a gradient window's layers in reverse unit
    order), and queues uploads around the previous step's gradients still
    leaving.  Every step must give the same loss and gradients, bit for
    bit, as one plain step."""
    w = STACK.with_(n_layers=n_layers, vocab=STACK.vocab if with_head else 0)
    say("engine-keep-pages", window, n_layers, with_head, w)
    layers, head = make_stack(w, n_layers)
    if not with_head:
        head = None
    if head is not None:
        d_in = torch.from_numpy(si.token_ids(w).reshape(-1)).cuda()
        d_dy = None
    else:
        d_in = rt.to_storage_tensor(si.layer_input(w), w).cuda()
        d_dy = rt.to_storage_tensor(si.upstream_grad(w), w).cuda()
    ref = rt.Engine(w, layers, head, window=window, n_grad_slots=n_layers, adam=False)
    loss0, st0 = ref.step(d_in, d_dy)
    ref.sync()
    ref_slots = [t.numpy().copy() for t in ref.h_slots]
    ref.close()
    eng = rt.Engine(w, layers, head, window=window, n_grad_slots=n_layers, adam=False, pipeline=True,
                    keep_turnaround=True)
    # three steps in one window: each step's forward overlaps the previous
    # step's last gradient copies, and every step writes the same slots
    losses = [eng.step(d_in, d_dy)[0] for _ in range(3)]
    agg = eng.sync()
    torch.cuda.synchronize()
    if head is not None:
        assert losses == [loss0] * 3
    for k in range(n_layers):
        assert np.array_equal(eng.h_slots[k].numpy(), ref_slots[k]), k
    assert agg["h2d_bytes"] == 3 * st0["h2d_bytes"] - 2 * window * eng.layout.param_bytes
    assert agg["d2h_bytes"] == 3 * st0["d2h_bytes"]
    eng.close()


def test_engine_window_covering_every_layer():
    """A window of at least the layer count (the degenerate sliding case):
    every layer stays in its own unit.  The first step uploads each layer
    once and nothing moves back in; with the parameters kept at the
    turnaround the next steps upload nothing.  Gradients equal a window-2
    step's bit for bit."""
    w = STACK.with_(vocab=0, n_layers=3)
    say("engine-window-all", w)
    layers = [si.layer_params(w, l, gains="random") for l in range(3)]
    d_x = rt.to_storage_tensor(si.layer_input(w), w).cuda()
    d_dy = rt.to_storage_tensor(si.upstream_grad(w), w).cuda()
    ref = rt.Engine(w, layers, None, window=2, n_grad_slots=3, adam=False)
    ref.step(d_x, d_dy)
    ref.sync()
    ref_slots = [t.numpy().copy() for t in ref.h_slots]
    ref.close()
    eng = rt.Engine(w, layers, None, window=5, n_grad_slots=3, adam=False, keep_turnaround=True)
    P = eng.layout.param_bytes
    for step in range(3):
        _, st = eng.step(d_x, d_dy)
        eng.sync()
        torch.cuda.synchronize()
        assert st["h2d_bytes"] == (3 * P if step == 0 else 0), step
        for k in range(3):
            assert np.array_equal(eng.h_slots[k].numpy(), ref_slots[k]), (step, k)
    eng.close()


def _run_engine(w, layers, head, x, dy, steps, **kw):
    """Steps an engine and returns per-step snapshots of everything it updates."""
    eng = rt.Engine(w, layers, head, n_grad_slots=2, adam=True, chunk=96, adam_hp=si.ADAM, **kw)
    d_in = torch.from_numpy(x.reshape(-1)).cuda() if head is not None else rt.to_storage_tensor(x, w).cuda()
    d_dy = None if head is not None else rt.to_storage_tensor(dy, w).cuda()
    n = w.tokens * w.hidden * 2
    base = eng.act.data_ptr()
    out = []
    for _ in range(steps):
        loss, st = eng.step(d_in, d_dy)
        torch.cuda.synchronize()
        snap = dict(loss=loss, st=st, master=[m.copy() for m in eng.h_master],
                    params=[p.numpy().view(np.uint16).copy() for p in eng.h_params])
        if head is not None:
            snap["head"] = [a.copy() for a in engine_head_state(eng)]
        od = sf.sf_engine_dx0(eng.eng) - base
        oy = sf.sf_engine_layer_input(eng.eng, w.n_layers) - base
        snap["dx0"] = eng.act[od:od + n].cpu().numpy().copy()
        snap["y"] = eng.act[oy:oy + n].cpu().numpy().copy()
        out.append(snap)
    info = dict(act_bytes=eng.act_bytes, x_bytes=eng.x_bytes, trace=eng.trace())
    eng.close()
    return out, info


@pytest.mark.parametrize("head_adam,window,n_layers", [("device", 2, 4), ("host", 3, 5), (None, 2, 3),
                                                       ("device", 2, 2), ("device", 2, 1)])
def test_engine_checkpointing_matches_plain_bitwise(head_adam, window, n_layers):
    """Sliding activation checkpointing only moves layer inputs through host
    memory and recomputes each layer's forward before its backward: every
    result of the iteration is the same bits as with all activations resident."""
    w = STACK.with_(n_layers=n_layers, vocab=STACK.vocab if head_adam else 0)
    say("engine-ckpt", head_adam, window, n_layers, w)
    layers = [si.layer_params(w, l, gains="random") for l in range(n_layers)]
    if head_adam:
        head = dict(E=si.embedding(w), gf=si.final_gain(w, gains="random"), Wlm=si.lm_head(w))
        x, dy = si.token_ids(w), None
        kw = dict(head_adam=head_adam)
    else:
        head, x, dy, kw = None, si.layer_input(w), si.upstream_grad(w), {}
    ref, ri = _run_engine(w, layers, head, x, dy, 2, window=window, **kw)
    got, gi = _run_engine(w, layers, head, x, dy, 2, window=window, ckpt=True, **kw)
    for t, (a, b) in enumerate(zip(ref, got)):
        if head is not None:  # (no loss without a head)
            assert a["loss"] == b["loss"], t
        for i in range(n_layers):
            assert np.array_equal(a["master"][i], b["master"][i]), (t, i)
            assert np.array_equal(a["params"][i], b["params"][i]), (t, i)
        if head is not None:
            assert np.array_equal(a["head"][0], b["head"][0]) and np.array_equal(a["head"][1], b["head"][1]), t
        else:
            assert np.array_equal(a["dx0"], b["dx0"]), t
        assert np.array_equal(a["y"], b["y"]), t
        # the checkpoints add one trip out and one back per layer input but
        # the last layer's (and, without a head, the caller's x_0)
        n_ck = max(n_layers - 1 - (0 if head is not None else 1), 0)
        assert b["st"]["d2h_bytes"] - a["st"]["d2h_bytes"] == n_ck * gi["x_bytes"], t
        assert b["st"]["h2d_bytes"] - a["st"]["h2d_bytes"] == n_ck * gi["x_bytes"], t
    if n_layers >= 4:
        assert gi["act_bytes"] < ri["act_bytes"]


def _run_pipelined(w, layers, head, x, dy, steps, **kw):
    """Steps a pipelined engine without draining in between (each forward
    waits on the previous step's Adam in flight); returns the per-step losses
    and, after one sync at the end, the final state as _run_engine does."""
    eng = rt.Engine(w, layers, head, n_grad_slots=2, adam=True, chunk=96, adam_hp=si.ADAM, pipeline=True, **kw)
    d_in = torch.from_numpy(x.reshape(-1)).cuda() if head is not None else rt.to_storage_tensor(x, w).cuda()
    d_dy = None if head is not None else rt.to_storage_tensor(dy, w).cuda()
    losses, walls = [], []
    for _ in range(steps):
        loss, st = eng.step(d_in, d_dy)
        losses.append(loss)
        walls.append(st["wall_ms"])
    agg = eng.sync()
    torch.cuda.synchronize()
    n = w.tokens * w.hidden * 2
    base = eng.act.data_ptr()
    snap = dict(master=[m.copy() for m in eng.h_master], params=[p.numpy().view(np.uint16).copy() for p in eng.h_params])
    if head is not None:
        snap["head"] = [a.copy() for a in engine_head_state(eng)]
    od = sf.sf_engine_dx0(eng.eng) - base
    oy = sf.sf_engine_layer_input(eng.eng, w.n_layers) - base
    snap["dx0"] = eng.act[od:od + n].cpu().numpy().copy()
    snap["y"] = eng.act[oy:oy + n].cpu().numpy().copy()
    trace = eng.trace()
    eng.close()
    return losses, snap, agg, trace


@pytest.mark.parametrize("head_adam,window,n_layers,ckpt", [("device", 2, 4, False), (None, 2, 3, False),
                                                            ("device", 3, 5, True), ("device", 2, 1, False),
                                                            ("device", 2, 7, False), (None, 3, 8, False)])
def test_engine_pipelined_matches_synchronous_bitwise(head_adam, window, n_layers, ckpt):
    """Running host Adam across the step boundary changes when updates are
    applied, never what is computed: three pipelined steps give the same
    losses and the same final parameters, moments, head state and outputs as
    three synchronous ones, bit for bit."""
    w = STACK.with_(n_layers=n_layers, vocab=STACK.vocab if head_adam else 0)
    say("engine-pipelined", head_adam, window, n_layers, ckpt, w)
    layers = [si.layer_params(w, l, gains="random") for l in range(n_layers)]
    if head_adam:
        head = dict(E=si.embedding(w), gf=si.final_gain(w, gains="random"), Wlm=si.lm_head(w))
        x, dy = si.token_ids(w), None
        kw = dict(head_adam=head_adam)
    else:
        head, x, dy, kw = None, si.layer_input(w), si.upstream_grad(w), {}
    steps = 3
    ref, _ = _run_engine(w, layers, head, x, dy, steps, window=window, ckpt=ckpt, **kw)
    losses, got, agg, trace = _run_pipelined(w, layers, head, x, dy, steps, window=window, ckpt=ckpt, **kw)
    if head is not None:
        assert losses == [r["loss"] for r in ref]
    last = ref[-1]
    for i in range(n_layers):
        assert np.array_equal(last["master"][i], got["master"][i]), i
        assert np.array_equal(last["params"][i], got["params"][i]), i
    if head is not None:
        assert np.array_equal(last["head"][0], got["head"][0]) and np.array_equal(last["head"][1], got["head"][1])
    else:
        assert np.array_equal(last["dx0"], got["dx0"])
    assert np.array_equal(last["y"], got["y"])
    # the sync's window covers all three steps: every byte the synchronous
    # steps moved, and one Adam pass per layer per step
    assert agg["h2d_bytes"] == sum(r["st"]["h2d_bytes"] for r in ref)
    assert agg["d2h_bytes"] == sum(r["st"]["d2h_bytes"] for r in ref)
    assert 0.0 <= agg["overlap_pct"] <= 100.0 + 1e-6
    assert {int(r[3]) for r in trace if r[0] == "adam"} == set(range(n_layers))


def test_engine_pipelined_rejects_host_head_adam():
    w = STACK.with_(n_layers=2)
    layers = [si.layer_params(w, l) for l in range(2)]
    head = dict(E=si.embedding(w), gf=si.final_gain(w), Wlm=si.lm_head(w))
    with pytest.raises(sf.SfError) as ei:
        rt.Engine(w, layers, head, adam=True, chunk=96, head_adam="host", pipeline=True)
    assert ei.value.code == sf.SF_ERR_UNSUPPORTED
