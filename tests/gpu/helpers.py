"""Shared plumbing of the GPU parity tests (all calls go through the C ABI)."""

import sys

import numpy as np
import torch

import oracle
import seeded_inputs as si
from layer_sliding_offloaded_amd import runtime as rt
from layer_sliding_offloaded_amd import sf


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-300))


def oracle_shape(w):
    return oracle.LayerShape(w.hidden, w.n_heads, w.n_kv_heads, w.head_dim, w.ffn, w.batch, w.seq, w.eps,
                             w.rope_base)


def f64(d):
    return {k: np.asarray(v, dtype=np.float64) for k, v in d.items()}


class LayerRun:
    """One decoder layer's forward and backward through sf_layer_fwd / sf_layer_bwd."""

    def __init__(self, w, params, x, dy):
        self.w = w
        self.c = rt.Context(w)
        L = self.c.layout
        self.L = L
        self.dw = rt.pack_params(L, params, w).cuda()
        self.x = rt.to_storage_tensor(x, w).cuda()
        self.dy = rt.to_storage_tensor(dy, w).cuda()
        self.y = rt.empty_like(self.x)
        self.dx = rt.empty_like(self.x)
        self.saved = rt.device_bytes(L.saved_bytes)
        self.grads = rt.empty(L.grad_bytes // 4, dtype=torch.float32)
        self.shapes = {k: v.shape for k, v in params.items()}

    def fwd(self):
        sf.sf_layer_fwd(self.c.ctx, self.dw.data_ptr(), self.x.data_ptr(), self.y.data_ptr(),
                        self.saved.data_ptr(), rt.stream_handle())

    def bwd(self):
        sf.sf_layer_bwd(self.c.ctx, self.dw.data_ptr(), self.x.data_ptr(), self.saved.data_ptr(),
                        self.dy.data_ptr(), self.dx.data_ptr(), self.grads.data_ptr(), rt.stream_handle())

    def results(self):
        torch.cuda.synchronize()
        y = self.y.float().cpu().numpy()
        dx = self.dx.float().cpu().numpy()
        g = rt.unpack_grads(self.L, self.grads.cpu().numpy(), self.shapes)
        return y, dx, g

    def close(self):
        self.c.close()


def layer_errors(w, p, x, dy, y, dx, g):
    """rel-L2 of every output against the oracle (y - x and dx - dy deltas too)."""
    sh = oracle_shape(w)
    yo, cache = oracle.layer_fwd(f64(p), x.astype(np.float64), sh)
    dxo, go = oracle.layer_bwd(f64(p), cache, dy.astype(np.float64), sh)
    errs = {"y": rel(y, yo), "y-x": rel(y - x, yo - x), "dx": rel(dx, dxo), "dx-dy": rel(dx - dy, dxo - dy)}
    for k in go:
        errs["d" + k] = rel(g[k], go[k])
    # The residual stream is stored in the storage dtype twice per layer (h
    # and y; dh and dx), each rounding within half an ulp (2^-9 relative in
    # bf16, 2^-12 in fp16), so a delta can be no more precise than 2^-8 |y|
    # in bf16 (2^-11 |y| in fp16): the delta checks get that floor, expressed
    # relative to the delta's own norm.
    ulp = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}.get(w.dtype)
    if ulp:
        errs["floor:y-x"] = ulp * np.linalg.norm(yo) / np.linalg.norm(yo - x)
        errs["floor:dx-dy"] = ulp * np.linalg.norm(dxo) / np.linalg.norm(dxo - dy)
    if w.seq == 1:
        # one key per query: softmax is constant, dq and dk vanish exactly;
        # bound their gradients against the scale of dWv instead
        scale = np.linalg.norm(go["Wv"])
        for k in ("Wq", "Wk"):
            errs["d" + k] = float(np.linalg.norm(g[k]) / scale)
    return errs


def check_errors(errs, tol):
    """Failing entries of layer_errors(): rel-L2 above tol (+ storage floor for deltas)."""
    bad = {}
    for k, v in errs.items():
        if k.startswith("floor:"):
            continue
        allowed = tol + errs.get("floor:" + k, 0.0)
        if not v <= allowed:
            bad[k] = (v, allowed)
    return bad


def make_layer_case(w, seed_layer=0, gains="random", scale=1.0):
    """Seeded weights and inputs.  scale < 1 draws x and dy at that scale so the
    residual branches are large against the residual stream itself (RMSNorm
    makes every branch independent of x's scale), which sharpens the y - x and
    dx - dy checks."""
    p = si.layer_params(w, seed_layer, gains=gains)
    x = si.layer_input(w, scale=scale)
    dy = si.upstream_grad(w, scale=scale)
    return p, x, dy


def stack_inputs(w):
    """Seeded layers (random gains), embedding / final gain / LM head and ids of a stack."""
    layers = [si.layer_params(w, l, gains="random") for l in range(w.n_layers)]
    head = dict(E=si.embedding(w), gf=si.final_gain(w, gains="random"), Wlm=si.lm_head(w))
    return layers, head, si.token_ids(w)


def oracle_trajectory(w, layers, head, ids, steps, hp, rnd):
    """`steps` oracle iterations of a stack: stack_step at the current
    (storage-rounded) weights, fp64 Adam on every tensor, then the next
    step's weights as rnd() of the fp64 masters (round_bf16 / round_f16).
    Returns per step: loss, layer and head gradients, masters after Adam."""
    sh = oracle_shape(w)
    lay = [f64(p) for p in layers]
    hd = f64(head)
    mlay = [{k: v.copy() for k, v in p.items()} for p in lay]
    mhd = {k: v.copy() for k, v in hd.items()}
    st_l = [{k: (np.zeros_like(v), np.zeros_like(v)) for k, v in p.items()} for p in lay]
    st_h = {k: (np.zeros_like(v), np.zeros_like(v)) for k, v in hd.items()}
    out = []
    for t in range(1, steps + 1):
        say("oracle step", t)
        loss, lg, dE, dgf, dWlm = oracle.stack_step(lay, hd["E"], hd["gf"], hd["Wlm"], ids, sh)
        out.append(dict(loss=loss, layers=lg, head=dict(E=dE, gf=dgf, Wlm=dWlm)))
        for i in range(len(lay)):
            mlay[i] = oracle.model.adam_all(mlay[i], lg[i], st_l[i], t, hp["lr"], hp["b1"], hp["b2"], hp["eps"])
            lay[i] = {k: rnd(v) for k, v in mlay[i].items()}
        mhd = oracle.model.adam_all(mhd, dict(E=dE, gf=dgf, Wlm=dWlm), st_h, t, hp["lr"], hp["b1"], hp["b2"],
                                    hp["eps"])
        hd = {k: rnd(v) for k, v in mhd.items()}
        out[-1]["master_layers"] = [{k: v.copy() for k, v in p.items()} for p in mlay]
        out[-1]["master_head"] = {k: v.copy() for k, v in mhd.items()}
    return out


def oracle_trajectory_skips(w, layers, head, ids, steps, hp, rnd, nonfinite):
    """Like oracle_trajectory, with fp16's loss-scaling skip rule: at step t,
    nonfinite(t) -> (head_bad, [layer_bad for layer 0 .. L-1]) says where a
    non-finite gradient appeared; oracle.applied_updates decides which groups
    update (oracle.adam_with_skip: a skipped group keeps tensor, moments and
    step count).  Returns per step: loss, gradients, masters after the step
    and the applied groups."""
    sh = oracle_shape(w)
    lay = [f64(p) for p in layers]
    hd = f64(head)
    mlay = [{k: v.copy() for k, v in p.items()} for p in lay]
    mhd = {k: v.copy() for k, v in hd.items()}
    st_l = [{k: [np.zeros_like(v), np.zeros_like(v), 0] for k, v in p.items()} for p in lay]
    st_h = {k: [np.zeros_like(v), np.zeros_like(v), 0] for k, v in hd.items()}
    a = (hp["lr"], hp["b1"], hp["b2"], hp["eps"])

    def upd(master, st, grads, apply):
        for k in master:
            m, v, t = st[k]
            master[k], st[k][0], st[k][1], st[k][2] = oracle.adam_with_skip(master[k], m, v, t, grads[k], apply, *a)

    out = []
    for t in range(1, steps + 1):
        say("oracle step", t)
        loss, lg, dE, dgf, dWlm = oracle.stack_step(lay, hd["E"], hd["gf"], hd["Wlm"], ids, sh)
        head_bad, layer_bad = nonfinite(t)
        ah, al, ae = oracle.applied_updates(head_bad, layer_bad)
        for i in range(len(lay)):
            upd(mlay[i], st_l[i], lg[i], al[i])
            lay[i] = {k: rnd(v) for k, v in mlay[i].items()}
        # the head's groups: final gain and LM head (ah), embedding (ae)
        hg = dict(E=dE, gf=dgf, Wlm=dWlm)
        for k, ok in (("gf", ah), ("Wlm", ah), ("E", ae)):
            m, v, tk = st_h[k]
            mhd[k], st_h[k][0], st_h[k][1], st_h[k][2] = oracle.adam_with_skip(mhd[k], m, v, tk, hg[k], ok, *a)
        hd = {k: rnd(v) for k, v in mhd.items()}
        out.append(dict(loss=loss, layers=lg, head=dict(E=dE, gf=dgf, Wlm=dWlm),
                        master_layers=[{k: v.copy() for k, v in p.items()} for p in mlay],
                        master_head={k: v.copy() for k, v in mhd.items()}, applied=(ah, al, ae)))
    return out
