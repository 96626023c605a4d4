"""Pins of the oracle's head, embedding, Adam and stack step.

* cross-entropy against ``torch.nn.functional.cross_entropy`` (float64),
  the W_lm = 0 closed form loss = ln V, dlogits rows summing to zero, and
  central finite differences of every head input;
* embedding scatter against a brute-force loop with repeated ids;
* Adam against ``torch.optim.Adam`` (float64) over several steps and the
  step-1 closed form w1 = w0 - lr g / (|g| + eps);
* bf16 rounding against torch's float32 -> bfloat16 conversion;
* the whole stack step against finite differences of its loss.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle.layer import LayerShape, PARAM_NAMES
from tests.oracle.test_layer_pins import fd_grad, rel_l2, tiny_params


def _head_inputs(seed=0, B=2, S=6, H=12, V=50):
    rng = np.random.default_rng(seed)
    return (1 + 0.1 * rng.normal(size=H), rng.normal(0, 0.3, (V, H)),
            rng.normal(size=(B, S, H)), rng.integers(0, V, (B, S)))


def test_ce_matches_torch():
    gf, Wlm, xL, ids = _head_inputs()
    loss, *_ = oracle.head_fwd_bwd(gf, Wlm, xL, ids, 1e-6)
    hf, _, _ = oracle.rmsnorm_fwd(xL, gf, 1e-6)
    logits = torch.tensor(hf @ Wlm.T)
    ref = torch.nn.functional.cross_entropy(logits[:, :-1].reshape(-1, 50),
                                            torch.tensor(ids[:, 1:]).reshape(-1))
    assert abs(loss - ref.item()) <= 1e-13


def test_ce_zero_weight_closed_form():
    B, S, H, V = 2, 5, 8, 32000
    rng = np.random.default_rng(1)
    ids = rng.integers(0, V, (B, S))
    loss, dxL, dgf, dWlm = oracle.head_fwd_bwd(np.ones(H), np.zeros((V, H)), rng.normal(size=(B, S, H)), ids, 1e-6)
    assert abs(loss - math.log(V)) <= 1e-12
    assert abs(math.log(32000) - 10.373491181781864) <= 1e-14
    assert np.all(dxL == 0) and np.all(dgf == 0)


def test_head_backward_matches_finite_differences():
    gf, Wlm, xL, ids = _head_inputs(seed=2)

    def loss():
        return oracle.head_fwd_bwd(gf, Wlm, xL, ids, 1e-6)[0]

    _, dxL, dgf, dWlm = oracle.head_fwd_bwd(gf, Wlm, xL, ids, 1e-6)
    assert rel_l2(dxL, fd_grad(loss, xL)) <= 1e-6
    assert rel_l2(dgf, fd_grad(loss, gf)) <= 1e-6
    assert rel_l2(dWlm, fd_grad(loss, Wlm)) <= 1e-6


def test_dlogits_rows_sum_to_zero():
    # dW_lm^T's column sums: sum_v dWlm[v, :] = sum_t (sum_v dlogits[t, v]) hf[t] = 0
    gf, Wlm, xL, ids = _head_inputs(seed=3)
    _, _, _, dWlm = oracle.head_fwd_bwd(gf, Wlm, xL, ids, 1e-6)
    assert np.max(np.abs(dWlm.sum(axis=0))) <= 1e-14


def test_embedding_scatter_brute_force():
    rng = np.random.default_rng(4)
    ids = np.array([[3, 1, 3, 0], [1, 1, 7, 3]])
    dx0 = rng.normal(size=(2, 4, 5))
    dE = oracle.embed_bwd(dx0, ids, 8)
    ref = np.zeros((8, 5))
    for b in range(2):
        for s in range(4):
            ref[ids[b, s]] += dx0[b, s]
    assert np.allclose(dE, ref, atol=1e-15)
    E = rng.normal(size=(8, 5))
    assert np.array_equal(oracle.embed_fwd(E, ids)[1, 2], E[7])


def test_adam_matches_torch_over_steps():
    rng = np.random.default_rng(5)
    w0 = rng.normal(size=100)
    gs = [rng.normal(size=100) * 10 ** rng.uniform(-6, 0, 100) for _ in range(4)]
    hp = dict(lr=1e-4, b1=0.9, b2=0.999, eps=1e-8)
    w, m, v = w0.copy(), np.zeros(100), np.zeros(100)
    tw = torch.nn.Parameter(torch.tensor(w0))
    opt = torch.optim.Adam([tw], lr=hp["lr"], betas=(hp["b1"], hp["b2"]), eps=hp["eps"])
    for t, g in enumerate(gs, start=1):
        w, m, v = oracle.adam_step(w, m, v, g, t, **hp)
        tw.grad = torch.tensor(g)
        opt.step()
        assert rel_l2(w - w0, tw.detach().numpy() - w0) <= 1e-12


def test_adam_step1_closed_form():
    g = np.array([1e-3, -2.0, 5e-9, 0.0])
    w0 = np.array([0.5, -0.25, 1.0, 2.0])
    w1, m1, v1 = oracle.adam_step(w0, np.zeros(4), np.zeros(4), g, 1, 1e-4, 0.9, 0.999, 1e-8)
    assert np.allclose(w1, w0 - 1e-4 * g / (np.abs(g) + 1e-8), rtol=0, atol=1e-17)


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(6)
    x32 = np.concatenate([rng.normal(size=10000).astype(np.float32) * np.float32(0.02),
                          rng.normal(size=1000).astype(np.float32) * np.float32(100),
                          # exact ties: 1 + 2^-8 + k 2^-7 sit halfway between bf16 neighbours
                          np.float32(1.0) + np.float32(2.0 ** -8) * np.arange(1, 40, 2, dtype=np.float32)])
    ref = torch.tensor(x32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.round_bf16(x32.astype(np.float64)), ref)


def test_stack_step_matches_finite_differences():
    sh = LayerShape(hidden=12, n_heads=3, n_kv_heads=1, head_dim=4, ffn=20, batch=2, seq=5)
    V = 30
    rng = np.random.default_rng(7)
    layers = [tiny_params(sh, seed=s)[0] for s in (21, 22)]
    E = rng.normal(0, 0.5, (V, 12))
    gf = 1 + 0.1 * rng.normal(size=12)
    Wlm = rng.normal(0, 0.3, (V, 12))
    ids = rng.integers(0, V, (2, 5))
    ids[1, 3] = ids[0, 0]  # a repeated id
    loss, lg, dE, dgf, dWlm = oracle.stack_step(layers, E, gf, Wlm, ids, sh)

    def f():
        return oracle.stack_step(layers, E, gf, Wlm, ids, sh)[0]

    assert rel_l2(dE, fd_grad(f, E)) <= 1e-6
    assert rel_l2(dWlm, fd_grad(f, Wlm)) <= 1e-6
    assert rel_l2(dgf, fd_grad(f, gf)) <= 1e-6
    for name in ("Wq", "Wd", "g1"):
        assert rel_l2(lg[0][name], fd_grad(f, layers[0][name])) <= 1e-6, name


def test_adam_all_matches_torch_over_a_dict():
    """The per-tensor Adam of a whole layer dict against torch.optim.Adam
    (float64) over three steps: updated weights and both moments of every
    tensor, so swapped moments, a wrong step index or a dropped state write
    show up."""
    from oracle.model import adam_all
    rng = np.random.default_rng(8)
    shapes = dict(Wq=(6, 4), Wd=(4, 5), g1=(4,))
    w0 = {k: rng.normal(size=s) for k, s in shapes.items()}
    hp = dict(lr=1e-3, b1=0.9, b2=0.999, eps=1e-8)
    tp = {k: torch.nn.Parameter(torch.tensor(v)) for k, v in w0.items()}
    opt = torch.optim.Adam(list(tp.values()), lr=hp["lr"], betas=(hp["b1"], hp["b2"]), eps=hp["eps"])
    params = {k: v.copy() for k, v in w0.items()}
    states = {k: (np.zeros(s), np.zeros(s)) for k, s in shapes.items()}
    for t in (1, 2, 3):
        grads = {k: rng.normal(size=s) * 10 ** rng.uniform(-4, 0, s) for k, s in shapes.items()}
        params = adam_all(params, grads, states, t, hp["lr"], hp["b1"], hp["b2"], hp["eps"])
        for k in shapes:
            tp[k].grad = torch.tensor(grads[k])
        opt.step()
        for k in shapes:
            ref = tp[k].detach().numpy()
            assert rel_l2(params[k] - w0[k], ref - w0[k]) <= 1e-12, (t, k)
            st = opt.state[tp[k]]
            assert rel_l2(states[k][0], st["exp_avg"].numpy()) <= 1e-13, (t, k)
            assert rel_l2(states[k][1], st["exp_avg_sq"].numpy()) <= 1e-13, (t, k)
