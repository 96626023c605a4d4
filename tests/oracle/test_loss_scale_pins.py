"""Pins of the oracle's fp16 rounding and dynamic loss scaling.

* round_f16 against numpy's float64 -> float16 conversion (IEEE round to
  nearest even from double) and, for float32 inputs, torch's float32 ->
  float16; plus hand-worked ties and the subnormal range;
* update_scale against torch's own loss-scale update
  (torch._amp_update_scale_, the step of torch.amp.GradScaler) over random
  sequences of overflowing and finite steps, including growth up to the
  largest fp32 scale; the floor at 1, which torch lacks, by closed form;
* applied_updates against brute force over every pattern of non-finite
  gradients for a 4-layer stack: a group applies iff no group computed at or
  before it in the backward (head, layer L-1 .. layer i, then the embedding)
  held a non-finite gradient;
* adam_with_skip: a skip changes nothing, an applied update is adam_step
  with the next step number.
"""

import itertools

import numpy as np
import torch

import oracle
from oracle.loss_scale import adam_with_skip, applied_updates, update_scale


def test_round_f16_matches_ieee_conversions():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(size=20000) * s for s in (1e-7, 1e-5, 1e-3, 0.02, 1.0, 100.0, 1e4)])
    assert np.array_equal(oracle.round_f16(x), x.astype(np.float16).astype(np.float64))
    x32 = x.astype(np.float32)
    ref = torch.tensor(x32).to(torch.float16).to(torch.float64).numpy()
    assert np.array_equal(oracle.round_f16(x32.astype(np.float64)), ref)


def test_round_f16_hand_worked_cases():
    # near 1 the spacing is 2^-10: midpoints round to the even neighbour
    assert oracle.round_f16(1 + 2.0 ** -11) == 1.0
    assert oracle.round_f16(1 + 3 * 2.0 ** -11) == 1 + 2.0 ** -9
    assert oracle.round_f16(1 + 2.0 ** -11 + 2.0 ** -30) == 1 + 2.0 ** -10
    # largest finite value and the subnormal spacing 2^-24
    assert oracle.round_f16(65504.0) == 65504.0
    assert oracle.round_f16(2.0 ** -24) == 2.0 ** -24
    assert oracle.round_f16(2.0 ** -25) == 0.0             # tie between 0 and 2^-24: even is 0
    assert oracle.round_f16(3 * 2.0 ** -25) == 2.0 ** -23  # tie between 2^-24 and 2^-23: even is 2^-23
    assert oracle.round_f16(-(2.0 ** -14) * 1.5) == -(2.0 ** -14) * 1.5


def test_update_scale_matches_torch_amp():
    rng = np.random.default_rng(1)
    for window in (1, 3, 2000):
        scale, good = 65536.0, 0
        ts = torch.tensor([65536.0])
        tg = torch.tensor([0], dtype=torch.int32)
        for overflow in rng.random(200) < 0.2:
            # torch has no floor: compare the rule without it (the floor at 1
            # is pinned by its own closed form below)
            scale, good = update_scale(scale, good, bool(overflow), window, floor=0.0)
            torch._amp_update_scale_(ts, tg, torch.tensor([1.0 if overflow else 0.0]), 2.0, 0.5, window)
            assert scale == ts.item() and good == tg.item()


def test_update_scale_floor_at_one():
    assert update_scale(1.0, 5, True, 2000) == (1.0, 0)
    assert update_scale(1.5, 0, True, 2000) == (1.0, 0)


def test_applied_updates_brute_force():
    L = 4
    for head_bad, *layer_bad in itertools.product([False, True], repeat=L + 1):
        head, layers, emb = applied_updates(head_bad, list(layer_bad))
        order = [("head", head_bad)] + [(i, layer_bad[i]) for i in range(L - 1, -1, -1)]
        seen_bad = False
        expect = {}
        for name, bad in order:
            seen_bad = seen_bad or bad
            expect[name] = not seen_bad
        assert head == expect["head"]
        assert layers == [expect[i] for i in range(L)]
        assert emb == (not (head_bad or any(layer_bad)))


def test_adam_with_skip():
    rng = np.random.default_rng(2)
    w, m, v, g = (rng.normal(size=8) for _ in range(4))
    v = np.abs(v)
    assert adam_with_skip(w, m, v, 3, g, False, 1e-3, 0.9, 0.999, 1e-8) == (w, m, v, 3)
    w2, m2, v2, t2 = adam_with_skip(w, m, v, 3, g, True, 1e-3, 0.9, 0.999, 1e-8)
    ref = oracle.adam_step(w, m, v, g, 4, 1e-3, 0.9, 0.999, 1e-8)
    assert t2 == 4 and all(np.array_equal(a, b) for a, b in zip((w2, m2, v2), ref))
