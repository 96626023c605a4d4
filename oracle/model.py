"""Oracle: one full training step of a layer stack with embedding and head.

Test infrastructure only (see the package docstring).

Layer sliding streams each layer's weights in from host memory for the
forward and again for the backward, and hands each layer's gradients to a
host Adam while the device continues with the next layer (de §2A, es §2A,
fr §2A).  None of that changes the arithmetic: the step equals the plain,
resident step below -- forward through every layer, head loss, backward in
reverse order, then Adam on every tensor with this iteration's gradients.
"""

import numpy as np

from .adam import adam_step
from .head import embed_bwd, embed_fwd, head_fwd_bwd
from .layer import layer_bwd, layer_fwd


def stack_step(layers, E, gf, Wlm, ids, sh):
    """Loss and every gradient of one step of an L-layer stack.

    layers: list of per-layer weight dicts (float64); E: [V, H] embedding;
    gf: [H] final norm gain; Wlm: [V, H]; ids: [B, S] int.
    Returns (loss, layer_grads list, dE, dgf, dWlm).
    """
    x = embed_fwd(E, ids)
    caches = []
    for p in layers:
        x, cache = layer_fwd(p, x, sh)
        caches.append(cache)
    loss, dx, dgf, dWlm = head_fwd_bwd(gf, Wlm, x, ids, sh.eps)
    layer_grads = [None] * len(layers)
    for i in reversed(range(len(layers))):
        dx, layer_grads[i] = layer_bwd(layers[i], caches[i], dx, sh)
    dE = embed_bwd(dx, ids, E.shape[0])
    return loss, layer_grads, dE, dgf, dWlm


def adam_all(params, grads, states, t, lr, b1, b2, eps):
    """Apply ``adam_step`` to every tensor of a dict; states holds (m, v)."""
    out = {}
    for name, w in params.items():
        m, v = states[name]
        w2, m2, v2 = adam_step(w, m, v, grads[name], t, lr, b1, b2, eps)
        out[name] = w2
        states[name] = (m2, v2)
    return out
