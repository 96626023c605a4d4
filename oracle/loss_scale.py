"""Oracle: dynamic loss scaling for fp16 storage (test infrastructure only).

The pages name fp16 beside bf16 as the format the host converts FP32 master
weights into through the shared buffers (de §2B "Gemeinsame Puffer auf der
CPU", es §2B, fr §2B) but say nothing of loss scaling; fp16's narrow range
makes it necessary (gradients of a large-vocabulary loss are ~1/N per entry,
mostly fp16 subnormals).  The plain scheme, written out here:

* the backward starts from the loss gradient times S, so every activation
  and weight gradient carries the factor S; the update takes g / S, which in
  exact arithmetic is the unscaled gradient (the oracle's own gradients are
  exact, so it never scales);
* after a step whose gradients held an infinity or a NaN, S halves (never
  below 1); after ``window`` consecutive steps without one, S doubles unless
  the double is no longer a finite fp32 value (S is an fp32 number);
* which updates a step applies (a reading adopted here: the layer-wise rule
  of a sliding engine whose host updates layer i while the device computes
  layer i-1): the backward computes the head's gradients first, then layer
  L-1 down to layer 0, then the embedding's; a tensor group is updated iff
  its own gradients and every gradient computed before it are finite.  A
  skipped update changes neither the tensor, nor its moments, nor its Adam
  step count.
"""

import numpy as np

from .adam import adam_step


def update_scale(scale, good_steps, overflow, window, growth=2.0, backoff=0.5, floor=1.0):
    """The loss scale and the count of consecutive finite steps after one step."""
    if overflow:
        return max(floor, scale * backoff), 0
    good_steps += 1
    if good_steps >= window:
        with np.errstate(over="ignore"):
            grown = np.float32(scale) * np.float32(growth)
        return (float(grown) if np.isfinite(grown) else scale), 0
    return scale, good_steps


def applied_updates(head_nonfinite, layer_nonfinite):
    """Which updates a step applies, given in which groups a non-finite
    gradient was found.  layer_nonfinite[i] is layer i's.  Returns
    (head, [layer 0 .. L-1], embedding) as booleans."""
    bad = head_nonfinite
    head = not bad
    layers = [False] * len(layer_nonfinite)
    for i in reversed(range(len(layer_nonfinite))):   # the backward's order
        bad = bad or layer_nonfinite[i]
        layers[i] = not bad
    embedding = not bad
    return head, layers, embedding


def adam_with_skip(w, m, v, t, g, apply, lr, b1, b2, eps):
    """One Adam update of a tensor that may be skipped: returns (w, m, v, t)
    with t the count of applied steps; the update uses step number t + 1."""
    if not apply:
        return w, m, v, t
    w, m, v = adam_step(w, m, v, g, t + 1, lr, b1, b2, eps)
    return w, m, v, t + 1
