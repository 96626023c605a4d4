"""Oracle: the host-side Adam step and the fp32 -> bf16 parameter copy.

Test infrastructure only (see the package docstring).

The pages place the optimizer on the CPU: while the device runs the backward
of L_{i-1}, the CPU updates L_i with optimizer states resident in host memory
(es §2A "Actualizacion Asincrona", de §2A, fr §2A), the states are flattened
host tensors (es §2B), and shared buffers perform the FP32 -> BF16/FP16
conversion (de §2B, es §2B, fr §2B).  The optimizer is named Adam (es §1,
es §2A).  The oracle is plain Adam with bias correction, no weight decay and
no clipping:

    m <- b1 m + (1 - b1) g
    v <- b2 v + (1 - b2) g^2
    w <- w - lr * (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps)
"""

import numpy as np


def adam_step(w, m, v, g, t, lr, b1, b2, eps):
    """One Adam step at step number t (t starts at 1).  Returns (w, m, v)."""
    m = b1 * m + (1.0 - b1) * g
    v = b2 * v + (1.0 - b2) * g * g
    mhat = m / (1.0 - b1 ** t)
    vhat = v / (1.0 - b2 ** t)
    w = w - lr * mhat / (np.sqrt(vhat) + eps)
    return w, m, v


def round_bf16(x):
    """Round float64 values to the nearest bfloat16 value (ties to even).

    bf16 keeps 8 significant bits.  frexp gives x = f * 2^e with
    0.5 <= |f| < 1, so f * 256 holds exactly the 8 kept bits before the
    point; numpy's round() breaks ties to even.  Inputs are finite and inside
    the normal bf16 range.
    """
    f, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(np.round(f * 256.0) / 256.0, e)


def round_f16(x):
    """Round float64 values to the nearest IEEE binary16 value (ties to even).

    binary16 keeps 11 significant bits for normal numbers (|x| >= 2^-14);
    below that the spacing is fixed at 2^-24 (subnormals).  The quantum of x
    is therefore 2^(max(e, -14) - 11) with x = f 2^e, 0.5 <= |f| < 1 from
    frexp, i.e. 2^(e-1) <= |x| < 2^e; numpy's round() breaks ties to even.
    Inputs are finite and below the largest binary16 value (65504).
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.ldexp(1.0, np.maximum(e - 1, -14) - 10)
    return np.round(x / q) * q
