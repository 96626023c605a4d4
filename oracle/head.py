"""Oracle: token embedding and the next-token cross-entropy head.

Test infrastructure only (see the package docstring).

The pages describe a fused LinearCrossEntropy kernel that projects to the
vocabulary and takes the loss in small row blocks so the full logits tensor is
never stored, with no loss of accuracy (de §2C "Fused LinearCrossEntropy",
es §2C, fr §2C), and a standard CrossEntropy loss (es §3).  Blocking does not
change the result, so the oracle takes the un-blocked definition:

    hf = RMSNorm(x_L; g_f) ;  logits = hf W_lm^T
    loss = mean over (b, s < S-1) of logsumexp(logits[b, s]) - logits[b, s, ids[b, s+1]]
"""

import numpy as np

from .layer import rmsnorm_bwd, rmsnorm_fwd


def embed_fwd(E, ids):
    """x0[b, s] = E[ids[b, s]]."""
    return E[ids]


def embed_bwd(dx0, ids, vocab):
    """dE[v] = sum of dx0[b, s] over every (b, s) with ids[b, s] == v."""
    H = dx0.shape[-1]
    dE = np.zeros((vocab, H), dtype=np.float64)
    np.add.at(dE, ids.reshape(-1), dx0.reshape(-1, H))
    return dE


def head_fwd_bwd(gf, Wlm, xL, ids, eps):
    """Loss and gradients of the final RMSNorm + LM head + next-token CE.

    xL: [B, S, H] output of the last block; ids: [B, S] int.
    The target of position s is ids[b, s + 1]; the last position of each row
    has no target and contributes nothing.  Returns (loss, dxL, dgf, dWlm).
    """
    B, S, H = xL.shape
    hf, nf, rf = rmsnorm_fwd(xL, gf, eps)
    logits = hf @ Wlm.T                                   # [B, S, V]
    V = logits.shape[-1]
    N = B * (S - 1)

    zmax = np.max(logits, axis=-1, keepdims=True)
    e = np.exp(logits - zmax)
    sumexp = np.sum(e, axis=-1, keepdims=True)
    lse = (zmax + np.log(sumexp))[..., 0]                 # [B, S]
    prob = e / sumexp

    tgt = ids[:, 1:]                                      # [B, S-1]
    picked = np.take_along_axis(logits[:, :-1, :], tgt[..., None], axis=-1)[..., 0]
    loss = np.sum(lse[:, :-1] - picked) / N

    dlogits = prob.copy()
    onehot = np.zeros_like(dlogits[:, :-1, :])
    np.put_along_axis(onehot, tgt[..., None], 1.0, axis=-1)
    dlogits[:, :-1, :] -= onehot
    dlogits[:, -1, :] = 0.0
    dlogits /= N

    dWlm = dlogits.reshape(-1, V).T @ hf.reshape(-1, H)
    dhf = dlogits @ Wlm
    dxL, dgf = rmsnorm_bwd(dhf, nf, rf, gf)
    return loss, dxL, dgf, dWlm
