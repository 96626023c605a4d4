"""Oracle: one pre-norm Llama decoder block, forward and hand-derived backward.

Test infrastructure only (see the package docstring).  Plain numpy float64,
one operation per line, in the order the block computes them.

The pages ("An Efficient Heterogeneous Co-Design for Fine-Tuning on a Single
GPU", gist.science summaries de/es/fr) name the supported families -- Llama,
Qwen, Mistral (de §5 "Bedeutung und Fazit", es §3 "Resultados Clave") -- and
the fused kernels RoPE, RMSNorm and SwiGLU (de §2C, es §2C, fr §2C), without
printing the block's equations.  The block below is the standard Llama one:

    xn = RMSNorm(x; g1)
    q, k, v = xn Wq^T, xn Wk^T, xn Wv^T         (bias-free)
    q', k' = RoPE(q), RoPE(k)                    (rotate-half pairs i, i+d/2)
    A = causal softmax(q' k'^T / sqrt(d)) v      (per head; GQA groups)
    h = x + A Wo^T
    hn = RMSNorm(h; g2)
    G, U = hn Wg^T, hn Wu^T ;  a = silu(G) * U
    y = h + a Wd^T

Weights are stored W[out, in]; every projection is y = x W^T.
"""

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class LayerShape:
    """Sizes of one decoder block and its input batch."""

    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    batch: int
    seq: int
    eps: float = 1e-6
    rope_base: float = 10000.0

    @property
    def tokens(self):
        return self.batch * self.seq


# --------------------------------------------------------------------------
# RMSNorm (fused kernel named in de §2C / es §2C / fr §2C)
# --------------------------------------------------------------------------

def rmsnorm_fwd(x, g, eps):
    """RMSNorm over the last axis.

    r = (mean_j x_j^2 + eps)^(-1/2) ;  n = x r ;  out = n * g.
    Returns (out, n, r); n and r are what the backward needs.
    """
    ms = np.mean(x * x, axis=-1)
    r = 1.0 / np.sqrt(ms + eps)
    n = x * r[..., None]
    return n * g, n, r


def rmsnorm_bwd(dout, n, r, g):
    """Backward of ``rmsnorm_fwd`` given its saved n and r.

    dn = dout * g
    dg = sum over every row of dout * n
    dx = r * (dn - n * mean_j(dn * n))
    """
    dn = dout * g
    dg = np.sum((dout * n).reshape(-1, n.shape[-1]), axis=0)
    proj = np.mean(dn * n, axis=-1)
    dx = r[..., None] * (dn - n * proj[..., None])
    return dx, dg


# --------------------------------------------------------------------------
# RoPE (fused kernel named in de §2C / es §2C / fr §2C)
# --------------------------------------------------------------------------

def rope_angles(seq, head_dim, base):
    """cos and sin of phi[s, i] = s * base^(-2i/d), s in [0, S), i in [0, d/2)."""
    half = head_dim // 2
    i = np.arange(half, dtype=np.float64)
    omega = base ** (-2.0 * i / head_dim)
    s = np.arange(seq, dtype=np.float64)
    phi = s[:, None] * omega[None, :]
    return np.cos(phi), np.sin(phi)


def rope_apply(u, cos, sin):
    """Rotate pairs (i, i + d/2) of every head by phi[s, i].

    u has shape [B, S, heads, d]; position s is the sequence index, so it
    restarts at 0 for every batch row.
    """
    half = u.shape[-1] // 2
    first = u[..., :half]
    second = u[..., half:]
    c = cos[None, :, None, :]
    s = sin[None, :, None, :]
    out = np.empty_like(u)
    out[..., :half] = first * c - second * s
    out[..., half:] = second * c + first * s
    return out


def rope_apply_inverse(du, cos, sin):
    """Backward of ``rope_apply``: the transpose (= inverse) rotation."""
    half = du.shape[-1] // 2
    first = du[..., :half]
    second = du[..., half:]
    c = cos[None, :, None, :]
    s = sin[None, :, None, :]
    out = np.empty_like(du)
    out[..., :half] = first * c + second * s
    out[..., half:] = second * c - first * s
    return out


# --------------------------------------------------------------------------
# Causal attention with grouped KV heads
# --------------------------------------------------------------------------

def _kv_head(h, n_heads, n_kv_heads):
    """Query head h reads KV head floor(h * n_kv / n_h) (contiguous groups)."""
    return (h * n_kv_heads) // n_heads


def _causal_probs(qh, kh):
    """Row-softmax of qh kh^T / sqrt(d) with s' > s masked out."""
    d = qh.shape[-1]
    z = (qh @ kh.T) / np.sqrt(d)
    S = z.shape[0]
    z = np.where(np.tril(np.ones((S, S), dtype=bool)), z, -np.inf)
    zmax = np.max(z, axis=1, keepdims=True)
    e = np.exp(z - zmax)
    return e / np.sum(e, axis=1, keepdims=True)


def attention_fwd(q, k, v):
    """o[b, s, h] = sum_{s' <= s} P[s, s'] v[b, s', kv(h)].

    q: [B, S, n_h, d]; k, v: [B, S, n_kv, d].  Returns o [B, S, n_h, d].
    """
    B, S, nh, d = q.shape
    nkv = k.shape[2]
    o = np.zeros_like(q)
    for b in range(B):
        for h in range(nh):
            kap = _kv_head(h, nh, nkv)
            P = _causal_probs(q[b, :, h], k[b, :, kap])
            o[b, :, h] = P @ v[b, :, kap]
    return o


def attention_bwd(q, k, v, do):
    """Backward of ``attention_fwd`` (probabilities recomputed).

    dv = P^T do ;  dP = do v^T ;  dz = P * (dP - rowsum(dP * P))
    dq = dz k / sqrt(d) ;  dk = dz^T q / sqrt(d)
    dk and dv of a KV head sum over the query heads of its group.
    """
    B, S, nh, d = q.shape
    nkv = k.shape[2]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(nh):
            kap = _kv_head(h, nh, nkv)
            qh, kh, vh, doh = q[b, :, h], k[b, :, kap], v[b, :, kap], do[b, :, h]
            P = _causal_probs(qh, kh)
            dv[b, :, kap] += P.T @ doh
            dP = doh @ vh.T
            dz = P * (dP - np.sum(dP * P, axis=1, keepdims=True))
            dq[b, :, h] = (dz @ kh) / np.sqrt(d)
            dk[b, :, kap] += (dz.T @ qh) / np.sqrt(d)
    return dq, dk, dv


# --------------------------------------------------------------------------
# SwiGLU (fused kernel named in de §2C / es §2C)
# --------------------------------------------------------------------------

def silu(z):
    """silu(z) = z / (1 + e^-z)."""
    return z / (1.0 + np.exp(-z))


def swiglu_fwd(G, U):
    """a = silu(G) * U."""
    return silu(G) * U


def swiglu_bwd(da, G, U):
    """dG = da * U * sig(G) (1 + G (1 - sig(G))) ;  dU = da * silu(G)."""
    sig = 1.0 / (1.0 + np.exp(-G))
    dG = da * U * sig * (1.0 + G * (1.0 - sig))
    dU = da * silu(G)
    return dG, dU


# --------------------------------------------------------------------------
# The block
# --------------------------------------------------------------------------

PARAM_NAMES = ("Wq", "Wk", "Wv", "Wo", "Wg", "Wu", "Wd", "g1", "g2")


def layer_fwd(p, x, sh):
    """Forward of one block.  p: dict of float64 weights; x: [B, S, H].

    Returns (y, cache) where cache holds what ``layer_bwd`` reads.
    """
    B, S, H = x.shape
    nh, nkv, d = sh.n_heads, sh.n_kv_heads, sh.head_dim

    xn, n1, r1 = rmsnorm_fwd(x, p["g1"], sh.eps)
    q = (xn @ p["Wq"].T).reshape(B, S, nh, d)
    k = (xn @ p["Wk"].T).reshape(B, S, nkv, d)
    v = (xn @ p["Wv"].T).reshape(B, S, nkv, d)
    cos, sin = rope_angles(S, d, sh.rope_base)
    qr = rope_apply(q, cos, sin)
    kr = rope_apply(k, cos, sin)
    o = attention_fwd(qr, kr, v)
    A = o.reshape(B, S, nh * d)
    h = x + A @ p["Wo"].T
    hn, n2, r2 = rmsnorm_fwd(h, p["g2"], sh.eps)
    G = hn @ p["Wg"].T
    U = hn @ p["Wu"].T
    a = swiglu_fwd(G, U)
    y = h + a @ p["Wd"].T

    cache = dict(x=x, xn=xn, n1=n1, r1=r1, qr=qr, kr=kr, v=v, A=A, h=h,
                 hn=hn, n2=n2, r2=r2, G=G, U=U, a=a, cos=cos, sin=sin)
    return y, cache


def layer_fwd_rows(p, x, rows, sh):
    """y of one sequence at selected positions only (for sequences too long
    for the full oracle).  x: [S, H] one sequence; rows: increasing indices.

    Same steps as ``layer_fwd``: keys and values are needed at every position
    up to the last selected row; queries, the attention output and the MLP
    only at the selected rows.
    """
    S, H = x.shape
    nh, nkv, d = sh.n_heads, sh.n_kv_heads, sh.head_dim
    last = int(rows[-1]) + 1
    xs = x[:last]
    xn, _, _ = rmsnorm_fwd(xs, p["g1"], sh.eps)
    cos, sin = rope_angles(last, d, sh.rope_base)
    k = (xn @ p["Wk"].T).reshape(1, last, nkv, d)
    v = (xn @ p["Wv"].T).reshape(1, last, nkv, d)
    kr = rope_apply(k, cos, sin)[0]                          # [last, nkv, d]
    v = v[0]
    xr = xn[rows]
    q = (xr @ p["Wq"].T).reshape(len(rows), nh, d)
    half = d // 2
    c, s = cos[rows][:, None, :], sin[rows][:, None, :]
    qr = np.empty_like(q)
    qr[..., :half] = q[..., :half] * c - q[..., half:] * s
    qr[..., half:] = q[..., half:] * c + q[..., :half] * s
    A = np.zeros((len(rows), nh * d))
    for i, r in enumerate(rows):
        for h in range(nh):
            kap = _kv_head(h, nh, nkv)
            z = (kr[: r + 1, kap] @ qr[i, h]) / np.sqrt(d)     # keys s' <= r
            e = np.exp(z - np.max(z))
            A[i, h * d:(h + 1) * d] = (e / np.sum(e)) @ v[: r + 1, kap]
    h_ = x[rows] + A @ p["Wo"].T
    hn, _, _ = rmsnorm_fwd(h_, p["g2"], sh.eps)
    a = swiglu_fwd(hn @ p["Wg"].T, hn @ p["Wu"].T)
    return h_ + a @ p["Wd"].T


def layer_bwd(p, cache, dy, sh):
    """Backward of one block given dy [B, S, H].

    Returns (dx, grads) with grads keyed like ``PARAM_NAMES``.
    """
    B, S, H = dy.shape
    T = B * S
    nh, nkv, d = sh.n_heads, sh.n_kv_heads, sh.head_dim
    c = cache

    def flat(t):
        return t.reshape(T, -1)

    # MLP branch: y = h + a Wd^T
    dWd = flat(dy).T @ flat(c["a"])
    da = dy @ p["Wd"]
    dG, dU = swiglu_bwd(da, c["G"], c["U"])
    dWg = flat(dG).T @ flat(c["hn"])
    dWu = flat(dU).T @ flat(c["hn"])
    dhn = dG @ p["Wg"] + dU @ p["Wu"]
    dh_norm, dg2 = rmsnorm_bwd(dhn, c["n2"], c["r2"], p["g2"])
    dh = dy + dh_norm

    # attention branch: h = x + A Wo^T
    dWo = flat(dh).T @ flat(c["A"])
    dA = dh @ p["Wo"]
    do = dA.reshape(B, S, nh, d)
    dqr, dkr, dv = attention_bwd(c["qr"], c["kr"], c["v"], do)
    dq = rope_apply_inverse(dqr, c["cos"], c["sin"])
    dk = rope_apply_inverse(dkr, c["cos"], c["sin"])
    dq = dq.reshape(B, S, nh * d)
    dk = dk.reshape(B, S, nkv * d)
    dv = dv.reshape(B, S, nkv * d)
    dWq = flat(dq).T @ flat(c["xn"])
    dWk = flat(dk).T @ flat(c["xn"])
    dWv = flat(dv).T @ flat(c["xn"])
    dxn = dq @ p["Wq"] + dk @ p["Wk"] + dv @ p["Wv"]
    dx_norm, dg1 = rmsnorm_bwd(dxn, c["n1"], c["r1"], p["g1"])
    dx = dh + dx_norm

    grads = dict(Wq=dWq, Wk=dWk, Wv=dWv, Wo=dWo, Wg=dWg, Wu=dWu, Wd=dWd,
                 g1=dg1, g2=dg2)
    return dx, grads
