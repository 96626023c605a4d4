"""Pins of the oracle's decoder block against things other than itself.

* central finite differences of the oracle forward (pins the hand-derived
  backward, every parameter and the input, MHA and GQA);
* the HF ``LlamaDecoderLayer`` in float64 (an independent implementation of
  the block the pages' model families use);
* torch's ``scaled_dot_product_attention`` / ``rms_norm`` / ``silu`` in float64;
* closed forms and invariants: softmax rows sum to 1, causal masking,
  RMSNorm scale invariance and gradient orthogonality, RoPE identity at s = 0,
  norm preservation, relative-position property, complex-multiply form.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.layer import LayerShape, PARAM_NAMES, _causal_probs

TINY_MHA = LayerShape(hidden=16, n_heads=4, n_kv_heads=4, head_dim=4, ffn=40, batch=2, seq=8)
TINY_GQA = LayerShape(hidden=16, n_heads=4, n_kv_heads=2, head_dim=4, ffn=40, batch=2, seq=8)


def tiny_params(sh, seed=0, gain_noise=0.1):
    rng = np.random.default_rng(seed)
    H, F = sh.hidden, sh.ffn
    qd, kvd = sh.n_heads * sh.head_dim, sh.n_kv_heads * sh.head_dim
    p = dict(
        Wq=rng.normal(0, 0.3, (qd, H)), Wk=rng.normal(0, 0.3, (kvd, H)),
        Wv=rng.normal(0, 0.3, (kvd, H)), Wo=rng.normal(0, 0.3, (H, qd)),
        Wg=rng.normal(0, 0.3, (F, H)), Wu=rng.normal(0, 0.3, (F, H)),
        Wd=rng.normal(0, 0.3, (H, F)),
        g1=1 + rng.normal(0, gain_noise, H), g2=1 + rng.normal(0, gain_noise, H),
    )
    x = rng.normal(0, 1, (sh.batch, sh.seq, H))
    dy = rng.normal(0, 1, (sh.batch, sh.seq, H))
    return p, x, dy


def rel_l2(a, b):
    return np.linalg.norm(np.ravel(a - b)) / max(np.linalg.norm(np.ravel(b)), 1e-300)


def fd_grad(f, arr, h_scale=1e-6):
    """Central finite differences of scalar f() with respect to every entry of arr."""
    g = np.zeros_like(arr)
    it = np.nditer(arr, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        old = arr[idx]
        h = h_scale * max(1.0, abs(old))
        arr[idx] = old + h
        fp = f()
        arr[idx] = old - h
        fm = f()
        arr[idx] = old
        g[idx] = (fp - fm) / (2 * h)
    return g


@pytest.mark.parametrize("sh", [TINY_MHA, TINY_GQA], ids=["mha", "gqa"])
def test_layer_backward_matches_finite_differences(sh):
    p, x, dy = tiny_params(sh)
    y, cache = oracle.layer_fwd(p, x, sh)
    dx, grads = oracle.layer_bwd(p, cache, dy, sh)

    def loss():
        return float(np.sum(oracle.layer_fwd(p, x, sh)[0] * dy))

    assert rel_l2(dx, fd_grad(loss, x)) <= 1e-6
    for name in PARAM_NAMES:
        fd = fd_grad(loss, p[name])
        err = rel_l2(grads[name], fd)
        assert err <= 1e-6, (name, err)


def _hf_layer(sh, p):
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaDecoderLayer, LlamaRotaryEmbedding

    cfg = LlamaConfig(hidden_size=sh.hidden, intermediate_size=sh.ffn,
                      num_attention_heads=sh.n_heads, num_key_value_heads=sh.n_kv_heads,
                      head_dim=sh.head_dim, rms_norm_eps=sh.eps, rope_theta=sh.rope_base,
                      attention_bias=False, mlp_bias=False, max_position_embeddings=4096,
                      attention_dropout=0.0)
    cfg._attn_implementation = "eager"
    layer = LlamaDecoderLayer(cfg, layer_idx=0).double().eval()
    t = lambda a: torch.tensor(a, dtype=torch.float64)
    with torch.no_grad():
        layer.self_attn.q_proj.weight.copy_(t(p["Wq"]))
        layer.self_attn.k_proj.weight.copy_(t(p["Wk"]))
        layer.self_attn.v_proj.weight.copy_(t(p["Wv"]))
        layer.self_attn.o_proj.weight.copy_(t(p["Wo"]))
        layer.mlp.gate_proj.weight.copy_(t(p["Wg"]))
        layer.mlp.up_proj.weight.copy_(t(p["Wu"]))
        layer.mlp.down_proj.weight.copy_(t(p["Wd"]))
        layer.input_layernorm.weight.copy_(t(p["g1"]))
        layer.post_attention_layernorm.weight.copy_(t(p["g2"]))
    rot = LlamaRotaryEmbedding(cfg)
    return layer, rot


@pytest.mark.parametrize("sh", [
    TINY_MHA, TINY_GQA,
    LayerShape(hidden=64, n_heads=4, n_kv_heads=1, head_dim=16, ffn=96, batch=2, seq=24),
], ids=["mha", "gqa", "mqa"])
def test_layer_forward_matches_hf_llama(sh):
    """The HF Llama block (float64 weights) computes the same y.

    HF evaluates RMSNorm and the RoPE angles in float32 internally, so the
    comparison is at 1e-5 on the branch delta y - x.
    """
    p, x, _ = tiny_params(sh, seed=3)
    y, _ = oracle.layer_fwd(p, x, sh)
    layer, rot = _hf_layer(sh, p)
    xt = torch.tensor(x, dtype=torch.float64)
    pos = torch.arange(sh.seq)[None, :].expand(sh.batch, -1)
    cos, sin = rot(xt, pos)
    mask = torch.full((sh.seq, sh.seq), float("-inf"), dtype=torch.float64).triu(1)
    mask = mask[None, None].expand(sh.batch, 1, -1, -1)
    with torch.no_grad():
        out = layer(xt, attention_mask=mask, position_ids=pos,
                    position_embeddings=(cos.double(), sin.double()))
    out = out[0] if isinstance(out, tuple) else out
    yh = out.numpy()
    assert rel_l2(y - x, yh - x) <= 1e-5


@pytest.mark.parametrize("sh", [TINY_MHA, TINY_GQA], ids=["mha", "gqa"])
def test_layer_fwd_rows_equals_full_forward(sh):
    """The row-restricted forward reproduces the full forward's rows."""
    p, x, _ = tiny_params(sh, seed=5)
    y, _ = oracle.layer_fwd(p, x, sh)
    rows = np.array([0, 3, 4, 7])
    for b in range(sh.batch):
        yr = oracle.layer_fwd_rows(p, x[b], rows, sh)
        assert np.max(np.abs(yr - y[b, rows])) <= 1e-13


def test_attention_matches_torch_sdpa_gqa():
    rng = np.random.default_rng(7)
    B, S, nh, nkv, d = 2, 11, 6, 2, 8
    q = rng.normal(size=(B, S, nh, d))
    k = rng.normal(size=(B, S, nkv, d))
    v = rng.normal(size=(B, S, nkv, d))
    o = oracle.attention_fwd(q, k, v)
    tq = torch.tensor(q).transpose(1, 2)
    tk = torch.tensor(k).transpose(1, 2)
    tv = torch.tensor(v).transpose(1, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, enable_gqa=True)
    assert rel_l2(o, ref.transpose(1, 2).numpy()) <= 1e-13


def test_attention_closed_forms():
    rng = np.random.default_rng(8)
    # S = 1: the only key is the query's own position, so o = v.
    q = rng.normal(size=(2, 1, 4, 8)); k = rng.normal(size=(2, 1, 2, 8)); v = rng.normal(size=(2, 1, 2, 8))
    o = oracle.attention_fwd(q, k, v)
    assert np.allclose(o[:, :, :2], v[:, :, :1], atol=1e-15) and np.allclose(o[:, :, 2:], v[:, :, 1:], atol=1e-15)
    # q = 0: softmax is uniform over s' <= s, o[s] = mean of v[:s+1].
    S = 9
    q = np.zeros((1, S, 2, 4)); k = rng.normal(size=(1, S, 2, 4)); v = rng.normal(size=(1, S, 2, 4))
    o = oracle.attention_fwd(q, k, v)
    cm = np.cumsum(v, axis=1) / np.arange(1, S + 1)[None, :, None, None]
    assert np.allclose(o, cm, atol=1e-14)


def test_softmax_rows_and_mask():
    rng = np.random.default_rng(9)
    P = _causal_probs(rng.normal(size=(13, 8)), rng.normal(size=(13, 8)))
    assert np.max(np.abs(P.sum(axis=1) - 1)) <= 1e-12
    assert np.all(P[np.triu_indices(13, 1)] == 0.0)
    assert np.all(P[np.tril_indices(13)] > 0.0)


def test_causality_forward_and_backward():
    sh = TINY_GQA
    p, x, dy = tiny_params(sh, seed=11)
    y, _ = oracle.layer_fwd(p, x, sh)
    s0 = 4
    x2 = x.copy()
    x2[:, s0 + 1:] += 5.0
    y2, _ = oracle.layer_fwd(p, x2, sh)
    assert np.max(np.abs(y2[:, :s0 + 1] - y[:, :s0 + 1])) <= 1e-14
    assert np.max(np.abs(y2[:, s0 + 1:] - y[:, s0 + 1:])) > 1e-3
    # upstream gradient only at position s0: no gradient reaches later positions
    dy0 = np.zeros_like(dy)
    dy0[:, s0] = dy[:, s0]
    _, cache = oracle.layer_fwd(p, x, sh)
    dx, _ = oracle.layer_bwd(p, cache, dy0, sh)
    assert np.all(dx[:, s0 + 1:] == 0.0)
    assert np.all(np.any(dx[:, :s0 + 1] != 0.0, axis=-1))


def test_rmsnorm_library_and_invariants():
    rng = np.random.default_rng(12)
    x = rng.normal(size=(5, 32))
    g = 1 + 0.1 * rng.normal(size=32)
    out, n, r = oracle.rmsnorm_fwd(x, g, 1e-6)
    ref = torch.nn.functional.rms_norm(torch.tensor(x), (32,), torch.tensor(g), eps=1e-6).numpy()
    assert rel_l2(out, ref) <= 1e-14
    # scale invariance with eps = 0
    a, _, _ = oracle.rmsnorm_fwd(x, g, 0.0)
    b, _, _ = oracle.rmsnorm_fwd(37.5 * x, g, 0.0)
    assert np.max(np.abs(a - b)) <= 1e-14
    # with eps = 1e-6 the deviation is O(eps / (alpha^2 ms))
    c, _, _ = oracle.rmsnorm_fwd(1e-2 * x, g, 1e-6)
    d, _, _ = oracle.rmsnorm_fwd(x, g, 1e-6)
    assert 0 < np.max(np.abs(c - d)) <= 1e-1
    # gradient orthogonal to x when g = 1, eps = 0
    _, n0, r0 = oracle.rmsnorm_fwd(x, np.ones(32), 0.0)
    dx, _ = oracle.rmsnorm_bwd(rng.normal(size=(5, 32)), n0, r0, np.ones(32))
    assert np.max(np.abs(np.sum(dx * x, axis=-1))) <= 1e-12


def test_rope_properties():
    rng = np.random.default_rng(13)
    S, d = 17, 8
    cos, sin = oracle.rope_angles(S, d, 10000.0)
    u = rng.normal(size=(2, S, 3, d))
    r = oracle.rope_apply(u, cos, sin)
    # identity at s = 0
    assert np.array_equal(r[:, 0], u[:, 0])
    # pair norms preserved
    h = d // 2
    assert np.allclose(r[..., :h] ** 2 + r[..., h:] ** 2, u[..., :h] ** 2 + u[..., h:] ** 2, atol=1e-12)
    # complex form: (u_i + i u_{i+d/2}) * e^{i phi}
    z = (u[..., :h] + 1j * u[..., h:]) * np.exp(1j * np.arctan2(sin, cos))[None, :, None, :]
    assert np.allclose(r[..., :h], z.real, atol=1e-13) and np.allclose(r[..., h:], z.imag, atol=1e-13)
    # angle of pair i at position s is s * 10000^(-2i/d)
    assert np.isclose(np.arctan2(sin[3, 1], cos[3, 1]), 3 * 10000.0 ** (-2 / d))
    # <R_m q, R_n k> depends only on m - n
    qv = rng.normal(size=d); kv = rng.normal(size=d)
    U = np.zeros((1, S, 2, d)); U[0, :, 0] = qv; U[0, :, 1] = kv
    R = oracle.rope_apply(U, cos, sin)[0]
    dots = R[:, 0] @ R[:, 1].T
    assert np.isclose(dots[5, 2], dots[12, 9], atol=1e-12) and np.isclose(dots[2, 5], dots[9, 12], atol=1e-12)
    # the backward is the inverse rotation
    assert np.allclose(oracle.rope_apply_inverse(r, cos, sin), u, atol=1e-13)


def test_swiglu_points_and_library():
    assert oracle.silu(np.array(0.0)) == 0.0
    dG, dU = oracle.swiglu_bwd(np.array(1.0), np.array(0.0), np.array(1.0))
    assert dG == 0.5 and dU == 0.0
    z = np.linspace(-6, 6, 101)
    assert rel_l2(oracle.silu(z), torch.nn.functional.silu(torch.tensor(z)).numpy()) <= 1e-15
    # a = 0 when U = 0
    assert np.all(oracle.swiglu_fwd(z, np.zeros_like(z)) == 0)
