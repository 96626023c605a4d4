"""Parity of the fused LinearCrossEntropy head and the embedding against the
oracle, chunk invariance, and deterministic embedding scatter."""

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from layer_sliding_offloaded_amd import runtime as rt
from layer_sliding_offloaded_amd import sf
from tests.gpu.helpers import rel, say

pytestmark = pytest.mark.gpu

BASE = si.WORKLOADS["layer-h256-fp32"].with_(vocab=1000, batch=2, seq=96)


def run_head(w, chunk, gf, Wlm, x, ids, grad_scale=None, dw_rows=0):
    c = rt.Context(w, head_chunk_rows=chunk, head_dw_rows=dw_rows)
    d_gf = rt.to_storage_tensor(gf, w).cuda()
    d_wlm = rt.to_storage_tensor(Wlm, w).cuda()
    d_x = rt.to_storage_tensor(x, w).cuda()
    d_ids = torch.from_numpy(ids.reshape(-1).astype(np.int32)).cuda()
    loss = rt.empty(1, dtype=torch.float32)
    dx = rt.empty_like(d_x)
    dgf = rt.empty(w.hidden, dtype=torch.float32)
    dwlm = rt.empty(w.vocab, w.hidden, dtype=torch.float32)
    if grad_scale is None:
        sf.sf_head_fwd_bwd(c.ctx, d_gf.data_ptr(), d_wlm.data_ptr(), d_x.data_ptr(), d_ids.data_ptr(),
                           loss.data_ptr(), dx.data_ptr(), dgf.data_ptr(), dwlm.data_ptr(), rt.stream_handle())
    else:
        sf.sf_head_fwd_bwd_scaled(c.ctx, d_gf.data_ptr(), d_wlm.data_ptr(), d_x.data_ptr(), d_ids.data_ptr(),
                                  loss.data_ptr(), dx.data_ptr(), dgf.data_ptr(), dwlm.data_ptr(), grad_scale,
                                  rt.stream_handle())
    torch.cuda.synchronize()
    out = (loss.item(), dx.float().cpu().numpy(), dgf.cpu().numpy(), dwlm.cpu().numpy())
    c.close()
    return out


@pytest.mark.parametrize("dtype,tol", [("f32", 1e-4), ("bf16", 2e-2)])
@pytest.mark.parametrize("chunk", [192, 64, 50])
def test_head_parity(dtype, tol, chunk):
    w = BASE.with_(dtype=dtype)
    say("head", dtype, "chunk", chunk, w)
    gf = si.final_gain(w, gains="random")
    Wlm = si.lm_head(w)
    x = si.layer_input(w)
    ids = si.token_ids(w)
    loss, dx, dgf, dwlm = run_head(w, chunk, gf, Wlm, x, ids)
    lo, dxo, dgfo, dwo = oracle.head_fwd_bwd(gf.astype(np.float64), Wlm.astype(np.float64), x.astype(np.float64),
                                             ids, w.eps)
    errs = {"loss": abs(loss - lo) / abs(lo), "dx": rel(dx, dxo), "dgf": rel(dgf, dgfo), "dWlm": rel(dwlm, dwo)}
    print({k: f"{v:.2e}" for k, v in errs.items()})
    assert all(v <= tol for v in errs.values()), errs


@pytest.mark.parametrize("dtype,tol", [("f32", 1e-4), ("bf16", 2e-2)])
@pytest.mark.parametrize("chunk,dw_rows", [(50, 150), (48, 100), (64, 10 ** 6)], ids=["50-150", "48-100", "64-all"])
def test_head_grouped_dw_parity(dtype, tol, chunk, dw_rows):
    """dW_lm in one product per group of chunks (sf_ctx_create_ex): 50-row
    chunks in groups of 150 rows over T = 192 (a ragged last group of 42),
    48-row chunks with 100 rounded up to 144, and every row in one group.
    Against the oracle at the dtype's bound; the loss, dx and dg_f do not
    depend on the grouping (same bits as one product per chunk), dW_lm only
    through the order of its fp32 sums."""
    w = BASE.with_(dtype=dtype)
    say("head-grouped", dtype, chunk, dw_rows, w)
    gf = si.final_gain(w, gains="random")
    Wlm = si.lm_head(w)
    x = si.layer_input(w)
    ids = si.token_ids(w)
    loss, dx, dgf, dwlm = run_head(w, chunk, gf, Wlm, x, ids, dw_rows=dw_rows)
    lo, dxo, dgfo, dwo = oracle.head_fwd_bwd(gf.astype(np.float64), Wlm.astype(np.float64), x.astype(np.float64),
                                             ids, w.eps)
    errs = {"loss": abs(loss - lo) / abs(lo), "dx": rel(dx, dxo), "dgf": rel(dgf, dgfo), "dWlm": rel(dwlm, dwo)}
    print({k: f"{v:.2e}" for k, v in errs.items()})
    assert all(v <= tol for v in errs.values()), errs
    l1, dx1, dgf1, dw1 = run_head(w, chunk, gf, Wlm, x, ids)
    assert loss == l1 and np.array_equal(dx, dx1) and np.array_equal(dgf, dgf1)
    assert rel(dwlm, dw1) <= 1e-6


def test_head_grouped_dw_layout():
    """The workspace holds dlogits of the group (rounded up to whole chunks,
    at most every row) instead of one chunk; the logits stay one chunk."""
    w = BASE.with_(dtype="bf16")
    shape = rt.shape_from(w)
    T, V = w.tokens, w.vocab
    base = sf.sf_layer_layout_ex(shape, 50, 0).head_workspace_bytes
    assert sf.sf_layer_layout_ex(shape, 50, 50).head_workspace_bytes == base
    assert sf.sf_layer_layout(shape, 50).head_workspace_bytes == base
    for want, eff in ((150, 150), (100, 100), (10 ** 6, 200)):
        got = sf.sf_layer_layout_ex(shape, 50, want).head_workspace_bytes
        assert base < got <= base + (eff - 50) * V * 2 + 256 * 4, (want, got)
    assert T == 192
    with pytest.raises(sf.SfError):
        sf.sf_layer_layout_ex(shape, 50, -1)


@pytest.mark.parametrize("dtype,tol,vocab", [("bf16", 2e-2, 65536), ("f32", 1e-4, 65544), ("bf16", 2e-2, 128256)])
def test_head_parity_vocab_paths(dtype, tol, vocab):
    """Cross-entropy rows held in registers (V <= 65536) and the two-pass
    kernel above that (65544; a Llama-3-sized 128256 vocabulary)."""
    w = BASE.with_(dtype=dtype, vocab=vocab, batch=2, seq=64)
    say("head-vocab", dtype, vocab, w)
    gf = si.final_gain(w, gains="random")
    Wlm = si.lm_head(w)
    x = si.layer_input(w)
    ids = si.token_ids(w)
    loss, dx, dgf, dwlm = run_head(w, 48, gf, Wlm, x, ids)
    lo, dxo, dgfo, dwo = oracle.head_fwd_bwd(gf.astype(np.float64), Wlm.astype(np.float64), x.astype(np.float64),
                                             ids, w.eps)
    errs = {"loss": abs(loss - lo) / abs(lo), "dx": rel(dx, dxo), "dgf": rel(dgf, dgfo), "dWlm": rel(dwlm, dwo)}
    print({k: f"{v:.2e}" for k, v in errs.items()})
    assert all(v <= tol for v in errs.values()), errs


@pytest.mark.parametrize("vocab,chunk,scale", [(1000, 64, 1024.0), (32000, 96, 65536.0)])
def test_head_parity_f16_scaled(vocab, chunk, scale):
    """fp16 storage with the gradients scaled by S (the loss-scaling seed):
    dx, dg_f and dW_lm divided by S against the oracle at the fp16 bound
    (2.5e-3: the bf16 bound's multiple of the unit roundoff), the loss
    unscaled."""
    w = BASE.with_(dtype="f16", vocab=vocab)
    say("head-f16", vocab, chunk, scale, w)
    gf = si.final_gain(w, gains="random")
    Wlm = si.lm_head(w)
    x = si.layer_input(w)
    ids = si.token_ids(w)
    loss, dx, dgf, dwlm = run_head(w, chunk, gf, Wlm, x, ids, grad_scale=scale)
    lo, dxo, dgfo, dwo = oracle.head_fwd_bwd(gf.astype(np.float64), Wlm.astype(np.float64), x.astype(np.float64),
                                             ids, w.eps)
    errs = {"loss": abs(loss - lo) / abs(lo), "dx": rel(dx / scale, dxo), "dgf": rel(dgf / scale, dgfo),
            "dWlm": rel(dwlm / scale, dwo)}
    print({k: f"{v:.2e}" for k, v in errs.items()})
    assert all(v <= 2.5e-3 for v in errs.values()), errs


def test_head_scaled_is_exact_power_of_two_multiple():
    """A power-of-two gradient scale multiplies every gradient of the head
    exactly: bf16 outputs with S = 256 are the unscaled ones times 256, bit
    for bit, and the loss is unchanged."""
    w = BASE.with_(dtype="bf16")
    say("head-scaled-exact", w)
    gf = si.final_gain(w, gains="random")
    args = (gf, si.lm_head(w), si.layer_input(w), si.token_ids(w))
    l1, dx1, dgf1, dw1 = run_head(w, 64, *args)
    l2, dx2, dgf2, dw2 = run_head(w, 64, *args, grad_scale=256.0)
    assert l1 == l2
    assert np.array_equal(dx1 * 256.0, dx2) and np.array_equal(dgf1 * 256.0, dgf2) and np.array_equal(dw1 * 256.0, dw2)


def test_head_zero_weight_loss_is_ln_v():
    w = BASE.with_(dtype="bf16", vocab=32000, seq=64)
    say("head-zero-weight", w)
    loss, dx, dgf, _ = run_head(w, 64, np.ones(w.hidden, np.float32), np.zeros((w.vocab, w.hidden), np.float32),
                                si.layer_input(w), si.token_ids(w))
    assert abs(loss - np.log(32000.0)) <= 1e-5 * np.log(32000.0)
    assert np.all(dx == 0) and np.all(dgf == 0)


def test_embedding_gather_and_scatter():
    w = BASE.with_(dtype="bf16", vocab=64, batch=4, seq=96)
    say("embedding", w)
    c = rt.Context(w, head_chunk_rows=64)
    E = si.embedding(w)
    ids = si.token_ids(w)  # 384 ids over 64 rows: many repeats
    d_E = rt.to_storage_tensor(E, w).cuda()
    d_ids = torch.from_numpy(ids.reshape(-1)).cuda()
    x0 = rt.empty(w.tokens, w.hidden, dtype=torch.bfloat16)
    sf.sf_embed_fwd(c.ctx, d_E.data_ptr(), d_ids.data_ptr(), x0.data_ptr(), rt.stream_handle())
    g = si.upstream_grad(w).reshape(w.tokens, w.hidden)
    d_g = rt.to_storage_tensor(g, w).cuda()
    dE1 = rt.empty(w.vocab, w.hidden, dtype=torch.float32)
    dE2 = rt.empty_like(dE1)
    sf.sf_embed_bwd(c.ctx, d_g.data_ptr(), d_ids.data_ptr(), dE1.data_ptr(), rt.stream_handle())
    sf.sf_embed_bwd(c.ctx, d_g.data_ptr(), d_ids.data_ptr(), dE2.data_ptr(), rt.stream_handle())
    torch.cuda.synchronize()
    assert np.array_equal(x0.float().cpu().numpy(), E[ids.reshape(-1)])
    ref = oracle.embed_bwd(g.astype(np.float64), ids.reshape(-1), w.vocab)
    assert rel(dE1.cpu().numpy(), ref) <= 1e-6
    assert torch.equal(dE1, dE2)
    c.close()
