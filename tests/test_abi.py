"""C-ABI contract tests that need no GPU: the library loads and exports every
symbol include/sf.h declares, layouts are consistent, arguments are
validated before any device is touched, and host Adam matches the oracle."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import seeded_inputs as si
from layer_sliding_offloaded_amd import sf
from layer_sliding_offloaded_amd import runtime as rt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sf.LIB_PATH):
        from layer_sliding_offloaded_amd import build
        build.build()
    return sf.load()


def header_symbols():
    text = open(os.path.join(ROOT, "include", "sf.h")).read()
    return sorted(set(re.findall(r"^\s*(?:sf_status|const char\*|size_t)\s+(sf_[a-z0-9_]+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported(lib):
    syms = header_symbols()
    assert len(syms) >= 16
    for s in syms:
        assert hasattr(lib, s), s
    assert set(syms) == set(sf.EXPORTS)


@pytest.mark.parametrize("name", list(si.WORKLOADS))
def test_layout_matches_tensor_shapes(lib, name):
    w = si.WORKLOADS[name]
    L = sf.sf_layer_layout(rt.shape_from(w), 2048)
    shapes = si.layer_tensor_shapes(w)
    e = 2 if w.dtype == "bf16" else 4
    n = 0
    for i, t in enumerate(sf.TENSOR_NAMES):
        cnt = int(np.prod(shapes[t]))
        n += cnt
        assert L.bytes[i] == cnt * e and L.grad_bytes_t[i] == cnt * 4
        assert L.off[i] % 16 == 0 and L.grad_off[i] % 16 == 0
    assert L.n_params == n
    # fused operand blocks: Wq|Wk|Wv and Wg|Wu are contiguous
    assert L.off[sf.SF_WK] == L.off[sf.SF_WQ] + L.bytes[sf.SF_WQ]
    assert L.off[sf.SF_WV] == L.off[sf.SF_WK] + L.bytes[sf.SF_WK]
    assert L.off[sf.SF_WU] == L.off[sf.SF_WG] + L.bytes[sf.SF_WG]
    assert L.grad_off[sf.SF_WU] == L.grad_off[sf.SF_WG] + L.grad_bytes_t[sf.SF_WG]
    for i in (sf.SF_WO, sf.SF_WG, sf.SF_WD, sf.SF_G1, sf.SF_G2):
        assert L.off[i] % 256 == 0
    assert L.param_bytes >= L.off[sf.SF_G2] + L.bytes[sf.SF_G2]
    assert L.grad_bytes >= L.grad_off[sf.SF_G2] + L.grad_bytes_t[sf.SF_G2]


def test_layout_param_count_of_named_shapes(lib):
    # per-layer parameter counts of the synthetic Llama shapes
    expect = {"layer-h256-fp32": 791040, "stack4-h1024-bf16": 12847104, "llama1.3b-bf16": 50597888,
              "llama6.7b-bf16": 202383360, "slice123b-gqa-bf16": 1384144896}
    for name, n in expect.items():
        L = sf.sf_layer_layout(rt.shape_from(si.WORKLOADS[name]), 2048)
        assert L.n_params == n, name


@pytest.mark.parametrize("field,value,code", [
    ("head_dim", 96, sf.SF_ERR_UNSUPPORTED),
    ("n_kv_heads", 3, sf.SF_ERR_UNSUPPORTED),
    ("hidden", 260, sf.SF_ERR_UNSUPPORTED),
    ("ffn", 690, sf.SF_ERR_UNSUPPORTED),
    ("batch", 0, sf.SF_ERR_ARG),
    ("dtype", 7, sf.SF_ERR_ARG),
])
def test_shape_validation(lib, field, value, code):
    shape = rt.shape_from(si.WORKLOADS["layer-h256-fp32"])
    setattr(shape, field, value)
    out = sf.SfLayout()
    rc = lib.sf_layer_layout(ctypes.byref(shape), 1, ctypes.byref(out))
    assert rc == code
    assert len(sf.sf_last_error()) > 0


def test_null_arguments_rejected(lib):
    out = sf.SfLayout()
    assert lib.sf_layer_layout(None, 1, ctypes.byref(out)) == sf.SF_ERR_ARG
    assert lib.sf_layer_fwd(None, 16, 16, 32, 48, None) == sf.SF_ERR_ARG
    assert lib.sf_slide_step(None, 16, None, None, None) == sf.SF_ERR_ARG
    assert lib.sf_engine_create(None, None, None) == sf.SF_ERR_ARG
    assert lib.sf_adam_host(None, None, None, None, None, 10, 1, 1e-4, 0.9, 0.999, 1e-8, 1) == sf.SF_ERR_ARG


def test_misaligned_pointer_rejected_before_device_use(lib):
    # a non-NULL context handle is never dereferenced when a buffer is misaligned
    bogus_ctx = ctypes.c_void_p(0x1000)
    rc = lib.sf_layer_fwd(bogus_ctx, 0x2000, 0x2008, 0x3000, 0x4000, None)
    assert rc == sf.SF_ERR_ALIGN


def test_ctx_create_without_device(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    shape = rt.shape_from(si.WORKLOADS["layer-h256-fp32"])
    ctx = ctypes.c_void_p()
    rc = lib.sf_ctx_create(ctypes.byref(shape), 1, 0x10000, 1 << 30, ctypes.byref(ctx))
    assert rc == sf.SF_ERR_NO_DEVICE
    assert ctx.value is None


def test_engine_act_bytes(lib):
    w = si.WORKLOADS["stack4-h1024-bf16"]
    shape = rt.shape_from(w)
    L = sf.sf_layer_layout(shape, 2048)
    xb = (w.tokens * w.hidden * 2 + 255) // 256 * 256
    assert sf.sf_engine_act_bytes(shape, 4) == 5 * xb + 4 * L.saved_bytes + xb + 256


@pytest.mark.parametrize("threads", [1, 3, 0])
def test_host_adam_matches_oracle(lib, threads):
    rng = np.random.default_rng(0)
    n = 300_001
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    pb = np.zeros(n, np.uint16)
    p64, m64, v64 = p.astype(np.float64), np.zeros(n), np.zeros(n)
    hp = si.ADAM
    for t in range(1, 4):
        g = (rng.standard_normal(n) * 10.0 ** rng.uniform(-5, 0, n)).astype(np.float32)
        sf.sf_adam_host(p.ctypes.data, m.ctypes.data, v.ctypes.data, g.ctypes.data, pb.ctypes.data, n, t,
                        hp["lr"], hp["b1"], hp["b2"], hp["eps"], threads)
        p64, m64, v64 = oracle.adam_step(p64, m64, v64, g.astype(np.float64), t, hp["lr"], hp["b1"], hp["b2"],
                                         hp["eps"])
        d = p.astype(np.float64) - p64
        assert np.linalg.norm(d) / np.linalg.norm(p64) <= 1e-6
        # the update itself (w_t - w_0) to 1e-3, the step-level tolerance
        assert np.all(np.isfinite(p))
    # bf16 copy is round-to-nearest-even of the fp32 master
    assert np.array_equal(si.f32_to_bf16_bits(p), pb)
    assert np.max(np.abs(si.bf16_bits_to_f32(pb).astype(np.float64) - oracle.round_bf16(p64))) <= \
        np.max(np.abs(p64)) * 2 ** -7


def test_host_adam_update_direction_matches_oracle(lib):
    # delta w of one step against the oracle's delta (relative 1e-3)
    rng = np.random.default_rng(1)
    n = 4096
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = rng.standard_normal(n).astype(np.float32)
    p = p0.copy(); m = np.zeros(n, np.float32); v = np.zeros(n, np.float32)
    sf.sf_adam_host(p.ctypes.data, m.ctypes.data, v.ctypes.data, g.ctypes.data, None, n, 1, 1e-4, 0.9, 0.999,
                    1e-8, 2)
    w1, _, _ = oracle.adam_step(p0.astype(np.float64), 0, 0, g.astype(np.float64), 1, 1e-4, 0.9, 0.999, 1e-8)
    dref = w1 - p0.astype(np.float64)
    assert np.linalg.norm((p - p0) - dref) / np.linalg.norm(dref) <= 1e-3


def test_engine_act_bytes_checkpointing(lib):
    """With SF_ENGINE_CKPT the activation region no longer grows with the
    layer count: six [T, H] buffers, two saved sets, the gradient buffer and
    the loss."""
    w = si.WORKLOADS["stack4-h1024-bf16"]
    shape = rt.shape_from(w)
    L = sf.sf_layer_layout(shape, 2048)
    xb = (w.tokens * w.hidden * 2 + 255) // 256 * 256
    for n in (1, 2, 4, 32):
        got = sf.sf_engine_act_bytes_flags(shape, n, sf.SF_ENGINE_CKPT)
        assert got == 6 * xb + 2 * L.saved_bytes + xb + 256, n
    assert sf.sf_engine_act_bytes_flags(shape, 4, 0) == sf.sf_engine_act_bytes(shape, 4)
