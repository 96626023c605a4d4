"""Failure handling of the sliding engine.

Every check of sf_engine_create and sf_slide_step fires before any device
work with the status the header names; a failed host Adam job (injected
through the SF_FAULT_ADAM_JOB test hook) surfaces as SF_ERR_HIP at the step
or sync that observes it and leaves the engine in the sticky error state;
and the engine's timing needs no event beyond those sf_engine_create made.
"""

import ctypes
import os

import numpy as np
import pytest
import torch

import seeded_inputs as si
from layer_sliding_offloaded_amd import runtime as rt
from layer_sliding_offloaded_amd import sf
from tests.gpu.helpers import say

pytestmark = pytest.mark.gpu

W = si.WORKLOADS["layer-h256-fp32"].with_(dtype="bf16", vocab=0, batch=2, seq=64, n_layers=3)


def _engine(**kw):
    w = kw.pop("w", W)
    layers = [si.layer_params(w, l) for l in range(w.n_layers)]
    return rt.Engine(w, layers, None, window=2, n_grad_slots=2, **kw)


def _copy_cfg(cfg):
    c = sf.SfEngineCfg()
    ctypes.memmove(ctypes.addressof(c), ctypes.addressof(cfg), ctypes.sizeof(cfg))
    return c


def _expect(ctx, cfg, code):
    with pytest.raises(sf.SfError) as ei:
        eng = sf.sf_engine_create(ctx, cfg)
        sf.sf_engine_destroy(eng)
    assert ei.value.code == code, str(ei.value)
    say("rejected", code, str(ei.value))


def test_engine_create_validation():
    say("engine-create-validation")
    eng = _engine(adam=True)
    ctx = eng.ctx.ctx
    base = eng.cfg
    keep = []

    c = _copy_cfg(base)
    c.window = 1
    _expect(ctx, c, sf.SF_ERR_ARG)
    c = _copy_cfg(base)
    c.n_grad_slots = 1
    _expect(ctx, c, sf.SF_ERR_ARG)
    c = _copy_cfg(base)
    c.n_layers = 0
    _expect(ctx, c, sf.SF_ERR_ARG)
    # undersized unit pool and activation region
    c = _copy_cfg(base)
    c.pool_bytes = base.pool_bytes - 256
    _expect(ctx, c, sf.SF_ERR_POOL)
    c = _copy_cfg(base)
    c.act_bytes = base.act_bytes - 256
    _expect(ctx, c, sf.SF_ERR_POOL)
    # misaligned device regions
    c = _copy_cfg(base)
    c.d_pool = base.d_pool + 16
    _expect(ctx, c, sf.SF_ERR_ALIGN)
    # pageable (unpinned) host parameters and gradient slot
    pageable = np.zeros(eng.layout.grad_bytes // 4 + 64, dtype=np.float32)
    keep.append(pageable)
    ptrs = [t.data_ptr() for t in eng.h_params]
    ptrs[1] = pageable.ctypes.data
    arr = sf.pointer_array(ptrs)
    keep.append(arr)
    c = _copy_cfg(base)
    c.h_params = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
    _expect(ctx, c, sf.SF_ERR_NOT_PINNED)
    sl = sf.pointer_array([eng.h_slots[0].data_ptr(), pageable.ctypes.data])
    keep.append(sl)
    c = _copy_cfg(base)
    c.h_grad_slots = ctypes.cast(sl, ctypes.POINTER(ctypes.c_void_p))
    _expect(ctx, c, sf.SF_ERR_NOT_PINNED)
    # Adam without host masters
    c = _copy_cfg(base)
    c.h_master = None
    _expect(ctx, c, sf.SF_ERR_ARG)
    # checkpointing needs a pinned checkpoint region
    c = _copy_cfg(base)
    c.flags = base.flags | sf.SF_ENGINE_CKPT
    c.h_ckpt = None
    _expect(ctx, c, sf.SF_ERR_ARG)
    c.h_ckpt = pageable.ctypes.data
    _expect(ctx, c, sf.SF_ERR_NOT_PINNED)
    # a head needs a context with a vocabulary
    c = _copy_cfg(base)
    c.flags = base.flags | sf.SF_ENGINE_HEAD
    _expect(ctx, c, sf.SF_ERR_ARG)
    # the original configuration still works after all of this
    x = rt.to_storage_tensor(si.layer_input(W), W).cuda()
    dy = rt.to_storage_tensor(si.upstream_grad(W), W).cuda()
    eng.step(x, dy)
    eng.sync()
    eng.close()


def test_slide_step_argument_checks_leave_engine_usable():
    say("slide-step-args")
    eng = _engine(adam=False)
    x = rt.to_storage_tensor(si.layer_input(W), W).cuda()
    dy = rt.to_storage_tensor(si.upstream_grad(W), W).cuda()
    with pytest.raises(sf.SfError) as ei:
        sf.sf_slide_step(eng.eng, x.data_ptr(), None)   # no head: dy is required
    assert ei.value.code == sf.SF_ERR_ARG
    with pytest.raises(sf.SfError) as ei:
        sf.sf_slide_step(eng.eng, x.data_ptr() + 2, dy.data_ptr())
    assert ei.value.code == sf.SF_ERR_ALIGN
    # argument errors are not sticky: the next valid step runs
    eng.step(x, dy)
    eng.sync()
    eng.close()


@pytest.mark.parametrize("pipeline", [False, True])
def test_injected_adam_failure_is_sticky(pipeline, monkeypatch):
    """The third host Adam job fails: the step (synchronous) or the next
    step / sync (pipelined) reports SF_ERR_HIP with the job's message, every
    later call returns SF_ERR_STATE, and destroy still releases everything."""
    say("injected-adam-failure", pipeline)
    monkeypatch.setenv("SF_FAULT_ADAM_JOB", "2")
    eng = _engine(adam=True, pipeline=pipeline)
    monkeypatch.delenv("SF_FAULT_ADAM_JOB")
    x = rt.to_storage_tensor(si.layer_input(W), W).cuda()
    dy = rt.to_storage_tensor(si.upstream_grad(W), W).cuda()
    with pytest.raises(sf.SfError) as ei:
        for _ in range(3):
            eng.step(x, dy)
        eng.sync()
    assert ei.value.code == sf.SF_ERR_HIP, str(ei.value)
    assert "injected failure of Adam job 2" in str(ei.value)
    with pytest.raises(sf.SfError) as ei:
        eng.step(x, dy)
    assert ei.value.code == sf.SF_ERR_STATE
    with pytest.raises(sf.SfError) as ei:
        eng.sync()
    assert ei.value.code == sf.SF_ERR_STATE
    eng.close()
    torch.cuda.synchronize()


def test_timing_events_fixed_across_pipelined_steps():
    """Pipelined steps without a sync in between reuse the timing events
    made at creation: the count never grows and every event is free again
    once the window closes."""
    w = W.with_(n_layers=4)
    say("timing-events-fixed", w)
    eng = _engine(w=w, adam=True, pipeline=True)
    x = rt.to_storage_tensor(si.layer_input(w), w).cuda()
    dy = rt.to_storage_tensor(si.upstream_grad(w), w).cuda()
    c0 = eng.counters()
    for _ in range(40):
        eng.step(x, dy)
        c = eng.counters()
        assert c["events"] == c0["events"], (c, c0)
        assert c["live_intervals"] * 2 <= c["events"]
    agg = eng.sync()
    c = eng.counters()
    say("counters", c0, c)
    assert c["events"] == c0["events"] and c["events_free"] == c["events"] and c["live_intervals"] == 0
    # the window's rows cover all 40 steps' copies
    assert agg["h2d_bytes"] > 0 and agg["d2h_bytes"] > 0
    eng.close()
