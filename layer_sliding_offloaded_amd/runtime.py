"""Host-side plumbing around the C ABI: torch device/pinned buffers, flat
parameter packing, and small helpers that drive one layer, the head or the
sliding engine.  No arithmetic of the training step happens here.
"""

import numpy as np
import torch

from . import sf

TENSORS = sf.TENSOR_NAMES


def shape_from(w, batch=None, seq=None):
    """sf_shape for a workload-like object (fields of seeded_inputs.Workload)."""
    return sf.make_shape(w.hidden, w.n_heads, w.n_kv_heads, w.head_dim, w.ffn, w.vocab,
                         batch if batch is not None else w.batch, seq if seq is not None else w.seq,
                         w.eps, w.rope_base, sf_dtype(w))


DTYPES = {"f32": (sf.SF_F32, torch.float32), "bf16": (sf.SF_BF16, torch.bfloat16), "f16": (sf.SF_F16, torch.float16)}


def sf_dtype(w):
    return DTYPES[w.dtype][0]


def storage_dtype(w):
    return DTYPES[w.dtype][1]


# When true, every buffer this module allocates (and empty() / empty_like())
# starts as all-ones bytes, which is NaN in fp32, bf16 and fp16: a kernel or
# copy that reads memory nothing wrote then spreads NaN into its results
# instead of whatever the allocator last held.  The parity tests turn it on.
POISON = False


def _poison(t):
    if POISON:
        t.view(torch.uint8).fill_(0xFF)
    return t


def device_bytes(n, device="cuda"):
    """Uninitialised device buffer of n bytes (torch allocations are >= 256-B aligned)."""
    return _poison(torch.empty(max(int(n), 256), dtype=torch.uint8, device=device))


def pinned_bytes(n):
    return _poison(torch.empty(max(int(n), 256), dtype=torch.uint8, pin_memory=True))


def empty(*shape, dtype=torch.float32, device="cuda", pin_memory=False):
    """torch.empty (poisoned when POISON is set)."""
    return _poison(torch.empty(*shape, dtype=dtype, device=device, pin_memory=pin_memory))


def empty_like(t):
    return _poison(torch.empty_like(t))


def to_storage_tensor(a, w):
    """float32 numpy array (storage-representable values) -> torch tensor of the storage dtype (CPU)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(storage_dtype(w))


def pack_params(layout, params, w, out=None):
    """Place each tensor at its layout offset in a flat byte buffer (CPU uint8 tensor)."""
    buf = out if out is not None else torch.zeros(layout.param_bytes, dtype=torch.uint8)
    for i, name in enumerate(TENSORS):
        t = to_storage_tensor(params[name], w).reshape(-1)
        nb = t.numel() * t.element_size()
        assert nb == layout.bytes[i], (name, nb, layout.bytes[i])
        buf[layout.off[i]:layout.off[i] + nb].copy_(t.view(torch.uint8))
    return buf


def master_from_params(layout, params):
    """fp32 master weights in the gradient layout (the host Adam layout)."""
    m = np.zeros(layout.grad_bytes // 4, dtype=np.float32)
    for i, name in enumerate(TENSORS):
        o = layout.grad_off[i] // 4
        a = np.asarray(params[name], dtype=np.float32).reshape(-1)
        m[o:o + a.size] = a
    return m


def unpack_grads(layout, flat, shapes):
    """fp32 flat gradient buffer (numpy, grad layout) -> dict name -> array."""
    out = {}
    for i, name in enumerate(TENSORS):
        o = layout.grad_off[i] // 4
        n = layout.grad_bytes_t[i] // 4
        out[name] = flat[o:o + n].reshape(shapes[name])
    return out


def unpack_params(layout, flat_bytes, shapes, w):
    """Storage-dtype flat parameter buffer (CPU uint8 tensor) -> dict of float32 arrays."""
    out = {}
    dt = storage_dtype(w)
    for i, name in enumerate(TENSORS):
        o, nb = layout.off[i], layout.bytes[i]
        t = flat_bytes[o:o + nb].view(dt).to(torch.float32)
        out[name] = t.numpy().reshape(shapes[name])
    return out


def stream_handle(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


class Context:
    """An sf_ctx plus the device workspace it borrows."""

    def __init__(self, w, head_chunk_rows=2048, batch=None, seq=None, head_dw_rows=0):
        """head_dw_rows: rows of dlogits kept for one LM-head weight-gradient
        product (sf_ctx_create_ex); 0 = one product per chunk."""
        self.w = w
        self.shape = shape_from(w, batch, seq)
        self.chunk = head_chunk_rows
        self.layout = sf.sf_layer_layout_ex(self.shape, head_chunk_rows, head_dw_rows)
        n = self.layout.workspace_bytes + (self.layout.head_workspace_bytes if w.vocab else 0)
        self.ws = device_bytes(n)
        self.ctx = sf.sf_ctx_create_ex(self.shape, head_chunk_rows, head_dw_rows, self.ws.data_ptr(),
                                       self.ws.numel())

    def close(self):
        if self.ctx:
            sf.sf_ctx_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Engine:
    """An sf_engine with every buffer it borrows: the device unit pool and
    activation region, pinned host parameters and gradient slots, host fp32
    master weights and Adam moments, and (with a head) the resident
    embedding / LM-head tensors.

    layers: list of per-layer parameter dicts (float32 storage values), or a
    callable l -> such a dict for l in range(w.n_layers); a callable's layers
    are drawn on `draw_threads` threads and packed into pinned memory one by
    one, so only a few of them exist unpacked at once.
    head: None or dict with E [V, H], gf [H], Wlm [V, H] (float32 storage values).
    ckpt: sliding activation checkpointing (layer inputs kept in pinned host
    memory, each layer's forward recomputed before its backward).
    pipeline: host Adam (or, without Adam, the last gradient copies) runs on
    across the step boundary (call sync() before reading host parameters,
    moments or gradient slots).
    keep_turnaround: without Adam, layers 0..window-1 stay in their units from
    one step's backward to the next step's forward (h_params unchanged).
    loss_scale, scale_window: fp16 storage's dynamic loss scaling (initial
    scale and growth window; 0 takes the library's defaults).
    head_dw_rows: rows of dlogits the LM head keeps for one dW_lm product
    (sf_ctx_create_ex; 0: one product per chunk).
    """

    def __init__(self, w, layers, head=None, window=2, n_grad_slots=2, adam=True, chunk=2048,
                 adam_threads=0, adam_hp=None, stream=None, head_adam="device", ckpt=False, pipeline=False,
                 draw_threads=1, keep_turnaround=False, loss_scale=0.0, scale_window=0, head_dw_rows=0):
        import ctypes
        from concurrent.futures import ThreadPoolExecutor
        hp = adam_hp or dict(lr=1e-4, b1=0.9, b2=0.999, eps=1e-8)
        self.w = w
        if callable(layers):
            layer_fn, self.nl = layers, w.n_layers
        else:
            layer_fn, self.nl = (lambda l: layers[l]), len(layers)
        self.ctx = Context(w, chunk, head_dw_rows=head_dw_rows)
        L = self.ctx.layout
        self.layout = L
        shape = self.ctx.shape
        W = min(window, self.nl)
        unit = (L.param_bytes + 255) // 256 * 256 + (L.grad_bytes + 255) // 256 * 256
        self.pool = device_bytes(W * unit)
        flags = (sf.SF_ENGINE_ADAM if adam else 0) | (sf.SF_ENGINE_HEAD if head is not None else 0)
        if head is not None and head_adam == "host":
            flags |= sf.SF_ENGINE_HEAD_HOST_ADAM
        if ckpt:
            flags |= sf.SF_ENGINE_CKPT
        if pipeline:
            flags |= sf.SF_ENGINE_PIPELINE
        if keep_turnaround:
            flags |= sf.SF_ENGINE_KEEP_TURNAROUND
        act = sf.sf_engine_act_bytes_flags(shape, self.nl, flags)
        self.act = device_bytes(act)
        self.act_bytes = act
        ebytes = 4 if w.dtype == "f32" else 2
        self.x_bytes = (shape.batch * shape.seq * shape.hidden * ebytes + 255) // 256 * 256
        self.h_ckpt = pinned_bytes(max(self.nl - 1, 1) * self.x_bytes) if ckpt else None
        def stage(l):
            p = layer_fn(l)
            # fp32 master weights (host, pageable): only with Adam
            return pack_params(L, p, w, pinned_bytes(L.param_bytes)), (master_from_params(L, p) if adam else None)

        with ThreadPoolExecutor(max(1, min(draw_threads, self.nl))) as ex:
            staged = list(ex.map(stage, range(self.nl)))
        self.h_params = [a for a, _ in staged]
        self.h_master = [m for _, m in staged] if adam else []
        del staged
        self.h_m = [np.zeros_like(m) for m in self.h_master]
        self.h_v = [np.zeros_like(m) for m in self.h_master]
        self.h_slots = [pinned_bytes(L.grad_bytes) for _ in range(n_grad_slots)]
        self._arrays = []

        def parr(ptrs):
            a = sf.pointer_array(ptrs)
            self._arrays.append(a)
            return ctypes.cast(a, ctypes.POINTER(ctypes.c_void_p))

        self.head_adam = head_adam
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        cfg = sf.SfEngineCfg()
        cfg.n_layers, cfg.window, cfg.n_grad_slots, cfg.flags = self.nl, window, n_grad_slots, flags
        cfg.adam_threads = adam_threads
        cfg.lr, cfg.b1, cfg.b2, cfg.eps = hp["lr"], hp["b1"], hp["b2"], hp["eps"]
        cfg.d_pool, cfg.pool_bytes = self.pool.data_ptr(), self.pool.numel()
        cfg.d_act, cfg.act_bytes = self.act.data_ptr(), self.act.numel()
        cfg.h_params = parr([t.data_ptr() for t in self.h_params])
        if adam:
            cfg.h_master = parr([m.ctypes.data for m in self.h_master])
            cfg.h_m = parr([m.ctypes.data for m in self.h_m])
            cfg.h_v = parr([m.ctypes.data for m in self.h_v])
        cfg.h_grad_slots = parr([t.data_ptr() for t in self.h_slots])
        cfg.compute_stream = self.stream.cuda_stream
        cfg.loss_scale, cfg.scale_window = loss_scale, scale_window
        if ckpt:
            cfg.h_ckpt = self.h_ckpt.data_ptr()
        if head is not None:
            V, H = w.vocab, w.hidden
            dt = storage_dtype(w)
            self.d_E = to_storage_tensor(head["E"], w).cuda()
            self.d_gf = to_storage_tensor(head["gf"], w).cuda()
            self.d_wlm = to_storage_tensor(head["Wlm"], w).cuda()
            self.d_head_grads = empty(2 * V * H + H, dtype=torch.float32)
            self.h_head_grads = empty(2 * V * H + H, dtype=torch.float32, device="cpu", pin_memory=True)
            flat = np.concatenate([head["E"].reshape(-1), head["gf"].reshape(-1), head["Wlm"].reshape(-1)])
            self.h_head_params = torch.empty(flat.size, dtype=dt, pin_memory=True)
            self.h_head_params.copy_(to_storage_tensor(flat, w))
            self.h_head_master = flat.astype(np.float32).copy()
            self.h_head_m = np.zeros_like(self.h_head_master)
            self.h_head_v = np.zeros_like(self.h_head_master)
            if head_adam == "device":
                nh = self.h_head_master.size
                self.d_head_state = torch.zeros(3 * nh, dtype=torch.float32, device="cuda")
                self.d_head_state[:nh].copy_(torch.from_numpy(self.h_head_master))
                cfg.d_head_state = self.d_head_state.data_ptr()
            cfg.d_E, cfg.d_gf, cfg.d_wlm = self.d_E.data_ptr(), self.d_gf.data_ptr(), self.d_wlm.data_ptr()
            cfg.d_head_grads = self.d_head_grads.data_ptr()
            cfg.h_head_params = self.h_head_params.data_ptr()
            cfg.h_head_master = self.h_head_master.ctypes.data
            cfg.h_head_m = self.h_head_m.ctypes.data
            cfg.h_head_v = self.h_head_v.ctypes.data
            cfg.h_head_grads = self.h_head_grads.data_ptr()
        self.cfg = cfg
        torch.cuda.synchronize()
        self.eng = sf.sf_engine_create(self.ctx.ctx, cfg)

    def step(self, d_in, d_dy=None):
        """d_in: device int32 ids [T] (head) or storage-dtype x [T, H]; returns (loss, stats dict)."""
        loss, st = sf.sf_slide_step(self.eng, d_in.data_ptr(), None if d_dy is None else d_dy.data_ptr())
        return loss, st.as_dict()

    def sync(self):
        """Wait for every step's copies and Adam jobs; returns the stats dict of
        the steps since the previous sync (pipelined) or of the last step."""
        return sf.sf_engine_sync(self.eng).as_dict()

    def counters(self):
        """The engine's timing bookkeeping (sf_engine_counters)."""
        return sf.sf_engine_counters(self.eng)

    def trace(self):
        """The last step's timeline: list of (kind name, start_ms, end_ms, info)."""
        return [(sf.TRACE_KINDS[int(k)], a, b, x) for k, a, b, x in sf.sf_engine_trace(self.eng)]

    def close(self):
        if getattr(self, "eng", None):
            sf.sf_engine_destroy(self.eng)
            self.eng = None
        self.ctx.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
