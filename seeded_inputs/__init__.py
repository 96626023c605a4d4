"""Seeded synthetic inputs shared by the oracle tests, the HIP parity tests and
the benchmark.

This module holds none of the method's arithmetic: it only names the
workloads, draws random numbers with fixed seeds and rounds them once to the
storage dtype.  Both the oracle and the HIP path consume these same arrays.

Seeds (numpy ``default_rng``): ``[0, l]`` for layer l's weights, ``[1]`` for
the layer input x, ``[2]`` for the upstream gradient dy, ``[3]`` for token
ids, ``[4]`` for the embedding table, ``[5]`` for the LM-head weight.
Values are drawn in float32 and rounded once (round to nearest, ties to even)
to the storage dtype.  Weights are N(0, 0.02^2); activations and upstream
gradients N(0, 1); token ids uniform in [0, vocab); RMSNorm gains are 1, or
1 + N(0, 0.1^2) when ``gains="random"`` (parity tests use that so a wrong gain
index cannot hide).
"""

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    """A synthetic Llama-shaped workload."""

    name: str
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int          # 0 = no embedding / LM head
    batch: int
    seq: int
    n_layers: int
    dtype: str          # "f32", "bf16" or "f16"
    window: int = 2
    eps: float = 1e-6
    rope_base: float = 10000.0

    @property
    def tokens(self):
        return self.batch * self.seq

    def with_(self, **kw):
        return replace(self, **kw)


WORKLOADS = {
    # one decoder layer in fp32: the small parity case
    "layer-h256-fp32": Workload("layer-h256-fp32", 256, 4, 4, 64, 688, 0, 1, 128, 1, "f32"),
    # 4-layer stack + LM head, window 2 layers of 4 resident
    "stack4-h1024-bf16": Workload("stack4-h1024-bf16", 1024, 16, 16, 64, 2816, 32000, 4, 512, 4, "bf16"),
    # 24-layer ~1.3B-shaped model
    "llama1.3b-bf16": Workload("llama1.3b-bf16", 2048, 16, 16, 128, 5504, 32000, 8, 1024, 24, "bf16"),
    # 32-layer ~6.7B-shaped model
    "llama6.7b-bf16": Workload("llama6.7b-bf16", 4096, 32, 32, 128, 11008, 32000, 4, 2048, 32, "bf16"),
    # slice of eight ~123B-shaped layers with 8 KV heads (GQA group 12)
    "slice123b-gqa-bf16": Workload("slice123b-gqa-bf16", 12288, 96, 8, 128, 28672, 0, 1, 4096, 8, "bf16"),
}

ADAM = dict(lr=1e-4, b1=0.9, b2=0.999, eps=1e-8)

LAYER_TENSORS = ("Wq", "Wk", "Wv", "Wo", "Wg", "Wu", "Wd", "g1", "g2")


def layer_tensor_shapes(w):
    """Shape of each per-layer tensor, in storage order."""
    H, F = w.hidden, w.ffn
    qd, kvd = w.n_heads * w.head_dim, w.n_kv_heads * w.head_dim
    return {
        "Wq": (qd, H), "Wk": (kvd, H), "Wv": (kvd, H), "Wo": (H, qd),
        "Wg": (F, H), "Wu": (F, H), "Wd": (H, F), "g1": (H,), "g2": (H,),
    }


# ---------------------------------------------------------------- rounding

def f32_to_bf16_bits(a):
    """float32 array -> uint16 bf16 bit patterns, round to nearest even."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(u):
    """uint16 bf16 bit patterns -> float32 values (exact)."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_storage(a, dtype):
    """Round a float32 array once to the storage dtype; returns float32."""
    a = np.asarray(a, dtype=np.float32)
    if dtype == "f32":
        return a
    if dtype == "bf16":
        return bf16_bits_to_f32(f32_to_bf16_bits(a))
    if dtype == "f16":
        return a.astype(np.float16).astype(np.float32)   # IEEE round to nearest even
    raise ValueError(dtype)


# ---------------------------------------------------------------- draws

def layer_params(w, layer, gains="one"):
    """Weights of layer ``layer`` (seed [0, layer]) as float32 storage values."""
    rng = np.random.default_rng([0, layer])
    out = {}
    for name, shp in layer_tensor_shapes(w).items():
        if name.startswith("W"):
            out[name] = to_storage(rng.standard_normal(shp, dtype=np.float32) * np.float32(0.02), w.dtype)
    for name in ("g1", "g2"):
        if gains == "one":
            out[name] = np.ones(w.hidden, dtype=np.float32)
        elif gains == "random":
            g = 1.0 + 0.1 * rng.standard_normal(w.hidden, dtype=np.float32)
            out[name] = to_storage(g, w.dtype)
        else:
            raise ValueError(gains)
    return out


def layer_input(w, seed=1, scale=1.0):
    """x ~ N(0, scale^2), shape [B, S, H] (scale 1 for every workload)."""
    rng = np.random.default_rng([seed])
    x = rng.standard_normal((w.batch, w.seq, w.hidden), dtype=np.float32)
    return to_storage(x * np.float32(scale) if scale != 1.0 else x, w.dtype)


def upstream_grad(w, seed=2, scale=1.0):
    """dy ~ N(0, scale^2), shape [B, S, H] (scale 1 for every workload)."""
    rng = np.random.default_rng([seed])
    g = rng.standard_normal((w.batch, w.seq, w.hidden), dtype=np.float32)
    return to_storage(g * np.float32(scale) if scale != 1.0 else g, w.dtype)


def token_ids(w, seed=3):
    """ids ~ U[0, vocab), int32 [B, S]."""
    rng = np.random.default_rng([seed])
    return rng.integers(0, w.vocab, size=(w.batch, w.seq), dtype=np.int32)


def embedding(w, seed=4):
    """Embedding table E [V, H] ~ N(0, 0.02^2)."""
    rng = np.random.default_rng([seed])
    return to_storage(rng.standard_normal((w.vocab, w.hidden), dtype=np.float32) * np.float32(0.02), w.dtype)


def lm_head(w, seed=5):
    """LM-head weight W_lm [V, H] ~ N(0, 0.02^2)."""
    rng = np.random.default_rng([seed])
    return to_storage(rng.standard_normal((w.vocab, w.hidden), dtype=np.float32) * np.float32(0.02), w.dtype)


def final_gain(w, gains="one", seed=6):
    """Final RMSNorm gain g_f [H]."""
    if gains == "one":
        return np.ones(w.hidden, dtype=np.float32)
    rng = np.random.default_rng([seed])
    return to_storage(1.0 + 0.1 * rng.standard_normal(w.hidden, dtype=np.float32), w.dtype)
