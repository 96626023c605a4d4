"""CPU fp64 oracle for the layer-sliding fine-tuning step (test infrastructure).

This package is test infrastructure, not product code. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The HIP library never calls it and shares no code with it; the two
meet only through the seeded inputs in ``seeded_inputs``.

Source pages (all three are summaries of the same paper, "An Efficient
Heterogeneous Co-Design for Fine-Tuning on a Single GPU", SlideFormer):

* de -- gist.science/de/paper/2603.16428, "Technische Zusammenfassung"
* es -- gist.science/es/paper/2603.16428, "Resumen tecnico"
* fr -- gist.science/fr/paper/2603.16428, technical summary

What the oracle computes and why that is the right thing:

* The pages name the model families (Llama, Qwen, Mistral: de §5, es §3) and
  the fused ops (RoPE, RMSNorm, SwiGLU, LinearCrossEntropy: de §2C, es §2C,
  fr §2C) but print no layer equations.  The oracle is therefore the plain
  definition of a pre-norm Llama decoder block (``layer.py``), its
  hand-derived backward, the next-token cross-entropy head (``head.py``),
  plain Adam (``adam.py``) and fp16's dynamic loss scaling
  (``loss_scale.py``).
* Layer sliding moves tensors between host and device and overlaps the host
  optimizer with the device backward (de §2A, es §2A, fr §2A); it changes
  where values live, not what is computed.  The oracle computes the plain,
  un-slid training step, which the sliding engine must reproduce.

Every routine works in float64 on numpy arrays.  Inputs are the exact stored
values (bf16- or fp32-representable numbers upcast to float64).

Parity status: every function here is pinned by ``tests/oracle`` against
something other than itself (central finite differences, torch autograd in
float64, the HF ``LlamaDecoderLayer`` in float64, ``torch.optim.Adam``,
closed forms and invariants).  No function is "parity unpinned"; the
conventions the pages leave open (block structure, RoPE pairing, Adam
epsilon) are readings, listed in the design notes.
"""

from .layer import (  # noqa: F401
    LayerShape,
    rmsnorm_fwd,
    rmsnorm_bwd,
    rope_angles,
    rope_apply,
    rope_apply_inverse,
    attention_fwd,
    attention_bwd,
    silu,
    swiglu_fwd,
    swiglu_bwd,
    layer_fwd,
    layer_fwd_rows,
    layer_bwd,
)
from .head import embed_fwd, embed_bwd, head_fwd_bwd  # noqa: F401
from .adam import adam_step, round_bf16, round_f16  # noqa: F401
from .loss_scale import adam_with_skip, applied_updates, update_scale  # noqa: F401
from .model import stack_step  # noqa: F401
