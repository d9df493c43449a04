"""fp64 CPU oracle for the fused row-wise normalisations (RMSNorm, residual add-RMSNorm,
LayerNorm, NormRope).

TEST INFRASTRUCTURE. This package is the slow, plain reference that the HIP library is
checked against. Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it. The product path (``transformer_row_wise_amd``) never imports,
calls or links it, and it never imports the product path: the two share no code. Inputs
come from the seeded generators in ``workloads.py``, which hold no arithmetic of the method.

What it computes, and where the pages define it:
  * ``rms_norm``      -- nuvec-core 0.5.0, enum ``fast::FastOp`` (docs.rs), variant ``RmsNorm``;
                         layer defaults from nuvec-nn 0.4.0 ``layers.rs``, ``RmsNorm``.
  * ``add_rms_norm``  -- ``fast::FastOp`` variant ``AddRmsNorm``; two-output form from the
                         MinivLLM API reference "Layers", section ``LayerNorm`` (``forward``).
  * ``layer_norm``    -- ``fast::FastOp`` variant ``LayerNorm``; nuvec-nn ``layers.rs``,
                         ``LayerNorm`` (affine / ``without_bias`` / ``affine(false)``).
  * ``norm_rope``     -- ``fast::FastOp`` variants ``NormRope`` and ``Rope``; nuvec-nn
                         ``layers.rs``, ``Rope`` (defaults, positions ``offset + l``).
  * ``rope_positions`` -- the positions-tensor form of RoPE on [T, H, D] rows (MinivLLM API
                         reference, "Layers", ``RotaryEmbedding.forward``).
  * ``rope_scaling``  -- frequency scalings named by nuvec-nn ``layers.rs``, ``Rope``
                         (Llama 3 NTK-by-parts, YaRN, LongRoPE "su"), each after its
                         published method.
  * ``softmax``       -- ``fast::FastOp`` variants ``Softmax``, ``CausalSoftmax``,
                         ``LogSumExp``, ``CrossEntropy``, ``CrossEntropyVjp``.
  * ``rms_norm_vjp``, ``layer_norm_vjp`` -- ``fast::FastOp`` variants ``RmsNormVjp`` and
                         ``LayerNormVjp``: the gradients of ``RmsNorm`` (for x, w) and of
                         ``LayerNorm`` (for x, w, b) given the output cotangent g.

Every value is computed in float64 from the exact input values (bf16 and fp32 decode
exactly) and rounded once, round-to-nearest-even, to the output dtype. Parameters that the
pages carry as ``f32::to_bits`` (eps, base, scale) enter as their exact float32 values.

Parity status: every function here is pinned by the CPU tests in ``tests/`` (closed forms,
invariants, library routines, brute force at 50 digits and hand-worked fixtures under
``tests/golden/``); none is "parity unpinned".
"""

from .rounding import round_bf16, round_f32, round_to, bf16_bits, f32_param
from .norms import rms_norm, add_rms_norm, layer_norm
from .rope import rope_frequencies, rope_angles, norm_rope, rope_positions
from . import rope_scaling
from . import softmax
from .vjp import rms_norm_vjp, layer_norm_vjp

__all__ = [
    "round_bf16", "round_f32", "round_to", "bf16_bits", "f32_param",
    "rms_norm", "add_rms_norm", "layer_norm",
    "rope_frequencies", "rope_angles", "norm_rope", "rope_positions", "rope_scaling",
    "rms_norm_vjp", "layer_norm_vjp", "softmax",
]
