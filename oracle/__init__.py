"""CPU oracle for the fused MoE forward layer -- TEST INFRASTRUCTURE.

Plain, slow, fp64 NumPy.  It defines what the layer computes so that the HIP
path can be checked against it.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` import it; the product package
``mixture_experts_layer_09_amd`` never does, and this package imports nothing
from it.  The two share no code: the seeded inputs of ``synth/`` are the only
thing both consume.

Sources (the method's pages, cited by page and section):
 * sglang PR 21321 page -- "FlashInfer TRTLLM-Gen MoE kernel optimisation:
   NemotronH support" (op signature with ``topk``/``renormalize``/
   ``activation_type``; ``_is_gated``; ``_align_fp8_moe_weights``; the
   [Up, Gate] -> [Gate, Up] swap; the fp8 per-tensor scale algebra).
 * flashinfer PR 4329 page -- "Gated MoE kernel optimisation for Blackwell"
   (generic vs gated kernels; gate/up branch pairing in FC1; FC2 non-gated).
 * sglang PR 26204 page -- "Qwen3-Next FP8 MoE: Shared-Expert Fusion"
   (fp8 w8a8 with 128x128 block scales; the shared expert as slot E=513).
 * sglang PR 32944 page -- "SwiGLU fusion into the MoE up-GEMM epilogue"
   (load-time gate/up interleave; SiLU*up in the epilogue; half-width store).
 * sglang PR 38220 page -- "W4A8 MoE GEMM for GLM-5.2 on H200"
   (int4 weights with group scales, fp8 activations, grouped problem list).

Parity pins: every function here is checked by ``tests/test_oracle_*.py``
against closed forms, invariants and independent library routines; none is
"parity unpinned".
"""
from . import codecs  # noqa: F401
from .moe import (  # noqa: F401
    route,
    align,
    quant_x,
    swap_halves,
    pad_intermediate,
    padded_intermediate,
    interleave_rows,
    dequant_w13,
    dequant_w2,
    store_intermediate,
    intermediate_window,
    gemm1_window,
    mfma_dot_model,
    activation_window,
    moe_forward,
)
