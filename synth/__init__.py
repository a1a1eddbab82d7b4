"""Seeded synthetic inputs for the fused MoE layer.

This package is the only code that the CPU oracle (``oracle/``) and the HIP
path (``mixture_experts_layer_09_amd/``) both consume.  It draws random
numbers and stores them in the storage formats the layer accepts (bf16 bits,
OCP e4m3 codes, packed int4); it computes nothing the layer computes.  The
conversions to storage formats are done with library casts (torch's bf16 and
float8_e4m3fn conversions, numpy's rint) so that neither side's codecs are
involved.
"""
from .configs import CONFIGS, MoEConfig, config_by_name  # noqa: F401
from .inputs import (  # noqa: F401
    make_weights,
    make_tokens,
    make_act_scales,
    weight_seed,
    token_seed,
)
