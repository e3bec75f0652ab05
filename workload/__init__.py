"""Seeded synthetic inputs for MLA absorbed decode.

This package is the only code shared by the CPU oracle (``oracle/``) and the
GPU path's tests and benchmark.  It draws random tensors, rounds them to
bfloat16, samples request lengths and builds page tables.  It contains none of
the attention arithmetic.
"""

from .gen import (  # noqa: F401
    CONFIGS,
    AppendCase,
    Case,
    WorkloadConfig,
    bf16_bits_to_f32,
    draw_latent_output,
    draw_latent_query,
    f32_to_bf16_bits,
    make_append_case,
    make_case,
    round_to_bf16,
)
