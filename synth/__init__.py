"""Seeded synthetic input generators.

This package produces the raw inputs (packed weight bytes, f32 activations,
expert ids, per-pair scales) that both the CPU oracle and the HIP path consume.
It holds none of the method's arithmetic: nothing here decodes a block or
contracts anything.  See ``synth.gen``.
"""

from .gen import (  # noqa: F401
    lcg_states,
    quant_bytes,
    unit_f32,
    nvfp4_rows,
    xorshift_f32,
    expert_ids,
    pair_scales,
    dense_weights,
    structured_exact,
)
