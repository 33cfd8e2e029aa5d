"""Seeded synthetic inputs for the TwELL sparse-FFN forward.

This package holds only input generation: random draws, the cast of those
draws to the storage dtype, and the per-token gate-bias schedule that sets the
activation density.  It contains none of the FFN or TwELL arithmetic, so both
the CPU oracle (``oracle/``) and the HIP path can be fed from it without
sharing any of the method's code.
"""

from .synth import (  # noqa: F401
    DTYPES,
    FfnInputs,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    ffn_inputs,
    gate_bias_for_density,
    pre_activations,
    to_storage,
)
from .configs import CONFIGS, Workload, workload  # noqa: F401
