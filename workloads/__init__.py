"""Seeded synthetic inputs for the LLM.int8() decomposed matmul.

This package holds only random-number generation and shapes. It contains none
of the method's arithmetic, so both the CPU oracle (``oracle/``) and the HIP
path (``int8_quantized_matmul_amd``) can be fed from it without sharing code.
"""

from .gen import (  # noqa: F401
    CONFIGS,
    SWEEP_POINTS,
    Workload,
    make_inputs,
    make_X,
    make_W,
    get_config,
    random_case,
    planted_on_row_subset,
)
