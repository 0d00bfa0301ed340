"""Seeded synthetic inputs for IKBO target attention and IKBO linear compression.

This package draws inputs only: sequence lengths, candidate-to-user mappings and
N(0,1) tensors quantised to the dtype the kernel receives (MXFP8 codes drawn with
torch's E4M3 conversion and randomly drawn block scales).  It holds none of the
attention or projection arithmetic, so both the fp64 oracle's tests and the GPU
path can use it without sharing any of the method's code.
"""

from .ikbo import (  # noqa: F401
    BWD_SEED_OFFSET,
    CONFIG_NAMES,
    Workload,
    add_output_grad,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_bwd_workload,
    make_custom,
    make_workload,
)
from .lce import (  # noqa: F401
    LCE_NAMES,
    LCE_NESTED_NAMES,
    LceNestedWorkload,
    LceWorkload,
    make_lce,
    make_lce_custom,
    make_lce_nested,
    make_lce_nested_custom,
)
from .mxfp8 import MX_NAMES, MxWorkload, make_mxfp8, make_mxfp8_custom  # noqa: F401
