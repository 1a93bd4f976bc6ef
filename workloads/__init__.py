"""Seeded synthetic inputs for the DSA forward hot path.

This package only draws random tensors and index routes; it holds none of the
method's arithmetic. Both the HIP path (through the tests and the bench) and
the CPU oracle consume what it produces.
"""

from .gen import (  # noqa: F401
    CONFIGS,
    Workload,
    bf16_to_numpy_bits,
    config_doc_lens,
    make_config,
    make_custom,
    make_split,
    quantize_fp8,
    qsa_routes,
    SplitWorkload,
)
