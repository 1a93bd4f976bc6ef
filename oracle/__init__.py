"""CPU fp64 oracle for the DSA forward hot path (test infrastructure only).

Only the test suite, the smoke check and the bench's CPU-baseline leg may
import this package. It shares no code with the HIP path.
"""

from .dsa_oracle import (  # noqa: F401
    bf16_bits_to_f64,
    indexer_scores,
    packed_metadata,
    sparse_attention,
    topk,
    topk_row,
)
