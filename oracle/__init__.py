"""CPU fp64 oracle for paged exact attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
bench's CPU-baseline leg, never by the library or its binding.  It shares no
code with the HIP path.
"""
from .attention import (  # noqa: F401
    bf16_to_f64, pages_needed, locate_token, gather_sequence, kv_head_of, row_positions,
    visible_mask, scores,
    softmax_rows, weighted_values, attend, paged_prefill, paged_decode,
)
