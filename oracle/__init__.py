"""fp64 CPU oracle for exact attention: forward, gradients and paged-cache
decoding (test infrastructure only).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package; the product path never does.
"""
from .attention import (attention_bwd_ref, attention_bwd_rows_ref, attention_probs_ref,
                        attention_ref, attention_rows_ref, attention_tiled_ref, kv_head,
                        visible)
from .decode import paged_decode_ref, paged_gather, paged_token_slots

__all__ = ["attention_bwd_ref", "attention_bwd_rows_ref", "attention_probs_ref",
           "attention_ref", "attention_rows_ref", "attention_tiled_ref", "kv_head", "visible",
           "paged_decode_ref", "paged_gather", "paged_token_slots"]
