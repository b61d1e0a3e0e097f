"""fp64 CPU oracle for causal GQA with RoPE.  TEST INFRASTRUCTURE: only the
tests, the smoke check and the benchmark's CPU-baseline leg may use it."""

from .gqa_oracle import (ROPE_THETA, inv_freq, rope, group_size, kv_group,
                         visible, softmax_rows, head_weights, attend, prefill,
                         prefill_rows, decode, prefill_brute)

__all__ = ["ROPE_THETA", "inv_freq", "rope", "group_size", "kv_group",
           "visible", "softmax_rows", "head_weights", "attend", "prefill",
           "prefill_rows", "decode", "prefill_brute"]
