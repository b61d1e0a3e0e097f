"""fp64 CPU oracle for causal GQA with RoPE.  TEST INFRASTRUCTURE: only the
tests, the smoke check and the benchmark's CPU-baseline leg may use it."""

from .gqa_oracle import (ROPE_THETA, YaRN, base_theta, yarn_ramp, rope_mscale,
                         inv_freq, rope, group_size, kv_group,
                         visible, softmax_rows, head_weights, attend, prefill,
                         prefill_rows, prefill_group_rows, decode, prefill_brute,
                         per_sequence, chunk_positions, cache_append,
                         attend_cached, prefill_chunk, decode_ragged,
                         decode_append, qkv_sections, qkv_epilogue,
                         paged_rows, decode_paged, paged_append)

__all__ = ["ROPE_THETA", "YaRN", "base_theta", "yarn_ramp", "rope_mscale", "inv_freq",
           "rope", "group_size", "kv_group",
           "visible", "softmax_rows", "head_weights", "attend", "prefill",
           "prefill_rows", "prefill_group_rows", "decode", "prefill_brute", "per_sequence",
           "chunk_positions", "cache_append", "attend_cached", "prefill_chunk",
           "decode_ragged", "decode_append", "qkv_sections", "qkv_epilogue",
           "paged_rows", "decode_paged", "paged_append"]
