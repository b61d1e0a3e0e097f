"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module only draws random numbers and rounds them to the storage type.
It holds none of the attention arithmetic (no rotation, no softmax, no
head-to-group mapping), so the fp64 oracle and the GPU path can both take
their inputs from here without sharing any of the method.

Every tensor is drawn from its own generator,
``numpy.random.default_rng([seed, tensor_id, b])``, one per (tensor, batch
index), as ``standard_normal(float32) * sigma`` in C order.  For bf16
workloads the float32 draw is then rounded to the nearest bf16 value (ties to
even) and kept in float32, so the host array holds exactly the values the
GPU receives.
"""

from .workloads import (WORKLOADS, Workload, bf16_round, gen_prefill, gen_prefill_b,
                        gen_decode_query, gen_decode_cache_b, gen_normal,
                        scaled_rows)

__all__ = ["WORKLOADS", "Workload", "bf16_round", "gen_prefill", "gen_prefill_b",
           "gen_decode_query", "gen_decode_cache_b", "gen_normal",
           "scaled_rows"]
