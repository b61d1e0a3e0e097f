"""The five attention workloads and their seeded input generators.

Shapes follow the Qwen2 size tables (query heads, KV heads, head size):
0.5B 14/2/64, 7B 28/4/128, 72B 64/8/128, with RoPE base 1e6.  Nothing here
rotates, scores or normalises; see the package docstring.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

# tensor ids of the per-tensor generators
TID_Q, TID_K, TID_V, TID_PICK = 0, 1, 2, 3


@dataclasses.dataclass(frozen=True)
class Workload:
    key: str
    name: str
    kind: str            # "prefill" or "decode"
    B: int
    L: int               # prefill: sequence length; decode: cached positions
    h_q: int
    h_kv: int
    d: int
    dtype: str           # "f32" or "bf16" (storage type of q, k, v)
    seed: int
    sigma: float = 1.0
    theta: float = 1.0e6
    boosted_rows: int = 0    # rows per Q/K head multiplied by 8 (0 = none)

    @property
    def g(self) -> int:
        return self.h_q // self.h_kv

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def q_pos(self) -> int:
        """Decode: position of the new query token (right after the cache)."""
        return self.L

    def prefill_flops(self) -> int:
        """QK^T + PV flops over the causal pairs j <= i only."""
        return 4 * self.B * self.h_q * self.d * self.L * (self.L + 1) // 2

    def decode_kv_bytes(self) -> int:
        """K and V cache bytes read once per KV group."""
        esz = 2 if self.dtype == "bf16" else 4
        return 2 * self.B * self.L * self.h_kv * self.d * esz


WORKLOADS = {
    "c1": Workload("c1", "qwen2-0.5b-gqa-prefill-f32", "prefill",
                   B=1, L=128, h_q=14, h_kv=2, d=64, dtype="f32", seed=1001),
    "c2": Workload("c2", "qwen2-7b-gqa-prefill-bf16", "prefill",
                   B=4, L=4096, h_q=28, h_kv=4, d=128, dtype="bf16", seed=1002),
    "c3": Workload("c3", "qwen2-7b-gqa-decode-bf16", "decode",
                   B=32, L=32768, h_q=28, h_kv=4, d=128, dtype="bf16", seed=1003),
    "c4": Workload("c4", "qwen2-72b-gqa-prefill-bf16", "prefill",
                   B=2, L=8192, h_q=64, h_kv=8, d=128, dtype="bf16", seed=1004),
    "c5": Workload("c5", "qwen2-7b-gqa-prefill-32k-bf16", "prefill",
                   B=1, L=32768, h_q=28, h_kv=4, d=128, dtype="bf16", seed=1005,
                   sigma=0.5, boosted_rows=4),
}


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even), kept as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32)


def gen_normal(seed: int, tid: int, b: int, shape, sigma: float,
               dtype: str) -> np.ndarray:
    """One batch slice: standard normal float32 * sigma, bf16-rounded if asked."""
    rng = np.random.default_rng([seed, tid, b])
    x = rng.standard_normal(size=tuple(shape), dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    if dtype == "bf16":
        x = bf16_round(x)
    return x


def scaled_rows(seed: int, which: int, head: int, L: int, n: int) -> np.ndarray:
    """n distinct seeded row indices of one head, at least one in the last quarter."""
    rng = np.random.default_rng([seed, TID_PICK, which, head])
    first = int(rng.integers(3 * L // 4, L))
    rows = [first]
    while len(rows) < min(n, L):
        r = int(rng.integers(0, L))
        if r not in rows:
            rows.append(r)
    return np.array(sorted(rows), dtype=np.int64)


def _boost(x: np.ndarray, seed: int, which: int, n: int) -> None:
    # x: [B, L, h, d]; the same rows are boosted in every batch slice
    L, h = x.shape[1], x.shape[2]
    for head in range(h):
        rows = scaled_rows(seed, which, head, L, n)
        x[:, rows, head, :] *= np.float32(8.0)


def gen_prefill(w: Workload, B: int | None = None, L: int | None = None):
    """(q, k, v) float32 host arrays shaped [B, L, h, d] for a prefill workload.

    ``B``/``L`` override the workload's sizes (same recipe, smaller draw).
    """
    B = w.B if B is None else B
    L = w.L if L is None else L
    q = np.empty((B, L, w.h_q, w.d), np.float32)
    k = np.empty((B, L, w.h_kv, w.d), np.float32)
    v = np.empty((B, L, w.h_kv, w.d), np.float32)
    for b in range(B):
        q[b] = gen_normal(w.seed, TID_Q, b, (L, w.h_q, w.d), w.sigma, w.dtype)
        k[b] = gen_normal(w.seed, TID_K, b, (L, w.h_kv, w.d), w.sigma, w.dtype)
        v[b] = gen_normal(w.seed, TID_V, b, (L, w.h_kv, w.d), w.sigma, w.dtype)
    if w.boosted_rows:
        _boost(q, w.seed, 0, w.boosted_rows)
        _boost(k, w.seed, 1, w.boosted_rows)
    return q, k, v


def gen_prefill_b(w: Workload, b: int, L: int | None = None):
    """(q, k, v) of batch slice b alone, each [L, h, d]: the same values as
    gen_prefill(w)[i][b] (per-slice generators; boosted rows are the same in
    every slice)."""
    L = w.L if L is None else L
    q = gen_normal(w.seed, TID_Q, b, (1, L, w.h_q, w.d), w.sigma, w.dtype)
    k = gen_normal(w.seed, TID_K, b, (1, L, w.h_kv, w.d), w.sigma, w.dtype)
    v = gen_normal(w.seed, TID_V, b, (1, L, w.h_kv, w.d), w.sigma, w.dtype)
    if w.boosted_rows:
        _boost(q, w.seed, 0, w.boosted_rows)
        _boost(k, w.seed, 1, w.boosted_rows)
    return q[0], k[0], v[0]


def gen_decode_query(w: Workload, B: int | None = None) -> np.ndarray:
    """New query tokens [B, h_q, d] (pre-rotation) for a decode workload."""
    B = w.B if B is None else B
    return np.stack([gen_normal(w.seed, TID_Q, b, (w.h_q, w.d), w.sigma, w.dtype)
                     for b in range(B)])


def gen_decode_cache_b(w: Workload, b: int, L: int | None = None):
    """Cached (already rotated) K and V of one sequence, each [L, h_kv, d]."""
    L = w.L if L is None else L
    k = gen_normal(w.seed, TID_K, b, (L, w.h_kv, w.d), w.sigma, w.dtype)
    v = gen_normal(w.seed, TID_V, b, (L, w.h_kv, w.d), w.sigma, w.dtype)
    return k, v
