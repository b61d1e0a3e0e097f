"""Synthetic workloads: shapes against the pages' size tables, the KV-cache
claims, seeding and bf16 rounding (CPU only)."""

import numpy as np
import torch

from synthetic import WORKLOADS, bf16_round, gen_prefill, scaled_rows
from tests.oracle_pins import read_table

SIZES = {r[0]: r for r in read_table("qwen2_attention_sizes.txt")}
MODEL_OF = {"c1": "0.5B", "c2": "7B", "c3": "7B", "c4": "72B", "c5": "7B"}


def test_workload_shapes_match_size_tables():
    for key, w in WORKLOADS.items():
        _, hidden, _layers, hq, hkv, hd, g, theta = SIZES[MODEL_OF[key]]
        assert (w.h_q, w.h_kv, w.d) == (int(hq), int(hkv), int(hd)), key
        assert w.g == int(g) and w.h_q * w.d == int(hidden), key
        assert w.theta == float(theta), key


def test_kv_cache_claims():
    """2 * layers * h_kv * d * seq_len elements per the pages' formula; the 7B
    ratio against same-shape MHA is 28/4 = 7 and the cut is 85.7%."""
    (model, seq, ratio, pct), = read_table("kv_cache_claims.txt")
    _, _, layers, hq, hkv, hd, _, _ = SIZES[model]
    gqa = 2 * int(layers) * int(hkv) * int(hd) * int(seq)
    mha = 2 * int(layers) * int(hq) * int(hd) * int(seq)
    assert mha // gqa == int(ratio) and mha % gqa == 0
    assert round(100 * (1 - gqa / mha), 1) == float(pct)
    # bf16, batch 1, 32K: 1.75 GiB vs 12.25 GiB
    assert gqa * 2 == int(1.75 * 2**30) and mha * 2 == int(12.25 * 2**30)


def test_bf16_round_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 7,
                        np.array([1.00390625, 1.01171875, -2.0039062, 0.0, -0.0],
                                 np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(bf16_round(x), want)


def test_generation_is_seeded_and_exact_bf16():
    w = WORKLOADS["c2"]
    a = gen_prefill(w, B=1, L=64)
    b = gen_prefill(w, B=1, L=64)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
        np.testing.assert_array_equal(bf16_round(x), x)
    # a different tensor id gives a different stream
    assert not np.array_equal(a[1][0, :, 0], a[2][0, :, 0])


def test_boosted_rows():
    w = WORKLOADS["c5"]
    L = 256
    q, k, v = gen_prefill(w, B=1, L=L)
    for head in range(w.h_kv):
        rows = scaled_rows(w.seed, 1, head, L, w.boosted_rows)
        assert len(set(rows.tolist())) == 4 and rows.max() >= 3 * L // 4
        norms = np.linalg.norm(k[0, :, head], axis=-1)
        assert np.all(norms[rows] > 4 * np.median(norms))
    assert np.all(np.isfinite(v))
