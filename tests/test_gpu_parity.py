"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Small shapes (several tiles, ragged tails, MHA/MQA/GQA, L = 1) are compared
element by element.  The five workloads run at full size in the launch
configuration the benchmark times; their outputs are compared on sampled
rows that the oracle evaluates one by one.

Tolerances: fp32 inputs max-abs <= 1e-4; bf16 inputs (fp32 accumulation)
max-abs <= 2e-2 and relative L2 <= 1e-2.
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import rope_causal_grouped_amd as gqa
from synthetic import (WORKLOADS, Workload, bf16_round, gen_decode_cache_b,
                       gen_decode_query, gen_prefill, scaled_rows)

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-4
TOL_BF16_ABS = 2e-2
TOL_BF16_REL = 1e-2


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device="cuda", dtype=dtype)


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def assert_parity(got, want, dtype, what):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, what
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - want)
    mx = float(err.max()) if err.size else 0.0
    rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30))
    note(f"  {what}: max-abs {mx:.3e} rel-L2 {rel:.3e}")
    if dtype == torch.float32:
        assert mx <= TOL_F32, f"{what}: max-abs {mx:.3e} > {TOL_F32}"
    else:
        assert mx <= TOL_BF16_ABS, f"{what}: max-abs {mx:.3e} > {TOL_BF16_ABS}"
        assert rel <= TOL_BF16_REL, f"{what}: rel-L2 {rel:.3e} > {TOL_BF16_REL}"


def small_case(B, L, h_q, h_kv, d, dtype, seed, sigma=1.0):
    w = Workload("t", "test", "prefill", B, L, h_q, h_kv, d,
                 "bf16" if dtype == torch.bfloat16 else "f32", seed, sigma)
    return gen_prefill(w)


# ------------------------------------------------------------------ RoPE --

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d,pos0", [(64, 0), (128, 0), (128, 32700)])
def test_rope_apply(dtype, d, pos0):
    note(f"rope_apply {dtype} d={d} pos0={pos0}")
    q, _, _ = small_case(2, 37, 3, 3, d, dtype, 11)
    x = dev(q, dtype)
    gqa.rope_apply(x, pos0=pos0)
    torch.cuda.synchronize()
    want = oracle.rope(q, np.arange(pos0, pos0 + 37))
    got = host(x)
    if dtype == torch.float32:
        assert np.max(np.abs(got - want)) <= 1e-5
    else:
        # rounding the fp32 rotation to bf16: half an ulp of the exact value
        # (<= 2^-8 |want|), plus the fp32 rotation's own error, which is
        # absolute (~1e-7 of the pair's size) and matters near zero
        assert np.all(np.abs(got - want) <= np.abs(want) * 2.0 ** -8 + 1e-5)


# ------------------------------------------------------- prefill, small --

SMALL_BF16 = [
    (2, 300, 14, 2, 64),     # Qwen2-0.5B heads, ragged tail vs 64-key tiles
    (1, 333, 28, 4, 128),    # Qwen2-7B heads
    (1, 257, 16, 2, 128),    # g = 8 (72B ratio), rows span 256-row blocks
    (2, 130, 8, 8, 128),     # MHA (g = 1)
    (1, 190, 8, 1, 64),      # MQA (h_kv = 1)
    (1, 1, 28, 4, 128),      # a single position
    (3, 64, 12, 2, 128),     # exactly one tile, g = 6 (1.5B ratio)
    (1, 65, 28, 4, 64),
    (1, 70, 40, 2, 128),     # g = 20 > 16
    (3, 100, 4, 1, 128),     # 3 (batch, group) units: each cut into 8 strided parts
    (5, 600, 12, 1, 64),     # 5 units, ragged part sizes across the XCDs
    (3, 700, 16, 4, 128),    # 12 units: halves of groups per XCD
]


@pytest.mark.parametrize("shape", SMALL_BF16, ids=lambda s: "B%d_L%d_%d/%d_d%d" % s)
def test_prefill_bf16_small(shape):
    B, L, h_q, h_kv, d = shape
    note(f"prefill bf16 {shape}")
    q, k, v = small_case(B, L, h_q, h_kv, d, torch.bfloat16, 100 + L)
    o = gqa.prefill(dev(q, torch.bfloat16), dev(k, torch.bfloat16), dev(v, torch.bfloat16))
    torch.cuda.synchronize()
    assert_parity(host(o), oracle.prefill(q, k, v), torch.bfloat16, f"prefill bf16 {shape}")


def attend_rounded_operands(q, k, v):
    """The oracle's attention on the operands the bf16 matrix cores see: the
    rotated Q times scale*log2(e) and the rotated K, each rounded to bf16
    (scores then in log2 units, hence softmax scale ln 2)."""
    B, L, h_q, d = q.shape
    h_kv = k.shape[2]
    pos = np.arange(L)
    sl2 = math.log2(math.e) / math.sqrt(d)
    qb = bf16_round((oracle.rope(q, pos) * sl2).astype(np.float32)).astype(np.float64)
    kb = bf16_round(oracle.rope(k, pos).astype(np.float32)).astype(np.float64)
    vis = oracle.visible(pos, pos)
    out = np.empty((B, L, h_q, d))
    for b in range(B):
        for t in range(h_q):
            u = oracle.kv_group(t, h_q, h_kv)
            out[b, :, t] = oracle.attend(qb[b, :, t], kb[b, :, u], v[b, :, u], math.log(2), vis)
    return out


@pytest.mark.parametrize("sigma,boosted", [(3.0, 0), (0.5, 24)], ids=["sigma3", "boosted"])
@pytest.mark.parametrize("shape", [(1, 333, 28, 4, 128), (2, 300, 14, 2, 64)],
                         ids=lambda s: "B%d_L%d_%d/%d_d%d" % s)
def test_prefill_bf16_large_scores(shape, sigma, boosted):
    """Score bounds past the 64 (log2) headroom: the kernel takes tile maxima
    first and shifts the scores by a nonzero reference.  With boosted rows
    (x8) only some rows of a wave need the shift, the rest keep m = 0.

    Rounding the rotated Q and K to bf16 perturbs a score by about 2^-9 of
    its size, so at logits of 70 (sigma 3) the output moves by up to ~0.1
    from the exact result whatever the softmax does: the relative-L2 bar is
    checked against the oracle, the max-abs bar against the oracle's
    attention on those rounded operands (where a one-ulp difference in an
    operand still moves a weight by a few percent; V is kept at unit scale
    so that this stays inside the bar)."""
    B, L, h_q, h_kv, d = shape
    note(f"prefill bf16 large scores {shape} sigma={sigma} boosted={boosted}")
    w = Workload("t", "test", "prefill", B, L, h_q, h_kv, d, "bf16", 300 + L, sigma,
                 boosted_rows=boosted)
    q, k, v = gen_prefill(w)
    v = bf16_round(v / np.float32(sigma))   # large scores, unit-scale values
    o = gqa.prefill(dev(q, torch.bfloat16), dev(k, torch.bfloat16), dev(v, torch.bfloat16))
    torch.cuda.synchronize()
    got = host(o)
    want = oracle.prefill(q, k, v)
    assert np.all(np.isfinite(got))
    rel = float(np.linalg.norm(got - want) / np.linalg.norm(want))
    note(f"  vs oracle: max-abs {np.abs(got - want).max():.3e} rel-L2 {rel:.3e}")
    assert rel <= TOL_BF16_REL
    assert_parity(got, attend_rounded_operands(q, k, v), torch.bfloat16,
                  f"prefill bf16 {shape} sigma={sigma} boosted={boosted} (rounded operands)")


def test_prefill_bf16_noncausal_and_bf16_out():
    B, L, h_q, h_kv, d = 2, 200, 14, 2, 128
    q, k, v = small_case(B, L, h_q, h_kv, d, torch.bfloat16, 7)
    qd, kd, vd = (dev(x, torch.bfloat16) for x in (q, k, v))
    o = gqa.prefill(qd, kd, vd, causal=False)
    ob = gqa.prefill(qd, kd, vd, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert_parity(host(o), oracle.prefill(q, k, v, causal=False), torch.bfloat16, "non-causal")
    assert ob.dtype == torch.bfloat16
    assert_parity(host(ob), oracle.prefill(q, k, v), torch.bfloat16, "bf16 output")


@pytest.mark.parametrize("shape", [(2, 77, 6, 2, 128), (1, 200, 14, 2, 64), (1, 5, 4, 4, 64),
                                   (1, 290, 8, 1, 128), (3, 17, 4, 2, 64)])
def test_prefill_f32_small(shape):
    """Causal and full attention, fp32 and bf16 output; the shapes cover one
    to five key tiles with ragged tails, partial 16-position row blocks, and
    rows whose later key quarters see no key."""
    B, L, h_q, h_kv, d = shape
    note(f"prefill f32 {shape}")
    q, k, v = small_case(B, L, h_q, h_kv, d, torch.float32, 200 + L)
    qd, kd, vd = (dev(x, torch.float32) for x in (q, k, v))
    o = gqa.prefill(qd, kd, vd)
    on = gqa.prefill(qd, kd, vd, causal=False)
    ob = gqa.prefill(qd, kd, vd, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    want = oracle.prefill(q, k, v)
    assert_parity(host(o), want, torch.float32, f"prefill f32 {shape}")
    assert_parity(host(on), oracle.prefill(q, k, v, causal=False), torch.float32, "non-causal")
    assert ob.dtype == torch.bfloat16
    assert_parity(host(ob), want, torch.bfloat16, "bf16 output")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_prefill_writes_cache_and_decode_continues(dtype):
    """Prefill writes rotated K and V into the cache; a decode step over that
    cache at the last position equals the last prefill row."""
    B, L, h_q, h_kv, d, cap = 2, 150, 14, 2, 128, 200
    q, k, v = small_case(B, L, h_q, h_kv, d, dtype, 5)
    kc = torch.full((B, cap, h_kv, d), 7.0, dtype=dtype, device="cuda")
    vc = torch.full((B, cap, h_kv, d), 7.0, dtype=dtype, device="cuda")
    qd = dev(q, dtype)
    gqa.prefill(qd, dev(k, dtype), dev(v, dtype), k_cache=kc, v_cache=vc)
    torch.cuda.synchronize()
    kr = oracle.rope(k, np.arange(L))
    tol = 1e-6 if dtype == torch.float32 else 2.0 ** -8
    assert np.all(np.abs(host(kc[:, :L]) - kr) <= np.abs(kr) * tol + 1e-5)
    np.testing.assert_array_equal(host(vc[:, :L]), v)
    assert torch.all(kc[:, L:] == 7.0) and torch.all(vc[:, L:] == 7.0)
    od = gqa.decode(qd[:, L - 1].contiguous(), kc, vc, kv_len=L, q_pos=L - 1)
    torch.cuda.synchronize()
    assert_parity(host(od), oracle.prefill(q, k, v)[:, L - 1], dtype, "decode = last prefill row")


# -------------------------------------------------------- decode, small --

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape", [(3, 2500, 2600, 28, 4, 128), (2, 1, 5, 14, 2, 64),
                                   (1, 1024, 1024, 16, 2, 128), (2, 700, 800, 8, 8, 64),
                                   (1, 300, 301, 40, 2, 128)],
                         ids=lambda s: "B%d_kv%d_qpos%d_%d/%d_d%d" % s)
def test_decode_small(dtype, shape):
    B, kv_len, q_pos, h_q, h_kv, d = shape
    note(f"decode {dtype} {shape}")
    cap = kv_len + 37
    w = Workload("t", "t", "decode", B, cap, h_q, h_kv, d,
                 "bf16" if dtype == torch.bfloat16 else "f32", 300 + kv_len)
    qh = gen_decode_query(w)
    kc = np.stack([gen_decode_cache_b(w, b)[0] for b in range(B)])
    vc = np.stack([gen_decode_cache_b(w, b)[1] for b in range(B)])
    kc[:, kv_len:] = 1e4   # rows past kv_len must not be read into the result
    o = gqa.decode(dev(qh, dtype), dev(kc, dtype), dev(vc, dtype), kv_len=kv_len, q_pos=q_pos)
    ob = gqa.decode(dev(qh, dtype), dev(kc, dtype), dev(vc, dtype), kv_len=kv_len, q_pos=q_pos,
                    out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    want = oracle.decode(qh, kc, vc, kv_len, q_pos)
    assert_parity(host(o), want, dtype, f"decode {shape}")
    if dtype == torch.bfloat16:
        assert_parity(host(ob), want, dtype, "decode bf16 out")


# ----------------------------------------------- full-size workloads -----

def sample_rows(w, n=48):
    rng = np.random.default_rng([w.seed, 99])
    rows = {(0, 0, 0), (w.B - 1, w.L - 1, w.h_q - 1), (0, w.L - 1, 0), (0, 63, w.g - 1),
            (0, 64, w.g), (w.B - 1, w.L // 2, w.h_q // 2)}
    while len(rows) < n:
        rows.add((int(rng.integers(w.B)), int(rng.integers(w.L)), int(rng.integers(w.h_q))))
    if w.boosted_rows:
        for t in (0, w.h_q - 1):
            for i in scaled_rows(w.seed, 0, t, w.L, w.boosted_rows)[:2]:
                rows.add((0, int(i), t))
        for u in range(w.h_kv):
            for i in scaled_rows(w.seed, 1, u, w.L, w.boosted_rows)[:2]:
                rows.add((0, min(int(i) + 1, w.L - 1), u * w.g))
    return sorted(rows)


@pytest.mark.parametrize("key", ["c1", "c2", "c4", "c5"])
def test_prefill_workload(key):
    w = WORKLOADS[key]
    note(f"workload {key} {w.name}: B{w.B} L{w.L} {w.h_q}/{w.h_kv} d{w.d} {w.dtype}")
    q, k, v = gen_prefill(w)
    dtype = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    qd, kd, vd = (dev(x, dtype) for x in (q, k, v))
    o = gqa.prefill(qd, kd, vd)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all())
    if key == "c1":
        assert_parity(host(o), oracle.prefill(q, k, v), dtype, key)
        return
    rows = sample_rows(w)
    got = np.stack([o[b, i, t].double().cpu().numpy() for b, i, t in rows])
    want = oracle.prefill_rows(q, k, v, rows)
    assert_parity(got, want, dtype, f"{key} ({len(rows)} sampled rows)")


def test_decode_workload():
    w = WORKLOADS["c3"]
    note(f"workload c3 {w.name}: B{w.B} cache {w.L} {w.h_q}/{w.h_kv} d{w.d}")
    qh = gen_decode_query(w)
    kc = torch.empty((w.B, w.L, w.h_kv, w.d), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    check_b = (0, 17, w.B - 1)
    host_cache = {}
    for b in range(w.B):
        kb, vb = gen_decode_cache_b(w, b)
        kc[b].copy_(torch.from_numpy(kb))
        vc[b].copy_(torch.from_numpy(vb))
        if b in check_b:
            host_cache[b] = (kb, vb)
    o = gqa.decode(dev(qh, torch.bfloat16), kc, vc, kv_len=w.L, q_pos=w.q_pos)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all())
    for b in check_b:
        kb, vb = host_cache[b]
        want = oracle.decode(qh[b:b + 1], kb[None], vb[None], w.L, w.q_pos)[0]
        assert_parity(host(o[b]), want, torch.bfloat16, f"c3 batch {b}")


def test_stream_read_runs():
    """The benchmark's streaming-read helper reads a buffer and leaves the
    sink alone for data whose XOR is not its marker value."""
    x = torch.ones(1 << 20, dtype=torch.bfloat16, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    gqa.stream_read(x, sink)
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0
