"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Small shapes (several tiles, ragged tails, MHA/MQA/GQA, L = 1) are compared
element by element.  The five workloads at full size are compared over their
whole outputs in tests/test_gpu_workloads.py.

Tolerances: fp32 inputs max-abs <= 1e-4; bf16 inputs (fp32 accumulation)
max-abs <= 2e-2 and relative L2 <= 1e-2.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import rope_causal_grouped_amd as gqa
from synthetic import Workload, bf16_round, gen_decode_cache_b, gen_decode_query, gen_prefill

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


@pytest.mark.parametrize("pos0", [0, 32768 - 2048, (1 << 24) - 2048])
def test_rope_cos_sin_error_bound(pos0):
    """Unit vectors (1 in the first half of each pair, 0 in the second) come
    out of an fp32 rotation as (cos, sin) of pos * omega_j themselves; every
    value lies within 2.5e-7 (about two fp32 ulps at 1) of cos and sin taken
    in extended precision of the fp64 angle, at positions up to 2^24."""
    d, L = 128, 2048
    note(f"rope cos/sin bound pos0={pos0}")
    x = torch.zeros((1, L, 1, d), dtype=torch.float32, device="cuda")
    x[..., : d // 2] = 1.0
    gqa.rope_apply(x, pos0=pos0)
    torch.cuda.synchronize()
    got = x.cpu().numpy().astype(np.float64)[0, :, 0]
    j = np.arange(d // 2, dtype=np.float64)
    omega = np.float64(gqa.ROPE_THETA) ** (-2.0 * j / d)
    ang = np.longdouble(np.arange(pos0, pos0 + L, dtype=np.float64))[:, None] * np.longdouble(omega)
    err_c = np.abs(got[:, : d // 2] - np.cos(ang).astype(np.float64)).max()
    err_s = np.abs(got[:, d // 2:] - np.sin(ang).astype(np.float64)).max()
    note(f"  max error cos {err_c:.3e} sin {err_s:.3e}")
    assert err_c <= 2.5e-7 and err_s <= 2.5e-7


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


@pytest.mark.parametrize("shape", [(2, 2048, 28, 4, 128), (1, 3000, 16, 2, 64)],
                         ids=lambda s: "B%d_L%d_%d/%d_d%d" % s)
def test_prefill_shared_tail_repeated_calls(shape):
    """Shapes whose work lists have a shared tail (items taken through a
    ticket counter in the workspace): three calls in a row on one workspace,
    the output poisoned with NaN before each, give the same bits every time
    (the counter starts over each call and every item is done exactly
    once), and sampled rows match the oracle -- the last rows of each group
    among them, which sit in the tail."""
    B, L, h_q, h_kv, d = shape
    note(f"prefill shared tail {shape}")
    q, k, v = small_case(B, L, h_q, h_kv, d, torch.bfloat16, 77 + L)
    qd, kd, vd = (dev(x, torch.bfloat16) for x in (q, k, v))
    ws = torch.empty(gqa.prefill_workspace_size(torch.bfloat16, B, L, h_kv, d), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty((B, L, h_q, d), dtype=torch.float32, device="cuda")
    outs = []
    for _ in range(3):
        o.fill_(float("nan"))
        gqa.prefill(qd, kd, vd, out=o, workspace=ws)
        torch.cuda.synchronize()
        outs.append(o.clone())
    assert not torch.isnan(outs[0]).any(), "rows left unwritten"
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    rng = np.random.default_rng(5)
    rows = [(b, i, t) for b in range(B) for i in (0, 1, L // 2, L - 2, L - 1)
            for t in (0, h_q - 1)]
    rows += [(int(rng.integers(B)), int(rng.integers(L)), int(rng.integers(h_q)))
             for _ in range(24)]
    got = host(outs[0])
    want = oracle.prefill_rows(q, k, v, rows)
    assert_parity(np.stack([got[b, i, t] for b, i, t in rows]), want, torch.bfloat16,
                  f"shared tail {shape}")


@pytest.mark.parametrize("sigma,boosted", [(3.0, 0), (0.5, 12)], ids=["sigma3", "boosted"])
@pytest.mark.parametrize("shape", [(1, 333, 28, 4, 128), (2, 300, 14, 2, 64)],
                         ids=lambda s: "B%d_L%d_%d/%d_d%d" % s)
def test_prefill_bf16_large_scores(shape, sigma, boosted):
    """Score bounds past the 64 (log2) headroom: the kernel takes tile maxima
    first and shifts the scores by a nonzero reference.  With boosted rows
    (x8) only some rows of a wave need the shift, the rest keep m = 0.
    Logits reach ~70 (sigma 3); the score operands are rounded to fp16, so
    both bars hold against the exact oracle (V kept at unit scale).  12 of
    ~300 rows per head scaled by 8 is ~900 times the 32K workload's density
    of such rows; a CPU model of the kernel's roundings (fp16 Q' and K',
    bf16 P) gives 1.4e-2 max-abs here and 1.8e-2 at 24 rows, the edge of
    what fp16 score operands hold to 2e-2."""
    B, L, h_q, h_kv, d = shape
    note(f"prefill bf16 large scores {shape} sigma={sigma} boosted={boosted}")
    w = Workload("t", "test", "prefill", B, L, h_q, h_kv, d, "bf16", 300 + L, sigma,
                 boosted_rows=boosted)
    q, k, v = gen_prefill(w)
    v = bf16_round(v / np.float32(sigma))   # large scores, unit-scale values
    o = gqa.prefill(dev(q, torch.bfloat16), dev(k, torch.bfloat16), dev(v, torch.bfloat16))
    torch.cuda.synchronize()
    assert_parity(host(o), oracle.prefill(q, k, v), torch.bfloat16,
                  f"prefill bf16 {shape} sigma={sigma} boosted={boosted}")


def test_prefill_bf16_fp16_range_gives_nan_rows():
    """Score operands are fp16: a rotated K element, or a Q element times
    scale*log2(e), of magnitude 2^14 or more is outside their range.  The
    rows that would use it come out NaN (every row of the query's group that
    sees the key; the one query row), and all other rows are unaffected."""
    B, L, h_q, h_kv, d = 1, 200, 28, 4, 128
    q, k, v = small_case(B, L, h_q, h_kv, d, torch.bfloat16, 77)
    k[0, 150, 1, :] = 40000.0          # group 1, position 150
    q[0, 10, 5, :] = 200000.0          # 200000 * log2(e) / sqrt(128) > 2^14
    o = host(gqa.prefill(dev(q, torch.bfloat16), dev(k, torch.bfloat16),
                         dev(v, torch.bfloat16)))
    torch.cuda.synchronize()
    g = h_q // h_kv
    assert np.all(np.isnan(o[0, 150:, g:2 * g])), "rows that see the large key"
    assert np.all(np.isnan(o[0, 10, 5])), "the large query row"
    want = oracle.prefill(q, k, v)
    keep = np.ones((L, h_q), bool)
    keep[:, g:2 * g] = False            # group 1 (rows before 150 may share a workgroup)
    keep[10, 5] = False
    got = o[0][keep]
    assert np.all(np.isfinite(got))
    assert_parity(got, want[0][keep], torch.bfloat16, "rows outside the large entries")


@pytest.mark.parametrize("shape", [(2, 200, 14, 2, 128), (2, 203, 16, 2, 64)],
                         ids=lambda s: "B%d_L%d_%d/%d_d%d" % s)
def test_prefill_bf16_noncausal_and_bf16_out(shape):
    """Full attention, and bf16 output; O leaves the kernel in 128-byte row
    pieces staged through LDS (32 fp32 or 64 bf16 dims; at d = 64 in two
    passes of 16 rows), with a ragged last row block (203 * 8 rows)."""
    B, L, h_q, h_kv, d = shape
    note(f"prefill bf16 non-causal / bf16 out {shape}")
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
                                   (1, 300, 301, 40, 2, 128),
                                   # chunk boundaries (2048 keys per bf16 chunk, 1024 per
                                   # fp32 chunk): exactly one chunk, one key into the next
                                   (1, 2048, 2048, 28, 4, 128), (2, 2049, 2049, 28, 4, 128),
                                   (1, 4095, 5000, 14, 2, 64),
                                   # four KV groups per workgroup (h_kv a multiple of 4)
                                   # with two 16-head blocks per group (g = 20), and
                                   # with g = 8 over two workgroup rows of groups
                                   (1, 2100, 2101, 80, 4, 128), (2, 3000, 3000, 64, 8, 64)],
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


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_timing_bound_to_dispatches(dtype):
    """With timing on, every call records its main kernel and the whole call
    through events bound to its own dispatches; the outputs are the same
    bits as with timing off, and each call spans at least its main kernel."""
    B, L, h_q, h_kv, d = 2, 300, 14, 2, 128
    q, k, v = small_case(B, L, h_q, h_kv, d, dtype, 41)
    qd, kd, vd = dev(q, dtype), dev(k, dtype), dev(v, dtype)
    cap = L + 16
    kc = torch.zeros((B, cap, h_kv, d), dtype=dtype, device="cuda")
    vc = torch.zeros_like(kc)
    ref_p = gqa.prefill(qd, kd, vd, k_cache=kc, v_cache=vc)
    ref_d = gqa.decode(qd[:, L - 1].contiguous(), kc, vc, kv_len=L, q_pos=L - 1)
    torch.cuda.synchronize()
    gqa.timing_enable(True)
    outs = []
    for _ in range(3):
        outs.append((gqa.prefill(qd, kd, vd, k_cache=kc, v_cache=vc),
                     gqa.decode(qd[:, L - 1].contiguous(), kc, vc, kv_len=L, q_pos=L - 1)))
    torch.cuda.synchronize()
    gqa.timing_enable(False)
    t = [gqa.timing_read(w) for w in range(4)]
    note(f"timing {dtype}: {t}")
    for op, od in outs:
        assert torch.equal(op, ref_p) and torch.equal(od, ref_d)
    for w in range(4):
        assert t[w][1] == 3 and t[w][0] > 0.0, (w, t[w])
    assert t[2][0] >= t[0][0] and t[3][0] >= t[1][0]
    # records stay readable until timing is enabled again, which drops them
    assert gqa.timing_read(0) == t[0]
    gqa.timing_enable(True)
    gqa.timing_enable(False)
    assert gqa.timing_read(2) == (0.0, 0)


def test_stream_read_runs():
    """The benchmark's streaming-read helper reads a buffer and leaves the
    sink alone for data whose XOR is not its marker value."""
    x = torch.ones(1 << 20, dtype=torch.bfloat16, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    gqa.stream_read(x, sink)
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0
