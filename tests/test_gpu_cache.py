"""GPU parity of the autoregressive entry points: KV append at decode,
ragged per-sequence lengths and positions, and chunked prefill against the
cache, through the C ABI, against the fp64 oracle.

Inputs are seeded N(0, 1) (bf16-rounded where the dtype is bf16).  The
cache rows that exist before a call are the oracle's rotated K (rounded to
the cache dtype) and the V rows, so both sides start from the same bytes.

Tolerances as for the one-shot calls: fp32 max-abs <= 1e-4; bf16 max-abs
<= 2e-2 and relative L2 <= 1e-2.  A K row the library rotates and rounds to
bf16 is within half an ulp of the exact rotation plus the fp32 rotation's
own absolute error.
"""

import numpy as np
import pytest
import torch

import oracle
import rope_causal_grouped_amd as gqa
from synthetic import Workload, gen_prefill
from tests.test_gpu_parity import assert_parity, dev, host, note

pytestmark = pytest.mark.gpu


def inputs(B, L, h_q, h_kv, d, dtype, seed):
    w = Workload("t", "test", "prefill", B, L, h_q, h_kv, d,
                 "bf16" if dtype == torch.bfloat16 else "f32", seed, 1.0)
    return gen_prefill(w)


def rounded(x, dtype):
    """x as the cache dtype stores it (bf16: round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype).double().numpy()


def prefilled_cache(k, v, n_rows, cap, dtype, fill=3.0):
    """Cache [B, cap, h_kv, d] whose rows < n_rows[b] hold the rotated K and
    the V of positions 0 .. n_rows[b]-1; later rows hold `fill`."""
    B, _, h_kv, d = k.shape
    kc = np.full((B, cap, h_kv, d), fill)
    vc = np.full((B, cap, h_kv, d), fill)
    kr = oracle.rope(k, np.arange(k.shape[1]))
    for b in range(B):
        n = int(n_rows[b])
        kc[b, :n] = kr[b, :n]
        vc[b, :n] = v[b, :n]
    return rounded(kc, dtype), rounded(vc, dtype)


def assert_rotated_rows(got, want, dtype, what):
    if np.size(got) == 0:
        return
    if dtype == torch.float32:
        assert np.max(np.abs(got - want)) <= 1e-5, what
    else:
        assert np.all(np.abs(got - want) <= np.abs(want) * 2.0 ** -8 + 1e-5), what


# ------------------------------------------------------------ decode -----

@pytest.mark.parametrize("dtype,heads", [(torch.bfloat16, (28, 4, 128)),
                                         (torch.bfloat16, (40, 2, 128)),
                                         (torch.float32, (14, 2, 64))],
                         ids=["bf16_28_4", "bf16_g20", "f32_14_2"])
def test_decode_append_ragged(dtype, heads):
    h_q, h_kv, d = heads
    pos = np.array([0, 1, 1023, 1024, 2500])
    B, cap = len(pos), 2600
    note(f"decode_append {dtype} {heads} pos={pos.tolist()}")
    q, k, v = inputs(B, cap, h_q, h_kv, d, dtype, 31)
    kc, vc = prefilled_cache(k, v, pos, cap, dtype)
    qn = np.stack([q[b, pos[b]] for b in range(B)])
    kn = np.stack([k[b, pos[b]] for b in range(B)])
    vn = np.stack([v[b, pos[b]] for b in range(B)])
    kcd, vcd = dev(kc, dtype), dev(vc, dtype)
    o = gqa.decode_append(dev(qn, dtype), dev(kn, dtype), dev(vn, dtype), kcd, vcd,
                          torch.tensor(pos, dtype=torch.int64), max_pos=int(pos.max()))
    torch.cuda.synchronize()
    want, kc_want, vc_want = oracle.decode_append(qn, kn, vn, kc, vc, pos)
    assert_parity(host(o), want, dtype, "decode_append")
    kc_got, vc_got = host(kcd), host(vcd)
    for b in range(B):
        p = int(pos[b])
        assert_rotated_rows(kc_got[b, p], kc_want[b, p], dtype, f"appended K row {b}")
        assert np.array_equal(vc_got[b, p], rounded(vn[b], dtype)), f"appended V row {b}"
    keep = np.ones((B, cap), bool)
    keep[np.arange(B), pos] = False
    assert np.array_equal(kc_got[keep], kc[keep]) and np.array_equal(vc_got[keep], vc[keep]), \
        "rows other than pos[b] changed"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_decode_ragged(dtype):
    h_q, h_kv, d = (28, 4, 128) if dtype == torch.bfloat16 else (14, 2, 64)
    # lengths on both sides of the chunk boundaries (1024 keys per fp32
    # chunk, 2048 per bf16 chunk)
    kv_len = np.array([1, 1024, 1025, 3000, 77, 2048, 2049])
    q_pos = np.array([0, 1023, 5000, 2999, 200, 2047, 2100])
    B, cap = len(kv_len), 3000
    note(f"decode_ragged {dtype} kv_len={kv_len.tolist()}")
    q, k, v = inputs(B, cap, h_q, h_kv, d, dtype, 32)
    kc, vc = prefilled_cache(k, v, np.full(B, cap), cap, dtype)
    o = gqa.decode_ragged(dev(q[:, 0], dtype), dev(kc, dtype), dev(vc, dtype),
                          torch.tensor(kv_len), torch.tensor(q_pos), max_kv_len=cap)
    torch.cuda.synchronize()
    assert_parity(host(o), oracle.decode_ragged(q[:, 0], kc, vc, kv_len, q_pos), dtype,
                  "decode_ragged")


def test_decode_ragged_matches_scalar_decode():
    """A ragged call whose sequences share one length equals gqa_decode."""
    B, cap, h_q, h_kv, d = 4, 1500, 28, 4, 128
    q, k, v = inputs(B, cap, h_q, h_kv, d, torch.bfloat16, 33)
    kc, vc = prefilled_cache(k, v, np.full(B, cap), cap, torch.bfloat16)
    qd, kcd, vcd = dev(q[:, 0], torch.bfloat16), dev(kc, torch.bfloat16), dev(vc, torch.bfloat16)
    a = gqa.decode(qd, kcd, vcd, 1300, 1400)
    b = gqa.decode_ragged(qd, kcd, vcd, [1300] * B, [1400] * B)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_decode_invalid_sequence_is_nan():
    """Entries that break the stated conditions give NaN rows for that
    sequence only, and an appending step then leaves its cache rows alone."""
    B, cap, h_q, h_kv, d = 3, 512, 28, 4, 128
    q, k, v = inputs(B, cap, h_q, h_kv, d, torch.bfloat16, 34)
    kc, vc = prefilled_cache(k, v, np.full(B, 300), cap, torch.bfloat16)
    kcd, vcd = dev(kc, torch.bfloat16), dev(vc, torch.bfloat16)
    qd = dev(q[:, 0], torch.bfloat16)
    # kv_len beyond max_kv_len, kv_len after the query's position
    o = gqa.decode_ragged(qd, kcd, vcd, [100, 400, 50], [99, 500, 10], max_kv_len=300)
    pos = np.array([299, 511, -1])   # valid, beyond max_pos, negative
    kn, vn = dev(k[:, 0], torch.bfloat16), dev(v[:, 0], torch.bfloat16)
    oa = gqa.decode_append(qd, kn, vn, kcd, vcd, torch.tensor(pos), max_pos=400)
    torch.cuda.synchronize()
    o, oa = host(o), host(oa)
    assert np.all(np.isfinite(o[0])) and np.all(np.isnan(o[1])) and np.all(np.isnan(o[2]))
    assert np.all(np.isfinite(oa[0])) and np.all(np.isnan(oa[1])) and np.all(np.isnan(oa[2]))
    kc_got = host(kcd)
    assert np.array_equal(kc_got[1:], kc[1:]), "an invalid sequence's cache was written"
    assert not np.array_equal(kc_got[0, 299], kc[0, 299])


# ----------------------------------------------------- chunked prefill ---

@pytest.mark.parametrize("dtype,heads,odt", [(torch.bfloat16, (28, 4, 128), torch.float32),
                                             (torch.bfloat16, (16, 2, 64), torch.float32),
                                             (torch.bfloat16, (16, 2, 64), torch.bfloat16),
                                             (torch.float32, (14, 2, 64), torch.float32)],
                         ids=["bf16_28_4", "bf16_d64_g8", "bf16_d64_g8_bf16out", "f32_14_2"])
def test_prefill_chunk_ragged(dtype, heads, odt):
    h_q, h_kv, d = heads
    start = np.array([0, 300, 1000, 64])
    length = np.array([200, 1, 137, 0])
    B, C, cap = len(start), 200, 1400
    note(f"prefill_chunk {dtype} {heads} start={start.tolist()} len={length.tolist()}")
    q, k, v = inputs(B, cap, h_q, h_kv, d, dtype, 35)
    kc, vc = prefilled_cache(k, v, start, cap, dtype)
    qc = np.zeros((B, C, h_q, d)); kn = np.zeros((B, C, h_kv, d)); vn = np.zeros_like(kn)
    for b in range(B):
        s0, n = int(start[b]), int(length[b])
        qc[b, :n], kn[b, :n], vn[b, :n] = q[b, s0:s0 + n], k[b, s0:s0 + n], v[b, s0:s0 + n]
    kcd, vcd = dev(kc, dtype), dev(vc, dtype)
    out = torch.full((B, C, h_q, d), 5.0, device="cuda", dtype=odt)
    gqa.prefill_chunk(dev(qc, dtype), dev(kn, dtype), dev(vn, dtype), kcd, vcd,
                      torch.tensor(start), torch.tensor(length), kend=1200, out=out)
    torch.cuda.synchronize()
    kc_want, vc_want = oracle.cache_append(kc, vc, kn, vn, start, length)
    want = oracle.prefill_chunk(qc, kc_want, vc_want, start, length)
    got = host(out)
    rows = np.zeros((B, C), bool)
    for b in range(B):
        rows[b, :length[b]] = True
    assert_parity(got[rows], want[rows], dtype, "prefill_chunk rows")
    assert np.all(got[~rows] == 5.0), "rows past len[b] were written"
    kc_got = host(kcd)
    for b in range(B):
        s0, n = int(start[b]), int(length[b])
        assert_rotated_rows(kc_got[b, s0:s0 + n], kc_want[b, s0:s0 + n], dtype, f"K rows {b}")
        assert np.array_equal(kc_got[b, :s0], kc[b, :s0])
        assert np.array_equal(kc_got[b, s0 + n:], kc[b, s0 + n:])


def test_prefill_chunk_fp16_range_gives_nan_rows():
    """The chunk path has the fp16 score-operand range of gqa_prefill: a
    cached rotated K element of magnitude 2^14 or more turns the rows of its
    group that see it into NaN, a query element past the range its own row;
    every other row matches the oracle."""
    B, cap, h_q, h_kv, d = 1, 300, 28, 4, 128
    dtype = torch.bfloat16
    start, length, C = np.array([200]), np.array([100]), 100
    q, k, v = inputs(B, cap, h_q, h_kv, d, dtype, 39)
    kc, vc = prefilled_cache(k, v, start, cap, dtype)
    kc[0, 150, 1, :] = 40000.0          # cached (rotated) key of group 1, position 150
    qc, kn, vn = q[:, 200:300].copy(), k[:, 200:300].copy(), v[:, 200:300].copy()
    qc[0, 10, 5, :] = 200000.0          # position 210, head 5 (group 0)
    out = torch.full((B, C, h_q, d), 5.0, device="cuda")
    gqa.prefill_chunk(dev(qc, dtype), dev(kn, dtype), dev(vn, dtype), dev(kc, dtype),
                      dev(vc, dtype), torch.tensor(start), torch.tensor(length), kend=cap,
                      out=out)
    torch.cuda.synchronize()
    got = host(out)[0]
    g = h_q // h_kv
    assert np.all(np.isnan(got[:, g:2 * g])), "group 1 rows see the large key"
    assert np.all(np.isnan(got[10, 5])), "the large query row"
    kc_want, vc_want = oracle.cache_append(kc, vc, kn, vn, start, length)
    want = oracle.prefill_chunk(qc, kc_want, vc_want, start, length)[0]
    keep = np.ones((C, h_q), bool)
    keep[:, g:2 * g] = False
    keep[10, 5] = False
    assert np.all(np.isfinite(got[keep]))
    assert_parity(got[keep], want[keep], dtype, "chunk rows outside the large entries")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_chunks_equal_one_shot_prefill(dtype):
    """Three chunks through the cache give the rows and the cache of one
    gqa_prefill call over the whole prompt."""
    B, L, h_q, h_kv, d = 2, 700, 28, 4, 128
    if dtype == torch.float32:
        h_q, h_kv, d = 14, 2, 64
    note(f"chunks vs one-shot {dtype}")
    q, k, v = inputs(B, L, h_q, h_kv, d, dtype, 36)
    qd, kd, vd = dev(q, dtype), dev(k, dtype), dev(v, dtype)
    cap = 768
    kc1 = torch.zeros((B, cap, h_kv, d), dtype=dtype, device="cuda")
    vc1 = torch.zeros_like(kc1)
    one = gqa.prefill(qd, kd, vd, k_cache=kc1, v_cache=vc1)
    kc2 = torch.zeros_like(kc1)
    vc2 = torch.zeros_like(kc1)
    parts = []
    for s0, n in ((0, 256), (256, 256), (512, 188)):
        parts.append(gqa.prefill_chunk(qd[:, s0:s0 + n].contiguous(), kd[:, s0:s0 + n].contiguous(),
                                       vd[:, s0:s0 + n].contiguous(), kc2, vc2, [s0] * B,
                                       kend=L))
    torch.cuda.synchronize()
    chunked = torch.cat(parts, dim=1)
    assert torch.equal(kc1, kc2) and torch.equal(vc1, vc2), "caches differ"
    assert_parity(host(chunked), host(one), dtype, "chunked vs one-shot")
    assert_parity(host(chunked), oracle.prefill(q, k, v), dtype, "chunked vs oracle")


def test_prefill_chunk_invalid_sequence_is_nan():
    B, C, h_q, h_kv, d, cap = 2, 64, 28, 4, 128, 256
    q, k, v = inputs(B, C, h_q, h_kv, d, torch.bfloat16, 37)
    kc = torch.zeros((B, cap, h_kv, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    o = gqa.prefill_chunk(dev(q, torch.bfloat16), dev(k, torch.bfloat16), dev(v, torch.bfloat16),
                          kc, vc, [0, 150], kend=200)   # 150 + 64 > 200
    torch.cuda.synchronize()
    o = host(o)
    assert np.all(np.isfinite(o[0])) and np.all(np.isnan(o[1]))
    assert torch.count_nonzero(kc[1]) == 0 and torch.count_nonzero(kc[0, :C]) > 0


# ------------------------------------------------------ QKV epilogue -----

def packed(B, C, h_q, h_kv, d, dtype, seed):
    """Packed projection output [B, C, (h_q + 2 h_kv) d] and a bias vector."""
    rng = np.random.default_rng([seed, 9])
    width = (h_q + 2 * h_kv) * d
    x = rounded(rng.standard_normal((B, C, width), dtype=np.float32), dtype)
    bias = rounded(0.5 * rng.standard_normal(width, dtype=np.float32), dtype)
    return x, bias


@pytest.mark.parametrize("dtype,heads", [(torch.bfloat16, (28, 4, 128)),
                                         (torch.float32, (14, 2, 64))],
                         ids=["bf16_28_4", "f32_14_2"])
def test_qkv_epilogue(dtype, heads):
    h_q, h_kv, d = heads
    B, C, cap = 3, 100, 700
    start, length = np.array([0, 500, 37]), np.array([100, 50, 0])
    note(f"qkv_epilogue {dtype} {heads}")
    x, bias = packed(B, C, h_q, h_kv, d, dtype, 40)
    kc0 = np.full((B, cap, h_kv, d), 2.0)
    vc0 = np.full((B, cap, h_kv, d), -2.0)
    kcd, vcd = dev(kc0, dtype), dev(vc0, dtype)
    q_out = torch.full((B, C, h_q, d), 9.0, dtype=dtype, device="cuda")
    gqa.qkv_epilogue(dev(x, dtype), dev(bias, dtype), kcd, vcd, h_q, torch.tensor(start),
                     torch.tensor(length), kend=650, q_out=q_out)
    torch.cuda.synchronize()
    q_want, kc_want, vc_want = oracle.qkv_epilogue(x, bias, kc0, vc0, h_q, h_kv, start, length)
    qg, kg, vg = host(q_out), host(kcd), host(vcd)
    for b in range(B):
        s0, n = int(start[b]), int(length[b])
        assert_rotated_rows(qg[b, :n], q_want[b, :n], dtype, f"q rows {b}")
        assert np.all(qg[b, n:] == 9.0), "q rows past len[b] were written"
        assert_rotated_rows(kg[b, s0:s0 + n], kc_want[b, s0:s0 + n], dtype, f"K rows {b}")
        assert_rotated_rows(vg[b, s0:s0 + n], vc_want[b, s0:s0 + n], dtype, f"V rows {b}")
        assert np.all(kg[b, :s0] == 2.0) and np.all(kg[b, s0 + n:] == 2.0)
        assert np.all(vg[b, :s0] == -2.0) and np.all(vg[b, s0 + n:] == -2.0)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_epilogue_then_attention(dtype):
    """Prompt: epilogue, then a chunk that attends to the rows it cached;
    next token: epilogue at position L, then a ragged decode over L + 1 rows."""
    h_q, h_kv, d = (28, 4, 128) if dtype == torch.bfloat16 else (14, 2, 64)
    B, L, cap = 2, 333, 400
    note(f"epilogue + attention {dtype}")
    x, bias = packed(B, L + 1, h_q, h_kv, d, dtype, 41)
    kcd = torch.zeros((B, cap, h_kv, d), dtype=dtype, device="cuda")
    vcd = torch.zeros_like(kcd)
    xd, bd = dev(x, dtype), dev(bias, dtype)
    qp = gqa.qkv_epilogue(xd[:, :L].contiguous(), bd, kcd, vcd, h_q, [0] * B)
    o = gqa.prefill_chunk(qp, None, None, kcd, vcd, [0] * B, kend=L, q_rotated=True)
    qn = gqa.qkv_epilogue(xd[:, L:].contiguous(), bd, kcd, vcd, h_q, [L] * B)
    od = gqa.decode_ragged(qn[:, 0].contiguous(), kcd, vcd, [L + 1] * B, [L] * B,
                           q_rotated=True)
    torch.cuda.synchronize()
    z = np.zeros((B, cap, h_kv, d))
    q_all, kc, vc = oracle.qkv_epilogue(x, bias, z, z, h_q, h_kv, 0)
    assert_parity(host(o), oracle.prefill_chunk(q_all[:, :L], kc, vc, 0, q_rotated=True), dtype,
                  "epilogue + chunk")
    assert_parity(host(od), oracle.decode_ragged(q_all[:, L], kc, vc, L + 1, L, q_rotated=True),
                  dtype, "epilogue + decode")


# --------------------------------------------------------- paged cache ---

def to_pages(kc, page_size, num_pages, seed, poison=4096.0):
    """Scatter a contiguous cache [B, cap, h_kv, d] into a page pool under a
    shuffled block table; unused pages hold `poison` (exact in bf16)."""
    B, cap, h_kv, d = kc.shape
    per_seq = -(-cap // page_size)
    perm = np.random.default_rng(seed).permutation(num_pages)[:B * per_seq].reshape(B, per_seq)
    pool = np.full((num_pages, h_kv, page_size, d), poison)
    for b in range(B):
        for n in range(per_seq):
            rows = kc[b, n * page_size:(n + 1) * page_size]
            pool[perm[b, n], :, :rows.shape[0]] = np.transpose(rows, (1, 0, 2))
    return pool, perm.astype(np.int32)


@pytest.mark.parametrize("dtype,page_size,heads",
                         [(torch.bfloat16, 16, (28, 4, 128)), (torch.bfloat16, 256, (28, 4, 128)),
                          (torch.bfloat16, 32, (64, 8, 128)), (torch.float32, 64, (14, 2, 64))],
                         ids=["bf16_ps16", "bf16_ps256", "bf16_ps32_72b_heads", "f32_ps64"])
def test_decode_paged(dtype, page_size, heads):
    h_q, h_kv, d = heads
    kv_len = np.array([1, 1024, 1025, 3000])
    q_pos = np.array([0, 1500, 1024, 2999])
    B, cap = len(kv_len), 3072
    num_pages = B * (cap // page_size) + 7
    note(f"decode_paged {dtype} page_size={page_size}")
    q, k, v = inputs(B, cap, h_q, h_kv, d, dtype, 42)
    kc, vc = prefilled_cache(k, v, np.full(B, cap), cap, dtype)
    kp, bt = to_pages(kc, page_size, num_pages, 1)
    vp, _ = to_pages(vc, page_size, num_pages, 1)
    kpd, vpd, btd = dev(kp, dtype), dev(vp, dtype), torch.from_numpy(bt).cuda()
    o = gqa.decode_paged(dev(q[:, 0], dtype), kpd, vpd, btd, torch.tensor(q_pos),
                         torch.tensor(kv_len))
    oc = gqa.decode_ragged(dev(q[:, 0], dtype), dev(kc, dtype), dev(vc, dtype),
                           torch.tensor(kv_len), torch.tensor(q_pos))
    torch.cuda.synchronize()
    assert_parity(host(o), oracle.decode_paged(q[:, 0], kp, vp, bt, page_size, kv_len, q_pos),
                  dtype, "decode_paged")
    assert torch.equal(o, oc), "paged and contiguous decode differ"


def test_decode_paged_append():
    dtype, page_size = torch.bfloat16, 32
    h_q, h_kv, d = 28, 4, 128
    pos = np.array([0, 31, 32, 2000])
    B, cap = len(pos), 2048
    num_pages = B * (cap // page_size) + 3
    note("decode_paged append")
    q, k, v = inputs(B, cap, h_q, h_kv, d, dtype, 43)
    kc, vc = prefilled_cache(k, v, pos, cap, dtype)
    kp, bt = to_pages(kc, page_size, num_pages, 2)
    vp, _ = to_pages(vc, page_size, num_pages, 2)
    qn = np.stack([q[b, pos[b]] for b in range(B)])
    kn = np.stack([k[b, pos[b]] for b in range(B)])
    vn = np.stack([v[b, pos[b]] for b in range(B)])
    kpd, vpd = dev(kp, dtype), dev(vp, dtype)
    o = gqa.decode_paged(dev(qn, dtype), kpd, vpd, torch.from_numpy(bt).cuda(), torch.tensor(pos),
                         k_new=dev(kn, dtype), v_new=dev(vn, dtype), max_kv_len=cap)
    torch.cuda.synchronize()
    kp_want, vp_want = oracle.paged_append(kp, vp, kn, vn, bt, page_size, pos)
    want = oracle.decode_paged(qn, kp_want, vp_want, bt, page_size, pos + 1, pos)
    assert_parity(host(o), want, dtype, "decode_paged append")
    kg = host(kpd)
    for b in range(B):
        page, row = bt[b, pos[b] // page_size], pos[b] % page_size
        assert_rotated_rows(kg[page, :, row], kp_want[page, :, row], dtype, f"appended K {b}")
        kg[page, :, row] = kp[page, :, row]
    assert np.array_equal(kg, kp), "pool rows other than the new tokens changed"


def test_decode_paged_bad_page_is_nan():
    dtype, page_size = torch.bfloat16, 64
    B, cap, h_q, h_kv, d = 2, 512, 28, 4, 128
    q, k, v = inputs(B, cap, h_q, h_kv, d, dtype, 44)
    kc, vc = prefilled_cache(k, v, np.full(B, cap), cap, dtype)
    kp, bt = to_pages(kc, page_size, 20, 3)
    vp, _ = to_pages(vc, page_size, 20, 3)
    bt[1, 5] = 99    # beyond the pool
    o = gqa.decode_paged(dev(q[:, 0], dtype), dev(kp, dtype), dev(vp, dtype),
                         torch.from_numpy(bt).cuda(), [511, 511], [512, 512])
    torch.cuda.synchronize()
    o = host(o)
    assert np.all(np.isfinite(o[0])) and np.all(np.isnan(o[1]))


# --------------------------------------------------------------- YaRN ----

@pytest.fixture
def yarn_4x():
    """Qwen2's long-context setting for the test's calls, reset afterwards."""
    gqa.set_rope_yarn(4.0, 32768.0, 32.0, 1.0)
    try:
        yield oracle.YaRN(theta=1.0e6, factor=4.0, original_max_position=32768.0)
    finally:
        gqa.set_rope_yarn(1.0)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_yarn_rope_apply(yarn_4x, dtype):
    q, _, _ = inputs(2, 37, 3, 3, 128, dtype, 45)
    x = dev(q, dtype)
    gqa.rope_apply(x, pos0=100000)
    torch.cuda.synchronize()
    assert_rotated_rows(host(x), oracle.rope(q, np.arange(100000, 100037), yarn_4x), dtype,
                        "YaRN rope")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_yarn_prefill_and_decode(yarn_4x, dtype):
    h_q, h_kv, d = (28, 4, 128) if dtype == torch.bfloat16 else (14, 2, 64)
    B, L = 2, 700
    note(f"YaRN prefill + decode {dtype}")
    q, k, v = inputs(B, L, h_q, h_kv, d, dtype, 46)
    qd, kd, vd = dev(q, dtype), dev(k, dtype), dev(v, dtype)
    kc = torch.zeros((B, L + 40000, h_kv, d), dtype=dtype, device="cuda")
    vc = torch.zeros_like(kc)
    o = gqa.prefill(qd, kd, vd, k_cache=kc, v_cache=vc)
    on = gqa.prefill(qd, kd, vd)   # no cache copy: another K path for fp32
    od = gqa.decode(qd[:, -1].contiguous(), kc, vc, kv_len=L, q_pos=L + 39000)
    torch.cuda.synchronize()
    want = oracle.prefill(q, k, v, theta=yarn_4x)
    assert_parity(host(o), want, dtype, "YaRN prefill")
    assert_parity(host(on), want, dtype, "YaRN prefill without a cache")
    kc_h, vc_h = host(kc), host(vc)
    assert_rotated_rows(kc_h[:, :L], oracle.rope(k, np.arange(L), yarn_4x), dtype, "YaRN cache")
    assert_parity(host(od), oracle.decode(q[:, -1], kc_h, vc_h, L, L + 39000, theta=yarn_4x),
                  dtype, "YaRN decode far past the cache")


def test_yarn_chunk_past_512_key_tiles(yarn_4x):
    """A bf16 chunk at the end of a 40960-position sequence (YaRN 4x, past
    the 32K window): the attention kernel walks 640 key tiles, more than one
    per thread of its workgroup, including the per-tile norm scan over all
    of them.  The whole chunk is compared."""
    L, C, h_q, h_kv, d = 40960, 256, 28, 4, 128
    s0 = L - C
    dtype = torch.bfloat16
    note(f"YaRN chunk at {s0}..{L - 1} over {L // 64} key tiles")
    q, k, v = inputs(1, L, h_q, h_kv, d, dtype, 48)
    kc = torch.zeros((1, L, h_kv, d), dtype=dtype, device="cuda")
    vc = torch.zeros_like(kc)
    kc[:, :s0].copy_(torch.from_numpy(k[:, :s0]))
    vc[:, :s0].copy_(torch.from_numpy(v[:, :s0]))
    gqa.rope_apply(kc[:, :s0])          # rows before the chunk: rotated K, as cached
    o = gqa.prefill_chunk(dev(q[:, s0:], dtype), dev(k[:, s0:], dtype), dev(v[:, s0:], dtype),
                          kc, vc, [s0], kend=L)
    torch.cuda.synchronize()
    g = h_q // h_kv
    want = np.concatenate([oracle.prefill_group_rows(q[0], k[0], v[0], u, s0, L,
                                                     theta=yarn_4x)
                           for u in range(h_kv)], axis=1)
    assert_parity(host(o)[0], want, dtype, f"YaRN chunk over {L // 64} key tiles")
    assert want.shape == (C, h_q, d) and g == 7
