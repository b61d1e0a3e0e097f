"""gqa_decode_noalloc (static per-GPU scratch, no workspace) against
gqa_decode (caller's workspace) through the C ABI: the same kernels on the
same chunk layout, so the outputs must agree bit for bit.  Two calls in a
row, the second smaller than the first, so the second reads scratch that the
first left behind; the small one is also held to the bf16/fp32 bars against
the fp64 oracle."""

import sys

import numpy as np
import pytest
import torch

import oracle
import rope_causal_grouped_amd as gqa
from synthetic import Workload, gen_decode_cache_b, gen_decode_query

pytestmark = pytest.mark.gpu


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device="cuda", dtype=dtype)


def small_inputs(B, cap, h_q, h_kv, d, dtype, seed):
    w = Workload("t", "t", "decode", B, cap, h_q, h_kv, d,
                 "bf16" if dtype == torch.bfloat16 else "f32", seed)
    qh = gen_decode_query(w)
    kc = np.stack([gen_decode_cache_b(w, b)[0] for b in range(B)])
    vc = np.stack([gen_decode_cache_b(w, b)[1] for b in range(B)])
    return qh, kc, vc


def both(q, kc, vc, kv_len, q_pos, out_dtype):
    B, h_q, d = q.shape
    want = gqa.decode(q, kc, vc, kv_len=kv_len, q_pos=q_pos, out_dtype=out_dtype)
    got = torch.full((B, h_q, d), float("nan"), dtype=out_dtype, device=q.device)
    gqa.decode_noalloc(q, kc, vc, kv_len=kv_len, q_pos=q_pos, out=got)
    torch.cuda.synchronize()
    return got, want


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noalloc_decode_equals_workspace_decode(dtype):
    # 1) the 7B decode step: B 32, cache 32768, 28/4 heads, d 128 (16 chunks
    #    per sequence in bf16, 32 in fp32: 7.5 / 14.9 MB of the 32 MiB scratch)
    B, cap, h_q, h_kv, d = 32, 32768, 28, 4, 128
    note(f"noalloc decode {dtype}: B{B} cache {cap} {h_q}/{h_kv} d{d}")
    g = torch.Generator(device="cuda").manual_seed(11)
    q = torch.randn((B, h_q, d), device="cuda", generator=g).to(dtype)
    kc = torch.randn((B, cap, h_kv, d), device="cuda", generator=g).to(dtype)
    vc = torch.randn((B, cap, h_kv, d), device="cuda", generator=g).to(dtype)
    for out_dtype in (torch.float32, torch.bfloat16):
        got, want = both(q, kc, vc, cap, cap, out_dtype)
        assert torch.isfinite(got.float()).all()
        assert torch.equal(got, want), f"large step, out {out_dtype}"
    del q, kc, vc
    torch.cuda.empty_cache()

    # 2) a smaller step right after (2 chunks in bf16, 3 in fp32; the scratch
    #    still holds the large step's states): equal to gqa_decode and within
    #    the bars
    B, kv_len, q_pos, h_q, h_kv, d = 3, 2500, 2600, 28, 4, 128
    note(f"noalloc decode {dtype}: B{B} kv {kv_len} qpos {q_pos} {h_q}/{h_kv} d{d}")
    qh, kch, vch = small_inputs(B, kv_len + 37, h_q, h_kv, d, dtype, 1300)
    q, kc, vc = dev(qh, dtype), dev(kch, dtype), dev(vch, dtype)
    got, want = both(q, kc, vc, kv_len, q_pos, torch.float32)
    assert torch.equal(got, want), "small step after the large one"
    ref = oracle.decode(qh, kch, vch, kv_len, q_pos)
    err = np.abs(got.double().cpu().numpy() - ref)
    rel = float(np.linalg.norm(got.double().cpu().numpy() - ref) / np.linalg.norm(ref))
    note(f"  small step vs oracle: max-abs {err.max():.3e} rel-L2 {rel:.3e}")
    if dtype == torch.float32:
        assert err.max() <= 1e-4
    else:
        assert err.max() <= 2e-2 and rel <= 1e-2

    # 3) smaller still (one chunk, d 64, MHA), bf16 output
    B, kv_len, q_pos, h_q, h_kv, d = 2, 700, 800, 8, 8, 64
    qh, kch, vch = small_inputs(B, kv_len, h_q, h_kv, d, dtype, 1700)
    got, want = both(dev(qh, dtype), dev(kch, dtype), dev(vch, dtype), kv_len, q_pos,
                     torch.bfloat16)
    assert torch.equal(got, want), "one-chunk step"


def test_noalloc_rejects_a_step_past_the_scratch():
    """A step whose chunk states exceed the static scratch is refused before
    anything is enqueued, with a message naming the limit."""
    B, cap, h_q, h_kv, d = 32, 1 << 18, 28, 4, 128     # 128 bf16 chunks: 59.6 MB of states
    q = torch.zeros((B, h_q, d), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((B, cap, h_kv, d), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((B, h_q, d), dtype=torch.float32, device="cuda")
    with pytest.raises(gqa.GQAError, match="scratch"):
        gqa.decode_noalloc(q, kc, kc, kv_len=cap, q_pos=cap, out=out)
    torch.cuda.synchronize()
    assert int(out.count_nonzero()) == 0


def test_noalloc_decode_replays_from_a_captured_graph():
    """The allocation-free decode inside a captured HIP graph, the kind of
    caller it is for.  One eager call first (it looks up the static scratch's
    device address, which is not done under capture); then the call is
    captured once and replayed three times, with new query values written
    eagerly and a synchronisation between replays.  Every replay must equal
    the eager gqa_decode (caller's workspace) on the same inputs, bit for
    bit."""
    B, cap, h_q, h_kv, d = 4, 4096, 28, 4, 128
    kv_len, q_pos = 3000, 3100                # two 2048-key chunks, the second partial
    note(f"noalloc decode under graph capture: B{B} kv {kv_len} {h_q}/{h_kv} d{d} bf16")
    gen = torch.Generator(device="cuda").manual_seed(29)
    q = torch.randn((B, h_q, d), device="cuda", generator=gen).to(torch.bfloat16)
    kc = torch.randn((B, cap, h_kv, d), device="cuda", generator=gen).to(torch.bfloat16)
    vc = torch.randn((B, cap, h_kv, d), device="cuda", generator=gen).to(torch.bfloat16)
    out = torch.empty((B, h_q, d), dtype=torch.float32, device="cuda")
    gqa.decode_noalloc(q, kc, vc, kv_len=kv_len, q_pos=q_pos, out=out)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gqa.decode_noalloc(q, kc, vc, kv_len=kv_len, q_pos=q_pos, out=out)
    torch.cuda.synchronize()
    for r in range(3):
        q.copy_(torch.randn((B, h_q, d), device="cuda", generator=gen).to(torch.bfloat16))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        want = gqa.decode(q, kc, vc, kv_len=kv_len, q_pos=q_pos)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all(), f"replay {r}"
        assert torch.equal(out, want), f"replay {r}"
