"""Whole-output parity of the five workloads at full size, and of one GPU's
share of the 72B prefill at 8-way tensor parallelism over KV heads.

Each workload runs through the C ABI in the launch configuration the
benchmark times (``gqa.prefill`` / ``gqa.decode`` with default arguments);
its entire output is then compared with the fp64 oracle, evaluated piece by
piece -- (sequence, KV group, query rows) for a prefill, one sequence for a
decode -- in a pool of worker processes on the host cores (oracle/pool.py).

Tolerances (over the whole output): fp32 inputs max-abs <= 1e-4; bf16
inputs (fp32 accumulation) max-abs <= 2e-2 and relative L2 <= 1e-2.
"""

import dataclasses
import time

import numpy as np
import pytest
import torch

import rope_causal_grouped_amd as gqa
from oracle import pool as opool
from synthetic import WORKLOADS, gen_decode_cache_b, gen_decode_query, gen_prefill

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-4
TOL_BF16_ABS = 2e-2
TOL_BF16_REL = 1e-2


@pytest.fixture(scope="module")
def pool():
    with opool.oracle_pool() as p:
        yield p


def say(capsys, msg):
    """Progress line straight to the terminal (long oracle runs)."""
    with capsys.disabled():
        print(msg, flush=True)


def check(cmp, dtype, what, capsys):
    say(capsys, f"  {what}: {cmp.summary()}")
    assert cmp.nonfinite == 0, f"{what}: non-finite outputs"
    if dtype == "f32":
        assert cmp.max_abs <= TOL_F32, f"{what}: max-abs {cmp.max_abs:.3e} > {TOL_F32}"
    else:
        assert cmp.max_abs <= TOL_BF16_ABS, f"{what}: max-abs {cmp.max_abs:.3e}"
        assert cmp.rel_l2 <= TOL_BF16_REL, f"{what}: rel-L2 {cmp.rel_l2:.3e}"


# one GPU's share of the 72B prefill at 8-way tensor parallelism over KV
# heads: the 72B recipe drawn at 8 query heads over 1 KV head
OVERRIDES = {"c4_tp8": ("c4", (("h_q", 8), ("h_kv", 1)))}


def gpu_prefill(w):
    """The benchmark's call on the workload; returns O as host float32."""
    q, k, v = gen_prefill(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    qd, kd, vd = (torch.from_numpy(x).to("cuda", dt) for x in (q, k, v))
    del q, k, v
    o = gqa.prefill(qd, kd, vd)
    torch.cuda.synchronize()
    out = o.cpu().numpy()
    del qd, kd, vd, o
    torch.cuda.empty_cache()
    return out


@pytest.mark.parametrize("key", ["c1", "c2", "c4", "c5", "c4_tp8"])
def test_prefill_workload_whole_output(key, pool, capsys):
    base, over = OVERRIDES.get(key, (key, ()))
    w = dataclasses.replace(WORKLOADS[base], **dict(over))
    say(capsys, f"\n[{key}] {w.name}: B{w.B} L{w.L} {w.h_q}/{w.h_kv} d{w.d} {w.dtype}")
    got = gpu_prefill(w)
    assert got.shape == (w.B, w.L, w.h_q, w.d)
    tasks = opool.prefill_tasks(base, over)
    cmp = opool.Comparison()
    seen = np.zeros((w.B, w.h_kv, w.L), bool)
    t0 = last = time.monotonic()
    for n, (b, u, r0, r1, want) in enumerate(opool.prefill_pieces(pool, tasks), 1):
        g = w.g
        cmp.add(got[b, r0:r1, u * g:(u + 1) * g], want, (b, u, r0, r1))
        seen[b, u, r0:r1] = True
        if time.monotonic() - last > 20.0:
            last = time.monotonic()
            say(capsys, f"  [{key}] oracle {n}/{len(tasks)} pieces, {last - t0:.0f} s")
    assert seen.all(), "oracle pieces do not cover the output"
    check(cmp, w.dtype, f"{key} whole output ({time.monotonic() - t0:.0f} s of oracle)",
          capsys)


def test_decode_workload_whole_output(pool, capsys):
    w = WORKLOADS["c3"]
    say(capsys, f"\n[c3] {w.name}: B{w.B} cache {w.L} {w.h_q}/{w.h_kv} d{w.d}")
    qh = gen_decode_query(w)
    kc = torch.empty((w.B, w.L, w.h_kv, w.d), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    for b in range(w.B):
        kb, vb = gen_decode_cache_b(w, b)
        kc[b].copy_(torch.from_numpy(kb))
        vc[b].copy_(torch.from_numpy(vb))
    o = gqa.decode(torch.from_numpy(qh).to("cuda", torch.bfloat16), kc, vc, kv_len=w.L,
                   q_pos=w.q_pos)
    torch.cuda.synchronize()
    got = o.cpu().numpy()
    del kc, vc, o
    torch.cuda.empty_cache()
    cmp = opool.Comparison()
    done = set()
    for b, want in opool.decode_pieces(pool, "c3"):
        cmp.add(got[b], want, b)
        done.add(b)
    assert done == set(range(w.B))
    check(cmp, w.dtype, "c3 whole output (all 32 sequences)", capsys)
