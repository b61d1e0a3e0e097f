#!/usr/bin/env python3
"""Benchmark: causal GQA prefill TFLOP/s + decode KV-stream GB/s on one MI355X.

One step = one pass of the whole hot path over resident synthetic inputs:
  * gqa_prefill on the Qwen2-7B-shaped workload (B=4, L=4096, 28 query heads
    over 4 KV heads, head size 128, bf16 in, fp32 accumulate and out, causal,
    RoPE theta 1e6): RoPE table, K/V preparation, attention;
  * gqa_decode on the Qwen2-7B-shaped decode workload (B=32 sequences, a
    32768-position bf16 cache, one new token at position 32768).
After the timed steps, the autoregressive entry points are measured on the
same shapes (reported under "next", outside the step): the last 1024-row
chunk of the prefill workload through gqa_prefill_chunk against a cache that
holds the first 3072 rows, one gqa_decode_append step for 32 sequences at
ragged positions 32767 - 256 b of a 32768-row cache, gqa_decode_paged on
the decode workload's cache cut into 16-position pages under a shuffled
block table, and gqa_qkv_epilogue over the packed projection output of the
prefill workload's 4 x 4096 tokens.  The same gqa_prefill call is then timed
on the other prefill workloads (72B heads at L 8192; 7B heads at L 32768;
the small fp32 0.5B case as a latency) under "other_prefill", and the HBM
context figures under "context".
`value` is the prefill rate in TFLOP/s over the causal pairs only
(4 * B * h_q * d * L(L+1)/2 flop per call) over the whole call, from the
start of its first kernel to the end of its last; the decode rate (K/V
cache bytes read once per KV group / call time) is reported beside it.
Call and kernel durations (the latter for the roofline objects) come from
HIP events that the library binds to its own kernel dispatches on the
launch stream (hipExtLaunchKernel), so no marker packet sits between the
kernels of a step; `ms_per_step` is the whole timed loop over K.  Before the W warm-up steps the step runs for a fixed
stretch of time (--clock-warmup-s), so that the timed steps see the
sustained shader clock rather than the ramp from idle, whatever W is.
After timing, the outputs of the timed calls are compared with the fp64
oracle (the whole 7B prefill output and all 32 decode sequences); the
oracle's prefill leg, run as a pool of single-threaded processes on the
host cores, is also the CPU baseline.

Prints one JSON line.  Only one GPU is supported.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GQA prefill TFLOP/s + decode KV-stream GB/s, % of MI355X roofline"
PEAK_BF16_TFLOPS = 2516.6    # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E peak
# HBM bytes per dispatch from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE
# (KiB per dispatch, each scaled by what the counter reads for a plain 1 GiB
# device copy: FETCH x 2.00, WRITE x 1.00).  Each figure is valid only for the
# kernel source it was measured on (sha256 prefix); otherwise it reports null.
TRAFFIC = {
    "prefill": ("prefill_bf16.hip", "d2bffe1f423a3633", (102977.3 * 2.0 + 229406.9) * 1024),
    "prefill_c4": ("prefill_bf16.hip", "d2bffe1f423a3633", (302314.0 * 2.0 + 524338.1) * 1024),
    "prefill_c5": ("prefill_bf16.hip", "d2bffe1f423a3633", (691369.8 * 2.0 + 458790.5) * 1024),
    "decode": ("decode.hip", "5d5c44530499b2f8", (1049670.9 * 2.0 + 7392.1) * 1024),
    "prefill_chunk": ("prefill_bf16.hip", "d2bffe1f423a3633", (41377.9 * 2.0 + 57344.0) * 1024),
    "decode_append": ("decode.hip", "5d5c44530499b2f8", (922583.2 * 2.0 + 7392.0) * 1024),
    "decode_paged": ("decode.hip", "5d5c44530499b2f8", (1049802.1 * 2.0 + 7392.0) * 1024),
    "qkv_epilogue": ("rope.hip", "b4d77aead74c0c45", (73825.9 * 2.0 + 147472.8) * 1024),
}


def traffic_bytes(which):
    import hashlib
    if which not in TRAFFIC:   # no counter figure taken for this call site
        return None
    src, digest, nbytes = TRAFFIC[which]
    path = os.path.join(ROOT, "rope_causal_grouped_amd", "csrc", src)
    with open(path, "rb") as f:
        cur = hashlib.sha256(f.read()).hexdigest()[:16]
    return nbytes if cur == digest else None


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    # the shader clock ramps up over the first tens of milliseconds of load;
    # this much untimed work first puts the timed steps at the sustained clock
    p.add_argument("--clock-warmup-s", type=float, default=0.5)
    p.add_argument("--only", choices=["prefill", "decode", "next"], default=None,
                   help="run one part only (for profiling)")
    p.add_argument("--no-cpu-baseline", action="store_true",
                   help="skip the oracle leg (CPU baseline and parity of the timed outputs)")
    p.add_argument("--calib-copy-mb", type=int, default=0,
                   help="also run a plain device copy of this many MiB (counter calibration)")
    return p.parse_args()


def oracle_leg(wp, wd, got_prefill, got_decode):
    """The fp64 oracle over the whole output of the timed prefill call (the
    CPU baseline: a pool of single-threaded processes, one per host core,
    over (sequence, KV group, query rows) pieces) and over every sequence of
    the decode call; both outputs are compared with it."""
    from oracle import pool as opool
    cores = opool.host_cores()
    res = {}
    with opool.oracle_pool(cores) as pool:
        tasks = opool.prefill_tasks(wp.key)
        cmp = opool.Comparison()
        t0 = time.perf_counter()
        for b, u, r0, r1, want in opool.prefill_pieces(pool, tasks):
            if got_prefill is not None:
                cmp.add(got_prefill[b, r0:r1, u * wp.g:(u + 1) * wp.g], want, (b, u, r0, r1))
        dt = time.perf_counter() - t0
        flops = wp.prefill_flops()
        res["cpu_baseline"] = {
            "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"the whole {wp.name} output (B{wp.B}, {wp.h_q} query heads, all {wp.L} "
                      f"positions): {flops / 1e9:.1f} causal GFLOP in {dt:.2f} s, fp64 NumPy "
                      f"in {cores} single-threaded processes over {len(tasks)} "
                      f"(sequence, KV group, rows) pieces"}
        log(f"[bench] oracle: whole prefill output in {dt:.1f} s on {cores} cores")
        parity = {}
        if got_prefill is not None:
            parity["prefill"] = {"workload": wp.name, "outputs": cmp.count,
                                 "max_abs": cmp.max_abs, "rel_l2": cmp.rel_l2,
                                 "nonfinite": cmp.nonfinite,
                                 "ok": bool(cmp.nonfinite == 0 and cmp.max_abs <= 2e-2
                                            and cmp.rel_l2 <= 1e-2)}
        if got_decode is not None:
            cmd = opool.Comparison()
            for b, want in opool.decode_pieces(pool, wd.key):
                cmd.add(got_decode[b], want, b)
            parity["decode"] = {"workload": wd.name, "outputs": cmd.count,
                                "max_abs": cmd.max_abs, "rel_l2": cmd.rel_l2,
                                "nonfinite": cmd.nonfinite,
                                "ok": bool(cmd.nonfinite == 0 and cmd.max_abs <= 2e-2
                                           and cmd.rel_l2 <= 1e-2)}
        for name, r in parity.items():
            log(f"[bench] parity of the timed {name} call vs the fp64 oracle: "
                f"max-abs {r['max_abs']:.3e}, rel-L2 {r['rel_l2']:.3e} over {r['outputs']} "
                f"outputs ({'ok' if r['ok'] else 'FAILED'})")
        res["parity"] = parity
    return res


def clock_warmup(torch, step, seconds):
    """Run the step until `seconds` of GPU time have passed; returns the
    number of steps run."""
    if seconds <= 0:
        return 0
    n, busy = 0, 0.0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    while busy < seconds * 1e3:
        e0.record()
        for _ in range(5):
            step()
        e1.record()
        torch.cuda.synchronize()
        busy += e0.elapsed_time(e1)
        n += 5
    return n


def timed_calls(torch, gqa, fam, fn, reps):
    """Runs fn() reps times back to back with the library's call timing on;
    returns the mean duration of the calls' main kernel (fam 0: prefill
    attention, 1: decode split-K) and of the whole calls (first kernel's
    start to last kernel's end), both in ms from HIP events bound to those
    kernel dispatches."""
    gqa.timing_enable(True)
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()
    gqa.timing_enable(False)
    k_ms, k_n = gqa.timing_read(fam)
    c_ms, c_n = gqa.timing_read(fam + 2)
    if k_n != reps or c_n != reps:
        raise RuntimeError(f"timed {k_n}/{c_n} calls, expected {reps}")
    return k_ms / reps, c_ms / reps


def no_children_left():
    """Child processes still running at exit, for the log; each is ended
    here.  The oracle pool's workers are joined when it closes, and its
    semaphore helper process is stopped after the oracle leg, so none is
    expected."""
    try:
        import psutil
    except ImportError:
        return "psutil unavailable"
    left = []
    for p in psutil.Process().children(recursive=True):
        try:
            left.append(" ".join(p.cmdline())[:100])
            p.kill()
            p.wait(timeout=5)
        except psutil.Error:
            pass
    return f"child processes at exit: {len(left)}{' (ended: ' + str(left) + ')' if left else ''}"


def measure_context(torch, gqa, dev):
    """HBM context figures for the HBM-bound rooflines: the library's plain
    streaming-read kernel over 2 GiB, and a 1 GiB framework device copy."""
    res = {}
    x = torch.ones(2**30, dtype=torch.bfloat16, device=dev)           # 2 GiB
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    a = torch.ones(2**28, dtype=torch.float32, device=dev)            # 1 GiB
    b = torch.empty_like(a)
    for name, fn, nbytes in (("read", lambda: gqa.stream_read(x, sink), 2**31),
                             ("copy", lambda: b.copy_(a), 2 * 2**30)):
        for _ in range(10):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[f"{name}_GBps"] = nbytes / (e0.elapsed_time(e1) / 20 * 1e-3) / 1e9
    res["kernels"] = ("read: gqa_stream_read over 2 GiB, 16-byte non-temporal loads (bytes "
                      "read); copy: torch copy_ of 1 GiB fp32 (bytes read + written)")
    del x, sink, a, b
    torch.cuda.empty_cache()
    return res


# One GPU's share of the 72B prefill under 8-way tensor parallelism over KV
# heads (each GPU owns one KV group and its 8 query heads): the 72B recipe
# drawn at 8/1 heads.
TP8_SHARE = ("c4", (("h_q", 8), ("h_kv", 1)))


def measure_other_prefills(torch, gqa, dev, keys=("c1", "c4", "c5", "c4_tp8"), warmup=10,
                           reps=20):
    """The same gqa_prefill call on the other prefill workloads, outside the
    timed step: the larger ones (72B heads at L 8192; 7B heads at L 32768
    with boosted rows), for the scaling of the attention kernel with L, the
    small fp32 one (0.5B heads, L 128), whose 29.6 MFLOP make it a latency
    figure (no roofline), and one GPU's share of the 72B prefill at 8-way
    tensor parallelism (B2 L8192, 8 query heads over 1 KV head)."""
    import dataclasses

    from synthetic import WORKLOADS, gen_prefill
    res = {}
    for key in keys:
        if key == "c4_tp8":
            base, over = TP8_SHARE
            w = dataclasses.replace(WORKLOADS[base], name=WORKLOADS[base].name + "-tp8-share",
                                    **dict(over))
        else:
            w = WORKLOADS[key]
        log(f"[bench] generating {w.name}")
        q, k, v = gen_prefill(w)
        dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        qd, kd, vd = (torch.from_numpy(x).to(dev, dt) for x in (q, k, v))
        del q, k, v
        od = torch.empty((w.B, w.L, w.h_q, w.d), dtype=torch.float32, device=dev)
        ws = torch.empty(gqa.prefill_workspace_size(dt, w.B, w.L, w.h_kv, w.d),
                         dtype=torch.uint8, device=dev)
        for _ in range(warmup):
            gqa.prefill(qd, kd, vd, out=od, workspace=ws)
        torch.cuda.synchronize()
        kern_ms, call_ms = timed_calls(
            torch, gqa, 0, lambda: gqa.prefill(qd, kd, vd, out=od, workspace=ws), reps)
        flops = w.prefill_flops()
        ach = flops / (kern_ms * 1e-3) / 1e12
        if w.dtype != "bf16":
            res[key] = {"workload": f"{w.name}: B{w.B} L{w.L} h_q{w.h_q} h_kv{w.h_kv} d{w.d} fp32",
                        "call_us": call_ms * 1e3, "kernel_us": kern_ms * 1e3,
                        "note": f"latency figure ({flops / 1e6:.1f} MFLOP); no roofline"}
            log(f"[bench] {key}: call {call_ms * 1e3:.1f} us, attention {kern_ms * 1e3:.1f} us")
            del qd, kd, vd, od, ws
            continue
        res[key] = {"workload": f"{w.name}: B{w.B} L{w.L} h_q{w.h_q} h_kv{w.h_kv} d{w.d} bf16 in / fp32 out",
                    "value": flops / (call_ms * 1e-3) / 1e12, "unit": "TFLOP/s", "call_ms": call_ms,
                    "roofline": {"bound": "mfma", "kernel": "prefill_bf16_kernel", "achieved": ach,
                                 "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                 "frac": ach / PEAK_BF16_TFLOPS, "kernel_ms": kern_ms,
                                 "traffic": traffic_bytes("prefill_" + key)}}
        log(f"[bench] {key}: attention {kern_ms:.3f} ms -> {ach:.0f} TFLOP/s")
        del qd, kd, vd, od, ws
        torch.cuda.empty_cache()
    return res


def measure_next(args, torch, gqa, dev, wp, wd, pre=None, dec=None):
    """Chunked prefill and appending decode on the prefill / decode shapes
    (``pre``/``dec``: the step's resident inputs, reused when present)."""
    from synthetic import gen_decode_cache_b, gen_decode_query, gen_prefill
    K = args.steps
    res = {}
    # -- chunked prefill: rows 3072..4095 of the prefill workload, cache holds 0..3071
    s0, C = wp.L - 1024, 1024
    if pre is None:
        q, k, v = gen_prefill(wp)
        pre = tuple(torch.from_numpy(x).to(dev, torch.bfloat16) for x in (q, k, v))
        del q, k, v
    qd, kd, vd = pre
    kc = torch.zeros((wp.B, wp.L, wp.h_kv, wp.d), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    ws = torch.empty(gqa.prefill_chunk_workspace_size(torch.bfloat16, wp.B, wp.L, wp.h_kv, wp.d),
                     dtype=torch.uint8, device=dev)
    for a in range(0, s0, C):   # fill the cache chunk by chunk (untimed)
        gqa.prefill_chunk(qd[:, a:a + C].contiguous(), kd[:, a:a + C].contiguous(),
                          vd[:, a:a + C].contiguous(), kc, vc, [a] * wp.B, kend=wp.L,
                          workspace=ws)
    qc, kn, vn = (x[:, s0:].contiguous() for x in (qd, kd, vd))
    start = torch.full((wp.B,), s0, dtype=torch.int64, device=dev)
    oc = torch.empty((wp.B, C, wp.h_q, wp.d), dtype=torch.float32, device=dev)

    def chunk():
        gqa.prefill_chunk(qc, kn, vn, kc, vc, start, kend=wp.L, out=oc, workspace=ws)

    for _ in range(args.warmup):
        chunk()
    torch.cuda.synchronize()
    attn_avg, call_ms = timed_calls(torch, gqa, 0, chunk, K)
    pos = np.arange(s0, wp.L, dtype=np.float64)
    flops = 4.0 * wp.B * wp.h_q * wp.d * float(np.sum(pos + 1))
    ach = flops / (attn_avg * 1e-3) / 1e12
    res["prefill_chunk"] = {
        "workload": f"{wp.name} last chunk: B{wp.B} rows {s0}..{wp.L - 1} ({C} per sequence) "
                    f"against {s0} cached rows, h_q{wp.h_q} h_kv{wp.h_kv} d{wp.d} bf16",
        "value": flops / (call_ms * 1e-3) / 1e12, "unit": "TFLOP/s", "call_ms": call_ms,
        "roofline": {"bound": "mfma", "kernel": "prefill_bf16_kernel", "achieved": ach,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": ach / PEAK_BF16_TFLOPS,
                     "kernel_ms": attn_avg, "traffic": traffic_bytes("prefill_chunk")}}
    del pre, qd, kd, vd, qc, kn, vn, kc, vc, ws, oc
    log(f"[bench] chunked prefill: {call_ms:.3f} ms per call")

    # -- appending decode: 32 sequences at ragged positions of a 32768-row cache
    cap = wd.L
    pos = np.array([cap - 1 - 256 * b for b in range(wd.B)], dtype=np.int64)
    if dec is None:
        qh = torch.from_numpy(gen_decode_query(wd)).to(dev, torch.bfloat16)
        kc = torch.empty((wd.B, cap, wd.h_kv, wd.d), dtype=torch.bfloat16, device=dev)
        vc = torch.empty_like(kc)
        for b in range(wd.B):
            kb, vb = gen_decode_cache_b(wd, b)
            kc[b].copy_(torch.from_numpy(kb))
            vc[b].copy_(torch.from_numpy(vb))
    else:
        qh, kc, vc = dec
    posd = torch.from_numpy(pos).to(dev)
    rows = torch.arange(wd.B, device=dev)
    kn = kc[rows, posd].clone()   # the new tokens' K and V (rewritten in place every step)
    vn = vc[rows, posd].clone()
    od = torch.empty((wd.B, wd.h_q, wd.d), dtype=torch.float32, device=dev)
    wsd = torch.empty(gqa.decode_workspace_size(wd.B, wd.h_q, wd.h_kv, wd.d, cap),
                      dtype=torch.uint8, device=dev)

    def app():
        gqa.decode_append(qh, kn, vn, kc, vc, posd, max_pos=int(pos.max()), out=od,
                          workspace=wsd)

    for _ in range(args.warmup):
        app()
    torch.cuda.synchronize()
    split_avg, call_ms = timed_calls(torch, gqa, 1, app, K)
    kvb = float(np.sum(pos + 1)) * wd.h_kv * wd.d * 2 * 2
    dach = kvb / (split_avg * 1e-3) / 1e9
    res["decode_append"] = {
        "workload": f"{wd.name} with append: B{wd.B} positions {int(pos.min())}..{int(pos.max())} "
                    f"(step 256) of a {cap}-row cache, h_q{wd.h_q} h_kv{wd.h_kv} d{wd.d} bf16",
        "value": kvb / (call_ms * 1e-3) / 1e9, "unit": "GB/s", "call_ms": call_ms,
        "roofline": {"bound": "hbm", "kernel": "decode_split_bf16_kernel", "achieved": dach,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": dach / PEAK_HBM_GBS,
                     "kernel_ms": split_avg, "traffic": traffic_bytes("decode_append")}}
    log(f"[bench] appending decode: {call_ms:.3f} ms per call")
    del kn, vn

    # -- paged decode: the same 32768-row caches cut into 16-position pages,
    #    scattered over the pool by a shuffled block table
    ps = 16
    n_pg = cap // ps
    perm = torch.randperm(wd.B * n_pg, generator=torch.Generator().manual_seed(wd.seed))
    permd = perm.to(dev)
    pools = []
    for c in (kc, vc):
        pool = c.view(wd.B, n_pg, ps, wd.h_kv, wd.d).permute(0, 1, 3, 2, 4).reshape(
            wd.B * n_pg, wd.h_kv, ps, wd.d)
        shuf = torch.empty(pool.shape, dtype=pool.dtype, device=dev)
        shuf[permd] = pool
        pools.append(shuf)
        del pool
    del kc, vc
    bt = permd.view(wd.B, n_pg).to(torch.int32)
    qpos = torch.full((wd.B,), wd.q_pos, dtype=torch.int64, device=dev)
    kvl = torch.full((wd.B,), cap, dtype=torch.int64, device=dev)

    def paged():
        gqa.decode_paged(qh, pools[0], pools[1], bt, qpos, kvl, out=od, workspace=wsd)

    for _ in range(args.warmup):
        paged()
    torch.cuda.synchronize()
    split_avg, call_ms = timed_calls(torch, gqa, 1, paged, K)
    kvb = wd.decode_kv_bytes()
    dach = kvb / (split_avg * 1e-3) / 1e9
    res["decode_paged"] = {
        "workload": f"{wd.name} over a paged cache: B{wd.B} x {cap} positions in {ps}-position "
                    f"pages (shuffled block table), h_q{wd.h_q} h_kv{wd.h_kv} d{wd.d} bf16",
        "value": kvb / (call_ms * 1e-3) / 1e9, "unit": "GB/s", "call_ms": call_ms,
        "roofline": {"bound": "hbm", "kernel": "decode_split_bf16_kernel", "achieved": dach,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": dach / PEAK_HBM_GBS,
                     "kernel_ms": split_avg, "traffic": traffic_bytes("decode_paged")}}
    log(f"[bench] paged decode: {call_ms:.3f} ms per call")
    del pools, bt, od, wsd

    # -- QKV epilogue on the prefill shape: packed projection output of all
    #    4096 tokens -> rotated Q, rotated K and V in a 4096-row cache
    width = (wp.h_q + 2 * wp.h_kv) * wp.d
    g = torch.Generator(device=dev).manual_seed(wp.seed)
    xq = torch.randn((wp.B, wp.L, width), generator=g, device=dev).to(torch.bfloat16)
    bq = torch.randn((width,), generator=g, device=dev).to(torch.bfloat16)
    kc = torch.empty((wp.B, wp.L, wp.h_kv, wp.d), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    qo = torch.empty((wp.B, wp.L, wp.h_q, wp.d), dtype=torch.bfloat16, device=dev)
    start = torch.zeros((wp.B,), dtype=torch.int64, device=dev)

    def epi():
        gqa.qkv_epilogue(xq, bq, kc, vc, wp.h_q, start, q_out=qo)

    for _ in range(args.warmup):
        epi()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(K):
        epi()
    e1.record()
    torch.cuda.synchronize()
    call_ms = e0.elapsed_time(e1) / K
    nbytes = 2.0 * wp.B * wp.L * (width + wp.h_q * wp.d + 2 * wp.h_kv * wp.d) + 2 * width
    rate = nbytes / (call_ms * 1e-3) / 1e9
    res["qkv_epilogue"] = {
        "workload": f"{wp.name} projections: B{wp.B} L{wp.L} packed ({wp.h_q}+2x{wp.h_kv}) "
                    f"x {wp.d} bf16 + bias -> rotated Q, rotated K and V into the cache",
        "value": rate, "unit": "GB/s", "call_ms": call_ms,
        "roofline": {"bound": "hbm", "kernel": "qkv_epilogue_kernel", "achieved": rate,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": rate / PEAK_HBM_GBS,
                     "kernel_ms": call_ms, "traffic": traffic_bytes("qkv_epilogue")}}
    log(f"[bench] QKV epilogue: {call_ms:.3f} ms per call")
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "this library has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch
    import rope_causal_grouped_amd as gqa
    from synthetic import WORKLOADS, gen_decode_cache_b, gen_decode_query, gen_prefill

    wp, wd = WORKLOADS["c2"], WORKLOADS["c3"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    run_p = args.only in (None, "prefill")
    run_d = args.only in (None, "decode")
    run_n = args.only in (None, "next")

    # ---- inputs resident in HBM
    if run_p:
        log(f"[bench] generating {wp.name}")
        q, k, v = gen_prefill(wp)
        qd, kd, vd = (torch.from_numpy(x).to(dev, torch.bfloat16) for x in (q, k, v))
        del q, k, v
        od = torch.empty((wp.B, wp.L, wp.h_q, wp.d), dtype=torch.float32, device=dev)
        wsp = torch.empty(gqa.prefill_workspace_size(torch.bfloat16, wp.B, wp.L, wp.h_kv, wp.d),
                          dtype=torch.uint8, device=dev)
    if run_d:
        log(f"[bench] generating {wd.name}")
        qh = torch.from_numpy(gen_decode_query(wd)).to(dev, torch.bfloat16)
        kc = torch.empty((wd.B, wd.L, wd.h_kv, wd.d), dtype=torch.bfloat16, device=dev)
        vc = torch.empty_like(kc)
        for b in range(wd.B):
            kb, vb = gen_decode_cache_b(wd, b)
            kc[b].copy_(torch.from_numpy(kb))
            vc[b].copy_(torch.from_numpy(vb))
        odd = torch.empty((wd.B, wd.h_q, wd.d), dtype=torch.float32, device=dev)
        wsd = torch.empty(gqa.decode_workspace_size(wd.B, wd.h_q, wd.h_kv, wd.d, wd.L),
                          dtype=torch.uint8, device=dev)

    def step():
        if run_p:
            gqa.prefill(qd, kd, vd, out=od, workspace=wsp)
        if run_d:
            gqa.decode(qh, kc, vc, kv_len=wd.L, q_pos=wd.q_pos, out=odd, workspace=wsd)

    n_clock = clock_warmup(torch, step, args.clock_warmup_s)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] clock warm-up {n_clock} steps ({args.clock_warmup_s:.2f} s), "
        f"warmup done ({args.warmup} steps)")

    K = args.steps
    # the calls time themselves (HIP events bound to their kernel dispatches:
    # no marker packets between the kernels of a step)
    gqa.timing_enable(True)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record()
    for s in range(K):
        step()
    t_end.record()
    torch.cuda.synchronize()
    gqa.timing_enable(False)
    total_ms = t_start.elapsed_time(t_end)
    attn_ms, attn_n = gqa.timing_read(0)
    split_ms, split_n = gqa.timing_read(1)
    pre_ms = gqa.timing_read(2)[0] / K
    dec_ms = gqa.timing_read(3)[0] / K
    log(f"[bench] timed {K} steps: {total_ms:.2f} ms total")
    # outputs of the last timed calls, for the parity check after all timing
    got_prefill = od.cpu().numpy() if run_p else None
    got_decode = odd.cpu().numpy() if run_d else None

    if run_n:
        out_next = measure_next(args, torch, gqa, dev, wp, wd,
                                (qd, kd, vd) if run_p else None,
                                (qh, kc, vc) if run_d else None)

    if args.calib_copy_mb:
        n = args.calib_copy_mb * 2**20 // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {args.calib_copy_mb} MiB x3 done")

    out = {"metric": METRIC, "n_gpus": 1, "steps": K, "warmup": args.warmup,
           "ms_per_step": total_ms / K, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "clock_warmup": {"steps": n_clock, "seconds": args.clock_warmup_s}}
    if run_p:
        flops = wp.prefill_flops()
        attn_avg = attn_ms / max(attn_n, 1)
        out["value"] = flops / (pre_ms * 1e-3) / 1e12
        out["unit"] = "TFLOP/s"
        out["config"] = {
            "workload": f"{wp.name}: B{wp.B} L{wp.L} h_q{wp.h_q} h_kv{wp.h_kv} d{wp.d} causal "
                        f"RoPE theta 1e6, bf16 in / fp32 out; plus {wd.name}: B{wd.B} "
                        f"cache {wd.L} h_q{wd.h_q} h_kv{wd.h_kv} d{wd.d} bf16",
            "global_batch": wp.B, "seq_len": wp.L, "parallelism": "single-gpu"}
        out["prefill_call_ms"] = pre_ms
        ach = flops / (attn_avg * 1e-3) / 1e12
        out["roofline"] = {"bound": "mfma", "kernel": "prefill_bf16_kernel",
                           "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": ach / PEAK_BF16_TFLOPS, "kernel_ms": attn_avg,
                           "traffic": traffic_bytes("prefill")}
        out["call_roofline"] = {"bound": "mfma", "achieved": out["value"],
                                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                "frac": out["value"] / PEAK_BF16_TFLOPS, "call_ms": pre_ms,
                                "outside_attention_us": (pre_ms - attn_avg) * 1e3}
    if run_d:
        kvb = wd.decode_kv_bytes()
        split_avg = split_ms / max(split_n, 1)
        dach = kvb / (split_avg * 1e-3) / 1e9
        dec = {"workload": f"{wd.name}: B{wd.B} cache {wd.L} h_q{wd.h_q} h_kv{wd.h_kv} "
                           f"d{wd.d} q_pos {wd.q_pos}",
               "value": kvb / (dec_ms * 1e-3) / 1e9, "unit": "GB/s", "call_ms": dec_ms,
               "roofline": {"bound": "hbm", "kernel": "decode_split_bf16_kernel",
                            "achieved": dach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": dach / PEAK_HBM_GBS, "kernel_ms": split_avg,
                            "traffic": traffic_bytes("decode")}}
        out["decode"] = dec
        if not run_p:
            out["value"], out["unit"] = dec["value"], "GB/s"
            out["config"] = {"workload": dec["workload"], "global_batch": wd.B,
                             "seq_len": wd.L, "parallelism": "single-gpu"}
            out["roofline"] = dec["roofline"]
    if run_n:
        out["next"] = out_next
        if not (run_p or run_d):
            nx = out_next["prefill_chunk"]
            out["value"], out["unit"] = nx["value"], nx["unit"]
            out["config"] = {"workload": nx["workload"], "global_batch": wp.B,
                             "seq_len": wp.L, "parallelism": "single-gpu"}
            out["roofline"] = nx["roofline"]
    if run_p and run_d:
        out["other_prefill"] = measure_other_prefills(torch, gqa, dev)
        out["context"] = measure_context(torch, gqa, dev)
        log(f"[bench] context: read {out['context']['read_GBps']:.0f} GB/s, "
            f"copy {out['context']['copy_GBps']:.0f} GB/s")
    if run_p and not args.no_cpu_baseline:
        log("[bench] fp64 oracle on the host cores: CPU baseline and parity of the timed calls")
        out.update(oracle_leg(wp, wd, got_prefill, got_decode))
        from oracle import pool as opool
        opool.stop_resource_tracker()
    log(f"[bench] {no_children_left()}")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
