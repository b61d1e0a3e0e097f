"""Host logic of bench.py (no GPU): the one-GPU guard, the traffic figures'
source-hash gating, and that each stored counter figure is the one the
committed profile summary lists."""

import hashlib
import importlib.util
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_follows_the_kernel_source(monkeypatch):
    bench = load_bench()
    for which, (src, digest, nbytes) in bench.TRAFFIC.items():
        path = os.path.join(ROOT, "rope_causal_grouped_amd", "csrc", src)
        cur = hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]
        want = nbytes if cur == digest else None
        assert bench.traffic_bytes(which) == want, which
    # a figure taken on another source is not reported
    monkeypatch.setitem(bench.TRAFFIC, "prefill", ("prefill_bf16.hip", "0" * 16, 1.0))
    assert bench.traffic_bytes("prefill") is None


def test_traffic_figures_match_the_profile_summary():
    """FETCH_SIZE / WRITE_SIZE KiB per dispatch in bench.py are the ones the
    committed counter summary lists for the same call site (FETCH x 2 and
    WRITE x 1, the copy calibration)."""
    bench = load_bench()
    prof_dir = os.path.join(ROOT, "profiles")
    text = "".join(open(os.path.join(prof_dir, f)).read() for f in os.listdir(prof_dir)
                   if f.startswith("hbm_traffic"))
    rows = {}
    for m in re.finditer(r"^\| `([^`]+)` \(([^)]*)\) \| ([\d,\.]+) \| ([\d,\.]+) \|", text, re.M):
        kern, site = m.group(1), m.group(2)
        rows[(kern, site)] = (float(m.group(3).replace(",", "")), float(m.group(4).replace(",", "")))
    pk = "prefill_bf16_kernel<128, false, true>"
    sites = {
        "prefill": (pk, "`gqa_prefill`, 7B B4 L4096"),
        "prefill_c4": (pk, "`gqa_prefill`, 72B B2 L8192"),
        "prefill_c5": (pk, "`gqa_prefill`, 7B B1 L32768"),
        "prefill_chunk": (pk, "`gqa_prefill_chunk`, rows 3072..4095"),
        "decode": ("decode_split_bf16_kernel<128, false, true>", "`gqa_decode`, 7B B32 x 32768"),
        "decode_append": ("decode_split_bf16_kernel<128, false, true>", "`gqa_decode_append`"),
        "decode_paged": ("decode_split_bf16_kernel<128, true, true>", "`gqa_decode_paged`"),
        "qkv_epilogue": ("qkv_epilogue_kernel<unsigned short>",
                         "`gqa_qkv_epilogue`, 7B B4 L4096 projections"),
    }
    assert set(sites) == set(bench.TRAFFIC)
    for which, key in sites.items():
        assert key in rows, key
        fetch, write = rows[key]
        assert bench.TRAFFIC[which][2] == pytest.approx((fetch * 2.0 + write) * 1024, rel=1e-9)
