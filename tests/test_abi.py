"""C-ABI checks that need no GPU: the library loads, exports every function
include/gqa.h declares, and rejects bad arguments on the host before any
HIP call (validation returns before anything is enqueued)."""

import os
import re

import pytest

from rope_causal_grouped_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa.h")

FAKE = 0x10000   # a 16-byte aligned non-NULL address; never dereferenced here


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gqa_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return _lib.lib()


def test_every_header_symbol_is_exported(lib):
    names = header_functions()
    assert len(names) >= 9
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(_lib.SIGNATURES), "binding signatures out of sync with gqa.h"


def test_version(lib):
    assert b"gfx950" in lib.gqa_version()


def prefill_call(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, in_dt=1, out_dt=0, B=1, L=16, h_q=28, h_kv=4,
             d=128, theta=1e6, scale=0.088, causal=1, kc=None, vc=None, cap=0,
             ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return lib.gqa_prefill(a["q"], a["k"], a["v"], a["o"], a["in_dt"], a["out_dt"], a["B"],
                           a["L"], a["h_q"], a["h_kv"], a["d"], a["theta"], a["scale"],
                           a["causal"], a["kc"], a["vc"], a["cap"], a["ws"], a["wsb"],
                           a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), _lib.GQA_ERR_INVALID_ARG),
    (dict(h_kv=0), _lib.GQA_ERR_INVALID_ARG),
    (dict(h_q=4, h_kv=28), _lib.GQA_ERR_INVALID_ARG),      # ratio written the wrong way round
    (dict(h_q=28, h_kv=3), _lib.GQA_ERR_INVALID_ARG),      # not a multiple
    (dict(d=127), _lib.GQA_ERR_INVALID_ARG),               # odd: no RoPE pairs
    (dict(d=96), _lib.GQA_ERR_UNSUPPORTED),
    (dict(B=0), _lib.GQA_ERR_INVALID_ARG),
    (dict(L=0), _lib.GQA_ERR_INVALID_ARG),
    (dict(L=(1 << 24) + 1), _lib.GQA_ERR_UNSUPPORTED),     # beyond the kernels' index range
    (dict(h_q=65536, h_kv=1), _lib.GQA_ERR_UNSUPPORTED),   # a grid dimension
    (dict(in_dt=7), _lib.GQA_ERR_INVALID_ARG),
    (dict(theta=float("nan")), _lib.GQA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), _lib.GQA_ERR_INVALID_ARG),
    (dict(kc=FAKE), _lib.GQA_ERR_INVALID_ARG),             # v_cache missing
    (dict(kc=FAKE, vc=FAKE, cap=8), _lib.GQA_ERR_INVALID_ARG),  # cap < L
    (dict(o=FAKE + 4), _lib.GQA_ERR_INVALID_ARG),          # misaligned
    (dict(ws=None), _lib.GQA_ERR_WORKSPACE),
    (dict(wsb=16), _lib.GQA_ERR_WORKSPACE),
])
def test_prefill_rejects(lib, kw, code):
    assert prefill_call(lib, **kw) == code
    assert lib.gqa_last_error()


def decode_call(lib, **kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, o=FAKE, in_dt=1, out_dt=0, B=2, h_q=28, h_kv=4, d=128,
             cap=64, kv_len=64, q_pos=64, theta=1e6, scale=0.088, ws=FAKE, wsb=1 << 40,
             stream=None)
    a.update(kw)
    return lib.gqa_decode(a["q"], a["kc"], a["vc"], a["o"], a["in_dt"], a["out_dt"], a["B"],
                          a["h_q"], a["h_kv"], a["d"], a["cap"], a["kv_len"], a["q_pos"],
                          a["theta"], a["scale"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(kc=None), _lib.GQA_ERR_INVALID_ARG),
    (dict(kv_len=0), _lib.GQA_ERR_INVALID_ARG),
    (dict(kv_len=65), _lib.GQA_ERR_INVALID_ARG),           # beyond cap
    (dict(q_pos=10), _lib.GQA_ERR_INVALID_ARG),            # keys after the query
    (dict(h_q=4, h_kv=28), _lib.GQA_ERR_INVALID_ARG),
    (dict(d=80), _lib.GQA_ERR_UNSUPPORTED),
    (dict(wsb=0), _lib.GQA_ERR_WORKSPACE),
])
def test_decode_rejects(lib, kw, code):
    assert decode_call(lib, **kw) == code
    assert lib.gqa_last_error()


def test_stream_read_rejects(lib):
    bad = _lib.GQA_ERR_INVALID_ARG
    assert lib.gqa_stream_read(None, 16, FAKE, None) == bad
    assert lib.gqa_stream_read(FAKE, 16, None, None) == bad
    assert lib.gqa_stream_read(FAKE, 0, FAKE, None) == bad
    assert lib.gqa_stream_read(FAKE, 24, FAKE, None) == bad
    assert lib.gqa_stream_read(FAKE + 8, 16, FAKE, None) == bad
    assert lib.gqa_last_error()


def test_rope_rejects(lib):
    assert lib.gqa_rope_apply(None, 1, 1, 4, 2, 64, 0, 1e6, None) == _lib.GQA_ERR_INVALID_ARG
    assert lib.gqa_rope_apply(FAKE, 1, 1, 4, 2, 63, 0, 1e6, None) == _lib.GQA_ERR_INVALID_ARG
    assert lib.gqa_rope_apply(FAKE, 1, 1, 4, 2, 64, -1, 1e6, None) == _lib.GQA_ERR_INVALID_ARG


def test_workspace_sizes(lib):
    # bf16 prefill: cos/sin table + rotated K + transposed V (64-key padded)
    # + the largest K row norm and the fp16 exponent per 64-key tile + 512
    # bytes for the attention kernel's work-ticket counters (8, 64 bytes apart)
    n = lib.gqa_prefill_workspace_size(1, 4, 4096, 4, 128)
    assert n == 4096 * 64 * 8 + 2 * 4 * 4 * 4096 * 128 * 2 + 2 * 4 * 4 * 64 * 4 + 512
    assert lib.gqa_prefill_workspace_size(1, 0, 10, 4, 128) == 0
    # decode: (m, l, o[d]) per (b, group, 1024-key chunk, head) and the
    # rotated queries of an appending step (fp32-sized)
    n = lib.gqa_decode_workspace_size(32, 28, 4, 128, 32768)
    assert n == 32 * 4 * 32 * 7 * (2 + 128) * 4 + 32 * 28 * 128 * 4
    assert lib.gqa_decode_workspace_size(1, 28, 3, 128, 10) == 0


def chunk_call(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, in_dt=1, out_dt=0, B=2, C=64, h_q=28, h_kv=4, d=128,
             start=FAKE, len=None, kend=512, theta=1e6, scale=0.088, kc=FAKE, vc=FAKE, cap=512,
             ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return lib.gqa_prefill_chunk(a["q"], a["k"], a["v"], a["o"], a["in_dt"], a["out_dt"], a["B"],
                                 a["C"], a["h_q"], a["h_kv"], a["d"], a["start"], a["len"],
                                 a["kend"], a["theta"], a["scale"], 0, a["kc"], a["vc"],
                                 a["cap"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(start=None), _lib.GQA_ERR_INVALID_ARG),          # positions are required
    (dict(kc=None), _lib.GQA_ERR_INVALID_ARG),             # chunks need the cache
    (dict(C=0), _lib.GQA_ERR_INVALID_ARG),
    (dict(kend=513), _lib.GQA_ERR_INVALID_ARG),            # beyond cap
    (dict(kend=0), _lib.GQA_ERR_INVALID_ARG),
    (dict(h_q=4, h_kv=28), _lib.GQA_ERR_INVALID_ARG),
    (dict(d=96), _lib.GQA_ERR_UNSUPPORTED),
    (dict(h_q=65536, h_kv=1), _lib.GQA_ERR_UNSUPPORTED),   # a grid dimension
    (dict(kc=FAKE + 8), _lib.GQA_ERR_INVALID_ARG),         # misaligned
    (dict(wsb=64), _lib.GQA_ERR_WORKSPACE),
    (dict(k=None), _lib.GQA_ERR_INVALID_ARG),              # k and v: both or neither
])
def test_prefill_chunk_rejects(lib, kw, code):
    assert chunk_call(lib, **kw) == code
    assert lib.gqa_last_error()


def ragged_call(lib, **kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, o=FAKE, in_dt=1, out_dt=0, B=2, h_q=28, h_kv=4, d=128,
             cap=64, kvl=FAKE, qpos=FAKE, max_kv=64, theta=1e6, scale=0.088, ws=FAKE,
             wsb=1 << 40, stream=None)
    a.update(kw)
    return lib.gqa_decode_ragged(a["q"], a["kc"], a["vc"], a["o"], a["in_dt"], a["out_dt"],
                                 a["B"], a["h_q"], a["h_kv"], a["d"], a["cap"], a["kvl"],
                                 a["qpos"], a["max_kv"], a["theta"], a["scale"], 0, a["ws"],
                                 a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(kvl=None), _lib.GQA_ERR_INVALID_ARG),
    (dict(max_kv=65), _lib.GQA_ERR_INVALID_ARG),           # longer than the cache
    (dict(max_kv=0), _lib.GQA_ERR_INVALID_ARG),
    (dict(out_dt=3), _lib.GQA_ERR_INVALID_ARG),
    (dict(wsb=0), _lib.GQA_ERR_WORKSPACE),
])
def test_decode_ragged_rejects(lib, kw, code):
    assert ragged_call(lib, **kw) == code
    assert lib.gqa_last_error()


def append_call(lib, **kw):
    a = dict(q=FAKE, kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, o=FAKE, in_dt=1, out_dt=0, B=2, h_q=28,
             h_kv=4, d=128, cap=64, pos=FAKE, max_pos=63, theta=1e6, scale=0.088, ws=FAKE,
             wsb=1 << 40, stream=None)
    a.update(kw)
    return lib.gqa_decode_append(a["q"], a["kn"], a["vn"], a["kc"], a["vc"], a["o"], a["in_dt"],
                                 a["out_dt"], a["B"], a["h_q"], a["h_kv"], a["d"], a["cap"],
                                 a["pos"], a["max_pos"], a["theta"], a["scale"], a["ws"],
                                 a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(pos=None), _lib.GQA_ERR_INVALID_ARG),
    (dict(kn=None), _lib.GQA_ERR_INVALID_ARG),
    (dict(max_pos=64), _lib.GQA_ERR_INVALID_ARG),          # row 64 is outside a 64-row cache
    (dict(max_pos=-1), _lib.GQA_ERR_INVALID_ARG),
    (dict(out_dt=5), _lib.GQA_ERR_INVALID_ARG),            # checked before the cache is touched
    (dict(h_q=30), _lib.GQA_ERR_INVALID_ARG),
    (dict(vn=FAKE + 2), _lib.GQA_ERR_INVALID_ARG),
    (dict(wsb=8), _lib.GQA_ERR_WORKSPACE),
])
def test_decode_append_rejects(lib, kw, code):
    assert append_call(lib, **kw) == code
    assert lib.gqa_last_error()


def test_chunk_workspace_sizes(lib):
    # bf16: the one-shot layout sized for kend keys; fp32: the size of a cos/sin
    # table, a region the fp32 kernels (which form their own cos/sin) leave unused
    assert (lib.gqa_prefill_chunk_workspace_size(1, 4, 4096, 4, 128)
            == lib.gqa_prefill_workspace_size(1, 4, 4096, 4, 128))
    assert lib.gqa_prefill_chunk_workspace_size(0, 1, 1000, 2, 64) == 1000 * 32 * 8


def epilogue_call(lib, **kw):
    a = dict(qkv=FAKE, bias=None, q_out=FAKE, kc=FAKE, vc=FAKE, dt=1, B=2, C=16, h_q=28, h_kv=4,
             d=128, cap=64, start=FAKE, len=None, kend=64, theta=1e6, stream=None)
    a.update(kw)
    return lib.gqa_qkv_epilogue(a["qkv"], a["bias"], a["q_out"], a["kc"], a["vc"], a["dt"],
                                a["B"], a["C"], a["h_q"], a["h_kv"], a["d"], a["cap"],
                                a["start"], a["len"], a["kend"], a["theta"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(qkv=None), _lib.GQA_ERR_INVALID_ARG),
    (dict(start=None), _lib.GQA_ERR_INVALID_ARG),
    (dict(vc=None), _lib.GQA_ERR_INVALID_ARG),
    (dict(kend=65), _lib.GQA_ERR_INVALID_ARG),
    (dict(h_q=4, h_kv=28), _lib.GQA_ERR_INVALID_ARG),
    (dict(d=96), _lib.GQA_ERR_UNSUPPORTED),
    (dict(bias=FAKE + 4), _lib.GQA_ERR_INVALID_ARG),       # misaligned bias
    (dict(dt=2), _lib.GQA_ERR_INVALID_ARG),
    (dict(theta=0.5), _lib.GQA_ERR_INVALID_ARG),
])
def test_qkv_epilogue_rejects(lib, kw, code):
    assert epilogue_call(lib, **kw) == code
    assert lib.gqa_last_error()


def paged_call(lib, **kw):
    a = dict(q=FAKE, kn=None, vn=None, kp=FAKE, vp=FAKE, o=FAKE, in_dt=1, out_dt=0, B=2, h_q=28,
             h_kv=4, d=128, ps=16, num_pages=64, bt=FAKE, max_pages=8, kvl=FAKE, qpos=FAKE,
             max_kv=128, theta=1e6, scale=0.088, qrot=0, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return lib.gqa_decode_paged(a["q"], a["kn"], a["vn"], a["kp"], a["vp"], a["o"], a["in_dt"],
                                a["out_dt"], a["B"], a["h_q"], a["h_kv"], a["d"], a["ps"],
                                a["num_pages"], a["bt"], a["max_pages"], a["kvl"], a["qpos"],
                                a["max_kv"], a["theta"], a["scale"], a["qrot"], a["ws"], a["wsb"],
                                a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(bt=None), _lib.GQA_ERR_INVALID_ARG),
    (dict(ps=24), _lib.GQA_ERR_INVALID_ARG),               # not a power of two
    (dict(ps=0), _lib.GQA_ERR_INVALID_ARG),
    (dict(max_kv=129), _lib.GQA_ERR_INVALID_ARG),          # beyond max_pages * page_size
    (dict(kn=FAKE), _lib.GQA_ERR_INVALID_ARG),             # v_new missing
    (dict(kn=FAKE, vn=FAKE), _lib.GQA_ERR_INVALID_ARG),    # append mode takes no kv_len
    (dict(kvl=None), _lib.GQA_ERR_INVALID_ARG),            # neither kv_len nor append
    (dict(num_pages=0), _lib.GQA_ERR_INVALID_ARG),
    (dict(h_q=30), _lib.GQA_ERR_INVALID_ARG),
    (dict(wsb=4), _lib.GQA_ERR_WORKSPACE),
])
def test_decode_paged_rejects(lib, kw, code):
    assert paged_call(lib, **kw) == code
    assert lib.gqa_last_error()


def test_set_rope_yarn_rejects(lib):
    assert lib.gqa_set_rope_yarn(0.5, 32768.0, 32.0, 1.0) == _lib.GQA_ERR_INVALID_ARG
    assert lib.gqa_set_rope_yarn(4.0, 0.0, 32.0, 1.0) == _lib.GQA_ERR_INVALID_ARG
    assert lib.gqa_set_rope_yarn(4.0, 32768.0, 1.0, 32.0) == _lib.GQA_ERR_INVALID_ARG
    assert lib.gqa_set_rope_yarn(float("nan"), 32768.0, 32.0, 1.0) == _lib.GQA_ERR_INVALID_ARG
    assert lib.gqa_set_rope_yarn(4.0, 32768.0, 32.0, 1.0) == _lib.GQA_OK
    assert lib.gqa_set_rope_yarn(1.0, 0.0, 0.0, 0.0) == _lib.GQA_OK   # back to plain RoPE


C_CONSUMER = os.path.join(ROOT, "tests", "c_abi", "consumer.c")


def test_c99_consumer_compiles_links_and_runs(lib, tmp_path):
    """A C99 translation unit that includes only gqa.h compiles warning-free
    under -pedantic, links against libgqa.so by name, and its host-side calls
    of every entry point behave as the header states."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    src = open(C_CONSUMER).read()
    missing = [n for n in header_functions() if re.search(r"\b%s\s*\(" % n, src) is None]
    assert not missing, f"consumer.c does not call {missing}"
    obj = tmp_path / "consumer.o"
    exe = tmp_path / "consumer"
    libdir = os.path.dirname(_lib.LIB_PATH)
    subprocess.run([gcc, "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror",
                    "-I", os.path.join(ROOT, "include"), "-c", C_CONSUMER, "-o", str(obj)],
                   check=True, capture_output=True, text=True)
    subprocess.run([gcc, str(obj), "-o", str(exe), "-L", libdir, "-lgqa",
                    "-Wl,-rpath," + libdir], check=True, capture_output=True, text=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "c99 consumer ok" in res.stdout
