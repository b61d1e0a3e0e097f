"""Pins for the fp64 oracle: checks that tie it to something other than itself.

Each ``pin_*`` takes the oracle module (or a deliberately broken copy of it,
see test_oracle_mutants.py) and raises AssertionError on a mismatch.  The
pins come from the pages' worked example, closed forms of a plane rotation,
PyTorch's SDPA in float64 (a library routine the GQA case reduces to),
brute-force loops and the invariants the pages state.
"""

from __future__ import annotations

import cmath
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def close(a, b, tol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


# ------------------------------------------------------------------ RoPE --

def pin_inv_freq_closed_form(orc):
    """omega_0 = 1 and omega_{d/4} = theta^(-1/2) = 1e-3 for theta = 1e6; the
    ratio of neighbours is theta^(-2/d) (geometric ladder over d/2 pairs)."""
    for d in (4, 8, 64, 128):
        w = orc.inv_freq(d, 1.0e6)
        assert w.shape == (d // 2,), "inv_freq length"
        close(w[0], 1.0, 0.0, "omega_0")
        close(w[d // 4], 1.0e-3, 1e-18, f"omega_(d/4) d={d}")
        close(w[1:] / w[:-1], np.full(d // 2 - 1, 10.0 ** (-12.0 / d)), 1e-14,
              f"omega ratio d={d}")
    close(orc.inv_freq(2, 1.0e6), [1.0], 0.0, "d=2")


def pin_rope_d2_is_plane_rotation(orc):
    """d = 2: one pair with omega = 1, so position m turns (a, b) by m radians,
    i.e. multiplies a + ib by e^{im}."""
    rng = _rng(1)
    for m in (0, 1, 2, 7, 1000, 32767, 32768):
        a, b = _rand(rng, 2)
        z = complex(a, b) * cmath.exp(1j * m)
        out = orc.rope(np.array([[[[a, b]]]]), [m], 1.0e6)[0, 0, 0]
        close(out, [z.real, z.imag], 1e-12, f"plane rotation m={m}")


def pin_rope_half_split_pairing(orc):
    """Dimension j pairs with j + d/2: a unit vector on dim j rotated at m has
    its only non-zeros on dims j (cos) and j + d/2 (sin of m*theta^(-2j/d))."""
    d = 8
    for j in range(d // 2):
        e = np.zeros((1, 1, 1, d))
        e[..., j] = 1.0
        m = 3
        ang = m * 1.0e6 ** (-2.0 * j / d)
        want = np.zeros(d)
        want[j] = math.cos(ang)
        want[j + d // 2] = math.sin(ang)
        close(orc.rope(e, [m], 1.0e6)[0, 0, 0], want, 1e-14, f"pair of dim {j}")


def pin_rope_norm(orc):
    """Rotation leaves every row's length unchanged (pages: RoPE keeps the
    vector length and only changes phases)."""
    rng = _rng(2)
    x = _rand(rng, 2, 5, 3, 128)
    pos = np.array([0, 1, 4095, 32767, 32768])
    r = orc.rope(x, pos, 1.0e6)
    close(np.linalg.norm(r, axis=-1), np.linalg.norm(x, axis=-1), 1e-12, "norms")


def pin_rope_relative(orc):
    """q'_m . k'_n depends only on m - n (pages: S_ij reflects i - j)."""
    rng = _rng(3)
    q = _rand(rng, 1, 1, 1, 64)
    k = _rand(rng, 1, 1, 1, 64)
    for m, n, c in ((5, 2, 100), (4096, 0, 28000), (32767, 1, 1), (9, 9, 32000)):
        a = np.sum(orc.rope(q, [m])[0, 0, 0] * orc.rope(k, [n])[0, 0, 0])
        b = np.sum(orc.rope(q, [m + c])[0, 0, 0] * orc.rope(k, [n + c])[0, 0, 0])
        close(a, b, 1e-10, f"relative m={m} n={n} c={c}")


def pin_rope_group_law(orc):
    """R(0) = I and R(n) R(m) = R(m + n)."""
    rng = _rng(4)
    x = _rand(rng, 1, 3, 2, 16)
    close(orc.rope(x, [0, 0, 0]), x, 0.0, "R(0)")
    m = np.array([1, 50, 20000])
    n = np.array([7, 3, 12767])
    close(orc.rope(orc.rope(x, m), n), orc.rope(x, m + n), 1e-10, "R(n)R(m)")


# ------------------------------------------------------------- grouping --

def pin_group_example(orc):
    """The pages' Qwen2-7B example: heads 1-7 read group 1, heads 8-14 group 2.
    V of group u is the constant u+1 everywhere, so output head t must equal
    the 1-based group the table lists for it."""
    rows = read_table("group_mapping_qwen2_7b.txt")
    h_q = int(rows[0][1])
    h_kv = int(rows[1][1])
    table = [(int(a), int(b)) for a, b in rows[2:]]
    rng = _rng(5)
    L, d = 4, 8
    q = _rand(rng, 1, L, h_q, d)
    k = _rand(rng, 1, L, h_kv, d)
    v = np.empty((1, L, h_kv, d))
    for u in range(h_kv):
        v[:, :, u, :] = u + 1
    o = orc.prefill(q, k, v)
    for t1, u1 in table:
        close(o[0, :, t1 - 1, :], np.full((L, d), float(u1)), 1e-12,
              f"head {t1} -> group {u1}")


def pin_repeat_interleave(orc):
    """GQA equals MHA after expanding K/V with repeat_interleave along heads
    (docs.keinmal.top pitfall 2), and differs from tiling the groups."""
    rng = _rng(6)
    B, L, h_q, h_kv, d = 2, 7, 6, 2, 8
    g = h_q // h_kv
    q = _rand(rng, B, L, h_q, d)
    k = _rand(rng, B, L, h_kv, d)
    v = _rand(rng, B, L, h_kv, d)
    o = orc.prefill(q, k, v)
    o_rep = orc.prefill(q, np.repeat(k, g, axis=2), np.repeat(v, g, axis=2))
    close(o, o_rep, 1e-12, "GQA vs repeat_interleave MHA")
    o_tile = orc.prefill(q, np.tile(k, (1, 1, g, 1)), np.tile(v, (1, 1, g, 1)))
    assert np.max(np.abs(o - o_tile)) > 1e-3, "GQA must differ from tiled repeat"


def pin_sdpa(orc):
    """With the rotation applied, the oracle equals PyTorch's SDPA in float64
    (causal, enable_gqa, default scale 1/sqrt(d)) for MHA (g = 1), MQA
    (h_kv = 1) and GQA (g = 7, the Qwen2 ratio)."""
    rng = _rng(7)
    F = torch.nn.functional
    for (B, L, h_q, h_kv, d) in ((1, 9, 4, 4, 8), (2, 11, 4, 1, 16),
                                 (1, 13, 14, 2, 64), (1, 5, 28, 4, 128)):
        q = _rand(rng, B, L, h_q, d)
        k = _rand(rng, B, L, h_kv, d)
        v = _rand(rng, B, L, h_kv, d)
        pos = np.arange(L)
        qt = torch.from_numpy(orc.rope(q, pos)).permute(0, 2, 1, 3)
        kt = torch.from_numpy(orc.rope(k, pos)).permute(0, 2, 1, 3)
        vt = torch.from_numpy(v).permute(0, 2, 1, 3)
        for causal in (True, False):
            ref = F.scaled_dot_product_attention(qt, kt, vt, is_causal=causal,
                                                 enable_gqa=(h_q != h_kv))
            o = orc.prefill(q, k, v, causal=causal)
            close(o, ref.permute(0, 2, 1, 3).numpy(), 1e-12,
                  f"SDPA B{B} L{L} {h_q}/{h_kv} d{d} causal={causal}")


def pin_brute(orc):
    """Scalar-loop definition vs the vectorised oracle on tiny inputs."""
    rng = _rng(8)
    for (B, L, h_q, h_kv, d, pos0) in ((1, 6, 4, 2, 8, 0), (1, 5, 3, 1, 4, 11),
                                       (2, 4, 2, 2, 2, 0)):
        q = _rand(rng, B, L, h_q, d)
        k = _rand(rng, B, L, h_kv, d)
        v = _rand(rng, B, L, h_kv, d)
        close(orc.prefill(q, k, v, pos0=pos0),
              orc.prefill_brute(q.tolist(), k.tolist(), v.tolist(), pos0=pos0),
              1e-12, f"brute B{B} L{L} {h_q}/{h_kv} d{d}")


# -------------------------------------------------------- softmax/causal --

def pin_softmax_causal(orc):
    """Rows of A sum to 1, weights above the diagonal are exactly 0, row 0 of
    every head is V[0] of its group, and equal rotated keys give the running
    mean of V (closed form A_ij = 1/(i+1))."""
    rng = _rng(9)
    L, d = 10, 16
    qr = _rand(rng, L, d)
    kr = _rand(rng, L, d)
    v = _rand(rng, L, d)
    vis = orc.visible(np.arange(L), np.arange(L))
    A = orc.head_weights(qr, kr, 0.25, vis)
    close(A.sum(axis=1), np.ones(L), 1e-14, "row sums")
    assert np.all(A[np.triu_indices(L, 1)] == 0.0), "future weight not zero"
    assert np.all(A[np.tril_indices(L)] > 0.0), "visible weight not positive"
    o = orc.attend(qr, kr, v, 0.25, vis)
    close(o[0], v[0], 1e-15, "row 0 = V[0]")
    keq = np.repeat(_rand(rng, 1, d), L, axis=0)
    o = orc.attend(qr, keq, v, 0.25, vis)
    close(o, np.cumsum(v, axis=0) / np.arange(1, L + 1)[:, None], 1e-13,
          "equal keys -> prefix mean")


def pin_future_invariance(orc):
    """Output row i does not change when K/V rows after i change."""
    rng = _rng(10)
    B, L, h_q, h_kv, d = 1, 12, 4, 2, 8
    q = _rand(rng, B, L, h_q, d)
    k = _rand(rng, B, L, h_kv, d)
    v = _rand(rng, B, L, h_kv, d)
    o = orc.prefill(q, k, v)
    i = 5
    k2, v2 = k.copy(), v.copy()
    k2[:, i + 1:] = _rand(rng, B, L - i - 1, h_kv, d) * 5
    v2[:, i + 1:] = _rand(rng, B, L - i - 1, h_kv, d) * 5
    o2 = orc.prefill(q, k2, v2)
    close(o2[:, :i + 1], o[:, :i + 1], 1e-13, "rows <= i unchanged")
    assert np.max(np.abs(o2[:, i + 1:] - o[:, i + 1:])) > 1e-3, "later rows must move"


def pin_softmax_extreme_logits(orc):
    """Scores far outside exp's range (|s| ~ 1e3, beyond fp64's e^709): with
    d = 2 the only pair turns by its position in radians, so the scores are
    set by hand.  Query 0 sees key 0 alone (score 1000; the masked key 1
    would score 3000), so its row is V[0] exactly; query 1 scores about
    -841 and -2524, so its weights are 1 and e^-1683 and its row is V[0]
    too.  The softmax must subtract the row max over the visible keys only."""
    c1, s1 = math.cos(1.0), math.sin(1.0)
    q = np.zeros((1, 2, 1, 2))
    q[0, 0, 0] = (1000.0, 0.0)
    q[0, 1, 0] = (0.0, 1000.0)            # turned by 1 rad: (-1000 sin 1, 1000 cos 1)
    k = np.zeros((1, 2, 1, 2))
    k[0, 0, 0] = (1.0, 0.0)
    k[0, 1, 0] = (3.0 * c1, -3.0 * s1)    # turned by 1 rad: (3, 0)
    v = np.zeros((1, 2, 1, 2))
    v[0, 0, 0] = (1.0, 2.0)
    v[0, 1, 0] = (5.0, -7.0)
    o = orc.prefill(q, k, v, scale=1.0)
    close(o[0, :, 0], np.repeat(v[0, :1, 0], 2, axis=0), 1e-12, "extreme logits")


def pin_shift_invariance(orc):
    """Moving every position by c leaves the prefill output unchanged."""
    rng = _rng(11)
    q = _rand(rng, 1, 8, 4, 16)
    k = _rand(rng, 1, 8, 2, 16)
    v = _rand(rng, 1, 8, 2, 16)
    close(orc.prefill(q, k, v, pos0=0), orc.prefill(q, k, v, pos0=32000), 1e-11,
          "shift by 32000")


# --------------------------------------------------------------- decode --

def pin_decode_is_prefill_row(orc):
    """A decode step at position p over the rotated cache rows 0..p equals
    row p of the prefill (the cache holds the same rotated K and V)."""
    rng = _rng(12)
    B, L, h_q, h_kv, d = 2, 9, 14, 2, 16
    q = _rand(rng, B, L, h_q, d)
    k = _rand(rng, B, L, h_kv, d)
    v = _rand(rng, B, L, h_kv, d)
    o = orc.prefill(q, k, v)
    cap = L + 3
    kc = np.zeros((B, cap, h_kv, d))
    vc = np.zeros((B, cap, h_kv, d))
    kc[:, :L] = orc.rope(k, np.arange(L))
    vc[:, :L] = v
    kc[:, L:] = 1e3   # rows past kv_len must be ignored
    vc[:, L:] = 1e3
    for p in (0, 4, L - 1):
        od = orc.decode(q[:, p], kc, vc, kv_len=p + 1, q_pos=p)
        close(od, o[:, p], 1e-12, f"decode at {p}")


def pin_prefill_rows(orc):
    """Sampled-row evaluation equals the full prefill at those rows."""
    rng = _rng(13)
    B, L, h_q, h_kv, d = 2, 17, 6, 3, 8
    q = _rand(rng, B, L, h_q, d)
    k = _rand(rng, B, L, h_kv, d)
    v = _rand(rng, B, L, h_kv, d)
    o = orc.prefill(q, k, v)
    rows = [(0, 0, 0), (1, 16, 5), (0, 9, 3), (1, 3, 2)]
    want = np.stack([o[b, i, t] for b, i, t in rows])
    close(orc.prefill_rows(q, k, v, rows), want, 1e-12, "prefill_rows")


def pin_prefill_group_rows(orc):
    """Row slices of one sequence and one KV group, tiling every row with
    ragged bounds, reassemble the full prefill (causal and not)."""
    rng = _rng(23)
    B, L, h_q, h_kv, d = 2, 23, 6, 2, 8
    q = _rand(rng, B, L, h_q, d)
    k = _rand(rng, B, L, h_kv, d)
    v = _rand(rng, B, L, h_kv, d)
    g = h_q // h_kv
    for causal in (True, False):
        want = orc.prefill(q, k, v, causal=causal)
        got = np.full(want.shape, np.nan)
        for b in range(B):
            for u in range(h_kv):
                for r0, r1 in ((0, 7), (7, 16), (16, 23)):
                    got[b, r0:r1, u * g:(u + 1) * g] = orc.prefill_group_rows(
                        q[b], k[b], v[b], u, r0, r1, causal=causal)
        close(got, want, 1e-12, f"prefill_group_rows (causal={causal})")


# ------------------------------------------------ cache, chunks, ragged --

def pin_chunked_prefill_is_prefill(orc):
    """Feeding a prompt in two chunks through the cache (ragged split points
    per sequence) gives the rows of the one-shot prefill, and leaves the
    cache holding the rotated K and the V of every position."""
    rng = _rng(14)
    B, L, h_q, h_kv, d = 2, 13, 6, 2, 16
    q = _rand(rng, B, L, h_q, d)
    k = _rand(rng, B, L, h_kv, d)
    v = _rand(rng, B, L, h_kv, d)
    want = orc.prefill(q, k, v)
    cap = L + 2
    kc = np.full((B, cap, h_kv, d), 7.0)   # rows never written must not be read
    vc = np.full((B, cap, h_kv, d), 7.0)
    split = np.array([5, 9])
    C1, C2 = 9, 8
    q1 = np.zeros((B, C1, h_q, d)); k1 = np.zeros((B, C1, h_kv, d)); v1 = np.zeros_like(k1)
    q2 = np.zeros((B, C2, h_q, d)); k2 = np.zeros((B, C2, h_kv, d)); v2 = np.zeros_like(k2)
    for b in range(B):
        s0 = split[b]
        q1[b, :s0], k1[b, :s0], v1[b, :s0] = q[b, :s0], k[b, :s0], v[b, :s0]
        n2 = L - s0
        q2[b, :n2], k2[b, :n2], v2[b, :n2] = q[b, s0:], k[b, s0:], v[b, s0:]
    kc, vc = orc.cache_append(kc, vc, k1, v1, 0, split)
    o1 = orc.prefill_chunk(q1, kc, vc, 0, split)
    kc, vc = orc.cache_append(kc, vc, k2, v2, split, L - split)
    o2 = orc.prefill_chunk(q2, kc, vc, split, L - split)
    for b in range(B):
        s0 = split[b]
        close(o1[b, :s0], want[b, :s0], 1e-12, f"first chunk, sequence {b}")
        close(o2[b, :L - s0], want[b, s0:], 1e-12, f"second chunk, sequence {b}")
        assert np.isnan(o1[b, s0:]).all() and np.isnan(o2[b, L - s0:]).all()
    close(kc[:, :L], orc.rope(k, np.arange(L)), 1e-12, "cached K")
    close(vc[:, :L], v, 0.0, "cached V")
    close(kc[:, L:], np.full((B, cap - L, h_kv, d), 7.0), 0.0, "rows past the prompt")


def pin_decode_append_is_prefill_row(orc):
    """A decode step that appends its own K, V at position p (ragged p per
    sequence) returns row p of the prefill over positions 0..p."""
    rng = _rng(15)
    B, L, h_q, h_kv, d = 3, 11, 8, 2, 16
    q = _rand(rng, B, L, h_q, d)
    k = _rand(rng, B, L, h_kv, d)
    v = _rand(rng, B, L, h_kv, d)
    want = orc.prefill(q, k, v)
    pos = np.array([0, 4, 10])
    cap = L
    kc = np.full((B, cap, h_kv, d), -3.0)
    vc = np.full((B, cap, h_kv, d), -3.0)
    kr = orc.rope(k, np.arange(L))
    for b in range(B):
        kc[b, :pos[b]] = kr[b, :pos[b]]
        vc[b, :pos[b]] = v[b, :pos[b]]
    qn = np.stack([q[b, pos[b]] for b in range(B)])
    kn = np.stack([k[b, pos[b]] for b in range(B)])
    vn = np.stack([v[b, pos[b]] for b in range(B)])
    o, kc2, vc2 = orc.decode_append(qn, kn, vn, kc, vc, pos)
    for b in range(B):
        close(o[b], want[b, pos[b]], 1e-12, f"sequence {b} at {pos[b]}")
        close(kc2[b, pos[b]], kr[b, pos[b]], 1e-12, "appended K")
        close(vc2[b, pos[b]], v[b, pos[b]], 0.0, "appended V")
        close(kc2[b, pos[b] + 1:], kc[b, pos[b] + 1:], 0.0, "rows after the new one")


def pin_cache_append_pair0(orc):
    """Pair 0 turns by exactly its position in radians (omega_0 = 1): as a
    complex number, (k'_0 + i k'_{d/2}) = (k_0 + i k_{d/2}) e^{i p}."""
    rng = _rng(16)
    B, C, h_kv, d, cap = 2, 3, 2, 8, 40
    k = _rand(rng, B, C, h_kv, d)
    v = _rand(rng, B, C, h_kv, d)
    start = np.array([30, 2])
    kc, vc = orc.cache_append(np.zeros((B, cap, h_kv, d)), np.zeros((B, cap, h_kv, d)),
                              k, v, start)
    for b in range(B):
        for i in range(C):
            p = int(start[b]) + i
            for u in range(h_kv):
                z = complex(k[b, i, u, 0], k[b, i, u, d // 2]) * cmath.exp(1j * p)
                assert abs(complex(kc[b, p, u, 0], kc[b, p, u, d // 2]) - z) < 1e-12, (b, i, u)


def pin_ragged_decode_is_single(orc):
    """Each sequence of a ragged decode equals a one-sequence decode with its
    own kv_len and position."""
    rng = _rng(17)
    B, cap, h_q, h_kv, d = 3, 20, 6, 3, 8
    q = _rand(rng, B, h_q, d)
    kc = _rand(rng, B, cap, h_kv, d)
    vc = _rand(rng, B, cap, h_kv, d)
    kv_len = np.array([1, 20, 7])
    q_pos = np.array([0, 25, 6])
    o = orc.decode_ragged(q, kc, vc, kv_len, q_pos)
    for b in range(B):
        one = orc.decode(q[b:b + 1], kc[b:b + 1], vc[b:b + 1], int(kv_len[b]), int(q_pos[b]))
        close(o[b], one[0], 1e-12, f"sequence {b}")


# ----------------------------------------------------- QKV epilogue -----

def _layout_code(section, head, dim):
    """A distinct value for every (section, head, dim) of the packed output."""
    return 100.0 * section + head + dim / 1000.0


def pin_qkv_layout(orc):
    """The packed projection output holds the h_q query heads, then the h_kv
    key heads, then the h_kv value heads, each head's d columns contiguous;
    the bias adds column by column.  At position 0 the rotation is the
    identity, so the cached K row shows the layout too."""
    B, h_q, h_kv, d = 2, 6, 2, 8
    width = (h_q + 2 * h_kv) * d
    qkv = np.zeros((B, 1, width))
    for col in range(width):
        if col < h_q * d:
            sec, rem = 0, col
        elif col < (h_q + h_kv) * d:
            sec, rem = 1, col - h_q * d
        else:
            sec, rem = 2, col - (h_q + h_kv) * d
        qkv[:, 0, col] = _layout_code(sec, rem // d, rem % d)
    bias = np.arange(width) * 1e-6
    cap = 3
    q, kc, vc = orc.qkv_epilogue(qkv, bias, np.zeros((B, cap, h_kv, d)),
                                 np.zeros((B, cap, h_kv, d)), h_q, h_kv, 0)
    for b in range(B):
        for t in range(h_q):
            for j in range(d):
                want = _layout_code(0, t, j) + (t * d + j) * 1e-6
                assert abs(q[b, 0, t, j] - want) < 1e-12, ("q", b, t, j)
        for u in range(h_kv):
            for j in range(d):
                kw = _layout_code(1, u, j) + (h_q * d + u * d + j) * 1e-6
                vw = _layout_code(2, u, j) + ((h_q + h_kv) * d + u * d + j) * 1e-6
                assert abs(kc[b, 0, u, j] - kw) < 1e-12, ("k", b, u, j)
                assert abs(vc[b, 0, u, j] - vw) < 1e-12, ("v", b, u, j)


def pin_qkv_epilogue_then_attention(orc):
    """Epilogue (which rotates Q and K), then a chunk attending to the cache
    it filled, equals the one-shot prefill of the biased projections."""
    rng = _rng(18)
    B, L, h_q, h_kv, d = 2, 9, 4, 2, 8
    width = (h_q + 2 * h_kv) * d
    qkv = _rand(rng, B, L, width)
    bias = _rand(rng, width)
    x = qkv + bias
    q = x[..., :h_q * d].reshape(B, L, h_q, d)
    k = x[..., h_q * d:(h_q + h_kv) * d].reshape(B, L, h_kv, d)
    v = x[..., (h_q + h_kv) * d:].reshape(B, L, h_kv, d)
    qe, kc, vc = orc.qkv_epilogue(qkv, bias, np.zeros((B, L, h_kv, d)),
                                  np.zeros((B, L, h_kv, d)), h_q, h_kv, 0)
    close(orc.prefill_chunk(qe, kc, vc, 0, q_rotated=True), orc.prefill(q, k, v), 1e-12,
          "epilogue + chunk")


# ------------------------------------------------------- paged cache ----

def _scatter_to_pages(kc, page_size, n_pages, rng):
    """Scatter a contiguous cache [B, cap, h_kv, d] into a pool under a random
    block table; unused pages hold a poison value."""
    B, cap, h_kv, d = kc.shape
    per_seq = cap // page_size
    perm = rng.permutation(n_pages)[:B * per_seq].reshape(B, per_seq)
    pool = np.full((n_pages, h_kv, page_size, d), 1e6)
    for b in range(B):
        for n in range(per_seq):
            pool[perm[b, n]] = np.transpose(kc[b, n * page_size:(n + 1) * page_size], (1, 0, 2))
    return pool, perm


def pin_paged_decode_is_contiguous(orc):
    """A paged cache holding the same rows under a shuffled block table gives
    the contiguous ragged decode; pages outside the table (poisoned) and
    rows past kv_len are never read."""
    rng = _rng(19)
    B, cap, h_q, h_kv, d, ps = 3, 24, 6, 2, 8, 4
    q = _rand(rng, B, h_q, d)
    kc = _rand(rng, B, cap, h_kv, d)
    vc = _rand(rng, B, cap, h_kv, d)
    kp, bt = _scatter_to_pages(kc, ps, 25, np.random.default_rng(5))
    vp, _ = _scatter_to_pages(vc, ps, 25, np.random.default_rng(5))
    kv_len, q_pos = np.array([1, 13, 24]), np.array([0, 20, 23])
    close(orc.decode_paged(q, kp, vp, bt, ps, kv_len, q_pos),
          orc.decode_ragged(q, kc, vc, kv_len, q_pos), 1e-12, "paged vs contiguous")


def pin_paged_append_is_contiguous(orc):
    """Appending into pages then decoding equals the contiguous appending step."""
    rng = _rng(20)
    B, cap, h_q, h_kv, d, ps = 2, 16, 4, 2, 8, 8
    q = _rand(rng, B, h_q, d)
    kn = _rand(rng, B, h_kv, d)
    vn = _rand(rng, B, h_kv, d)
    kc = _rand(rng, B, cap, h_kv, d)
    vc = _rand(rng, B, cap, h_kv, d)
    pos = np.array([9, 0])
    want, kc2, vc2 = orc.decode_append(q, kn, vn, kc, vc, pos)
    kp, bt = _scatter_to_pages(kc, ps, 7, np.random.default_rng(6))
    vp, _ = _scatter_to_pages(vc, ps, 7, np.random.default_rng(6))
    kp2, vp2 = orc.paged_append(kp, vp, kn, vn, bt, ps, pos)
    close(orc.decode_paged(q, kp2, vp2, bt, ps, pos + 1, pos), want, 1e-12, "paged append")
    for b in range(B):
        close(orc.paged_rows(kp2, bt, b, cap, ps), kc2[b], 1e-12, "pool after append")


# --------------------------------------------------------------- YaRN ----

def pin_yarn_factor_one_is_plain(orc):
    """A YaRN factor of 1 leaves RoPE unchanged."""
    rng = _rng(21)
    x = _rand(rng, 2, 5, 3, 64)
    y = orc.YaRN(factor=1.0)
    close(orc.inv_freq(64, y), orc.inv_freq(64), 0.0, "frequencies")
    close(orc.rope(x, np.arange(100, 105), y), orc.rope(x, np.arange(100, 105)), 0.0, "rotation")


def pin_yarn_regions(orc):
    """Per pair, count the turns n = L_orig * omega / (2 pi) over the original
    context (Qwen2: 32768 positions, base 1e6, extension 4x to 128K).  Pairs
    turning at least twice beta_fast = 32 times keep their frequency; pairs
    turning at most half of beta_slow = 1 times are slowed by the factor
    exactly; every pair lies between, and the slow-down never decreases
    towards low frequencies."""
    d, s = 128, 4.0
    y = orc.YaRN(theta=1.0e6, factor=s, original_max_position=32768.0)
    w = np.array([1.0e6 ** (-2.0 * j / d) for j in range(d // 2)])
    w2 = orc.inv_freq(d, y)
    turns = 32768.0 * w / (2.0 * math.pi)
    keep, slow = turns >= 64.0, turns <= 0.5
    assert keep.sum() >= 8 and slow.sum() >= 8
    assert np.allclose(w2[keep], w[keep], rtol=1e-13, atol=0.0), "kept pairs"
    assert np.allclose(w2[slow], w[slow] / s, rtol=1e-13, atol=0.0), "slowed pairs"
    assert np.all(w2 <= w * (1 + 1e-15)) and np.all(w2 >= w / s * (1 - 1e-15))
    ratio = w / w2
    assert np.all(np.diff(ratio) >= -1e-12)


def _yarn_golden():
    """tests/golden/yarn_qwen2.txt: Qwen2's 4x YaRN setting, closed form in
    decimal arithmetic (pairs 0, 20-43, 63; ramp bounds; attention factor)."""
    meta, pairs = {}, []
    for row in read_table("yarn_qwen2.txt"):
        if row[0] in ("lo", "hi", "mscale"):
            meta[row[0]] = float(row[1])
        else:
            num, _, den = row[1].partition("/")
            pairs.append((int(row[0]), float(num) / float(den or 1), float(row[2]),
                          float(row[3])))
    return meta, pairs


QWEN2_YARN = dict(theta=1.0e6, factor=4.0, original_max_position=32768.0, beta_fast=32.0,
                  beta_slow=1.0)


def pin_yarn_golden_frequencies(orc):
    """Every pair of Qwen2's long-context setting (d 128, base 1e6, 32K window,
    4x) against the closed-form values of tests/golden/yarn_qwen2.txt
    ("Qwen-2 详解" (yudonglee.me) §6.2; walkthrough §5.3): the unscaled
    frequencies, the ramp (0 up to pair 23, k/17 at pair 23 + k, 1 from pair
    40) and the blended frequencies, including the whole ramp interior."""
    meta, pairs = _yarn_golden()
    assert (meta["lo"], meta["hi"]) == (23.0, 40.0)
    y = orc.YaRN(**QWEN2_YARN)
    ramp = orc.yarn_ramp(y, 128)
    w0 = orc.inv_freq(128)
    w = orc.inv_freq(128, y)
    for j, r, om, om2 in pairs:
        assert abs(ramp[j] - r) <= 1e-15, f"ramp of pair {j}: {ramp[j]!r} vs {r!r}"
        assert abs(w0[j] - om) <= 1e-14 * om, f"omega of pair {j}: {w0[j]!r} vs {om!r}"
        assert abs(w[j] - om2) <= 1e-14 * om2, f"scaled omega of pair {j}: {w[j]!r} vs {om2!r}"


def pin_yarn_attention_factor(orc):
    """Under Qwen2's 4x setting every rotated row is longer by the golden
    factor 0.1 ln 4 + 1 = 1.1386... (tests/golden/yarn_qwen2.txt), so q'.k'
    at equal positions is q.k times its square (the logit rescale of
    walkthrough §5.3), and q'.k' still depends on m - n only."""
    meta, _ = _yarn_golden()
    ms = meta["mscale"]
    assert abs(ms - 1.1386294361119891) < 1e-15
    rng = _rng(22)
    y = orc.YaRN(**QWEN2_YARN)
    x = _rand(rng, 1, 7, 2, 128)
    xr = orc.rope(x, np.arange(100000, 100007), y)
    close(np.linalg.norm(xr, axis=-1), np.linalg.norm(x, axis=-1) * ms, 1e-12, "norm")
    q = _rand(rng, 1, 1, 1, 128)
    k = _rand(rng, 1, 1, 1, 128)
    same = np.sum(orc.rope(q, [70000], y) * orc.rope(k, [70000], y))
    assert abs(same - ms * ms * np.sum(q * k)) < 1e-11, (same, np.sum(q * k))
    a = np.sum(orc.rope(q, [120000], y) * orc.rope(k, [119990], y))
    b = np.sum(orc.rope(q, [10], y) * orc.rope(k, [0], y))
    assert abs(a - b) < 1e-9, (a, b)


ALL_PINS = [pin_inv_freq_closed_form, pin_rope_d2_is_plane_rotation,
            pin_rope_half_split_pairing, pin_rope_norm, pin_rope_relative,
            pin_rope_group_law, pin_group_example, pin_repeat_interleave,
            pin_sdpa, pin_brute, pin_softmax_causal, pin_softmax_extreme_logits,
            pin_future_invariance,
            pin_shift_invariance, pin_decode_is_prefill_row, pin_prefill_rows,
            pin_prefill_group_rows,
            pin_chunked_prefill_is_prefill, pin_decode_append_is_prefill_row,
            pin_cache_append_pair0, pin_ragged_decode_is_single, pin_qkv_layout,
            pin_qkv_epilogue_then_attention, pin_paged_decode_is_contiguous,
            pin_paged_append_is_contiguous, pin_yarn_factor_one_is_plain, pin_yarn_regions,
            pin_yarn_golden_frequencies, pin_yarn_attention_factor]
