"""fp64 CPU oracle: causal grouped-query attention with RoPE (base 1e6).

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline may import or run this module.  The library never calls it, and it
shares no code with the GPU path: the only thing both sides use is the seeded
input generator in ``synthetic/``.

It is the plain definition, written out in float64 with NumPy, in the order
the pages state it, with no tiling, fusion or reordering.

Sources (web pages on the Qwen2 decoder, cited by title/host and section):
  [evo]  "从 Qwen 1 到 Qwen 2 架构演进到底改了什么" (nxmr.cn)
  [ip]   "Qwen2架构解析：GQA与MoE技术在大模型中的创新应用" (intelliparadigm.com)
  [csdn] Qwen2 technical-report walkthrough (aicoding.csdn.net)
  [yd]   "Qwen-2 详解" (yudonglee.me)
  [kn]   "Qwen2 / Qwen3 的实测配置差异与三个坑" (docs.keinmal.top)

Readings taken where the pages are silent or disagree:
  * RoPE rotates dimension j together with dimension j + d/2 ("half-split"
    pairing); the pages only say "each dimension pair".
  * The frequency exponent uses the head size d (the rotation happens inside
    each head's d_k dims, [csdn] §4.1.3 step 3; Q and K share one table,
    [kn] pitfall 3); [ip] §2.3 writes d_model there, read as a slip.
  * Masked scores are -inf (exact zero weight) ([csdn] §4.1.3 step 4 allows
    "-inf or a very large negative number").
  * Prefill: query i and key j both sit at position (offset + index); key j
    is visible to query i iff pos(j) <= pos(i).
  * Decode: the cache holds keys that are already rotated; the new query is
    rotated at its own position inside; every cached row < kv_len is visible.

Every function here is pinned by tests that do not re-type its formulas:
closed forms of the rotation, SDPA from PyTorch in fp64, the pages' group
example, brute-force loops, and the invariants the pages state.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

ROPE_THETA = 1.0e6   # Qwen2's RoPE base: [evo] §2.3/§3.2, [csdn] §5.2, [kn] config table


# ---------------------------------------------------------------- RoPE ----

@dataclass(frozen=True)
class YaRN:
    """RoPE with YaRN context extension, usable wherever a base theta is.

    The pages: beyond the 32K training window Qwen2 enables YaRN at inference
    to reach 128K ([yd] §6.2), which scales each pair's frequency as
    theta'_i = theta_i / s * alpha_i with a per-dimension ramp alpha_i, and
    rescales the attention logits for length extrapolation ([csdn] §5.3).
    The ramp is the one of the YaRN paper (Peng et al., 2023): pairs that
    turn at least beta_fast times over the original context keep their
    frequency, pairs below beta_slow turns are divided by the factor s, and
    the blend is linear in the pair index between the two correction
    dimensions; cos and sin carry the factor 0.1 ln s + 1."""
    theta: float = ROPE_THETA
    factor: float = 4.0
    original_max_position: float = 32768.0
    beta_fast: float = 32.0
    beta_slow: float = 1.0


def base_theta(theta) -> float:
    return theta.theta if isinstance(theta, YaRN) else float(theta)


def yarn_ramp(spec: YaRN, d: int) -> np.ndarray:
    """Blend weight per pair (0: frequency kept, 1: divided by the factor).
    Pair index of a frequency that turns n times over the original context:
    D(n) = d ln(L_orig / (2 pi n)) / (2 ln theta); the ramp rises linearly
    from floor(D(beta_fast)) to ceil(D(beta_slow)) (bounds clamped to
    [0, d-1])."""
    def corr_dim(n):
        return d * math.log(spec.original_max_position / (n * 2.0 * math.pi)) / (
            2.0 * math.log(spec.theta))
    lo = max(math.floor(corr_dim(spec.beta_fast)), 0)
    hi = min(math.ceil(corr_dim(spec.beta_slow)), d - 1)
    if hi == lo:
        hi += 0.001
    j = np.arange(d // 2, dtype=np.float64)
    return np.clip((j - lo) / (hi - lo), 0.0, 1.0)


def rope_mscale(theta) -> float:
    """Factor on cos and sin: 0.1 ln s + 1 under YaRN with s > 1, else 1."""
    if isinstance(theta, YaRN) and theta.factor > 1.0:
        return 0.1 * math.log(theta.factor) + 1.0
    return 1.0


def inv_freq(d: int, theta=ROPE_THETA) -> np.ndarray:
    """omega_j = theta^(-2j/d), j = 0 .. d/2-1 ([ip] §2.3 angle m*base^(-2i/d);
    [csdn] §5.2: the base generates the inverse frequencies); under YaRN
    blended towards omega_j / s by yarn_ramp."""
    if d % 2:
        raise ValueError("RoPE needs an even head size")
    j = np.arange(d // 2, dtype=np.float64)
    w = np.power(np.float64(base_theta(theta)), -2.0 * j / d)
    if isinstance(theta, YaRN) and theta.factor != 1.0:
        r = yarn_ramp(theta, d)
        w = w * (1.0 - r) + (w / theta.factor) * r
    return w


def rope(x: np.ndarray, positions, theta=ROPE_THETA) -> np.ndarray:
    """Rotate every row of x[..., L, h, d] at its position ([csdn] §3.5.2 and
    §4.1.3 step 3: rotate Q and K per position and per dimension pair; the
    shape is unchanged).  ``positions`` has shape [L] (or broadcasts to
    x.shape[:-2]).  Pair (j, j + d/2) turns by the angle pos * omega_j."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    pos = np.asarray(positions, dtype=np.float64)
    ang = pos[..., None] * inv_freq(d, theta)          # [..., L, d/2]
    ms = rope_mscale(theta)
    c = ms * np.cos(ang)[..., None, :]                 # broadcast over heads
    s = ms * np.sin(ang)[..., None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


# ---------------------------------------------------------- grouping ------

def group_size(h_q: int, h_kv: int) -> int:
    """g = h_q / h_kv ([csdn] §4.1.2); h_q must be a multiple of h_kv."""
    if h_kv < 1 or h_q < 1 or h_q % h_kv:
        raise ValueError(f"h_q={h_q} is not a positive multiple of h_kv={h_kv}")
    return h_q // h_kv


def kv_group(t: int, h_q: int, h_kv: int) -> int:
    """0-based KV group of query head t: u = floor(t / g), the 0-based form of
    [csdn] §4.1.2 / [evo] §2.2 u = floor((t-1)/g) + 1."""
    return t // group_size(h_q, h_kv)


# ---------------------------------------------------------- attention -----

def visible(q_pos, k_pos) -> np.ndarray:
    """Causal mask [Lq, Lk]: key j may be seen by query i iff pos_j <= pos_i
    ([csdn] §4.1.3 step 4: positions j > i are masked)."""
    return np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[:, None]


def softmax_rows(s: np.ndarray, vis: np.ndarray) -> np.ndarray:
    """Row softmax of scores with masked entries at -inf (exact zero weight).
    Subtracts the row max first; every row must see at least one key."""
    s = np.where(vis, s, -np.inf)
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def head_weights(q_rot: np.ndarray, k_rot: np.ndarray, scale: float,
                 vis: np.ndarray) -> np.ndarray:
    """A = softmax(Q' K'^T * scale + M) for one query head and its KV group
    ([csdn] §3.5.2 S_ij = Q'[i].K'[j]/sqrt(d_k); §4.1.3 step 4)."""
    return softmax_rows((q_rot @ k_rot.T) * scale, vis)


def attend(q_rot, k_rot, v, scale, vis) -> np.ndarray:
    """head = A V ([csdn] §4.1.3 step 4)."""
    return head_weights(q_rot, k_rot, scale, vis) @ np.asarray(v, np.float64)


def prefill(q, k, v, theta: float = ROPE_THETA, scale: float | None = None,
            causal: bool = True, pos0: int = 0) -> np.ndarray:
    """Causal GQA prefill.  q [B, L, h_q, d], k/v [B, L, h_kv, d] (pre-RoPE);
    rows sit at positions pos0 .. pos0+L-1.  Returns O [B, L, h_q, d] fp64
    (the per-head outputs side by side, i.e. the concat layout of [csdn]
    §4.1.3 step 5, before W_O).

    Steps as in [csdn] §4.1.3: 3) rotate Q and K; 4) per query head t with
    its group u: scores, causal mask, softmax, times V^(u)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, L, h_q, d = q.shape
    h_kv = k.shape[2]
    group_size(h_q, h_kv)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    pos = np.arange(pos0, pos0 + L)
    qr = rope(q, pos, theta)
    kr = rope(k, pos, theta)
    vis = visible(pos, pos) if causal else np.ones((L, L), bool)
    out = np.empty((B, L, h_q, d), np.float64)
    for b in range(B):
        for t in range(h_q):
            u = kv_group(t, h_q, h_kv)
            out[b, :, t, :] = attend(qr[b, :, t, :], kr[b, :, u, :],
                                     v[b, :, u, :], scale, vis)
    return out


def prefill_rows(q, k, v, rows, theta: float = ROPE_THETA,
                 scale: float | None = None) -> np.ndarray:
    """The same causal prefill, evaluated one output row at a time for a list
    of (b, i, t) triples; returns [len(rows), d].  Row i only needs keys
    0..i, so this serves as the oracle for sampled rows of large inputs."""
    d = q.shape[-1]
    h_q, h_kv = q.shape[2], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.empty((len(rows), d), np.float64)
    for n, (b, i, t) in enumerate(rows):
        u = kv_group(t, h_q, h_kv)
        qr = rope(np.asarray(q[b, i:i + 1, t:t + 1, :], np.float64), [i], theta)[:, 0, :]
        kr = rope(np.asarray(k[b, :i + 1, u:u + 1, :], np.float64),
                  np.arange(i + 1), theta)[:, 0, :]
        out[n] = attend(qr, kr, v[b, :i + 1, u, :], scale,
                        visible([i], np.arange(i + 1)))[0]
    return out


def prefill_group_rows(q_b, k_b, v_b, u: int, r0: int, r1: int,
                       theta: float = ROPE_THETA, scale: float | None = None,
                       causal: bool = True) -> np.ndarray:
    """Rows r0 .. r1-1 of the prefill of one sequence for the g query heads
    of KV group u: q_b [L, h_q, d], k_b/v_b [L, h_kv, d] (pre-RoPE, positions
    0 .. L-1).  Returns [r1 - r0, g, d], equal to
    prefill(q_b[None], k_b[None], v_b[None])[0, r0:r1, u*g:(u+1)*g].

    The same steps as prefill ([csdn] §4.1.3 steps 3-4) restricted to those
    query rows: a causal row i only sees keys 0..i, so keys past r1 - 1 are
    not formed.  Cutting the output into such slices lets the full
    workloads be evaluated piece by piece (and in parallel)."""
    L, h_q, d = np.shape(q_b)
    h_kv = np.shape(k_b)[1]
    g = group_size(h_q, h_kv)
    if not 0 <= r0 < r1 <= L:
        raise ValueError("row range outside the sequence")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    pos = np.arange(L)
    nk = r1 if causal else L
    qr = rope(np.asarray(q_b[r0:r1, u * g:(u + 1) * g], np.float64), pos[r0:r1], theta)
    kr = rope(np.asarray(k_b[:nk, u:u + 1], np.float64), pos[:nk], theta)[:, 0]
    vu = np.asarray(v_b[:nk, u], np.float64)
    vis = visible(pos[r0:r1], pos[:nk]) if causal else np.ones((r1 - r0, nk), bool)
    out = np.empty((r1 - r0, g, d), np.float64)
    for c in range(g):
        if kv_group(u * g + c, h_q, h_kv) != u:
            raise AssertionError("head outside its group")
        out[:, c, :] = attend(qr[:, c, :], kr, vu, scale, vis)
    return out


def decode(q, k_cache, v_cache, kv_len: int, q_pos: int,
           theta: float = ROPE_THETA, scale: float | None = None) -> np.ndarray:
    """One new query token per sequence.  q [B, h_q, d] (pre-RoPE, rotated
    here at q_pos); k_cache/v_cache [B, cap, h_kv, d] hold rotated keys and
    values; rows 0..kv_len-1 are attended ([csdn] §4.1.3: the cache keeps only
    the h_kv groups' K, V, appended each step).  Returns O [B, h_q, d]."""
    q = np.asarray(q, np.float64)
    B, h_q, d = q.shape
    h_kv = k_cache.shape[2]
    if not 1 <= kv_len <= k_cache.shape[1]:
        raise ValueError("kv_len out of range")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    qr = rope(q[:, None, :, :], [q_pos], theta)[:, 0]
    out = np.empty((B, h_q, d), np.float64)
    vis = np.ones((1, kv_len), bool)   # every cached row precedes the query
    for b in range(B):
        kb = np.asarray(k_cache[b, :kv_len], np.float64)
        vb = np.asarray(v_cache[b, :kv_len], np.float64)
        for t in range(h_q):
            u = kv_group(t, h_q, h_kv)
            out[b, t] = attend(qr[b, t][None, :], kb[:, u, :], vb[:, u, :],
                               scale, vis)[0]
    return out


# ------------------------------------------- cache append and chunks -----
#
# Autoregressive use around the path: every step appends the current K and V
# of the h_kv groups to the per-layer cache ([csdn] §4.1.3 closing note), a
# decode step attends to everything cached so far, and a long prompt may be
# fed in chunks whose queries see the cache plus the chunk itself.

def per_sequence(values, B: int) -> np.ndarray:
    """One int64 value per sequence: a scalar is shared, an array is ragged."""
    return np.broadcast_to(np.asarray(values, np.int64), (B,)).copy()


def chunk_positions(start: int, n: int) -> np.ndarray:
    """Positions of the n new rows of a sequence whose first new row sits at
    ``start`` (the rows already cached occupy positions 0 .. start-1)."""
    return np.arange(start, start + n)


def cache_append(k_cache, v_cache, k_new, v_new, start, length=None,
                 theta: float = ROPE_THETA):
    """Append rows to the cache.  k_new/v_new [B, C, h_kv, d] are pre-RoPE;
    row i < length[b] (default C) of sequence b sits at position
    p = start[b] + i, its K is rotated at p and stored, with its V, in cache
    row p.  Returns updated fp64 copies of (k_cache, v_cache)."""
    kc = np.array(k_cache, np.float64, copy=True)
    vc = np.array(v_cache, np.float64, copy=True)
    B, C = np.shape(k_new)[:2]
    start = per_sequence(start, B)
    n_new = per_sequence(C if length is None else length, B)
    for b in range(B):
        n = int(n_new[b])
        if n == 0:
            continue
        pos = chunk_positions(int(start[b]), n)
        if pos[0] < 0 or pos[-1] >= kc.shape[1] or n > C:
            raise ValueError("rows outside the cache")
        kc[b, pos] = rope(np.asarray(k_new[b, :n], np.float64), pos, theta)
        vc[b, pos] = np.asarray(v_new[b, :n], np.float64)
    return kc, vc


def attend_cached(q, q_pos, k_cache, v_cache, kv_len: int,
                  theta: float = ROPE_THETA, scale: float | None = None,
                  q_rotated: bool = False):
    """Queries of one sequence at explicit positions against its cache:
    q [n, h_q, d] pre-RoPE (rotated here at q_pos[n]; already rotated if
    q_rotated); cache rows j < kv_len hold the rotated key and the value of
    position j, visible to a query iff j <= its position.  Returns
    [n, h_q, d]."""
    q = np.asarray(q, np.float64)
    n, h_q, d = q.shape
    h_kv = np.shape(k_cache)[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    qp = np.asarray(q_pos)
    qr = q if q_rotated else rope(q, qp, theta)
    kb = np.asarray(k_cache[:kv_len], np.float64)
    vb = np.asarray(v_cache[:kv_len], np.float64)
    vis = visible(qp, np.arange(kv_len))
    out = np.empty((n, h_q, d), np.float64)
    for t in range(h_q):
        u = kv_group(t, h_q, h_kv)
        out[:, t, :] = attend(qr[:, t, :], kb[:, u, :], vb[:, u, :], scale, vis)
    return out


def prefill_chunk(q, k_cache, v_cache, start, length=None,
                  theta: float = ROPE_THETA, scale: float | None = None,
                  q_rotated: bool = False):
    """Chunked causal prefill against a cache that already holds the chunk's
    own rows (see cache_append): query i < length[b] of sequence b sits at
    position start[b] + i and sees cache rows 0 .. start[b] + i.
    q [B, C, h_q, d]; returns O [B, C, h_q, d] with rows i >= length[b] NaN."""
    q = np.asarray(q, np.float64)
    B, C = q.shape[:2]
    start = per_sequence(start, B)
    n_new = per_sequence(C if length is None else length, B)
    out = np.full(q.shape, np.nan)
    for b in range(B):
        n = int(n_new[b])
        if n == 0:
            continue
        pos = chunk_positions(int(start[b]), n)
        out[b, :n] = attend_cached(q[b, :n], pos, k_cache[b], v_cache[b],
                                   int(pos[-1]) + 1, theta, scale, q_rotated)
    return out


def decode_ragged(q, k_cache, v_cache, kv_len, q_pos,
                  theta: float = ROPE_THETA, scale: float | None = None,
                  q_rotated: bool = False):
    """Decode with one length and one query position per sequence: q [B, h_q,
    d]; sequence b attends to its cache rows 0 .. kv_len[b]-1 from position
    q_pos[b] (kv_len[b] <= q_pos[b] + 1).  Returns O [B, h_q, d]."""
    q = np.asarray(q, np.float64)
    B = q.shape[0]
    kv_len = per_sequence(kv_len, B)
    q_pos = per_sequence(q_pos, B)
    out = np.empty(q.shape, np.float64)
    for b in range(B):
        if not 1 <= kv_len[b] <= min(np.shape(k_cache)[1], q_pos[b] + 1):
            raise ValueError("kv_len out of range")
        out[b] = attend_cached(q[b][None], q_pos[b:b + 1], k_cache[b], v_cache[b],
                               int(kv_len[b]), theta, scale, q_rotated)[0]
    return out


def decode_append(q, k_new, v_new, k_cache, v_cache, pos,
                  theta: float = ROPE_THETA, scale: float | None = None):
    """One autoregressive step: the new token of sequence b sits at position
    pos[b]; its K (rotated there) and V are appended at cache row pos[b],
    then its query attends to rows 0 .. pos[b].  q [B, h_q, d], k_new/v_new
    [B, h_kv, d].  Returns (O [B, h_q, d], k_cache', v_cache')."""
    B = np.shape(q)[0]
    pos = per_sequence(pos, B)
    kc, vc = cache_append(k_cache, v_cache, np.asarray(k_new)[:, None],
                          np.asarray(v_new)[:, None], pos, 1, theta)
    return decode_ragged(q, kc, vc, pos + 1, pos, theta, scale), kc, vc


# --------------------------------------------------------- paged cache ---
#
# A paged cache keeps K (and V) in a pool of fixed-size pages instead of one
# contiguous [cap] range per sequence; PagedAttention manages its memory in
# blocks per KV head ([evo] §2, GQA's effect on inference).  Here a page
# holds page_size consecutive positions of every KV head:
# pool [num_pages, h_kv, page_size, d]; block_table[b][n] is the page that
# holds positions n*page_size .. (n+1)*page_size - 1 of sequence b.

def paged_rows(pool, block_table, b: int, n_rows: int, page_size: int):
    """Rows 0 .. n_rows-1 of sequence b, gathered from the pool in
    position order: [n_rows, h_kv, d]."""
    pos = np.arange(n_rows)
    pages = np.asarray(block_table)[b][pos // page_size]
    return np.asarray(pool, np.float64)[pages, :, pos % page_size, :]


def decode_paged(q, k_pool, v_pool, block_table, page_size: int, kv_len, q_pos,
                 theta: float = ROPE_THETA, scale: float | None = None,
                 q_rotated: bool = False):
    """decode_ragged over a paged cache: sequence b's position j lives in
    page block_table[b][j // page_size], row j % page_size."""
    q = np.asarray(q, np.float64)
    B = q.shape[0]
    kv_len = per_sequence(kv_len, B)
    q_pos = per_sequence(q_pos, B)
    out = np.empty(q.shape, np.float64)
    for b in range(B):
        n = int(kv_len[b])
        kb = paged_rows(k_pool, block_table, b, n, page_size)
        vb = paged_rows(v_pool, block_table, b, n, page_size)
        out[b] = decode_ragged(q[b:b + 1], kb[None], vb[None], n, int(q_pos[b]), theta,
                               scale, q_rotated)[0]
    return out


def paged_append(k_pool, v_pool, k_new, v_new, block_table, page_size: int, pos,
                 theta: float = ROPE_THETA):
    """Write the new token of each sequence (k_new/v_new [B, h_kv, d],
    pre-RoPE) at its position pos[b] of the paged cache, K rotated there.
    Returns updated fp64 copies of both pools."""
    kp = np.array(k_pool, np.float64, copy=True)
    vp = np.array(v_pool, np.float64, copy=True)
    B = np.shape(k_new)[0]
    pos = per_sequence(pos, B)
    for b in range(B):
        p = int(pos[b])
        page = int(np.asarray(block_table)[b][p // page_size])
        kp[page, :, p % page_size, :] = rope(np.asarray(k_new[b], np.float64)[None], [p], theta)[0]
        vp[page, :, p % page_size, :] = np.asarray(v_new[b], np.float64)
    return kp, vp


# ------------------------------------------------ QKV projection epilogue -

def qkv_sections(h_q: int, h_kv: int, d: int):
    """Column ranges of Q, K and V in the packed projection output
    [..., (h_q + 2 h_kv) d]: the h_q query heads, then the h_kv key heads,
    then the h_kv value heads, each head's d columns contiguous."""
    return ((0, h_q * d), (h_q * d, (h_q + h_kv) * d),
            ((h_q + h_kv) * d, (h_q + 2 * h_kv) * d))


def qkv_epilogue(qkv, bias, k_cache, v_cache, h_q: int, h_kv: int, start,
                 length=None, theta: float = ROPE_THETA):
    """The step before attention in a Qwen2 layer: each projection adds its
    bias and the flat output is cut into heads ([csdn] §4.1.3 steps 1-2;
    §4.2: Qwen2 keeps the QKV bias), Q and K are rotated at their position
    (step 3), and the K, V of the h_kv groups go to the cache (closing note
    of §4.1.3).  qkv [B, C, (h_q + 2 h_kv) d] is the packed projection
    output without bias, bias [(h_q + 2 h_kv) d]; token i < length[b] of
    sequence b sits at position start[b] + i.  Returns (q [B, C, h_q, d]
    with bias and rotated -- rows past length[b] NaN --, k_cache',
    v_cache')."""
    x = np.asarray(qkv, np.float64) + np.asarray(bias, np.float64)
    B, C, _ = x.shape
    d = x.shape[-1] // (h_q + 2 * h_kv)
    (q0, q1), (k0, k1), (v0, v1) = qkv_sections(h_q, h_kv, d)
    q = x[..., q0:q1].reshape(B, C, h_q, d)
    k = x[..., k0:k1].reshape(B, C, h_kv, d)
    v = x[..., v0:v1].reshape(B, C, h_kv, d)
    kc, vc = cache_append(k_cache, v_cache, k, v, start, length, theta)
    n_new = per_sequence(C if length is None else length, B)
    q_out = np.full(q.shape, np.nan)
    start = per_sequence(start, B)
    for b in range(B):
        n = int(n_new[b])
        if n:
            q_out[b, :n] = rope(q[b, :n], chunk_positions(int(start[b]), n), theta)
    return q_out, kc, vc


# ------------------------------------------------------- brute force ------

def prefill_brute(q, k, v, theta: float = ROPE_THETA, scale: float | None = None,
                  pos0: int = 0):
    """Scalar-loop causal GQA prefill for tiny inputs (nested Python lists or
    arrays).  Written independently of the vectorised functions above: it
    uses math.cos/sin and plain loops only."""
    B, L, h_q, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    h_kv = len(k[0][0])
    g = h_q // h_kv
    half = d // 2
    if scale is None:
        scale = 1.0 / math.sqrt(d)

    def rot(vec, p):
        outv = [0.0] * d
        for j in range(half):
            a = p * theta ** (-2.0 * j / d)
            c, s = math.cos(a), math.sin(a)
            outv[j] = vec[j] * c - vec[j + half] * s
            outv[j + half] = vec[j + half] * c + vec[j] * s
        return outv

    out = [[[[0.0] * d for _ in range(h_q)] for _ in range(L)] for _ in range(B)]
    for b in range(B):
        for t in range(h_q):
            u = t // g
            kr = [rot([float(x) for x in k[b][j][u]], pos0 + j) for j in range(L)]
            for i in range(L):
                qi = rot([float(x) for x in q[b][i][t]], pos0 + i)
                sc = []
                for j in range(i + 1):
                    sc.append(sum(qi[e] * kr[j][e] for e in range(d)) * scale)
                mx = max(sc)
                w = [math.exp(s - mx) for s in sc]
                tot = sum(w)
                for e in range(d):
                    out[b][i][t][e] = sum(w[j] * float(v[b][j][u][e])
                                          for j in range(i + 1)) / tot
    return np.array(out, dtype=np.float64)
