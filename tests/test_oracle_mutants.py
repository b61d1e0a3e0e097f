"""Plant plausible mistakes in a private copy of the oracle (on the CPU) and
check that at least one pin catches each of them."""

import importlib.util
import math
import os
import sys

import numpy as np
import pytest

from tests.oracle_pins import ALL_PINS

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "gqa_oracle.py")


def fresh_oracle():
    spec = importlib.util.spec_from_file_location("oracle_mutant", ORACLE_SRC)
    mod = importlib.util.module_from_spec(spec)
    sys.modules["oracle_mutant"] = mod    # dataclasses look the module up by name
    spec.loader.exec_module(mod)
    return mod


def _rope_variant(mod, kind):
    orig_inv = mod.inv_freq

    def rope(x, positions, theta=mod.ROPE_THETA):
        x = np.asarray(x, np.float64)
        d = x.shape[-1]
        half = d // 2
        pos = np.asarray(positions, np.float64)
        ang = pos[..., None] * orig_inv(d, theta)
        c = np.cos(ang)[..., None, :]
        s = np.sin(ang)[..., None, :]
        if kind == "interleaved":
            x1, x2 = x[..., 0::2], x[..., 1::2]
            out = np.empty_like(x)
            out[..., 0::2] = x1 * c - x2 * s
            out[..., 1::2] = x2 * c + x1 * s
            return out
        x1, x2 = x[..., :half], x[..., half:]
        if kind == "clockwise":
            return np.concatenate([x1 * c + x2 * s, x2 * c - x1 * s], axis=-1)
        if kind == "dropped_term":
            return np.concatenate([x1 * c, x2 * c + x1 * s], axis=-1)
        raise AssertionError(kind)
    return rope


def m_group_tiled(mod):
    mod.kv_group = lambda t, h_q, h_kv: t % h_kv


def m_group_off_by_one(mod):
    mod.kv_group = lambda t, h_q, h_kv: min((t + 1) // (h_q // h_kv), h_kv - 1)


def m_rope_interleaved(mod):
    mod.rope = _rope_variant(mod, "interleaved")


def m_rope_clockwise(mod):
    mod.rope = _rope_variant(mod, "clockwise")


def m_rope_dropped_term(mod):
    mod.rope = _rope_variant(mod, "dropped_term")


def m_freq_no_factor_two(mod):
    mod.inv_freq = lambda d, theta=1e6: np.power(theta, -np.arange(d // 2) / d)


def m_theta_1e4(mod):
    orig = mod.inv_freq
    mod.inv_freq = lambda d, theta=1e6: orig(d, 1.0e4)


def m_mask_strict(mod):
    mod.visible = lambda qp, kp: np.asarray(kp)[None, :] < np.asarray(qp)[:, None]


def m_mask_transposed(mod):
    mod.visible = lambda qp, kp: np.asarray(kp)[None, :] >= np.asarray(qp)[:, None]


def m_no_scale(mod):
    orig = mod.head_weights
    mod.head_weights = lambda q, k, scale, vis: orig(q, k, 1.0, vis)


def m_transposed_weights(mod):
    orig = mod.head_weights

    def attend(q, k, v, scale, vis):
        return orig(q, k, scale, vis).T @ np.asarray(v, np.float64)
    mod.attend = attend


def m_softmax_no_norm(mod):
    def softmax_rows(s, vis):
        s = np.where(vis, s, -np.inf)
        return np.exp(s - np.max(s, axis=-1, keepdims=True))
    mod.softmax_rows = softmax_rows


def m_decode_unrotated_query(mod):
    orig = mod.rope

    def rope(x, positions, theta=mod.ROPE_THETA):
        x = np.asarray(x)
        if x.ndim == 4 and x.shape[1] == 1 and np.size(positions) == 1 and x.shape[0] > 1:
            return np.asarray(x, np.float64)
        return orig(x, positions, theta)
    mod.rope = rope


def m_chunk_position_shift(mod):
    mod.chunk_positions = lambda start, n: np.arange(start + 1, start + 1 + n)


def m_ragged_first_value(mod):
    def per_sequence(values, B):
        a = np.asarray(values, np.int64).reshape(-1)
        return np.full(B, a[0], np.int64)
    mod.per_sequence = per_sequence


def m_cached_key_unrotated(mod):
    orig = mod.cache_append

    def cache_append(k_cache, v_cache, k_new, v_new, start, length=None, theta=mod.ROPE_THETA):
        saved = mod.rope
        mod.rope = lambda x, positions, theta=theta: np.asarray(x, np.float64)
        try:
            return orig(k_cache, v_cache, k_new, v_new, start, length, theta)
        finally:
            mod.rope = saved
    mod.cache_append = cache_append


def m_qkv_k_v_swapped(mod):
    orig = mod.qkv_sections

    def qkv_sections(h_q, h_kv, d):
        q, k, v = orig(h_q, h_kv, d)
        return q, v, k
    mod.qkv_sections = qkv_sections


def m_qkv_bias_dropped(mod):
    orig = mod.qkv_epilogue
    mod.qkv_epilogue = lambda qkv, bias, *a, **kw: orig(qkv, np.zeros_like(bias), *a, **kw)


def m_qkv_heads_transposed(mod):
    orig = mod.qkv_epilogue

    def qkv_epilogue(qkv, bias, k_cache, v_cache, h_q, h_kv, start, length=None,
                     theta=mod.ROPE_THETA):
        x = np.asarray(qkv, np.float64)
        B, C, width = x.shape
        d = width // (h_q + 2 * h_kv)
        perm = []
        for lo, n in ((0, h_q), (h_q * d, h_kv), ((h_q + h_kv) * d, h_kv)):
            perm += [lo + j * n + h for h in range(n) for j in range(d)]   # dim-major heads
        return orig(x[..., perm], np.asarray(bias)[perm], k_cache, v_cache, h_q, h_kv, start,
                    length, theta)
    mod.qkv_epilogue = qkv_epilogue


def m_paged_row_major_page(mod):
    def paged_rows(pool, block_table, b, n_rows, page_size):
        pos = np.arange(n_rows)
        pages = np.asarray(block_table)[b][pos // page_size]
        pool = np.asarray(pool, np.float64)
        flat = pool.reshape(pool.shape[0], -1, pool.shape[-1])      # page as [ps*h_kv] token-major
        h_kv = pool.shape[1]
        return np.stack([flat[pages, (pos % page_size) * h_kv + u] for u in range(h_kv)], axis=1)
    mod.paged_rows = paged_rows


def m_paged_page_of_next_block(mod):
    orig = mod.paged_rows

    def paged_rows(pool, block_table, b, n_rows, page_size):
        bt = np.asarray(block_table)
        shifted = np.concatenate([bt[:, 1:], bt[:, -1:]], axis=1)
        return orig(pool, shifted, b, n_rows, page_size)
    mod.paged_rows = paged_rows


def m_yarn_ramp_reversed(mod):
    orig = mod.yarn_ramp
    mod.yarn_ramp = lambda spec, d: 1.0 - orig(spec, d)


def m_yarn_no_attention_factor(mod):
    mod.rope_mscale = lambda theta: 1.0


def m_yarn_factor_squared(mod):
    orig = mod.inv_freq

    def inv_freq(d, theta=mod.ROPE_THETA):
        if isinstance(theta, mod.YaRN) and theta.factor != 1.0:
            import dataclasses
            theta = dataclasses.replace(theta, factor=theta.factor ** 2)
        return orig(d, theta)
    mod.inv_freq = inv_freq


def m_yarn_round_bounds(mod):
    """Ramp bounds rounded to the nearest pair instead of floor / ceil."""
    def yarn_ramp(spec, d):
        def corr_dim(n):
            return d * math.log(spec.original_max_position / (n * 2.0 * math.pi)) / (
                2.0 * math.log(spec.theta))
        lo = max(round(corr_dim(spec.beta_fast)), 0)
        hi = min(round(corr_dim(spec.beta_slow)), d - 1)
        j = np.arange(d // 2, dtype=np.float64)
        return np.clip((j - lo) / (hi - lo), 0.0, 1.0)
    mod.yarn_ramp = yarn_ramp


def m_yarn_blend_in_turns(mod):
    """Ramp linear in the number of turns over the window, not in the pair index."""
    def yarn_ramp(spec, d):
        j = np.arange(d // 2, dtype=np.float64)
        turns = spec.original_max_position * spec.theta ** (-2.0 * j / d) / (2.0 * math.pi)
        return np.clip((spec.beta_fast - turns) / (spec.beta_fast - spec.beta_slow), 0.0, 1.0)
    mod.yarn_ramp = yarn_ramp


def m_group_rows_short_keys(mod):
    """Row slices that drop the diagonal key of their last row."""
    orig = mod.prefill_group_rows

    def prefill_group_rows(q_b, k_b, v_b, u, r0, r1, theta=mod.ROPE_THETA, scale=None,
                           causal=True):
        out = orig(q_b, k_b, v_b, u, r0, r1, theta, scale, causal)
        if causal and r1 - r0 > 1:
            out[-1] = orig(q_b[:r1 - 1], k_b[:r1 - 1], v_b[:r1 - 1], u, r1 - 2, r1 - 1, theta,
                           scale, causal)[0]
        return out
    mod.prefill_group_rows = prefill_group_rows


def m_softmax_no_max(mod):
    """exp of the raw scores (no max subtraction): overflows for large scores."""
    def softmax_rows(s, vis):
        s = np.where(vis, s, -np.inf)
        e = np.exp(s)
        return e / np.sum(e, axis=-1, keepdims=True)
    mod.softmax_rows = softmax_rows


def m_softmax_max_over_masked(mod):
    """Row max taken before masking, so a masked key's score can underflow
    every visible weight."""
    def softmax_rows(s, vis):
        m = np.max(s, axis=-1, keepdims=True)
        e = np.where(vis, np.exp(s - m), 0.0)
        return e / np.sum(e, axis=-1, keepdims=True)
    mod.softmax_rows = softmax_rows


def m_cache_v_rotated(mod):
    """The appended V rows are rotated like K."""
    orig = mod.cache_append

    def cache_append(k_cache, v_cache, k_new, v_new, start, length=None,
                     theta=mod.ROPE_THETA):
        B, C = np.shape(k_new)[:2]
        kc, vc = orig(k_cache, v_cache, k_new, v_new, start, length, theta)
        st = mod.per_sequence(start, B)
        nn = mod.per_sequence(C if length is None else length, B)
        for b in range(B):
            n = int(nn[b])
            if n:
                pos = mod.chunk_positions(int(st[b]), n)
                vc[b, pos] = mod.rope(np.asarray(v_new[b, :n], np.float64), pos, theta)
        return kc, vc
    mod.cache_append = cache_append


def m_qkv_bias_after_rope(mod):
    """The QKV bias is added after the rotation instead of before it."""
    orig = mod.qkv_epilogue

    def qkv_epilogue(qkv, bias, k_cache, v_cache, h_q, h_kv, start, length=None,
                     theta=mod.ROPE_THETA):
        x = np.asarray(bias, np.float64)
        q_out, kc, vc = orig(qkv, np.zeros_like(x), k_cache, v_cache, h_q, h_kv, start,
                             length, theta)
        d = x.shape[-1] // (h_q + 2 * h_kv)
        (q0, q1), (k0, k1), (v0, v1) = mod.qkv_sections(h_q, h_kv, d)
        q_out = q_out + x[q0:q1].reshape(h_q, d)
        B, C = np.shape(qkv)[:2]
        st = mod.per_sequence(start, B)
        nn = mod.per_sequence(C if length is None else length, B)
        for b in range(B):
            n = int(nn[b])
            if n:
                pos = mod.chunk_positions(int(st[b]), n)
                kc[b, pos] += x[k0:k1].reshape(h_kv, d)
                vc[b, pos] += x[v0:v1].reshape(h_kv, d)
        return q_out, kc, vc
    mod.qkv_epilogue = qkv_epilogue


def m_cached_query_misses_own_key(mod):
    """Queries against the cache see keys strictly before their position
    (position 0 keeps its own key, so no row is empty)."""
    orig, orig_vis = mod.attend_cached, mod.visible

    def strict(qp, kp):
        kp, qp = np.asarray(kp)[None, :], np.asarray(qp)[:, None]
        return (kp < qp) | ((kp == 0) & (qp == 0))

    def attend_cached(q, q_pos, k_cache, v_cache, kv_len, theta=mod.ROPE_THETA, scale=None,
                      q_rotated=False):
        mod.visible = strict
        try:
            return orig(q, q_pos, k_cache, v_cache, kv_len, theta, scale, q_rotated)
        finally:
            mod.visible = orig_vis
    mod.attend_cached = attend_cached


MUTANTS = [m_group_tiled, m_group_off_by_one, m_rope_interleaved,
           m_rope_clockwise, m_rope_dropped_term, m_freq_no_factor_two,
           m_theta_1e4, m_mask_strict, m_mask_transposed, m_no_scale,
           m_transposed_weights, m_softmax_no_norm, m_decode_unrotated_query,
           m_chunk_position_shift, m_ragged_first_value, m_cached_key_unrotated,
           m_qkv_k_v_swapped, m_qkv_bias_dropped, m_qkv_heads_transposed,
           m_paged_row_major_page, m_paged_page_of_next_block, m_yarn_ramp_reversed,
           m_yarn_no_attention_factor, m_yarn_factor_squared, m_yarn_round_bounds,
           m_yarn_blend_in_turns, m_group_rows_short_keys, m_softmax_no_max,
           m_softmax_max_over_masked, m_cache_v_rotated, m_qkv_bias_after_rope,
           m_cached_query_misses_own_key]


def failing_pins(mod):
    failed = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except Exception as e:   # any error counts as the pin catching it
            failed.append((pin.__name__, type(e).__name__))
    return failed


def test_unmutated_copy_passes():
    assert failing_pins(fresh_oracle()) == []


@pytest.mark.parametrize("mutate", MUTANTS, ids=lambda m: m.__name__)
def test_mutant_is_caught(mutate):
    mod = fresh_oracle()
    mutate(mod)
    assert failing_pins(mod), f"no pin catches {mutate.__name__}"
