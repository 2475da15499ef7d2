"""Plant plausible mistakes in copies of the oracle and check that a pin catches each.

The mutants live only here, on the CPU.  A mutant is caught when at least one
pin check raises.
"""
import math

import numpy as np
import pytest

import oracle
import oracle_pins as pins


def _naive_variant(q, k, v, scale, *, mask="causal", max_sub=True, group="div",
                   axis=1, transpose=False, return_probs=False):
    B, H, T, D = q.shape
    Hkv = k.shape[1]
    out = np.empty((B, H, T, v.shape[-1]))
    for b in range(B):
        for h in range(H):
            g = h // (H // Hkv) if group == "div" else h % Hkv
            s = ((k[b, g] @ q[b, h].T) if transpose else (q[b, h] @ k[b, g].T)) * scale
            if mask == "causal":
                s[np.triu(np.ones((T, T), bool), 1)] = -np.inf
            elif mask == "strict":
                s[np.triu(np.ones((T, T), bool), 0)] = -np.inf
            elif mask == "anti":
                s[np.tril(np.ones((T, T), bool), -1)] = -np.inf
            if max_sub:
                s = s - s.max(axis=axis, keepdims=True)
            e = np.exp(s)
            p = e / e.sum(axis=axis, keepdims=True)
            out[b, h] = p @ v[b, g]
    return out


NAIVE_MUTANTS = {
    "no_scale": lambda q, k, v, s, **kw: oracle.naive_causal(q, k, v, 1.0),
    "inverted_scale": lambda q, k, v, s, **kw: oracle.naive_causal(q, k, v, 1.0 / s),
    "no_mask": lambda q, k, v, s, **kw: _naive_variant(q, k, v, s, mask="none"),
    "strict_mask": lambda q, k, v, s, **kw: _naive_variant(q, k, v, s, mask="strict"),
    "anti_causal": lambda q, k, v, s, **kw: _naive_variant(q, k, v, s, mask="anti"),
    "no_max_subtraction": lambda q, k, v, s, **kw: _naive_variant(q, k, v, s, max_sub=False),
    "interleaved_gqa": lambda q, k, v, s, **kw: _naive_variant(q, k, v, s, group="mod"),
    "softmax_over_queries": lambda q, k, v, s, **kw: _naive_variant(q, k, v, s, axis=0),
    "transposed_scores": lambda q, k, v, s, **kw: _naive_variant(q, k, v, s, transpose=True),
    "v_from_k": lambda q, k, v, s, **kw: oracle.naive_causal(q, k, k, s),
}


def _chunked_no_rescale(q, k, v, scale, cq, ck):
    B, H, T, D = q.shape
    Hkv = k.shape[1]
    out = np.empty_like(q)
    for b in range(B):
        for h in range(H):
            g = h // (H // Hkv)
            for i0 in range(0, T, cq):
                i1 = min(i0 + cq, T)
                rows = np.arange(i0, i1)
                m = np.full(i1 - i0, -np.inf); l = np.zeros(i1 - i0); u = np.zeros((i1 - i0, D))
                for j0 in range(0, i1, ck):
                    j1 = min(j0 + ck, T)
                    s = (q[b, h, i0:i1] @ k[b, g, j0:j1].T) * scale
                    s[np.arange(j0, j1)[None, :] > rows[:, None]] = -np.inf
                    m_new = np.maximum(m, s.max(axis=1))
                    e = np.exp(s - m_new[:, None])
                    l = l + e.sum(axis=1)          # planted: missing exp(m - m') rescale
                    u = u + e @ v[b, g, j0:j1]
                    m = m_new
                out[b, h, i0:i1] = u / l[:, None]
    return out


def _decode_short_by_one(q, ck, cv, lengths, scale):
    return oracle.decode_cached(q, ck, cv, np.maximum(np.asarray(lengths) - 1, 1), scale)


def _attend_row_no_normalise(q_row, K, V, scale):
    s = (K @ q_row) * scale
    e = np.exp(s - s.max())
    return e @ V


class _CacheModelOffByOne(oracle.CacheModel):
    def append(self, layer, k_new, v_new):   # planted: writes one slot too far
        for b in range(self.k.shape[1]):
            pos = min(self.lengths[layer, b] + 1, self.max_T - 1)
            self.k[layer, b, :, pos] = k_new[b, :, 0]
            self.v[layer, b, :, pos] = v_new[b, :, 0]
        self.lengths[layer] += 1


def _run_all(overrides):
    """Run every pin with the overridden functions; return the names that failed."""
    failed = []
    naive = overrides.get("naive", oracle.naive_causal)
    calls = {
        "check_kv_bytes": lambda: pins.check_kv_bytes(overrides.get("kv_bytes", oracle.kv_bytes)),
        "check_brute": lambda: pins.check_brute(naive),
        "check_row0_is_v0": lambda: pins.check_row0_is_v0(naive),
        "check_zero_query_prefix_mean": lambda: pins.check_zero_query_prefix_mean(naive),
        "check_two_key_logistic": lambda: pins.check_two_key_logistic(naive),
        "check_rows_sum_to_one": lambda: pins.check_rows_sum_to_one(naive),
        "check_large_scores": lambda: pins.check_large_scores(naive),
        "check_causality": lambda: pins.check_causality(naive),
        "check_gqa_equals_repeated_mha": lambda: pins.check_gqa_equals_repeated_mha(naive),
        "check_torch_sdpa": lambda: pins.check_torch_sdpa(naive),
        "check_chunked": lambda: pins.check_chunked(overrides.get("chunked", oracle.chunked), oracle.naive_causal),
        "check_decode_single_key": lambda: pins.check_decode_single_key(overrides.get("attend_row", oracle.attend_row)),
        "check_decode_permutation": lambda: pins.check_decode_permutation(overrides.get("attend_row", oracle.attend_row)),
        "check_decode_matches_prefill_rows": lambda: pins.check_decode_matches_prefill_rows(
            overrides.get("decode_cached", oracle.decode_cached), oracle.naive_causal),
        "check_cached_equals_recompute": lambda: pins.check_cached_equals_recompute(
            overrides.get("decode_cached", oracle.decode_cached), oracle.decode_recompute,
            overrides.get("CacheModel", oracle.CacheModel)),
        "check_extend_matches_prefill_rows": lambda: pins.check_extend_matches_prefill_rows(
            overrides.get("extend", oracle.extend), oracle.naive_causal),
        "check_chunked_prefill_by_extend": lambda: pins.check_chunked_prefill_by_extend(
            overrides.get("extend", oracle.extend), oracle.naive_causal),
        "check_extend_brute": lambda: pins.check_extend_brute(overrides.get("extend", oracle.extend)),
        "check_window_special_cases": lambda: pins.check_window_special_cases(
            overrides.get("naive_windowed", oracle.naive_windowed), oracle.naive_causal),
        "check_window_brute": lambda: pins.check_window_brute(overrides.get("naive_windowed", oracle.naive_windowed)),
        "check_window_decode_and_extend_rows": lambda: pins.check_window_decode_and_extend_rows(
            overrides.get("decode_cached", oracle.decode_cached), overrides.get("extend", oracle.extend),
            overrides.get("naive_windowed", oracle.naive_windowed)),
        "check_window_ignores_hidden_keys": lambda: pins.check_window_ignores_hidden_keys(
            overrides.get("naive_windowed", oracle.naive_windowed)),
        "check_paged_addressing": lambda: pins.check_paged_addressing(
            overrides.get("PagedCacheModel", oracle.PagedCacheModel)),
        "check_paged_equals_contiguous": lambda: pins.check_paged_equals_contiguous(
            overrides.get("PagedCacheModel", oracle.PagedCacheModel), oracle.decode_paged, oracle.CacheModel),
        "check_paged_prefix_sharing": lambda: pins.check_paged_prefix_sharing(
            overrides.get("PagedCacheModel", oracle.PagedCacheModel), oracle.decode_paged),
        "check_paged_extend_and_window": lambda: pins.check_paged_extend_and_window(
            overrides.get("PagedCacheModel", oracle.PagedCacheModel),
            overrides.get("extend_paged", oracle.extend_paged), overrides.get("decode_paged", oracle.decode_paged)),
    }
    with np.errstate(all="ignore"):
        for name, fn in calls.items():
            try:
                fn()
            except Exception:
                failed.append(name)
    return failed


def _decode_cached_with(attend_row):
    def f(q, ck, cv, lengths, scale):
        B, H, D = q.shape
        Hkv = ck.shape[1]
        out = np.empty((B, H, D))
        for b in range(B):
            for h in range(H):
                g = h // (H // Hkv)
                out[b, h] = attend_row(q[b, h], ck[b, g, :lengths[b]], cv[b, g, :lengths[b]], scale)
        return out
    return f


def _extend_visible(count):
    """An extend whose new query t sees count(off, t, T) keys instead of off + t + 1."""
    def f(q_new, ck, cv, offsets, scale):
        B, H, T, D = q_new.shape
        Hkv = ck.shape[1]
        out = np.empty((B, H, T, cv.shape[-1]))
        for b in range(B):
            for h in range(H):
                g = h // (H // Hkv)
                for t in range(T):
                    n = max(1, count(int(offsets[b]), t, T))
                    out[b, h, t] = oracle.attend_row(q_new[b, h, t], ck[b, g, :n], cv[b, g, :n], scale)
        return out
    return f


def _extend_paged_offset(shift):
    """extend_paged taking each slot's prefix as len - T + shift."""
    def f(q_new, model, layer, scale, dtype, to_f64, window=0, sink=0):
        B, H, T, D = q_new.shape
        out = np.empty((B, H, T, D))
        for s in range(B):
            kg, vg = model.gather(layer, s)
            off = min(max(kg.shape[1] - T + shift, 0), kg.shape[1] - T)
            out[s:s + 1] = oracle.extend(q_new[s:s + 1], to_f64(kg[None], dtype), to_f64(vg[None], dtype),
                                         [off], scale, window, sink)
        return out
    return f


def _decode_paged_window_dropped(q, model, layer, scale, dtype, to_f64, window=0, sink=0):
    return oracle.decode_paged(q, model, layer, scale, dtype, to_f64)


def _paged_variant(where):
    """PagedCacheModel with another position -> (block, row) placement."""
    class Variant(oracle.PagedCacheModel):
        def where(self, slot, pos):
            return where(self, slot, pos)
    return Variant


def _windowed_variant(rule):
    """naive_windowed with another visibility rule(i, j, W, S)."""
    def f(q, k, v, scale, W, S):
        B, H, T, D = q.shape
        Hkv = k.shape[1]
        out = np.empty((B, H, T, v.shape[-1]))
        hidden = np.array([[not rule(i, j, W, S) for j in range(T)] for i in range(T)])
        for b in range(B):
            for h in range(H):
                g = h // (H // Hkv)
                s = (q[b, h] @ k[b, g].T) * scale
                s[hidden] = -np.inf
                s = s - s.max(axis=1, keepdims=True)
                e = np.exp(s)
                out[b, h] = (e / e.sum(axis=1, keepdims=True)) @ v[b, g]
        return out
    return f


MUTANTS = {f"naive_{n}": {"naive": fn} for n, fn in NAIVE_MUTANTS.items()}
MUTANTS.update({
    "kv_bytes_without_factor_2": {"kv_bytes": lambda L, Hk, D, T, e, B: L * Hk * D * T * e * B},
    "kv_bytes_bits_not_bytes": {"kv_bytes": lambda L, Hk, D, T, e, B: 2 * L * Hk * D * T * e * 8 * B},
    "chunked_no_rescale": {"chunked": _chunked_no_rescale},
    "decode_short_by_one": {"decode_cached": _decode_short_by_one},
    "decode_unnormalised": {"attend_row": _attend_row_no_normalise,
                            "decode_cached": _decode_cached_with(_attend_row_no_normalise)},
    "cache_append_off_by_one": {"CacheModel": _CacheModelOffByOne},
    "extend_ignores_offset": {"extend": _extend_visible(lambda off, t, T: t + 1)},
    "extend_misses_own_key": {"extend": _extend_visible(lambda off, t, T: off + t)},
    "extend_sees_whole_block": {"extend": _extend_visible(lambda off, t, T: off + T)},
    "window_one_too_wide": {"naive_windowed": _windowed_variant(
        lambda i, j, W, S: j <= i and (W <= 0 or i - j <= W or j < S))},
    "window_sink_ignored": {"naive_windowed": _windowed_variant(
        lambda i, j, W, S: j <= i and (W <= 0 or i - j < W))},
    "window_sink_one_too_many": {"naive_windowed": _windowed_variant(
        lambda i, j, W, S: j <= i and (W <= 0 or i - j < W or j <= S))},
    "paged_ignores_table": {"PagedCacheModel": _paged_variant(lambda m, slot, pos: (pos // m.block_size, pos % m.block_size))},
    "paged_row_and_block_swapped": {"PagedCacheModel": _paged_variant(
        lambda m, slot, pos: (m.tables[slot][pos % len(m.tables[slot])], (pos // len(m.tables[slot])) % m.block_size))},
    "paged_block_off_by_one": {"PagedCacheModel": _paged_variant(
        lambda m, slot, pos: (m.tables[slot][min((pos + 1) // m.block_size, len(m.tables[slot]) - 1)], pos % m.block_size))},
    "paged_extend_offset_from_start": {"extend_paged": _extend_paged_offset(-99)},
    "paged_extend_offset_one_short": {"extend_paged": _extend_paged_offset(-1)},
    "paged_decode_window_dropped": {"decode_paged": _decode_paged_window_dropped},
    "window_not_causal": {"naive_windowed": _windowed_variant(
        lambda i, j, W, S: W <= 0 and j <= i or W > 0 and (abs(i - j) < W or j < S))},
})


def test_pins_pass_on_the_oracle():
    assert _run_all({}) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    failed = _run_all(MUTANTS[name])
    assert failed, f"no pin caught the planted mistake {name}"
