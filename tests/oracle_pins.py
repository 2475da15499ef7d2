"""Pins of the CPU oracle against facts outside the oracle itself.

Each ``check_*`` takes the functions under test as arguments (defaulting to the
oracle's own), so that ``test_oracle_mutations.py`` can plant plausible
mistakes in copies of the oracle and show that some pin catches each one.

What the pins rest on:
* the inference chapter's worked KV-bytes example (section 9.3), stored in
  ``tests/golden/kv_bytes_worked_example.json``;
* closed forms: row 0 of causal attention is v_0 exactly; a zero query (or
  identical keys) gives the running mean of V; a two-key row is a logistic
  blend; V = 1 gives outputs of exactly 1 (rows sum to one);
* brute force: pure-Python ``math.fsum`` loops on tiny shapes;
* a library routine: PyTorch's CPU float64 scaled_dot_product_attention with
  is_causal (square prefill only, where its top-left mask coincides);
* invariants the pages state: chunked == naive for any chunk size (README
  correctness notes), cached == uncached (README, chapter 9.3), and the
  structural facts that GQA equals MHA on repeated K/V heads (roadmap project
  12), that future keys never change a row, and that decode is invariant
  under permutations of the cached keys.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle
from synth_inputs import round_to, to_f64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _to_lists(a):
    return a.tolist()


# ---------------------------------------------------------------- capacity
def check_kv_bytes(kv_bytes=oracle.kv_bytes):
    with open(os.path.join(GOLDEN, "kv_bytes_worked_example.json")) as f:
        gold = json.load(f)
    for c in gold["cases"]:
        got = kv_bytes(c["layers"], c["kv_heads"], c["head_dim"], c["seq_len"],
                       c["bytes_per_elem"], c["batch"])
        assert got == c["exact_bytes"], (c, got)
    # linear in every factor: doubling T or batch doubles the bytes
    base = kv_bytes(2, 3, 4, 5, 2, 1)
    assert kv_bytes(2, 3, 4, 10, 2, 1) == 2 * base
    assert kv_bytes(2, 3, 4, 5, 2, 3) == 3 * base
    assert kv_bytes(1, 1, 1, 1, 1, 1) == 2


# ---------------------------------------------------------------- prefill
TINY_SHAPES = [  # (B, H, Hkv, T, D)
    (1, 1, 1, 1, 1), (1, 1, 1, 2, 3), (1, 2, 1, 5, 4), (2, 4, 2, 9, 5),
    (2, 4, 4, 7, 2), (1, 4, 1, 8, 5), (2, 2, 2, 3, 1),
]


def check_brute(naive=oracle.naive_causal):
    for n, (B, H, Hkv, T, D) in enumerate(TINY_SHAPES):
        q = _rand((B, H, T, D), 100 + n)
        k = _rand((B, Hkv, T, D), 200 + n)
        v = _rand((B, Hkv, T, D), 300 + n)
        scale = 1.0 / math.sqrt(D)
        got = naive(q, k, v, scale)
        ref = np.array(oracle.brute(_to_lists(q), _to_lists(k), _to_lists(v), scale))
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def check_row0_is_v0(naive=oracle.naive_causal):
    q = _rand((2, 4, 6, 8), 1)
    k = _rand((2, 2, 6, 8), 2)
    v = _rand((2, 2, 6, 8), 3)
    o = naive(q, k, v, 0.35)
    for h in range(4):
        assert np.array_equal(o[:, h, 0], v[:, h // 2, 0]), "row 0 must equal v_0 exactly"


def check_zero_query_prefix_mean(naive=oracle.naive_causal):
    B, H, T, D = 2, 3, 11, 6
    q = np.zeros((B, H, T, D))
    k = _rand((B, H, T, D), 4)
    v = _rand((B, H, T, D), 5)
    o = naive(q, k, v, 0.5)
    mean = np.cumsum(v, axis=2) / np.arange(1, T + 1)[None, None, :, None]
    np.testing.assert_allclose(o, mean, rtol=1e-13, atol=1e-13)
    # identical keys give the same uniform weights whatever the query
    k_same = np.broadcast_to(_rand((B, H, 1, D), 6), (B, H, T, D)).copy()
    o2 = naive(_rand((B, H, T, D), 7), k_same, v, 0.5)
    np.testing.assert_allclose(o2, mean, rtol=1e-13, atol=1e-13)


def check_two_key_logistic(naive=oracle.naive_causal):
    B, H, T, D = 1, 2, 2, 4
    q = _rand((B, H, T, D), 8)
    k = _rand((B, H, T, D), 9)
    v = _rand((B, H, T, D), 10)
    scale = 0.7
    o = naive(q, k, v, scale)
    for h in range(H):
        s0 = scale * float(np.dot(q[0, h, 1], k[0, h, 0]))
        s1 = scale * float(np.dot(q[0, h, 1], k[0, h, 1]))
        p0 = 1.0 / (1.0 + math.exp(s1 - s0))
        ref = p0 * v[0, h, 0] + (1.0 - p0) * v[0, h, 1]
        np.testing.assert_allclose(o[0, h, 1], ref, rtol=1e-13, atol=1e-13)


def check_rows_sum_to_one(naive=oracle.naive_causal):
    # with V = 1 every output element is the row's probability sum
    q = _rand((2, 4, 13, 5), 11, 3.0)
    k = _rand((2, 2, 13, 5), 12, 3.0)
    o = naive(q, k, np.ones((2, 2, 13, 5)), 0.9)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-13)


def check_large_scores(naive=oracle.naive_causal):
    # scores near +-1000 overflow exp() unless the row max is subtracted
    D = 4
    q = np.zeros((1, 1, 2, D)); q[0, 0, :, 0] = 100.0
    k = np.zeros((1, 1, 2, D)); k[0, 0, 0, 0] = 10.0; k[0, 0, 1, 0] = 9.9
    v = _rand((1, 1, 2, D), 13)
    o = naive(q, k, v, 1.0)
    assert np.isfinite(o).all()
    p0 = 1.0 / (1.0 + math.exp(100.0 * 9.9 - 100.0 * 10.0))
    np.testing.assert_allclose(o[0, 0, 1], p0 * v[0, 0, 0] + (1 - p0) * v[0, 0, 1], rtol=1e-12)


def check_causality(naive=oracle.naive_causal):
    B, H, Hkv, T, D = 2, 4, 2, 10, 6
    q = _rand((B, H, T, D), 14)
    k = _rand((B, Hkv, T, D), 15)
    v = _rand((B, Hkv, T, D), 16)
    o = naive(q, k, v, 0.4)
    for cut in (0, 3, 8):
        k2, v2 = k.copy(), v.copy()
        k2[:, :, cut + 1:] = _rand(k2[:, :, cut + 1:].shape, 17 + cut, 5.0)
        v2[:, :, cut + 1:] = _rand(v2[:, :, cut + 1:].shape, 27 + cut, 5.0)
        o2 = naive(q, k2, v2, 0.4)
        assert np.array_equal(o[:, :, :cut + 1], o2[:, :, :cut + 1]), "a future key changed a row"
        assert not np.array_equal(o[:, :, cut + 1:], o2[:, :, cut + 1:])


def check_gqa_equals_repeated_mha(naive=oracle.naive_causal):
    B, H, T, D = 2, 8, 9, 4
    q = _rand((B, H, T, D), 18)
    for Hkv in (1, 2, 4, 8):
        k = _rand((B, Hkv, T, D), 19 + Hkv)
        v = _rand((B, Hkv, T, D), 29 + Hkv)
        G = H // Hkv
        o_gqa = naive(q, k, v, 0.5)
        o_mha = naive(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), 0.5)
        np.testing.assert_allclose(o_gqa, o_mha, rtol=0, atol=0)


def check_torch_sdpa(naive=oracle.naive_causal):
    import torch
    import torch.nn.functional as F
    for n, (B, H, T, D) in enumerate([(1, 2, 16, 8), (2, 3, 33, 16), (1, 1, 64, 32)]):
        q = _rand((B, H, T, D), 40 + n)
        k = _rand((B, H, T, D), 50 + n)
        v = _rand((B, H, T, D), 60 + n)
        scale = 1.0 / math.sqrt(D)
        ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k),
                                             torch.from_numpy(v), is_causal=True, scale=scale).numpy()
        np.testing.assert_allclose(naive(q, k, v, scale), ref, rtol=1e-11, atol=1e-12)


def check_chunked(chunked=oracle.chunked, naive=oracle.naive_causal):
    B, H, Hkv, T, D = 2, 4, 2, 23, 8
    q = _rand((B, H, T, D), 70, 2.0)
    k = _rand((B, Hkv, T, D), 71, 2.0)
    v = _rand((B, Hkv, T, D), 72)
    ref = naive(q, k, v, 0.3)
    for cq in (1, 2, 3, 7, 64, T - 1, T, T + 5):
        for ck in (1, 2, 3, 7, 64, T - 1, T, T + 5):
            np.testing.assert_allclose(chunked(q, k, v, 0.3, cq, ck), ref, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- decode
def check_decode_single_key(attend_row=oracle.attend_row):
    K = _rand((1, 8), 80)
    V = _rand((1, 8), 81)
    assert np.array_equal(attend_row(_rand(8, 82), K, V, 0.3), V[0])


def check_decode_permutation(attend_row=oracle.attend_row):
    L, D = 37, 16
    K = _rand((L, D), 83, 2.0)
    V = _rand((L, D), 84)
    q = _rand(D, 85)
    perm = np.random.default_rng(86).permutation(L)
    np.testing.assert_allclose(attend_row(q, K[perm], V[perm], 0.25), attend_row(q, K, V, 0.25),
                               rtol=1e-13, atol=1e-14)


def check_decode_matches_prefill_rows(decode_cached=oracle.decode_cached, naive=oracle.naive_causal):
    B, H, Hkv, T, D = 2, 4, 2, 12, 8
    q = _rand((B, H, T, D), 87)
    k = _rand((B, Hkv, T, D), 88)
    v = _rand((B, Hkv, T, D), 89)
    full = naive(q, k, v, 0.35)
    for p in (0, 5, T - 1):
        got = decode_cached(q[:, :, p], k, v, np.full(B, p + 1), 0.35)
        np.testing.assert_allclose(got, full[:, :, p], rtol=1e-12, atol=1e-13)


def check_cached_equals_recompute(decode_cached=oracle.decode_cached,
                                  decode_recompute=oracle.decode_recompute,
                                  CacheModel=oracle.CacheModel, dtype="f16"):
    """Token-by-token decode through the cache equals recomputing the whole prefix,
    bit for bit, at every step, for batch 1 and batch 2, with a rollback in between."""
    storage = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]
    for B in (1, 2):
        H, Hkv, D, T, steps = 4, 2, 8, 6, 7
        max_T = T + steps
        rng = np.random.default_rng(90 + B)
        qh = round_to(rng.standard_normal((B, H, max_T, D)), dtype)
        kh = round_to(rng.standard_normal((B, Hkv, max_T, D)), dtype)
        vh = round_to(rng.standard_normal((B, Hkv, max_T, D)), dtype)
        cache = CacheModel(1, B, Hkv, D, max_T, storage)
        cache.prefill(0, kh[:, :, :T], vh[:, :, :T])
        for s in range(steps):
            pos = T + s
            if s == 3:
                # roll back two positions (rejected draft tokens) and re-append them
                cache.set_lengths(0, cache.lengths[0] - 2)
                for r in (pos - 2, pos - 1):
                    cache.append(0, kh[:, :, r:r + 1], vh[:, :, r:r + 1])
            cache.append(0, kh[:, :, pos:pos + 1], vh[:, :, pos:pos + 1])
            assert (cache.lengths[0] == pos + 1).all()
            got = decode_cached(to_f64(qh[:, :, pos], dtype), to_f64(cache.k[0], dtype),
                                to_f64(cache.v[0], dtype), cache.lengths[0], 0.3)
            ref = decode_recompute(to_f64(qh[:, :, :pos + 1], dtype), to_f64(kh[:, :, :pos + 1], dtype),
                                   to_f64(vh[:, :, :pos + 1], dtype), 0.3)
            assert np.array_equal(got, ref), f"cached != recompute at step {s}, B={B}"


def check_extend_matches_prefill_rows(extend=oracle.extend, naive=oracle.naive_causal):
    """New positions after ragged cached prefixes equal the matching rows of one
    causal prefill over the whole sequence (matrix form, written independently)."""
    B, H, Hkv, S, D, T = 3, 4, 2, 23, 6, 5
    q = _rand((B, H, S, D), 141)
    k = _rand((B, Hkv, S, D), 142)
    v = _rand((B, Hkv, S, D), 143)
    full = naive(q, k, v, 0.4)
    offsets = [0, 9, S - T]
    q_new = np.stack([q[b, :, o:o + T] for b, o in enumerate(offsets)])
    got = extend(q_new, k, v, offsets, 0.4)
    for b, o in enumerate(offsets):
        np.testing.assert_allclose(got[b], full[b, :, o:o + T], rtol=1e-12, atol=1e-13)


def check_chunked_prefill_by_extend(extend=oracle.extend, naive=oracle.naive_causal):
    """A prompt fed in chunks of any sizes (the README's chunked form) equals one prefill."""
    B, H, Hkv, S, D = 2, 2, 1, 19, 5
    q = _rand((B, H, S, D), 151)
    k = _rand((B, Hkv, S, D), 152)
    v = _rand((B, Hkv, S, D), 153)
    full = naive(q, k, v, 0.5)
    for sizes in ([S], [1] * S, [5, 1, 7, 6], [18, 1]):
        outs, off = [], 0
        for n in sizes:
            outs.append(extend(q[:, :, off:off + n], k, v, [off] * B, 0.5))
            off += n
        np.testing.assert_allclose(np.concatenate(outs, axis=2), full, rtol=1e-12, atol=1e-13)


def check_extend_brute(extend=oracle.extend):
    """Brute force (pure Python, fsum) on the whole sequence, rows after a prefix."""
    B, H, Hkv, S, D, T = 1, 2, 1, 7, 3, 3
    q = _rand((B, H, S, D), 161)
    k = _rand((B, Hkv, S, D), 162)
    v = _rand((B, Hkv, S, D), 163)
    ref = np.array(oracle.brute(_to_lists(q), _to_lists(k), _to_lists(v), 0.7))
    got = extend(q[:, :, S - T:], k, v, [S - T], 0.7)
    np.testing.assert_allclose(got, ref[:, :, S - T:], rtol=1e-12, atol=1e-13)


def check_window_special_cases(naive_windowed=oracle.naive_windowed, naive=oracle.naive_causal):
    """Sliding window + sink reduce to plain causal attention when nothing is cut
    (W = 0, W >= T, sink >= T), to v_i when a query sees only itself (W = 1, no
    sink), and to the two-key logistic mix of v_0 and v_i when W = 1, sink = 1."""
    B, H, Hkv, T, D = 2, 2, 1, 11, 4
    q = _rand((B, H, T, D), 171)
    k = _rand((B, Hkv, T, D), 172)
    v = _rand((B, Hkv, T, D), 173)
    full = naive(q, k, v, 0.6)
    for W, S in ((0, 0), (T, 0), (T + 5, 2), (3, T)):
        np.testing.assert_allclose(naive_windowed(q, k, v, 0.6, W, S), full, rtol=1e-12, atol=1e-13)
    own = naive_windowed(q, k, v, 0.6, 1, 0)
    np.testing.assert_array_equal(own, np.repeat(v, H // Hkv, axis=1))
    two = naive_windowed(q, k, v, 0.6, 1, 1)
    for i in range(1, T):
        s0 = 0.6 * np.einsum("bhd,bd->bh", q[:, :, i], k[:, 0, 0])
        si = 0.6 * np.einsum("bhd,bd->bh", q[:, :, i], k[:, 0, i])
        p0 = 1.0 / (1.0 + np.exp(si - s0))
        expect = p0[..., None] * v[:, 0, 0][:, None] + (1 - p0)[..., None] * v[:, 0, i][:, None]
        np.testing.assert_allclose(two[:, :, i], expect, rtol=1e-12, atol=1e-13)


def check_window_brute(naive_windowed=oracle.naive_windowed):
    """Row-by-row pure-Python loops (math.fsum) with the window/sink rule spelled out."""
    B, H, Hkv, T, D = 1, 2, 2, 9, 3
    q = _rand((B, H, T, D), 181)
    k = _rand((B, Hkv, T, D), 182)
    v = _rand((B, Hkv, T, D), 183)
    for W, S in ((2, 0), (3, 1), (4, 2)):
        got = naive_windowed(q, k, v, 0.8, W, S)
        for h in range(H):
            for i in range(T):
                keys = [j for j in range(T) if j <= i and (i - j < W or j < S)]
                sc = [0.8 * math.fsum(float(q[0, h, i, d]) * float(k[0, h, j, d]) for d in range(D)) for j in keys]
                top = max(sc)
                w = [math.exp(x - top) for x in sc]
                z = math.fsum(w)
                ref = [math.fsum(w[n] * float(v[0, h, j, d]) for n, j in enumerate(keys)) / z for d in range(D)]
                np.testing.assert_allclose(got[0, h, i], ref, rtol=1e-12, atol=1e-13)


def check_window_decode_and_extend_rows(decode_cached=oracle.decode_cached, extend=oracle.extend,
                                        naive_windowed=oracle.naive_windowed):
    """Decode at each position and extend after ragged prefixes give the rows of one windowed prefill."""
    B, H, Hkv, T, D = 2, 4, 2, 21, 5
    q = _rand((B, H, T, D), 191)
    k = _rand((B, Hkv, T, D), 192)
    v = _rand((B, Hkv, T, D), 193)
    for W, S in ((4, 0), (5, 3), (1, 1)):
        full = naive_windowed(q, k, v, 0.45, W, S)
        for p in (0, 3, 12, T - 1):
            got = decode_cached(q[:, :, p], k, v, np.full(B, p + 1), 0.45, W, S)
            np.testing.assert_allclose(got, full[:, :, p], rtol=1e-12, atol=1e-13)
        offsets = [2, 13]
        n = 6
        q_new = np.stack([q[b, :, o:o + n] for b, o in enumerate(offsets)])
        got = extend(q_new, k, v, offsets, 0.45, W, S)
        for b, o in enumerate(offsets):
            np.testing.assert_allclose(got[b], full[b, :, o:o + n], rtol=1e-12, atol=1e-13)


def check_window_ignores_hidden_keys(naive_windowed=oracle.naive_windowed):
    """Changing keys/values a query cannot see leaves its row bit-identical."""
    B, H, Hkv, T, D = 1, 2, 1, 16, 4
    q = _rand((B, H, T, D), 201)
    k = _rand((B, Hkv, T, D), 202)
    v = _rand((B, Hkv, T, D), 203)
    W, S, i = 4, 2, 12
    base = naive_windowed(q, k, v, 0.5, W, S)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, S:i - W + 1] *= -3.0
    v2[:, :, S:i - W + 1] += 7.0
    k2[:, :, i + 1:] = 0.0
    got = naive_windowed(q, k2, v2, 0.5, W, S)
    assert np.array_equal(got[:, :, i], base[:, :, i])


def check_paged_addressing(PagedCacheModel=oracle.PagedCacheModel):
    """Hand-worked placement: block size 2, table [5, 1, 3]; positions 0..5 land
    at (block, row) = (5,0) (5,1) (1,0) (1,1) (3,0) (3,1); the 7th append is
    refused (the slot holds 3 * 2 positions)."""
    m = PagedCacheModel(1, 1, 6, 2, 1, 1, np.float32)
    m.set_blocks(0, [5, 1, 3])
    expect = [(5, 0), (5, 1), (1, 0), (1, 1), (3, 0), (3, 1)]
    for p in range(6):
        m.append(0, np.full((1, 1, 1, 1), 10.0 + p, np.float32), np.full((1, 1, 1, 1), -p, np.float32))
    for p, (blk, row) in enumerate(expect):
        assert m.k[0, blk, 0, row, 0] == 10.0 + p and m.v[0, blk, 0, row, 0] == -p
    assert set(np.flatnonzero(m.k[0, :, 0, :, 0].any(axis=1))) == {1, 3, 5}
    try:
        m.append(0, np.zeros((1, 1, 1, 1), np.float32), np.zeros((1, 1, 1, 1), np.float32))
    except RuntimeError:
        pass
    else:
        raise AssertionError("append past the slot's blocks was accepted")


def check_paged_equals_contiguous(PagedCacheModel=oracle.PagedCacheModel, decode_paged=oracle.decode_paged,
                                  CacheModel=oracle.CacheModel, dtype="bf16"):
    """The same prefill and appends through a paged cache with permuted block
    tables and through the contiguous cache model: every slot gathers to the
    contiguous rows bit for bit, and the paged decode equals the contiguous one
    exactly, at every step."""
    storage = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]
    B, H, Hkv, D, T, steps, bs = 3, 4, 2, 8, 5, 9, 4
    max_T = T + steps
    nb = -(-max_T // bs)
    rng = np.random.default_rng(301)
    perm = rng.permutation(B * nb + 3)  # a few pool blocks stay unused
    tables = [list(perm[s * nb:(s + 1) * nb]) for s in range(B)]
    paged = PagedCacheModel(2, B, B * nb + 3, bs, Hkv, D, storage)
    for s in range(B):
        paged.set_blocks(s, tables[s])
    flat = CacheModel(2, B, Hkv, D, max_T, storage)
    kh = round_to(rng.standard_normal((B, Hkv, max_T, D)), dtype)
    vh = round_to(rng.standard_normal((B, Hkv, max_T, D)), dtype)
    qh = round_to(rng.standard_normal((B, H, max_T, D)), dtype)
    layer = 1
    for c in (paged, flat):
        c.prefill(layer, kh[:, :, :T], vh[:, :, :T])
    for t in range(T, max_T):
        for c in (paged, flat):
            c.append(layer, kh[:, :, t:t + 1], vh[:, :, t:t + 1])
        for s in range(B):
            kg, vg = paged.gather(layer, s)
            assert np.array_equal(kg, flat.k[layer, s, :, :t + 1]) and np.array_equal(vg, flat.v[layer, s, :, :t + 1])
        got = decode_paged(to_f64(qh[:, :, t], dtype), paged, layer, 0.35, dtype, to_f64)
        ref = oracle.decode_cached(to_f64(qh[:, :, t], dtype), to_f64(flat.k[layer], dtype),
                                   to_f64(flat.v[layer], dtype), flat.lengths[layer], 0.35)
        assert np.array_equal(got, ref), f"paged decode differs at position {t}"


def check_paged_prefix_sharing(PagedCacheModel=oracle.PagedCacheModel, decode_paged=oracle.decode_paged):
    """Two slots whose prompts share their first 8 positions: with the two full
    blocks of that prefix shared between the tables, both slots decode exactly
    as with private copies; the shared blocks hold the prefix once."""
    dtype, B, H, Hkv, D, bs, T = "f16", 2, 2, 1, 8, 4, 10
    rng = np.random.default_rng(311)
    k = round_to(rng.standard_normal((B, Hkv, T + 1, D)), dtype)
    v = round_to(rng.standard_normal((B, Hkv, T + 1, D)), dtype)
    k[1, :, :8], v[1, :, :8] = k[0, :, :8], v[0, :, :8]
    q = round_to(rng.standard_normal((B, H, D)), dtype)
    shared = PagedCacheModel(1, B, 6, bs, Hkv, D, np.float16)
    shared.set_blocks(0, [4, 0, 2])
    shared.set_blocks(1, [4, 0, 5])
    private = PagedCacheModel(1, B, 6, bs, Hkv, D, np.float16)
    private.set_blocks(0, [4, 0, 2])
    private.set_blocks(1, [1, 3, 5])
    for c in (shared, private):
        c.prefill(0, k[:, :, :T], v[:, :, :T])
        c.append(0, k[:, :, T:T + 1], v[:, :, T:T + 1])
    a = decode_paged(to_f64(q, dtype), shared, 0, 0.4, dtype, to_f64)
    b = decode_paged(to_f64(q, dtype), private, 0, 0.4, dtype, to_f64)
    assert np.array_equal(a, b)
    assert not shared.k[0, [1, 3]].any(), "shared prefix was written twice"


def check_paged_extend_and_window(PagedCacheModel=oracle.PagedCacheModel, extend_paged=oracle.extend_paged,
                                  decode_paged=oracle.decode_paged, dtype="f16"):
    """Ragged extends (rollback to lengths 5, 2, 7, then 6 new rows) through a
    paged cache with permuted 4-position blocks and through the contiguous
    cache model: the slots gather to the contiguous rows bit for bit; the
    paged extend equals ``extend`` on the contiguous rows exactly, with and
    without a window and sink; a windowed paged decode equals the windowed
    contiguous decode exactly."""
    storage = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]
    B, H, Hkv, D, T0, T, bs = 3, 4, 2, 8, 8, 6, 4
    max_T = T0 + T + 1
    nb = -(-max_T // bs)
    rng = np.random.default_rng(331)
    perm = rng.permutation(B * nb + 2)
    tables = [list(perm[s * nb:(s + 1) * nb]) for s in range(B)]
    kh = round_to(rng.standard_normal((B, Hkv, max_T, D)), dtype)
    vh = round_to(rng.standard_normal((B, Hkv, max_T, D)), dtype)
    qn = round_to(rng.standard_normal((B, H, T, D)), dtype)
    qd = round_to(rng.standard_normal((B, H, D)), dtype)
    base = [5, 2, 7]
    for W, S in ((0, 0), (4, 2)):
        paged = PagedCacheModel(1, B, B * nb + 2, bs, Hkv, D, storage)
        for s in range(B):
            paged.set_blocks(s, tables[s])
        flat = oracle.CacheModel(1, B, Hkv, D, max_T, storage)
        for c in (paged, flat):
            c.prefill(0, kh[:, :, :T0], vh[:, :, :T0])
            c.set_lengths(0, base)
        kn = np.stack([kh[s, :, base[s]:base[s] + T] for s in range(B)])
        vn = np.stack([vh[s, :, base[s]:base[s] + T] for s in range(B)])
        for c in (paged, flat):
            c.extend(0, kn, vn)
        for s in range(B):
            kg, vg = paged.gather(0, s)
            L = base[s] + T
            assert np.array_equal(kg, flat.k[0, s, :, :L]) and np.array_equal(vg, flat.v[0, s, :, :L])
        got = extend_paged(to_f64(qn, dtype), paged, 0, 0.3, dtype, to_f64, W, S)
        ref = oracle.extend(to_f64(qn, dtype), to_f64(flat.k[0], dtype), to_f64(flat.v[0], dtype), base, 0.3, W, S)
        assert np.array_equal(got, ref), f"paged extend differs (window {W}, sink {S})"
        got = decode_paged(to_f64(qd, dtype), paged, 0, 0.3, dtype, to_f64, W, S)
        ref = oracle.decode_cached(to_f64(qd, dtype), to_f64(flat.k[0], dtype), to_f64(flat.v[0], dtype),
                                   flat.lengths[0], 0.3, W, S)
        assert np.array_equal(got, ref), f"paged decode differs (window {W}, sink {S})"


ALL_CHECKS = [
    check_kv_bytes, check_brute, check_row0_is_v0, check_zero_query_prefix_mean,
    check_two_key_logistic, check_rows_sum_to_one, check_large_scores, check_causality,
    check_gqa_equals_repeated_mha, check_torch_sdpa, check_chunked, check_decode_single_key,
    check_decode_permutation, check_decode_matches_prefill_rows, check_cached_equals_recompute,
    check_extend_matches_prefill_rows, check_chunked_prefill_by_extend, check_extend_brute,
    check_window_special_cases, check_window_brute, check_window_decode_and_extend_rows,
    check_window_ignores_hidden_keys, check_paged_addressing, check_paged_equals_contiguous,
    check_paged_prefix_sharing, check_paged_extend_and_window,
]
