"""Plain CPU fp64 oracle of exact causal softmax attention over a KV cache.

TEST INFRASTRUCTURE.  Only ``tests/``, the smoke check and the CPU-baseline leg
of the benchmark may import this module.  The GPU library never calls it and
shares no code with it; the two meet only through the seeded inputs of
``synth_inputs``.

Sources (the three web pages this method is described on):

* Inference chapter ("9. 推理：从生成到性能优化"), section 9.3 "KV Cache": the
  prefill builds each layer's K/V cache, decode reads the cache and appends one
  position, only K and V are cached (never Q), the cache must not change the
  result, and the KV-bytes capacity formula with its 32-layer worked example.
* Roadmap page ("项目 9-16"), project 11 "实现 KV cache": the
  ``CachedSelfAttention`` snippet -- scores ``q @ k^T`` divided by sqrt(D),
  softmax over the key axis, times V, with past K/V concatenated along the
  time axis of a (B, H, T, D) layout; and the cached-vs-uncached generation
  loops.  Project 12: MQA/GQA share K/V heads between query heads.
  Project 15: the naive form that materialises the T x T score matrix.
* llm-perf-lab README: cached and uncached outputs must agree, and chunked
  attention must equal naive attention for any chunk size (its correctness
  notes); the inference chapter, section 9.7: flash-style tiling is exact up to
  ordinary floating-point rounding.

Readings where the pages are silent:
causal mask with the diagonal visible, bottom-right aligned for a decode
query; scale = the float32 value 1/sqrt(D) passed by the caller; query head h
uses KV head h // (H // Hkv).

Every function computes in float64 on inputs already rounded to the device
storage dtype (``synth_inputs.to_f64``).  Each function is pinned to facts
outside itself (closed forms, brute force, a library routine, invariants the
pages state) by ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import math

import numpy as np


# --------------------------------------------------------------------------
# capacity (inference chapter, section 9.3, memory formula)
# --------------------------------------------------------------------------
def kv_bytes(layers: int, kv_heads: int, head_dim: int, seq_len: int,
             bytes_per_elem: int, batch: int) -> int:
    """K and V payload bytes: 2 x layers x kv_heads x head_dim x T x bytes x batch.

    The leading 2 counts K and V.  Alignment, page tables and workspace are not
    part of the formula (the chapter says so next to its worked example).
    """
    return 2 * layers * kv_heads * head_dim * seq_len * bytes_per_elem * batch


def kv_head_of(h: int, q_heads: int, kv_heads: int) -> int:
    """GQA/MQA sharing (roadmap page, project 12): contiguous groups of query heads."""
    return h // (q_heads // kv_heads)


# --------------------------------------------------------------------------
# the plain definition (roadmap page, project 15 naive form + causal mask)
# --------------------------------------------------------------------------
def naive_causal(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                 return_probs: bool = False):
    """Causal attention that materialises the full T x T score matrix per head.

    q: (B, H, T, D); k, v: (B, Hkv, T, D), float64.  Key j is visible to query
    i iff j <= i.  Returns o: (B, H, T, D) and, if asked, P: (B, H, T, T).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, T, D = q.shape
    Hkv = k.shape[1]
    if H % Hkv:
        raise ValueError("H must be a multiple of Hkv")
    above_diag = np.triu(np.ones((T, T), dtype=bool), k=1)
    out = np.empty((B, H, T, v.shape[-1]), dtype=np.float64)
    probs = np.empty((B, H, T, T), dtype=np.float64) if return_probs else None
    for b in range(B):
        for h in range(H):
            g = kv_head_of(h, H, Hkv)
            s = (q[b, h] @ k[b, g].T) * scale
            s[above_diag] = -np.inf
            s = s - s.max(axis=1, keepdims=True)
            e = np.exp(s)
            p = e / e.sum(axis=1, keepdims=True)
            out[b, h] = p @ v[b, g]
            if return_probs:
                probs[b, h] = p
    return (out, probs) if return_probs else out


# --------------------------------------------------------------------------
# sliding window and attention sink (roadmap page, project 13 long context)
# --------------------------------------------------------------------------
def visible(i: int, j: int, window: int = 0, sink: int = 0) -> bool:
    """Key j is visible to the query at position i: causal (j <= i) and, with a
    window W > 0, within the last W positions (i - j < W) or among the first
    `sink` positions (j < sink).  W = 0 means no window."""
    return j <= i and (window <= 0 or i - j < window or j < sink)


def naive_windowed(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                   window: int, sink: int) -> np.ndarray:
    """Causal attention restricted to a sliding window plus attention-sink keys,
    with the full T x T score matrix materialised per head (matrix form)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, T, D = q.shape
    Hkv = k.shape[1]
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    hidden = j > i
    if window > 0:
        hidden |= (i - j >= window) & (j >= sink)
    out = np.empty((B, H, T, v.shape[-1]), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            g = kv_head_of(h, H, Hkv)
            s = (q[b, h] @ k[b, g].T) * scale
            s[hidden] = -np.inf
            s = s - s.max(axis=1, keepdims=True)
            e = np.exp(s)
            out[b, h] = (e / e.sum(axis=1, keepdims=True)) @ v[b, g]
    return out


def visible_keys(pos: int, window: int, sink: int) -> np.ndarray:
    """Indices of the keys the query at position `pos` sees, in increasing order."""
    return np.array([j for j in range(pos + 1) if visible(pos, j, window, sink)], dtype=np.int64)


# --------------------------------------------------------------------------
# the tiled form (README: chunked == naive; chapter 9.7: flash-style tiling)
# --------------------------------------------------------------------------
def chunked(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
            q_chunk: int, k_chunk: int) -> np.ndarray:
    """Causal attention over query chunks and key blocks with the online recurrence.

    For each query chunk, key blocks are visited in order from key 0 up to the
    chunk's last row.  Running row state (m, l, u):
        m' = max(m, block row max)
        l' = exp(m - m') * l + sum_block exp(s - m')
        u' = exp(m - m') * u + sum_block exp(s - m') * v
    and finally o = u / l.  The same recurrence merges decode splits.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if q_chunk < 1 or k_chunk < 1:
        raise ValueError("chunk sizes must be >= 1")
    B, H, T, D = q.shape
    Hkv = k.shape[1]
    Dv = v.shape[-1]
    out = np.empty((B, H, T, Dv), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            g = kv_head_of(h, H, Hkv)
            for i0 in range(0, T, q_chunk):
                i1 = min(i0 + q_chunk, T)
                rows = np.arange(i0, i1)
                m = np.full(i1 - i0, -np.inf)
                l = np.zeros(i1 - i0)
                u = np.zeros((i1 - i0, Dv))
                for j0 in range(0, i1, k_chunk):
                    j1 = min(j0 + k_chunk, T)
                    cols = np.arange(j0, j1)
                    s = (q[b, h, i0:i1] @ k[b, g, j0:j1].T) * scale
                    s[cols[None, :] > rows[:, None]] = -np.inf
                    m_new = np.maximum(m, s.max(axis=1))
                    # key block 0 holds key 0, visible to every row, so m_new is
                    # finite from the first block on
                    alpha = np.exp(m - m_new)
                    e = np.exp(s - m_new[:, None])
                    l = alpha * l + e.sum(axis=1)
                    u = alpha[:, None] * u + e @ v[b, g, j0:j1]
                    m = m_new
                out[b, h, i0:i1] = u / l[:, None]
    return out


# --------------------------------------------------------------------------
# decode: one query over a cache prefix (chapter 9.3; roadmap project 11)
# --------------------------------------------------------------------------
def attend_row(q_row: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """One query against keys/values K, V of shape (L, D), L >= 1.

    The single row routine that both the cached and the recompute decode paths
    use, so that their agreement can be checked bit for bit.
    """
    s = (K @ q_row) * scale
    s = s - s.max()
    e = np.exp(s)
    p = e / e.sum()
    return p @ V


def decode_cached(q: np.ndarray, cache_k: np.ndarray, cache_v: np.ndarray,
                  lengths, scale: float, window: int = 0, sink: int = 0) -> np.ndarray:
    """Decode step from a cache: q (B, H, D); cache_k/v (B, Hkv, >=L, D); lengths (B,).

    Sequence b's query sits at position L_b - 1 and sees the L_b cached keys,
    including the one appended this step (bottom-right aligned causal mask);
    with a window, only the keys ``visible`` to it.
    """
    q = np.asarray(q, dtype=np.float64)
    B, H, D = q.shape
    Hkv = cache_k.shape[1]
    out = np.empty((B, H, cache_v.shape[-1]), dtype=np.float64)
    for b in range(B):
        L = int(lengths[b])
        if L < 1:
            raise ValueError("decode needs at least one cached key")
        keys = visible_keys(L - 1, window, sink) if window > 0 else slice(0, L)
        for h in range(H):
            g = kv_head_of(h, H, Hkv)
            out[b, h] = attend_row(q[b, h], np.asarray(cache_k[b, g, keys], np.float64),
                                   np.asarray(cache_v[b, g, keys], np.float64), scale)
    return out


def decode_recompute(q_hist: np.ndarray, k_hist: np.ndarray, v_hist: np.ndarray,
                     scale: float) -> np.ndarray:
    """The uncached path: recompute attention for every position of the history.

    q_hist (B, H, P+1, D), k_hist/v_hist (B, Hkv, P+1, D) hold the whole
    sequence so far (prompt plus every decoded position).  Every row 0..P is
    recomputed, as the uncached generation loop reruns the whole prefix; the
    last row is returned, shape (B, H, D).
    """
    q_hist = np.asarray(q_hist, dtype=np.float64)
    k_hist = np.asarray(k_hist, dtype=np.float64)
    v_hist = np.asarray(v_hist, dtype=np.float64)
    B, H, P1, D = q_hist.shape
    Hkv = k_hist.shape[1]
    out = np.empty((B, H, v_hist.shape[-1]), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            g = kv_head_of(h, H, Hkv)
            row = None
            for i in range(P1):
                row = attend_row(q_hist[b, h, i], k_hist[b, g, :i + 1], v_hist[b, g, :i + 1], scale)
            out[b, h] = row
    return out


# --------------------------------------------------------------------------
# extend: T new positions after a cached prefix (chunked prefill, multi-token
# verification of the README's speculative loop; chapter 9.3's cache)
# --------------------------------------------------------------------------
def extend(q_new: np.ndarray, cache_k: np.ndarray, cache_v: np.ndarray, offsets,
           scale: float, window: int = 0, sink: int = 0) -> np.ndarray:
    """Attention of T new queries appended after a cached prefix.

    q_new (B, H, T, D); cache_k/v (B, Hkv, >= off_b + T, D) already hold the
    prefix in rows [0, off_b) and the T new keys/values in rows [off_b,
    off_b + T).  New query t of sequence b sits at absolute position off_b + t
    and sees keys 0 .. off_b + t (the causal mask aligned to the bottom right).
    Every row goes through ``attend_row``, the routine of the decode paths.
    """
    q_new = np.asarray(q_new, dtype=np.float64)
    B, H, T, D = q_new.shape
    Hkv = cache_k.shape[1]
    out = np.empty((B, H, T, cache_v.shape[-1]), dtype=np.float64)
    for b in range(B):
        off = int(offsets[b])
        if off < 0 or off + T > cache_k.shape[2]:
            raise ValueError("new positions must fit the cache")
        for h in range(H):
            g = kv_head_of(h, H, Hkv)
            for t in range(T):
                keys = visible_keys(off + t, window, sink) if window > 0 else slice(0, off + t + 1)
                out[b, h, t] = attend_row(q_new[b, h, t], np.asarray(cache_k[b, g, keys], np.float64),
                                          np.asarray(cache_v[b, g, keys], np.float64), scale)
    return out


# --------------------------------------------------------------------------
# textbook brute force (pure Python loops)
# --------------------------------------------------------------------------
def brute(q, k, v, scale: float) -> list:
    """Pure-Python causal attention with math.exp and math.fsum, for tiny shapes.

    Nested lists [b][h][i][d] of floats.  Query head h reads KV head h * Hkv // H
    (the same contiguous grouping, written without the group size).
    """
    B, H, T, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv = len(k[0])
    Dv = len(v[0][0][0])
    out = []
    for b in range(B):
        ob = []
        for h in range(H):
            g = (h * Hkv) // H
            oh = []
            for i in range(T):
                scores = [scale * math.fsum(float(q[b][h][i][d]) * float(k[b][g][j][d]) for d in range(D))
                          for j in range(i + 1)]
                top = max(scores)
                w = [math.exp(s - top) for s in scores]
                z = math.fsum(w)
                oh.append([math.fsum(w[j] * float(v[b][g][j][d]) for j in range(i + 1)) / z
                           for d in range(Dv)])
            ob.append(oh)
        out.append(ob)
    return out


# --------------------------------------------------------------------------
# cache bookkeeping model (chapter 9.3; README kv_cache module description)
# --------------------------------------------------------------------------
class CacheModel:
    """Bit-level model of the preallocated per-layer cache.

    Storage arrays keep the raw storage dtype (bf16 as uint16 bits), laid out
    [layer][B][Hkv][max_T][D] for K and for V, plus lengths[layer][B].
    prefill writes rows [0, T) and sets the length to T; append writes one row
    at the current length and increments it; extend writes T rows there and
    advances it by T; set_lengths truncates or rolls back.  Rows at or past a sequence's length are never read.
    """

    def __init__(self, layers, batch, kv_heads, head_dim, max_T, storage_dtype):
        shape = (layers, batch, kv_heads, max_T, head_dim)
        self.k = np.zeros(shape, dtype=storage_dtype)
        self.v = np.zeros(shape, dtype=storage_dtype)
        self.lengths = np.zeros((layers, batch), dtype=np.int64)
        self.max_T = max_T

    def prefill(self, layer, k, v):
        T = k.shape[2]
        if (self.lengths[layer] != 0).any():
            raise RuntimeError("prefill needs an empty cache")
        if T > self.max_T:
            raise RuntimeError("prompt longer than the cache")
        self.k[layer, :, :, :T] = k
        self.v[layer, :, :, :T] = v
        self.lengths[layer] = T

    def append(self, layer, k_new, v_new):
        if (self.lengths[layer] >= self.max_T).any():
            raise RuntimeError("cache full")
        for b in range(self.k.shape[1]):
            pos = self.lengths[layer, b]
            self.k[layer, b, :, pos] = k_new[b, :, 0]
            self.v[layer, b, :, pos] = v_new[b, :, 0]
        self.lengths[layer] += 1

    def extend(self, layer, k_new, v_new):
        """Write T rows per sequence at its current length, then advance it by T."""
        T = k_new.shape[2]
        if (self.lengths[layer] + T > self.max_T).any():
            raise RuntimeError("cache full")
        for b in range(self.k.shape[1]):
            pos = self.lengths[layer, b]
            self.k[layer, b, :, pos:pos + T] = k_new[b]
            self.v[layer, b, :, pos:pos + T] = v_new[b]
        self.lengths[layer] += T

    def set_lengths(self, layer, lengths):
        lengths = np.asarray(lengths, dtype=np.int64)
        if (lengths < 0).any() or (lengths > self.max_T).any():
            raise RuntimeError("length out of range")
        self.lengths[layer] = lengths


# --------------------------------------------------------------------------
# paged cache model (inference chapter, section 9.6: the cache managed in
# blocks instead of one contiguous max-length region per sequence; llm-perf-lab
# README roadmap: vLLM-style paging with prefix sharing)
# --------------------------------------------------------------------------
class PagedCacheModel:
    """Bit-level model of a block-paged cache.

    A pool of ``num_blocks`` blocks per layer, K and V each laid out
    [layer][block][Hkv][block_size][D] in the raw storage dtype.  Each of the
    ``slots`` sequences owns a block table (a list of pool block indices, the
    same for every layer): its logical position p lives in block
    ``table[p // block_size]`` at row ``p % block_size``.  Two tables may name
    the same block (prefix sharing); both then read, and may write, the same
    rows.  Lengths are per (layer, slot); a slot holds at most
    ``len(table) * block_size`` positions.
    """

    def __init__(self, layers, slots, num_blocks, block_size, kv_heads, head_dim, storage_dtype):
        shape = (layers, num_blocks, kv_heads, block_size, head_dim)
        self.k = np.zeros(shape, dtype=storage_dtype)
        self.v = np.zeros(shape, dtype=storage_dtype)
        self.block_size = block_size
        self.tables = [[] for _ in range(slots)]
        self.lengths = np.zeros((layers, slots), dtype=np.int64)

    def capacity(self, slot):
        return len(self.tables[slot]) * self.block_size

    def set_blocks(self, slot, block_ids):
        ids = [int(x) for x in block_ids]
        if any(i < 0 or i >= self.k.shape[1] for i in ids):
            raise RuntimeError("block index out of the pool")
        if (self.lengths[:, slot] > len(ids) * self.block_size).any():
            raise RuntimeError("table too short for the slot's length")
        self.tables[slot] = ids

    def where(self, slot, pos):
        """(block, row) of logical position ``pos`` of ``slot``."""
        return self.tables[slot][pos // self.block_size], pos % self.block_size

    def _write(self, layer, slot, pos, k_row, v_row):
        blk, row = self.where(slot, pos)
        self.k[layer, blk, :, row] = k_row
        self.v[layer, blk, :, row] = v_row

    def prefill(self, layer, k, v):
        T = k.shape[2]
        if (self.lengths[layer] != 0).any():
            raise RuntimeError("prefill needs an empty cache")
        for s in range(len(self.tables)):
            if T > self.capacity(s):
                raise RuntimeError("prompt longer than the slot's blocks")
        for s in range(len(self.tables)):
            for t in range(T):
                self._write(layer, s, t, k[s, :, t], v[s, :, t])
        self.lengths[layer] = T

    def append(self, layer, k_new, v_new):
        for s in range(len(self.tables)):
            if self.lengths[layer, s] >= self.capacity(s):
                raise RuntimeError("slot full")
        for s in range(len(self.tables)):
            self._write(layer, s, int(self.lengths[layer, s]), k_new[s, :, 0], v_new[s, :, 0])
        self.lengths[layer] += 1

    def extend(self, layer, k_new, v_new):
        """T rows per slot (k_new/v_new (slots, Hkv, T, D)) written at logical
        positions [len, len + T) of each slot, then len += T."""
        T = k_new.shape[2]
        for s in range(len(self.tables)):
            if self.lengths[layer, s] + T > self.capacity(s):
                raise RuntimeError("slot full")
        for s in range(len(self.tables)):
            L = int(self.lengths[layer, s])
            for t in range(T):
                self._write(layer, s, L + t, k_new[s, :, t], v_new[s, :, t])
        self.lengths[layer] += T

    def set_lengths(self, layer, lengths):
        lengths = np.asarray(lengths, dtype=np.int64)
        for s, L in enumerate(lengths):
            if L < 0 or L > self.capacity(s):
                raise RuntimeError("length out of range")
        self.lengths[layer] = lengths

    def gather(self, layer, slot):
        """The slot's K and V rows in logical order: two (Hkv, L, D) arrays."""
        L = int(self.lengths[layer, slot])
        Hkv, D = self.k.shape[2], self.k.shape[4]
        kg = np.empty((Hkv, L, D), dtype=self.k.dtype)
        vg = np.empty((Hkv, L, D), dtype=self.v.dtype)
        for p in range(L):
            blk, row = self.where(slot, p)
            kg[:, p] = self.k[layer, blk, :, row]
            vg[:, p] = self.v[layer, blk, :, row]
        return kg, vg


def decode_paged(q: np.ndarray, model: PagedCacheModel, layer: int, scale: float, dtype: str,
                 to_f64, window: int = 0, sink: int = 0) -> np.ndarray:
    """Decode step over a paged cache: each slot's rows gathered in logical
    order, then the contiguous decode (``decode_cached``, with the same window
    and sink).  ``to_f64`` widens the raw storage values (bf16 bits included)
    to float64."""
    q = np.asarray(q, dtype=np.float64)
    B, H, D = q.shape
    out = np.empty((B, H, D), dtype=np.float64)
    for s in range(B):
        kg, vg = model.gather(layer, s)
        L = kg.shape[1]
        out[s:s + 1] = decode_cached(q[s:s + 1], to_f64(kg[None], dtype), to_f64(vg[None], dtype), [L], scale,
                                     window, sink)
    return out


def extend_paged(q_new: np.ndarray, model: PagedCacheModel, layer: int, scale: float, dtype: str,
                 to_f64, window: int = 0, sink: int = 0) -> np.ndarray:
    """Extend over a paged cache, after ``model.extend`` has written the T new
    rows: each slot's rows gathered in logical order, then ``extend`` with
    the slot's prefix length len - T as its offset."""
    q_new = np.asarray(q_new, dtype=np.float64)
    B, H, T, D = q_new.shape
    out = np.empty((B, H, T, D), dtype=np.float64)
    for s in range(B):
        kg, vg = model.gather(layer, s)
        off = kg.shape[1] - T
        out[s:s + 1] = extend(q_new[s:s + 1], to_f64(kg[None], dtype), to_f64(vg[None], dtype), [off], scale,
                              window, sink)
    return out
