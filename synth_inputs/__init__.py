"""Seeded synthetic inputs for the KV-cached causal attention workloads.

This module is the one piece shared by the CPU oracle side (``oracle/``, the
tests) and the GPU side (the tests, ``bench.py``, the smoke check).  It holds
none of the attention arithmetic: it only draws i.i.d. N(0, 1) samples, rounds
them to the storage dtype with round-to-nearest-even, picks the heavy key rows
and the ragged sequence lengths, and describes the workload shapes.

Seeding: every tensor comes from its own ``numpy.random.Generator`` built from
``SeedSequence(BASE_SEED, spawn_key=(cfg, layer, step + 1, tensor, *extra))``.
``step = -1`` is the prompt / cache history, ``step = s >= 0`` is decode step
``s``.  Samples are drawn as float64 in C order of the logical shape and then
rounded: float32 by IEEE RNE, float16 by numpy's RNE cast, bfloat16 by RNE on
the float32 bit pattern.  bfloat16 arrays are carried as ``uint16`` bit
patterns, so that the exact bits can be uploaded to the device unchanged.

Workload shapes follow the pages' workloads: the 8-layer, 512-wide, 16-head
model of the llm-perf-lab README (KV-cache and attention tables), the
B=4, H=12, T=2048, D=64 shape of the naive-vs-SDPA comparison (roadmap page,
project 15) and the 32-layer, D=128, 4096-token capacity example of the
inference chapter (section 9.3).
"""
from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np

BASE_SEED = 0x6B76_6361  # fixed base of every seed sequence

# tensor ids inside the spawn key
Q, K, V, HEAVY, LENGTHS = 0, 1, 2, 3, 4

DTYPES = ("f32", "f16", "bf16")
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}


def generator(cfg: int, layer: int, step: int, tensor: int, *extra: int) -> np.random.Generator:
    """Independent generator for one (config, layer, step, tensor[, extra]) stream."""
    if step < -1:
        raise ValueError("step must be >= -1")
    key = (int(cfg), int(layer), int(step) + 1, int(tensor)) + tuple(int(e) for e in extra)
    if min(key) < 0:
        raise ValueError("spawn key entries must be non-negative")
    return np.random.default_rng(np.random.SeedSequence(BASE_SEED, spawn_key=key))


def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (RNE on the bit pattern); returns uint16 bits."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    bits = x32.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x32)
    if nan.any():
        rounded[nan] = 0x7FC0
    return rounded


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64/float32 values to the storage dtype (RNE)."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    if dtype == "f16":
        return np.asarray(x, dtype=np.float64).astype(np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))
    raise ValueError(f"unknown dtype {dtype!r}")


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of storage values to float64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a).astype(np.float64)


def normal(cfg: int, layer: int, step: int, tensor: int, shape, dtype: str, *extra: int) -> np.ndarray:
    """i.i.d. N(0,1) tensor of ``shape``, rounded to ``dtype`` storage."""
    g = generator(cfg, layer, step, tensor, *extra)
    x = g.standard_normal(size=tuple(shape), dtype=np.float64)
    return round_to(x, dtype)


def heavy_count(n: int, frac: float = 0.01) -> int:
    """Number of heavy rows among n positions: frac*n rounded half up."""
    return int(math.floor(frac * n + 0.5))


def heavy_rows(cfg: int, layer: int, step: int, b: int, h: int, n: int, frac: float = 0.01) -> np.ndarray:
    """Sorted positions (out of n) of the K rows that are scaled by 8."""
    g = generator(cfg, layer, step, HEAVY, b, h)
    c = heavy_count(n, frac)
    return np.sort(g.choice(n, size=c, replace=False)).astype(np.int64)


def scale_rows(a: np.ndarray, rows: np.ndarray, factor: float, dtype: str) -> np.ndarray:
    """Multiply whole rows (last axis = D) of a 2-D storage array by a power of two.

    Scaling by 8 is exact in binary floating point for these magnitudes, so the
    re-rounding below returns the exact product.
    """
    out = a.copy()
    if len(rows):
        x = to_f64(out[rows], dtype) * factor
        out[rows] = round_to(x, dtype)
    return out


def ragged_lengths(cfg: int, batch: int, lo: int, hi: int) -> np.ndarray:
    """Per-sequence context lengths drawn uniformly from the inclusive range [lo, hi]."""
    g = generator(cfg, 0, -1, LENGTHS)
    return g.integers(lo, hi, size=batch, endpoint=True).astype(np.int64)


@dataclass(frozen=True)
class Workload:
    """Shape and dtype of one workload (one attention layer stack)."""

    cfg: int
    name: str
    dtype: str
    layers: int
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    prompt: int            # prefill length T (0: no prefill, cache is filled directly)
    steps: int             # decode steps after the prompt
    max_T: int             # cache capacity
    ctx_lo: int = 0        # ragged decode contexts (keys attended, incl. the appended row)
    ctx_hi: int = 0
    heavy_frac: float = 0.0
    extra_prefill_T: int = 0   # a separate B=1 prefill at this length
    extra_prefill_batch: int = 1
    note: str = field(default="", compare=False)

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(D) as the float32 value passed across the C ABI."""
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))


WORKLOADS = {
    1: Workload(1, "c1_f32_mha_b1h4d64_t128", "f32", 1, 1, 4, 4, 64, 128, 32, 160,
                note="correctness case: prefill 128 then 32 decode steps"),
    2: Workload(2, "c2_f16_mha_b4h12d64_t2048", "f16", 1, 4, 12, 12, 64, 2048, 128, 2176,
                note="naive-vs-SDPA shape with 128 decode steps"),
    3: Workload(3, "c3_f16_8l_b1h16d32_t4096", "f16", 8, 1, 16, 16, 32, 4096, 128, 4224,
                extra_prefill_T=8192,
                note="8L x 512d, 16-head model: prompt 4096 + 128 steps; separate prefill at 8192"),
    4: Workload(4, "c4_bf16_gqa32x8_32l_b16_ctx4096", "bf16", 32, 16, 32, 8, 128, 0, 1, 4096,
                ctx_lo=4096, ctx_hi=4096,
                note="GQA decode, every sequence at context 4096"),
    5: Workload(5, "c5_f16_mha32_32l_b32_ragged", "f16", 32, 32, 32, 32, 128, 0, 1, 4096,
                ctx_lo=512, ctx_hi=4096, heavy_frac=0.01, extra_prefill_T=8192,
                note="ragged batch-32 decode with 1% heavy keys; separate B=1 prefill at 8192"),
}


def decode_contexts(w: Workload) -> np.ndarray:
    """Keys attended by each sequence's decode query (after its own append)."""
    if w.ctx_lo == w.ctx_hi:
        return np.full(w.batch, w.ctx_hi, dtype=np.int64)
    return ragged_lengths(w.cfg, w.batch, w.ctx_lo, w.ctx_hi)


# --------------------------------------------------------------------------
# per-phase inputs of a workload
# --------------------------------------------------------------------------
def _apply_heavy(w: Workload, k: np.ndarray, layer: int, step: int, b: int, n_total: int,
                 first_pos: int) -> np.ndarray:
    """Scale by 8 the heavy rows (chosen among n_total positions) that fall in
    k's positions [first_pos, first_pos + k.shape[-2]), per KV head."""
    if w.heavy_frac <= 0:
        return k
    out = k.copy()
    n_here = k.shape[-2]
    for h in range(k.shape[0]):
        rows = heavy_rows(w.cfg, layer, step, b, h, n_total, w.heavy_frac)
        rows = rows[(rows >= first_pos) & (rows < first_pos + n_here)] - first_pos
        out[h] = scale_rows(out[h], rows, 8.0, w.dtype)
    return out


def prefill_inputs(w: Workload, layer: int, T: int, batch: int | None = None, variant: int = 0):
    """Prompt q (B,H,T,D), k, v (B,Hkv,T,D) for one layer, storage dtype.

    variant 0 is the workload's own prompt; variant 1 its separate long prefill.
    """
    B = w.batch if batch is None else batch
    q = normal(w.cfg, layer, -1, Q, (B, w.q_heads, T, w.head_dim), w.dtype, variant)
    k = normal(w.cfg, layer, -1, K, (B, w.kv_heads, T, w.head_dim), w.dtype, variant)
    v = normal(w.cfg, layer, -1, V, (B, w.kv_heads, T, w.head_dim), w.dtype, variant)
    if w.heavy_frac > 0:
        for b in range(B):
            k[b] = _apply_heavy(w, k[b], layer, 1000 + variant, b, T, 0)
    return q, k, v


def decode_history(w: Workload, layer: int, b: int, L: int):
    """Cached rows [0, L-1) of sequence b before its decode step: k, v (Hkv, L-1, D)."""
    k = normal(w.cfg, layer, -1, K, (w.kv_heads, L - 1, w.head_dim), w.dtype, 2, b)
    v = normal(w.cfg, layer, -1, V, (w.kv_heads, L - 1, w.head_dim), w.dtype, 2, b)
    return _apply_heavy(w, k, layer, 0, b, L, 0), v


def decode_step_inputs(w: Workload, layer: int, step: int, contexts=None):
    """q (B,H,1,D) and the appended k_new, v_new (B,Hkv,1,D) of one decode step.

    With ``contexts`` (keys attended per sequence after the append), the heavy
    rows of position L_b - 1 are applied to k_new.
    """
    q = normal(w.cfg, layer, step, Q, (w.batch, w.q_heads, 1, w.head_dim), w.dtype)
    k = normal(w.cfg, layer, step, K, (w.batch, w.kv_heads, 1, w.head_dim), w.dtype)
    v = normal(w.cfg, layer, step, V, (w.batch, w.kv_heads, 1, w.head_dim), w.dtype)
    if contexts is not None and w.heavy_frac > 0:
        for b in range(w.batch):
            L = int(contexts[b])
            k[b] = _apply_heavy(w, k[b], layer, 0, b, L, L - 1)
    return q, k, v


# --------------------------------------------------------------------------
# random-weight decoder (the README's minimal decoder-only model: 8 layers,
# 512 wide, 16 heads, vocabulary 4096)
# --------------------------------------------------------------------------
MODEL_CFG = 6  # config id of the model's seed streams
W_TOK, W_POS, W_LN1, W_QKV, W_O, W_LN2, W_UP, W_DOWN, W_LNF, W_HEAD, W_TOKENS = range(11)


@dataclass(frozen=True)
class ModelSpec:
    layers: int = 8
    d_model: int = 512
    heads: int = 16
    vocab: int = 4096
    max_T: int = 4224      # prompt 4096 + 128 generated tokens
    mlp_mult: int = 4

    @property
    def head_dim(self) -> int:
        return self.d_model // self.heads

    @property
    def d_mlp(self) -> int:
        return self.mlp_mult * self.d_model


TINYGPT = ModelSpec()


def model_weight_shapes(s: ModelSpec):
    """(name, shape) of every weight in packing order: token and position
    embeddings, then per layer norm-1 gain, fused QKV (3d x d, rows q | k | v,
    head-major inside each), output projection (d x d), norm-2 gain, MLP up
    (4d x d) and down (d x 4d), then the final norm gain and the LM head
    (vocab x d).  Matrices are (out, in), row-major."""
    d = s.d_model
    out = [("tok_emb", (s.vocab, d)), ("pos_emb", (s.max_T, d))]
    for l in range(s.layers):
        out += [(f"ln1.{l}", (d,)), (f"wqkv.{l}", (3 * d, d)), (f"wo.{l}", (d, d)),
                (f"ln2.{l}", (d,)), (f"w_up.{l}", (s.d_mlp, d)), (f"w_down.{l}", (d, s.d_mlp))]
    out += [("ln_f", (d,)), ("lm_head", (s.vocab, d))]
    return out


def model_weights(s: ModelSpec, dtype: str = "f16", seed: int = 0) -> dict:
    """Random weights: matrices and embeddings N(0, 0.02^2), norm gains 1 + N(0, 0.1^2),
    rounded to ``dtype``.  Seeded per tensor (``seed`` selects an independent model)."""
    ids = {"tok_emb": W_TOK, "pos_emb": W_POS, "ln1": W_LN1, "wqkv": W_QKV, "wo": W_O, "ln2": W_LN2,
           "w_up": W_UP, "w_down": W_DOWN, "ln_f": W_LNF, "lm_head": W_HEAD}
    w = {}
    for name, shape in model_weight_shapes(s):
        base, _, layer = name.partition(".")
        g = generator(MODEL_CFG, int(layer or 0), -1, ids[base], seed)
        x = g.standard_normal(shape)
        x = 1.0 + 0.1 * x if base.startswith("ln") else 0.02 * x
        w[name] = round_to(x, dtype)
    return w


def pack_model_weights(s: ModelSpec, w: dict) -> np.ndarray:
    """All weights concatenated in packing order (one flat array)."""
    return np.concatenate([np.ascontiguousarray(w[name]).reshape(-1) for name, _ in model_weight_shapes(s)])


def model_tokens(s: ModelSpec, batch: int, T: int, seed: int = 0) -> np.ndarray:
    """Seeded prompt token ids (batch, T), uniform over the vocabulary."""
    g = generator(MODEL_CFG, 0, -1, W_TOKENS, seed)
    return g.integers(0, s.vocab, size=(batch, T)).astype(np.int32)
