"""fp64 oracle of the random-weight decoder around the attention path.

TEST INFRASTRUCTURE.  Only ``tests/``, the smoke check and the CPU-baseline leg
of the benchmark may import this module.

The model is the llm-perf-lab README's minimal decoder-only Transformer (its
``model.py`` entry: RMSNorm and a GELU MLP, incremental decoding), at the
README's benchmark shape (8 layers, 512 wide, 16 heads, vocabulary 4096).
Readings where the README is silent: pre-norm residual blocks
``x += attn(rmsnorm(x))`` and ``x += mlp(rmsnorm(x))``; RMSNorm
``x / sqrt(mean(x^2) + 1e-5) * gain``; the exact (erf) GELU; an MLP four times
as wide; learned absolute position embeddings added to the token embeddings;
no biases; a final RMSNorm and an untied LM head; the fused QKV projection's
rows ordered q | k | v, head-major inside each.  The attention is the oracle's
own causal attention (``naive_causal`` for a prompt, ``decode_cached`` over the
cache model for a decode step) on q, k, v rounded to the cache's storage dtype
(float16): the cache holds K and V in that dtype and the kernels take q in it.
Everything else is float64.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import CacheModel, decode_cached, naive_causal

EPS = 1e-5


def rmsnorm(x: np.ndarray, gain: np.ndarray) -> np.ndarray:
    """Root-mean-square normalisation over the last axis, times the gain."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + EPS) * np.asarray(gain, np.float64)


_erf = np.vectorize(math.erf, otypes=[np.float64])


def gelu(x: np.ndarray) -> np.ndarray:
    """Exact GELU: x * Phi(x) with the standard normal CDF written through erf."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + _erf(x / math.sqrt(2.0)))


def _f64(w: dict) -> dict:
    return {k: np.asarray(v, dtype=np.float64) for k, v in w.items()}


def _to_storage(x: np.ndarray) -> np.ndarray:
    """Round to float16 (the cache's storage dtype) and widen back."""
    return np.asarray(x, np.float64).astype(np.float16).astype(np.float64)


def _heads(x: np.ndarray, H: int) -> np.ndarray:
    """(B, T, d) -> (B, H, T, d / H)."""
    B, T, d = x.shape
    return x.reshape(B, T, H, d // H).transpose(0, 2, 1, 3)


def forward(spec, weights: dict, tokens: np.ndarray) -> np.ndarray:
    """Logits (B, T, vocab) of the whole prompt, computed at once."""
    W = _f64(weights)
    tokens = np.asarray(tokens)
    B, T = tokens.shape
    d, H = spec.d_model, spec.heads
    scale = float(np.float32(1.0 / math.sqrt(d // H)))
    x = W["tok_emb"][tokens] + W["pos_emb"][:T][None]
    for l in range(spec.layers):
        qkv = rmsnorm(x, W[f"ln1.{l}"]) @ W[f"wqkv.{l}"].T
        q, k, v = (_to_storage(_heads(qkv[..., i * d:(i + 1) * d], H)) for i in range(3))
        a = naive_causal(q, k, v, scale)                      # (B, H, T, D)
        x = x + a.transpose(0, 2, 1, 3).reshape(B, T, d) @ W[f"wo.{l}"].T
        x = x + gelu(rmsnorm(x, W[f"ln2.{l}"]) @ W[f"w_up.{l}"].T) @ W[f"w_down.{l}"].T
    return rmsnorm(x, W["ln_f"]) @ W["lm_head"].T


class Decoder:
    """Incremental decoding: prefill a prompt into per-layer caches, then one
    position per sequence per step (append, then attend the cache)."""

    def __init__(self, spec, weights: dict, batch: int):
        self.spec, self.W, self.B = spec, _f64(weights), batch
        self.cache = CacheModel(spec.layers, batch, spec.heads, spec.head_dim, spec.max_T, np.float16)
        self.pos = 0

    def prefill(self, tokens: np.ndarray) -> np.ndarray:
        """Logits of the prompt's last position (B, vocab); fills the caches."""
        spec, W = self.spec, self.W
        B, T = tokens.shape
        d, H = spec.d_model, spec.heads
        scale = float(np.float32(1.0 / math.sqrt(d // H)))
        x = W["tok_emb"][tokens] + W["pos_emb"][:T][None]
        for l in range(spec.layers):
            qkv = rmsnorm(x, W[f"ln1.{l}"]) @ W[f"wqkv.{l}"].T
            q, k, v = (_to_storage(_heads(qkv[..., i * d:(i + 1) * d], H)) for i in range(3))
            self.cache.prefill(l, k.astype(np.float16), v.astype(np.float16))
            a = naive_causal(q, k, v, scale)
            x = x + a.transpose(0, 2, 1, 3).reshape(B, T, d) @ W[f"wo.{l}"].T
            x = x + gelu(rmsnorm(x, W[f"ln2.{l}"]) @ W[f"w_up.{l}"].T) @ W[f"w_down.{l}"].T
        self.pos = T
        return rmsnorm(x[:, -1], W["ln_f"]) @ W["lm_head"].T

    def step(self, tokens: np.ndarray) -> np.ndarray:
        """Feed one token per sequence at the next position; logits (B, vocab)."""
        spec, W = self.spec, self.W
        d, H, D = spec.d_model, spec.heads, spec.head_dim
        scale = float(np.float32(1.0 / math.sqrt(D)))
        x = W["tok_emb"][np.asarray(tokens)] + W["pos_emb"][self.pos][None]    # (B, d)
        for l in range(spec.layers):
            qkv = rmsnorm(x, W[f"ln1.{l}"]) @ W[f"wqkv.{l}"].T
            q, k, v = (_to_storage(qkv[:, i * d:(i + 1) * d].reshape(self.B, H, D)) for i in range(3))
            self.cache.append(l, k[:, :, None].astype(np.float16), v[:, :, None].astype(np.float16))
            a = decode_cached(q, self.cache.k[l].astype(np.float64), self.cache.v[l].astype(np.float64),
                              self.cache.lengths[l], scale)            # (B, H, D)
            x = x + a.reshape(self.B, d) @ W[f"wo.{l}"].T
            x = x + gelu(rmsnorm(x, W[f"ln2.{l}"]) @ W[f"w_up.{l}"].T) @ W[f"w_down.{l}"].T
        self.pos += 1
        return rmsnorm(x, W["ln_f"]) @ W["lm_head"].T
