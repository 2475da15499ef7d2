"""Prompts whose scores rise, fall or jump along the keys.

The fused-softmax prefill keeps, per query row, a reference point that it
subtracts from the scaled scores before exp2, and moves it to the row maximum
only when P against the old one would grow too large (chunked-attention
recurrence: any reference point gives the same softmax once the accumulated
numerator and denominator are rescaled by exp2(old - new)).  Random scores set
the reference in a row's first key tile and rarely move it again; these inputs
force the other cases:

* rising: the scaled score grows by about 24 (exp2 units) per 64 keys, so the
  reference moves in almost every key tile of every row;
* falling: the first keys dominate and later tiles contribute P far below one
  (down to underflow);
* jumps: mostly random scores with a spike every 300 keys, each spike larger
  than the last, so the reference moves in the tiles that hold a spike.

Checked against the CPU oracle on every row at the output tolerance of the
other prefill tests, for prompts that run whole, as two key halves (split
query tiles), and after a cached prefix (extend).
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_util import TORCH_DT, check_output, free_gpu, say, to_dev

pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634


def _kv():
    import kv_cached_causal_amd as kv
    return kv


def _inputs(pattern, B, H, Hkv, T, D, dtype, seed):
    """q, k, v (fp64 values already rounded to dtype) with the given score pattern along the keys."""
    rng = np.random.default_rng(seed)
    scale = float(np.float32(1 / np.sqrt(D)))
    c = scale * LOG2E  # scaled-score units per unit of q . k
    q = 0.5 * rng.standard_normal((B, H, T, D))
    k = 0.5 * rng.standard_normal((B, Hkv, T, D))
    v = rng.standard_normal((B, Hkv, T, D))
    q[..., 0] = 1.0
    t = np.arange(T, dtype=np.float64)
    if pattern == "rising":
        k[..., 0] = (24.0 / 64.0 / c) * t
    elif pattern == "falling":
        k[..., 0] = -(24.0 / 64.0 / c) * t
    elif pattern == "jumps":
        spikes = (t % 300 == 7)
        k[..., 0] = np.where(spikes, (20.0 + 12.0 * (t // 300)) / c, 0.0)
    else:
        raise ValueError(pattern)
    return (si.round_to(q, dtype), si.round_to(k, dtype), si.round_to(v, dtype), scale)


PATTERNS = ["rising", "falling", "jumps"]
# (dtype, D, H, Hkv, T): whole prompts over several key tiles with a ragged tail
WHOLE = [("f16", 128, 4, 4, 2100), ("f16", 64, 4, 2, 1500), ("f16", 32, 4, 4, 2100),
         ("bf16", 128, 4, 2, 1100), ("bf16", 64, 2, 2, 1300)]


@pytest.mark.parametrize("pattern", PATTERNS)
@pytest.mark.parametrize("case", WHOLE, ids=lambda c: f"{c[0]}_D{c[1]}_H{c[2]}kv{c[3]}_T{c[4]}")
def test_prefill_reference_point_moves(pattern, case):
    kv = _kv()
    dtype, D, H, Hkv, T = case
    B = 1
    say(f"prefill scores {pattern}: dtype={dtype} D={D} H={H} Hkv={Hkv} T={T}")
    q, k, v, scale = _inputs(pattern, B, H, Hkv, T, D, dtype, 7 + T)
    ref = oracle.naive_causal(si.to_f64(q, dtype), si.to_f64(k, dtype), si.to_f64(v, dtype), scale)
    c = kv.KVCache(1, B, H, Hkv, D, T, TORCH_DT[dtype])
    o = c.prefill(0, to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), scale=scale, out_dtype=torch.float32)
    check_output(o, ref, dtype, f"{pattern} o(f32)")
    c.close()
    free_gpu()


@pytest.mark.parametrize("pattern", PATTERNS)
def test_split_prefill_reference_point_moves(pattern):
    """9 query tiles x 16 heads: the heavier tiles run as two key halves."""
    kv = _kv()
    dtype, D, H, T = "f16", 128, 16, 2048 + 255
    say(f"split prefill scores {pattern}: D={D} H={H} T={T}")
    q, k, v, scale = _inputs(pattern, 1, H, H, T, D, dtype, 11)
    ref = oracle.naive_causal(si.to_f64(q, dtype), si.to_f64(k, dtype), si.to_f64(v, dtype), scale)
    c = kv.KVCache(1, 1, H, H, D, T, TORCH_DT[dtype])
    o = c.prefill(0, to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), scale=scale, out_dtype=torch.float32)
    check_output(o, ref, dtype, f"split {pattern} o(f32)")
    c.close()
    free_gpu()


@pytest.mark.parametrize("pattern", PATTERNS)
def test_extend_reference_point_moves(pattern):
    """A 700-row prefix, then 900 rows attending to it and to themselves."""
    kv = _kv()
    dtype, D, H, Hkv, T0, T1 = "f16", 128, 4, 2, 700, 900
    T = T0 + T1
    say(f"extend scores {pattern}: prefix {T0}, {T1} new rows")
    q, k, v, scale = _inputs(pattern, 1, H, Hkv, T, D, dtype, 13)
    ref = oracle.naive_causal(si.to_f64(q, dtype), si.to_f64(k, dtype), si.to_f64(v, dtype), scale)
    c = kv.KVCache(1, 1, H, Hkv, D, T, TORCH_DT[dtype])
    qd, kd, vd = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    c.prefill(0, qd[:, :, :T0].contiguous(), kd[:, :, :T0].contiguous(), vd[:, :, :T0].contiguous(), scale=scale)
    o = c.extend(0, qd[:, :, T0:].contiguous(), kd[:, :, T0:].contiguous(), vd[:, :, T0:].contiguous(), scale=scale,
                 out_dtype=torch.float32)
    check_output(o, ref[:, :, T0:], dtype, f"extend {pattern} o(f32)")
    c.close()
    free_gpu()
