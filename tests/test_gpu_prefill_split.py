"""Prompts whose heavier query tiles are split across two workgroups.

When a prompt's per-sequence grid (query tiles of 256 rows x query heads)
fills between half a round and one round of the pipelined prefill kernel (128
to 256 workgroups) and has at least 8 query tiles, the heavier half of the query tiles each run as two workgroups over the first and
second half of their key tiles, and the second to finish merges the two
partial softmax states (the README's chunked-attention recurrence: any split
of the keys gives the same attention).  Checked against the CPU oracle on
every row, with the cache write bit for bit; repeated calls give the same
bits (the split counters return to zero); a sequence's output does not depend
on the batch it is in (the split is a function of T and H only).
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_util import TORCH_DT, check_output, free_gpu, host_bits, say, to_dev

pytestmark = pytest.mark.gpu


def _kv():
    import kv_cached_causal_amd as kv
    return kv


def _rand(shape, dtype, seed):
    return si.round_to(np.random.default_rng(seed).standard_normal(shape), dtype)


# (dtype, D, H, Hkv, T): 8 to 17 query tiles, 128 to 256 (query tile, head)
# pairs per sequence, MHA and GQA; the third is the 8-layer model's prompt
CASES = [
    ("f16", 128, 16, 16, 2048),
    ("f16", 64, 16, 8, 2048 + 100),
    ("f16", 32, 16, 16, 4096),
    ("bf16", 128, 16, 16, 2048 + 255),
    ("bf16", 64, 12, 4, 3000),
    ("f16", 128, 8, 8, 4096 + 1),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}_D{c[1]}_H{c[2]}kv{c[3]}_T{c[4]}")
def test_split_prefill_matches_oracle(case):
    kv = _kv()
    dtype, D, H, Hkv, T = case
    B = 2
    scale = float(np.float32(1 / np.sqrt(D)))
    say(f"split prefill dtype={dtype} D={D} H={H} Hkv={Hkv} T={T}")
    q = _rand((B, H, T, D), dtype, 10 + T)
    k = _rand((B, Hkv, T, D), dtype, 11 + T)
    v = _rand((B, Hkv, T, D), dtype, 12 + T)
    ref = oracle.naive_causal(si.to_f64(q, dtype), si.to_f64(k, dtype), si.to_f64(v, dtype), scale)
    c = kv.KVCache(1, B, H, Hkv, D, T + 5, TORCH_DT[dtype])
    qd, kd, vd = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    o32 = c.prefill(0, qd, kd, vd, scale=scale, out_dtype=torch.float32)
    check_output(o32, ref, dtype, "split prefill o(f32)")
    kb, vb = host_bits(c.k_view(0)), host_bits(c.v_view(0))
    assert np.array_equal(kb[:, :, :T], k.view(kb.dtype)) and np.array_equal(vb[:, :, :T], v.view(vb.dtype))
    # the same call again: the same bits
    c.set_lengths([0] * B)
    o32b = c.prefill(0, qd, kd, vd, scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(o32), host_bits(o32b)), "repeated split prefill differs"
    c.set_lengths([0] * B)
    on = c.prefill(0, qd, kd, vd, scale=scale)
    check_output(on, ref, dtype, f"split prefill o({dtype})")
    # sequence 1 alone gives the bits it gave in the batch
    c1 = kv.KVCache(1, 1, H, Hkv, D, T + 5, TORCH_DT[dtype])
    o1 = c1.prefill(0, qd[1:].contiguous(), kd[1:].contiguous(), vd[1:].contiguous(), scale=scale,
                    out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(o1)[0], host_bits(o32)[1]), "a sequence's output depends on its batch"
    c.close()
    c1.close()
    free_gpu()
