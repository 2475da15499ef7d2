"""GPU parity of kvattn_extend: T new positions after a cached prefix.

Chunked prefill and the multi-token verification step of a speculative loop
(with rollback by set_lengths).  Every case calls the HIP path through the C
ABI and compares with the CPU oracle (oracle.extend / naive_causal) on the
same seeded inputs; cache rows are compared bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_util import TORCH_DT, check_output, host_bits, say, to_dev

pytestmark = pytest.mark.gpu


def _kv():
    import kv_cached_causal_amd as kv
    return kv


def _rand(shape, dtype, seed):
    return si.round_to(np.random.default_rng(seed).standard_normal(shape), dtype)


def _fill_prefix(c, layer, k_hist, v_hist, dtype, lengths):
    """Write the history into the cache views and set ragged lengths; rows at or past
    each length are poisoned with NaN (they must never be read)."""
    B, Hkv, S, D = k_hist.shape
    kv_k, kv_v = c.k_view(layer), c.v_view(layer)
    kv_k.fill_(float("nan"))
    kv_v.fill_(float("nan"))
    for b, L in enumerate(lengths):
        if L:
            kv_k[b, :, :L] = to_dev(k_hist[b, :, :L], dtype)
            kv_v[b, :, :L] = to_dev(v_hist[b, :, :L], dtype)
    c.set_lengths(lengths, layer=layer)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("heads", [(4, 4), (4, 2), (4, 1)], ids=lambda x: f"H{x[0]}kv{x[1]}")
@pytest.mark.parametrize("T", [1, 5, 70])
def test_extend_matches_oracle(dtype, D, heads, T):
    kv = _kv()
    H, Hkv = heads
    B = 3
    lengths = [0, 37, 130]
    max_T = max(lengths) + T + 3
    say(f"extend dtype={dtype} D={D} H={H} Hkv={Hkv} T={T} lengths={lengths}")
    seed = 1000 * D + 10 * H + Hkv + T
    k_hist = _rand((B, Hkv, max_T, D), dtype, seed)
    v_hist = _rand((B, Hkv, max_T, D), dtype, seed + 1)
    q = _rand((B, H, T, D), dtype, seed + 2)
    k_new = np.stack([k_hist[b, :, L:L + T] for b, L in enumerate(lengths)])
    v_new = np.stack([v_hist[b, :, L:L + T] for b, L in enumerate(lengths)])
    c = kv.KVCache(1, B, H, Hkv, D, max_T, TORCH_DT[dtype])
    _fill_prefix(c, 0, k_hist, v_hist, dtype, lengths)
    o = c.extend(0, to_dev(q, dtype), to_dev(k_new, dtype), to_dev(v_new, dtype), out_dtype=torch.float32)
    torch.cuda.synchronize()
    f = lambda a: si.to_f64(a, dtype)
    ref = oracle.extend(f(q), f(k_hist), f(v_hist), lengths, 1.0 / np.sqrt(D))
    check_output(o, ref, dtype, "extend")
    assert c.lengths(0) == [L + T for L in lengths]
    kb = host_bits(c.k_view(0))
    vb = host_bits(c.v_view(0))
    for b, L in enumerate(lengths):
        assert np.array_equal(kb[b, :, L:L + T], k_new[b].view(kb.dtype)), "new K rows not bit-exact"
        assert np.array_equal(vb[b, :, L:L + T], v_new[b].view(vb.dtype)), "new V rows not bit-exact"
    c.close()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("heads", [(8, 8), (8, 2)], ids=lambda x: f"H{x[0]}kv{x[1]}")
def test_extend_long_ragged_prefixes(dtype, heads):
    """Extends after long cached prefixes whose lengths are not multiples of the
    32-row wave slice or the 64-key tile (a wave's rows then straddle two key
    tiles deep in the cache), with several 256-row query tiles per head; f16 at
    D=128 runs the pipelined kernel, bf16 the plain one."""
    kv = _kv()
    H, Hkv = heads
    B, D, T = 3, 128, 600
    lengths = [1000, 3001, 77]
    max_T = max(lengths) + T + 5
    say(f"extend long prefixes dtype={dtype} H={H} Hkv={Hkv} T={T} lengths={lengths}")
    seed = 7000 + 10 * H + Hkv
    k_hist = _rand((B, Hkv, max_T, D), dtype, seed)
    v_hist = _rand((B, Hkv, max_T, D), dtype, seed + 1)
    q = _rand((B, H, T, D), dtype, seed + 2)
    k_new = np.stack([k_hist[b, :, L:L + T] for b, L in enumerate(lengths)])
    v_new = np.stack([v_hist[b, :, L:L + T] for b, L in enumerate(lengths)])
    c = kv.KVCache(1, B, H, Hkv, D, max_T, TORCH_DT[dtype])
    _fill_prefix(c, 0, k_hist, v_hist, dtype, lengths)
    o = c.extend(0, to_dev(q, dtype), to_dev(k_new, dtype), to_dev(v_new, dtype), out_dtype=torch.float32)
    torch.cuda.synchronize()
    f = lambda a: si.to_f64(a, dtype)
    ref = oracle.extend(f(q), f(k_hist), f(v_hist), lengths, 1.0 / np.sqrt(D))
    check_output(o, ref, dtype, "extend after long prefixes")
    assert c.lengths(0) == [L + T for L in lengths]
    c.close()


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("D", [32, 128])
@pytest.mark.parametrize("GT", [(1, 2), (1, 3), (1, 4), (1, 8), (2, 2), (2, 4), (4, 2)],
                         ids=lambda x: f"G{x[0]}T{x[1]}")
def test_short_extend_on_decode_kernels(dtype, D, GT):
    """Extends of T = 2..8 positions whose G * T query rows fit one workgroup run
    on the decode kernels (token t of a sequence sees the keys up to its own
    position).  Prefix lengths put the new tokens on both sides of split
    boundaries (384 / 512 / 1024 keys) and start one sequence empty."""
    kv = _kv()
    G, T = GT
    Hkv = 2
    H = G * Hkv
    lengths = [0, 381, 510, 1022, 1500]
    B = len(lengths)
    max_T = max(lengths) + 2 * T + 3
    say(f"short extend dtype={dtype} D={D} G={G} T={T}")
    seed = 7000 + 100 * D + 10 * G + T
    k_hist = _rand((B, Hkv, max_T, D), dtype, seed)
    v_hist = _rand((B, Hkv, max_T, D), dtype, seed + 1)
    q = _rand((B, H, T, D), dtype, seed + 2)
    k_new = np.stack([k_hist[b, :, L:L + T] for b, L in enumerate(lengths)])
    v_new = np.stack([v_hist[b, :, L:L + T] for b, L in enumerate(lengths)])
    c = kv.KVCache(1, B, H, Hkv, D, max_T, TORCH_DT[dtype])
    _fill_prefix(c, 0, k_hist, v_hist, dtype, lengths)
    o = c.extend(0, to_dev(q, dtype), to_dev(k_new, dtype), to_dev(v_new, dtype), out_dtype=torch.float32)
    torch.cuda.synchronize()
    f = lambda a: si.to_f64(a, dtype)
    ref = oracle.extend(f(q), f(k_hist), f(v_hist), lengths, float(np.float32(1.0 / np.sqrt(D))))
    check_output(o, ref, dtype, "short extend")
    assert c.lengths(0) == [L + T for L in lengths]
    # the native output dtype too, and a second extend on top of the first
    q2 = _rand((B, H, T, D), dtype, seed + 3)
    k2 = np.stack([k_hist[b, :, L + T:L + 2 * T] for b, L in enumerate(lengths)])
    v2 = np.stack([v_hist[b, :, L + T:L + 2 * T] for b, L in enumerate(lengths)])
    o2 = c.extend(0, to_dev(q2, dtype), to_dev(k2, dtype), to_dev(v2, dtype))
    torch.cuda.synchronize()
    ref2 = oracle.extend(f(q2), f(k_hist), f(v_hist), [L + T for L in lengths], float(np.float32(1.0 / np.sqrt(D))))
    check_output(o2, ref2, dtype, "second short extend, native dtype")
    assert c.lengths(0) == [L + 2 * T for L in lengths]
    c.close()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_chunked_prefill_equals_one_shot(dtype):
    """A prompt fed through extend in uneven chunks equals one prefill (and the oracle)."""
    kv = _kv()
    B, H, Hkv, D, S = 2, 4, 2, 128, 300
    say(f"chunked prefill dtype={dtype} S={S}")
    q = _rand((B, H, S, D), dtype, 71)
    k = _rand((B, Hkv, S, D), dtype, 72)
    v = _rand((B, Hkv, S, D), dtype, 73)
    f = lambda a: si.to_f64(a, dtype)
    ref = oracle.naive_causal(f(q), f(k), f(v), 1.0 / np.sqrt(D))
    one = kv.KVCache(1, B, H, Hkv, D, S, TORCH_DT[dtype])
    o_one = one.prefill(0, to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), out_dtype=torch.float32)
    ch = kv.KVCache(1, B, H, Hkv, D, S, TORCH_DT[dtype])
    outs, off = [], 0
    for n in (100, 1, 64, 135):
        sl = slice(off, off + n)
        outs.append(ch.extend(0, to_dev(q[:, :, sl], dtype), to_dev(k[:, :, sl], dtype), to_dev(v[:, :, sl], dtype),
                              out_dtype=torch.float32))
        off += n
    torch.cuda.synchronize()
    o_ch = torch.cat(outs, dim=2)
    check_output(o_ch, ref, dtype, "chunked prefill vs oracle")
    check_output(o_one, ref, dtype, "one-shot prefill vs oracle")
    assert np.array_equal(host_bits(ch._buf), host_bits(one._buf)), "caches differ"
    assert ch.lengths(0) == [S] * B
    one.close()
    ch.close()


def test_speculative_verify_with_rollback():
    """Prefill, verify 4 draft positions, reject the last 2, verify 3 new ones."""
    kv = _kv()
    dtype = "f16"
    B, H, Hkv, D, P = 2, 8, 2, 64, 40
    max_T = P + 8
    say("speculative verify + rollback")
    qh = _rand((B, H, max_T, D), dtype, 81)
    kh = _rand((B, Hkv, max_T, D), dtype, 82)
    vh = _rand((B, Hkv, max_T, D), dtype, 83)
    # the second round re-uses positions P+2, P+3 with different (accepted) tokens
    kh2 = _rand((B, Hkv, max_T, D), dtype, 84)
    vh2 = _rand((B, Hkv, max_T, D), dtype, 85)
    qh2 = _rand((B, H, max_T, D), dtype, 86)
    c = kv.KVCache(1, B, H, Hkv, D, max_T, TORCH_DT[dtype])
    d = lambda a: to_dev(np.ascontiguousarray(a), dtype)
    c.prefill(0, d(qh[:, :, :P]), d(kh[:, :, :P]), d(vh[:, :, :P]))
    o1 = c.extend(0, d(qh[:, :, P:P + 4]), d(kh[:, :, P:P + 4]), d(vh[:, :, P:P + 4]), out_dtype=torch.float32)
    c.set_lengths([P + 2] * B)  # reject two draft positions
    o2 = c.extend(0, d(qh2[:, :, P + 2:P + 5]), d(kh2[:, :, P + 2:P + 5]), d(vh2[:, :, P + 2:P + 5]),
                  out_dtype=torch.float32)
    torch.cuda.synchronize()
    f = lambda a: si.to_f64(a, dtype)
    scale = 1.0 / np.sqrt(D)
    ref1 = oracle.extend(f(qh[:, :, P:P + 4]), f(kh), f(vh), [P] * B, scale)
    kmix = kh.copy()
    vmix = vh.copy()
    kmix[:, :, P + 2:P + 5] = kh2[:, :, P + 2:P + 5]
    vmix[:, :, P + 2:P + 5] = vh2[:, :, P + 2:P + 5]
    ref2 = oracle.extend(f(qh2[:, :, P + 2:P + 5]), f(kmix), f(vmix), [P + 2] * B, scale)
    check_output(o1, ref1, dtype, "first verification")
    check_output(o2, ref2, dtype, "second verification after rollback")
    assert c.lengths(0) == [P + 5] * B
    kb = host_bits(c.k_view(0))
    assert np.array_equal(kb[:, :, :P + 5], kmix[:, :, :P + 5].view(kb.dtype))
    c.close()


def test_extend_capacity_error_changes_nothing():
    kv = _kv()
    B, H, Hkv, D, max_T = 2, 2, 2, 64, 10
    c = kv.KVCache(1, B, H, Hkv, D, max_T, torch.float16)
    c.set_lengths([3, 8])
    before = host_bits(c._buf)
    q = torch.zeros((B, H, 3, D), dtype=torch.float16, device="cuda")
    k = torch.ones((B, Hkv, 3, D), dtype=torch.float16, device="cuda")
    with pytest.raises(kv.KVAttnError) as e:
        c.extend(0, q, k, k.clone())
    assert e.value.status == -3
    torch.cuda.synchronize()
    assert c.lengths(0) == [3, 8]
    assert np.array_equal(host_bits(c._buf), before)
    c.close()
