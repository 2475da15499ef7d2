"""GPU parity of the block-paged cache (kvattn_paged_*).

The pool, the block tables and the lengths are mirrored in the oracle's
PagedCacheModel; prefill and appends must leave the pool bit-identical to
the model, and decode and extend must match oracle.decode_paged /
oracle.extend_paged (each slot gathered in logical order, then the plain
decode or extend), with and without a sliding window.  Pool blocks no table names hold NaN,
so a read through a wrong table entry reaches the output.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_util import TORCH_DT, check_output, host_bits, say, to_dev

pytestmark = pytest.mark.gpu

STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}


def _kv():
    import kv_cached_causal_amd as kv
    return kv


def _rand(shape, dtype, seed):
    return si.round_to(np.random.default_rng(seed).standard_normal(shape), dtype)


def _nan_bits(dtype):
    return {"f32": np.float32(np.nan), "f16": np.float16(np.nan), "bf16": np.uint16(0x7FC0)}[dtype]


def _upload_pool(c, model, layer, dtype):
    for view, arr in ((c.k_view(layer), model.k[layer]), (c.v_view(layer), model.v[layer])):
        view.copy_(to_dev(arr, dtype))


def _tables(rng, slots, nblk, num_blocks):
    perm = [int(x) for x in rng.permutation(num_blocks)]
    return [perm[s * nblk:(s + 1) * nblk] for s in range(slots)]


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("heads", [(4, 4), (8, 2), (4, 1)], ids=lambda x: f"H{x[0]}kv{x[1]}")
@pytest.mark.parametrize("bs", [16, 64])
def test_paged_decode_matches_oracle(dtype, heads, bs):
    kv = _kv()
    H, Hkv = heads
    D = 128
    lens = [1, 17, 300, 1100]
    slots = len(lens)
    nblk = -(-max(lens) // bs) + 1
    num_blocks = slots * nblk + 5
    say(f"paged decode dtype={dtype} H={H} Hkv={Hkv} bs={bs} lens={lens}")
    rng = np.random.default_rng(7 * bs + H)
    tables = _tables(rng, slots, nblk, num_blocks)
    model = oracle.PagedCacheModel(1, slots, num_blocks, bs, Hkv, D, STORAGE[dtype])
    model.k[0] = _rand(model.k.shape[1:], dtype, 11)
    model.v[0] = _rand(model.v.shape[1:], dtype, 12)
    used = {b for t in tables for b in t}
    for blk in range(num_blocks):
        if blk not in used:
            model.k[0, blk] = _nan_bits(dtype)
            model.v[0, blk] = _nan_bits(dtype)
    for s in range(slots):
        model.set_blocks(s, tables[s])
    model.set_lengths(0, lens)
    c = kv.PagedKVCache(1, slots, nblk, num_blocks, bs, H, Hkv, D, TORCH_DT[dtype])
    _upload_pool(c, model, 0, dtype)
    for s in range(slots):
        c.set_blocks(s, tables[s])
    c.set_lengths(lens)
    q = _rand((slots, H, 1, D), dtype, 13)
    o = c.decode(0, to_dev(q, dtype), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.decode_paged(si.to_f64(q[:, :, 0], dtype), model, 0, 1.0 / np.sqrt(D), dtype, si.to_f64)
    check_output(o[:, :, 0], ref, dtype, "paged decode")
    c.close()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_paged_decode_equals_contiguous_bitwise(dtype):
    """The same rows through a paged cache (shuffled blocks) and a contiguous
    cache of the same capacity give bit-identical decode outputs."""
    kv = _kv()
    H, Hkv, D, bs = 8, 2, 128, 32
    lens = [5, 385, 999]
    slots = len(lens)
    nblk = -(-max(lens) // bs)
    cap = nblk * bs
    say(f"paged == contiguous dtype={dtype}")
    rng = np.random.default_rng(5)
    tables = _tables(rng, slots, nblk, slots * nblk)
    k = _rand((slots, Hkv, cap, D), dtype, 21)
    v = _rand((slots, Hkv, cap, D), dtype, 22)
    q = _rand((slots, H, 1, D), dtype, 23)
    flat = kv.KVCache(1, slots, H, Hkv, D, cap, TORCH_DT[dtype])
    flat.k_view(0).copy_(to_dev(k, dtype))
    flat.v_view(0).copy_(to_dev(v, dtype))
    flat.set_lengths(lens)
    paged = kv.PagedKVCache(1, slots, nblk, slots * nblk, bs, H, Hkv, D, TORCH_DT[dtype])
    pk, pv = paged.k_view(0), paged.v_view(0)
    for s in range(slots):
        for j, blk in enumerate(tables[s]):
            pk[blk] = to_dev(np.ascontiguousarray(k[s, :, j * bs:(j + 1) * bs]), dtype)
            pv[blk] = to_dev(np.ascontiguousarray(v[s, :, j * bs:(j + 1) * bs]), dtype)
        paged.set_blocks(s, tables[s])
    paged.set_lengths(lens)
    a = flat.decode(0, to_dev(q, dtype), out_dtype=torch.float32)
    b = paged.decode(0, to_dev(q, dtype), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    flat.close()
    paged.close()


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("bs", [16, 128])
def test_paged_prefill_append_decode(dtype, bs):
    """Prefill 100 positions per slot, then append and decode 40 steps across
    block boundaries: the pool stays bit-identical to the model, prefill and
    every fifth decode match the oracle."""
    kv = _kv()
    H, Hkv, D, T, steps = 4, 2, 64, 100, 40
    slots = 3
    nblk = -(-(T + steps) // bs)
    num_blocks = slots * nblk + 2
    say(f"paged prefill/append dtype={dtype} bs={bs}")
    rng = np.random.default_rng(31 + bs)
    tables = _tables(rng, slots, nblk, num_blocks)
    model = oracle.PagedCacheModel(1, slots, num_blocks, bs, Hkv, D, STORAGE[dtype])
    c = kv.PagedKVCache(1, slots, nblk, num_blocks, bs, H, Hkv, D, TORCH_DT[dtype])
    c.k_view(0).zero_()
    c.v_view(0).zero_()
    for s in range(slots):
        model.set_blocks(s, tables[s])
        c.set_blocks(s, tables[s])
    qh = _rand((slots, H, T + steps, D), dtype, 41)
    kh = _rand((slots, Hkv, T + steps, D), dtype, 42)
    vh = _rand((slots, Hkv, T + steps, D), dtype, 43)
    f = lambda a: si.to_f64(a, dtype)
    o = c.prefill(0, to_dev(qh[:, :, :T], dtype), to_dev(kh[:, :, :T], dtype), to_dev(vh[:, :, :T], dtype),
                  out_dtype=torch.float32)
    model.prefill(0, kh[:, :, :T], vh[:, :, :T])
    check_output(o, oracle.naive_causal(f(qh[:, :, :T]), f(kh[:, :, :T]), f(vh[:, :, :T]), 1.0 / np.sqrt(D)),
                 dtype, "paged prefill")
    assert c.lengths(0) == [T] * slots
    for t in range(T, T + steps):
        kn, vn = kh[:, :, t:t + 1], vh[:, :, t:t + 1]
        c.append(0, to_dev(kn, dtype), to_dev(vn, dtype))
        model.append(0, kn, vn)
        if (t - T) % 5 == 0 or t == T + steps - 1:
            od = c.decode(0, to_dev(qh[:, :, t:t + 1], dtype), out_dtype=torch.float32)
            torch.cuda.synchronize()
            ref = oracle.decode_paged(f(qh[:, :, t]), model, 0, 1.0 / np.sqrt(D), dtype, si.to_f64)
            check_output(od[:, :, 0], ref, dtype, f"paged decode at position {t}")
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(c.k_view(0)), model.k[0].view(host_bits(c.k_view(0)).dtype))
    assert np.array_equal(host_bits(c.v_view(0)), model.v[0].view(host_bits(c.v_view(0)).dtype))
    assert c.lengths(0) == [T + steps] * slots
    c.close()


def test_paged_prefix_sharing():
    """Two slots whose prompts share 64 positions share those two blocks; each
    decodes as the oracle says, and the shared blocks hold the prefix once."""
    kv = _kv()
    dtype, H, Hkv, D, bs, T = "f16", 4, 1, 128, 32, 80
    say("paged prefix sharing")
    k = _rand((2, Hkv, T + 1, D), dtype, 51)
    v = _rand((2, Hkv, T + 1, D), dtype, 52)
    k[1, :, :64], v[1, :, :64] = k[0, :, :64], v[0, :, :64]
    q = _rand((2, H, T + 1, D), dtype, 53)
    tables = [[6, 2, 4], [6, 2, 0]]
    model = oracle.PagedCacheModel(1, 2, 8, bs, Hkv, D, np.float16)
    c = kv.PagedKVCache(1, 2, 3, 8, bs, H, Hkv, D, torch.float16)
    c.k_view(0).zero_()
    c.v_view(0).zero_()
    for s in range(2):
        model.set_blocks(s, tables[s])
        c.set_blocks(s, tables[s])
    c.prefill(0, to_dev(q[:, :, :T], dtype), to_dev(k[:, :, :T], dtype), to_dev(v[:, :, :T], dtype))
    model.prefill(0, k[:, :, :T], v[:, :, :T])
    c.append(0, to_dev(k[:, :, T:], dtype), to_dev(v[:, :, T:], dtype))
    model.append(0, k[:, :, T:], v[:, :, T:])
    o = c.decode(0, to_dev(q[:, :, T:], dtype), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.decode_paged(si.to_f64(q[:, :, T], dtype), model, 0, 1.0 / np.sqrt(D), dtype, si.to_f64)
    check_output(o[:, :, 0], ref, dtype, "shared-prefix decode")
    assert np.array_equal(host_bits(c.k_view(0)), model.k[0].view(np.uint16))
    assert not model.k[0, [1, 3, 5, 7]].any()
    c.close()


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("bs", [16, 64])
def test_paged_extend_matches_oracle(dtype, bs):
    """Prefill 70 positions, roll the slots back to 70, 33 and 0, extend each
    by 37 (crossing block boundaries; slot 2 starts empty, a prefill), by 2
    (on the decode kernels) and by 5 more under a window: outputs match
    oracle.extend_paged, the pool stays bit-identical to the model, and a
    windowed decode follows."""
    kv = _kv()
    H, Hkv, D, T0, T1, T2, T3 = 8, 2, 64, 70, 37, 2, 5
    slots = 3
    nblk = -(-(T0 + T1 + T2 + T3) // bs)
    num_blocks = slots * nblk + 3
    say(f"paged extend dtype={dtype} bs={bs}")
    rng = np.random.default_rng(61 + bs)
    tables = _tables(rng, slots, nblk, num_blocks)
    model = oracle.PagedCacheModel(1, slots, num_blocks, bs, Hkv, D, STORAGE[dtype])
    c = kv.PagedKVCache(1, slots, nblk, num_blocks, bs, H, Hkv, D, TORCH_DT[dtype])
    c.k_view(0).zero_()
    c.v_view(0).zero_()
    for s in range(slots):
        model.set_blocks(s, tables[s])
        c.set_blocks(s, tables[s])
    f = lambda a: si.to_f64(a, dtype)
    kp, vp = _rand((slots, Hkv, T0, D), dtype, 62), _rand((slots, Hkv, T0, D), dtype, 63)
    c.prefill(0, to_dev(_rand((slots, H, T0, D), dtype, 64), dtype), to_dev(kp, dtype), to_dev(vp, dtype))
    model.prefill(0, kp, vp)
    base = [70, 33, 0]
    c.set_lengths(base)
    model.set_lengths(0, base)
    # 37 rows (prefill kernels), 2 rows (G * T = 8: the decode kernels), 5 rows under a window
    for T, (W, S), seed in ((T1, (0, 0), 65), (T2, (0, 0), 75), (T3, (24, 3), 68)):
        c.set_window(W, S)
        q, kn, vn = (_rand((slots, n, T, D), dtype, seed + i) for i, n in enumerate((H, Hkv, Hkv)))
        o = c.extend(0, to_dev(q, dtype), to_dev(kn, dtype), to_dev(vn, dtype), out_dtype=torch.float32)
        model.extend(0, kn, vn)
        torch.cuda.synchronize()
        ref = oracle.extend_paged(f(q), model, 0, 1.0 / np.sqrt(D), dtype, si.to_f64, W, S)
        check_output(o, ref, dtype, f"paged extend by {T} (window {W}, sink {S})")
        assert c.lengths(0) == [int(x) for x in model.lengths[0]]
    qd = _rand((slots, H, 1, D), dtype, 71)
    od = c.decode(0, to_dev(qd, dtype), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.decode_paged(f(qd[:, :, 0]), model, 0, 1.0 / np.sqrt(D), dtype, si.to_f64, 24, 3)
    check_output(od[:, :, 0], ref, dtype, "windowed paged decode after the extends")
    assert np.array_equal(host_bits(c.k_view(0)), model.k[0].view(host_bits(c.k_view(0)).dtype))
    assert np.array_equal(host_bits(c.v_view(0)), model.v[0].view(host_bits(c.v_view(0)).dtype))
    c.close()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("heads", [(8, 2), (8, 8)], ids=lambda x: f"H{x[0]}kv{x[1]}")
def test_paged_extend_equals_contiguous_bitwise(dtype, heads):
    """A 4-token verification after ragged prefixes, through shuffled 32-position
    blocks and through a contiguous cache.  Where both run the same kernel the
    outputs are bit-identical: the decode kernels' short-extend form (G = 1).
    An extend at D = 128 with G = 4 runs the pipelined kernel (32x32 MFMA) on
    the contiguous cache and the plain kernel through the block tables: the
    two sum in different orders, so they agree to rounding (each is checked
    against the oracle in its own test)."""
    kv = _kv()
    (H, Hkv), D, bs, T = heads, 128, 32, 4
    lens = [5, 385, 999]
    slots = len(lens)
    nblk = -(-(max(lens) + T) // bs)
    cap = nblk * bs
    say(f"paged extend == contiguous dtype={dtype}")
    rng = np.random.default_rng(73)
    tables = _tables(rng, slots, nblk, slots * nblk)
    k = _rand((slots, Hkv, cap, D), dtype, 74)
    v = _rand((slots, Hkv, cap, D), dtype, 75)
    q, kn, vn = _rand((slots, H, T, D), dtype, 76), _rand((slots, Hkv, T, D), dtype, 77), _rand((slots, Hkv, T, D), dtype, 78)
    flat = kv.KVCache(1, slots, H, Hkv, D, cap, TORCH_DT[dtype])
    flat.k_view(0).copy_(to_dev(k, dtype))
    flat.v_view(0).copy_(to_dev(v, dtype))
    flat.set_lengths(lens)
    paged = kv.PagedKVCache(1, slots, nblk, slots * nblk, bs, H, Hkv, D, TORCH_DT[dtype])
    pk, pv = paged.k_view(0), paged.v_view(0)
    for s in range(slots):
        for j, blk in enumerate(tables[s]):
            pk[blk] = to_dev(np.ascontiguousarray(k[s, :, j * bs:(j + 1) * bs]), dtype)
            pv[blk] = to_dev(np.ascontiguousarray(v[s, :, j * bs:(j + 1) * bs]), dtype)
        paged.set_blocks(s, tables[s])
    paged.set_lengths(lens)
    a = flat.extend(0, to_dev(q, dtype), to_dev(kn, dtype), to_dev(vn, dtype), out_dtype=torch.float32)
    b = paged.extend(0, to_dev(q, dtype), to_dev(kn, dtype), to_dev(vn, dtype), out_dtype=torch.float32)
    torch.cuda.synchronize()
    if H // Hkv == 4:
        err = (a - b).abs().max().item()
        assert err <= 1e-3, err
    else:
        assert torch.equal(a, b)
    assert paged.lengths(0) == flat.lengths(0) == [L + T for L in lens]
    flat.close()
    paged.close()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("heads", [(8, 8), (8, 2)], ids=lambda x: f"H{x[0]}kv{x[1]}")
@pytest.mark.parametrize("bs", [16, 128])
def test_paged_window_decode(dtype, heads, bs):
    """Window 600 + sink 5 over contexts up to 4100 (splits that hold sink rows,
    window rows, or both runs): matches the oracle, and equals the contiguous
    windowed decode of the same rows bit for bit."""
    kv = _kv()
    H, Hkv = heads
    D, W, S = 128, 600, 5
    lens = [1, 7, 600, 606, 1500, 4100]
    slots = len(lens)
    nblk = -(-max(lens) // bs)
    cap = nblk * bs
    say(f"paged window decode dtype={dtype} H={H} Hkv={Hkv} bs={bs}")
    rng = np.random.default_rng(81 + bs + H)
    tables = _tables(rng, slots, nblk, slots * nblk + 1)
    k = _rand((slots, Hkv, cap, D), dtype, 82)
    v = _rand((slots, Hkv, cap, D), dtype, 83)
    q = _rand((slots, H, 1, D), dtype, 84)
    flat = kv.KVCache(1, slots, H, Hkv, D, cap, TORCH_DT[dtype])
    flat.k_view(0).copy_(to_dev(k, dtype))
    flat.v_view(0).copy_(to_dev(v, dtype))
    flat.set_lengths(lens)
    flat.set_window(W, S)
    paged = kv.PagedKVCache(1, slots, nblk, slots * nblk + 1, bs, H, Hkv, D, TORCH_DT[dtype])
    pk, pv = paged.k_view(0), paged.v_view(0)
    pk[slots * nblk] = float("nan")   # the one block no table names
    pv[slots * nblk] = float("nan")
    for s in range(slots):
        for j, blk in enumerate(tables[s]):
            pk[blk] = to_dev(np.ascontiguousarray(k[s, :, j * bs:(j + 1) * bs]), dtype)
            pv[blk] = to_dev(np.ascontiguousarray(v[s, :, j * bs:(j + 1) * bs]), dtype)
        paged.set_blocks(s, tables[s])
    paged.set_lengths(lens)
    paged.set_window(W, S)
    assert paged.window(0) == (W, S)
    a = flat.decode(0, to_dev(q, dtype), out_dtype=torch.float32)
    b = paged.decode(0, to_dev(q, dtype), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.decode_cached(si.to_f64(q[:, :, 0], dtype), si.to_f64(k, dtype), si.to_f64(v, dtype), lens,
                               float(np.float32(1 / np.sqrt(D))), W, S)
    check_output(b[:, :, 0], ref, dtype, "windowed paged decode")
    assert torch.equal(a, b), "paged windowed decode differs from the contiguous one"
    flat.close()
    paged.close()


def test_paged_window_prefill():
    """A windowed prompt on the paged cache: attention as oracle.naive_windowed."""
    kv = _kv()
    dtype, H, Hkv, D, bs, T, W, S = "f16", 4, 2, 128, 64, 300, 50, 4
    say("paged windowed prefill")
    q, k, v = _rand((2, H, T, D), dtype, 91), _rand((2, Hkv, T, D), dtype, 92), _rand((2, Hkv, T, D), dtype, 93)
    c = kv.PagedKVCache(1, 2, 5, 10, bs, H, Hkv, D, torch.float16)
    c.set_blocks(0, [9, 0, 8, 1, 7])
    c.set_blocks(1, [2, 6, 3, 5, 4])
    c.set_window(W, S)
    o = c.prefill(0, to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), out_dtype=torch.float32)
    torch.cuda.synchronize()
    f = lambda a: si.to_f64(a, dtype)
    check_output(o, oracle.naive_windowed(f(q), f(k), f(v), 1.0 / np.sqrt(D), W, S), dtype, "paged windowed prefill")
    c.close()


def test_paged_validation():
    kv = _kv()
    say("paged validation")
    c = kv.PagedKVCache(2, 2, 2, 6, 16, 4, 2, 64, torch.float16)
    with pytest.raises(kv.KVAttnError):       # block index outside the pool
        c.set_blocks(0, [0, 6])
    with pytest.raises(kv.KVAttnError):       # more entries than max_blocks
        c.set_blocks(0, [0, 1, 2])
    c.set_blocks(0, [3, 1])
    c.set_blocks(1, [2])
    q = torch.randn(2, 4, 1, 64, device="cuda").half()
    with pytest.raises(kv.KVAttnError):       # decode at length 0
        c.decode(0, q)
    with pytest.raises(kv.KVAttnError):       # prompt longer than slot 1's single block
        c.prefill(0, torch.zeros(2, 4, 17, 64, device="cuda").half(), torch.zeros(2, 2, 17, 64, device="cuda").half(),
                  torch.zeros(2, 2, 17, 64, device="cuda").half())
    c.set_lengths([32, 16], layer=0)
    with pytest.raises(kv.KVAttnError):       # both slots full
        c.append(0, torch.zeros(2, 2, 1, 64, device="cuda").half(), torch.zeros(2, 2, 1, 64, device="cuda").half())
    with pytest.raises(kv.KVAttnError):       # shrinking slot 0's table below its length
        c.set_blocks(0, [3])
    with pytest.raises(kv.KVAttnError):       # prefill on a non-empty layer
        c.prefill(0, torch.zeros(2, 4, 4, 64, device="cuda").half(), torch.zeros(2, 2, 4, 64, device="cuda").half(),
                  torch.zeros(2, 2, 4, 64, device="cuda").half())
    with pytest.raises(kv.KVAttnError):       # extend past slot 1's single block
        c.extend(0, torch.zeros(2, 4, 1, 64, device="cuda").half(), torch.zeros(2, 2, 1, 64, device="cuda").half(),
                 torch.zeros(2, 2, 1, 64, device="cuda").half())
    with pytest.raises(kv.KVAttnError):       # negative window
        c.set_window(-1, 0)
    assert c.lengths(0) == [32, 16] and c.lengths(1) == [0, 0]
    c.close()
