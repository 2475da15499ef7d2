"""GPU invariants that hold bit for bit, whatever the rounding of the kernels.

* Causality: K/V rows after position i never change query row i's output
  (the pages' cached == uncached argument rests on this).
* Determinism: the same call twice gives the same bits.
* Batch independence: a sequence's output depends only on its own query,
  cache rows and length, not on the other sequences of the batch or their
  order (the verification protocol of the inference chapter runs batch 1 and
  batch 2 and names batch reordering as a failure mode).
* Guard bytes just before and after the cache payload are never written.

Every call goes through the C ABI (the ctypes binding).
"""
import ctypes

import numpy as np
import pytest
import torch

import synth_inputs as si
from gpu_util import TORCH_DT, host_bits, say, to_dev

pytestmark = pytest.mark.gpu


def _kv():
    import kv_cached_causal_amd as kv
    return kv


def _rand(shape, dtype, seed):
    return si.round_to(np.random.default_rng(seed).standard_normal(shape), dtype)


# (dtype, head dim): the pipelined kernel (f16, 128), the plain kernel with one-
# and two-part P (f16 64, bf16 128) and the vector kernel (f32 64)
KERNELS = [("f16", 128), ("f16", 64), ("bf16", 128), ("f32", 64)]


@pytest.mark.parametrize("dtype,D", KERNELS, ids=lambda x: str(x))
def test_prefill_causality_and_determinism(dtype, D):
    kv = _kv()
    B, H, Hkv, T = 2, 4, 2, 600
    say(f"prefill causality dtype={dtype} D={D} T={T}")
    q = _rand((B, H, T, D), dtype, 501)
    k = _rand((B, Hkv, T, D), dtype, 502)
    v = _rand((B, Hkv, T, D), dtype, 503)
    c = kv.KVCache(1, B, H, Hkv, D, T, TORCH_DT[dtype])

    def run(kk, vv):
        c.set_lengths([0] * B)
        o = c.prefill(0, to_dev(q, dtype), to_dev(kk, dtype), to_dev(vv, dtype), out_dtype=torch.float32)
        torch.cuda.synchronize()
        return host_bits(o)

    base = run(k, v)
    assert np.array_equal(base, run(k, v)), "prefill is not deterministic"
    for i0 in (0, 37, 255, 300, T - 2):
        k2, v2 = k.copy(), v.copy()
        k2[:, :, i0 + 1:] = _rand(k2[:, :, i0 + 1:].shape, dtype, 600 + i0)
        v2[:, :, i0 + 1:] = _rand(v2[:, :, i0 + 1:].shape, dtype, 700 + i0)
        pert = run(k2, v2)
        assert np.array_equal(pert[:, :, :i0 + 1], base[:, :, :i0 + 1]), f"rows <= {i0} changed"
        assert not np.array_equal(pert[:, :, i0 + 1:], base[:, :, i0 + 1:])
    c.close()


@pytest.mark.parametrize("dtype,D", KERNELS, ids=lambda x: str(x))
def test_prefill_batch_independence(dtype, D):
    kv = _kv()
    H, Hkv, T = 4, 2, 333
    say(f"prefill batch independence dtype={dtype} D={D}")
    q = _rand((2, H, T, D), dtype, 511)
    k = _rand((2, Hkv, T, D), dtype, 512)
    v = _rand((2, Hkv, T, D), dtype, 513)

    def run(idx):
        c = kv.KVCache(1, len(idx), H, Hkv, D, T, TORCH_DT[dtype])
        o = c.prefill(0, to_dev(q[idx], dtype), to_dev(k[idx], dtype), to_dev(v[idx], dtype),
                      out_dtype=torch.float32)
        torch.cuda.synchronize()
        bits = host_bits(o)
        c.close()
        return bits

    both = run([0, 1])
    swapped = run([1, 0])
    for b in range(2):
        alone = run([b])
        assert np.array_equal(both[b], alone[0]), f"sequence {b}: batch of 2 != alone"
        assert np.array_equal(swapped[1 - b], alone[0]), f"sequence {b}: swapped batch != alone"


@pytest.mark.parametrize("heads", [(8, 8), (8, 2)], ids=lambda x: f"H{x[0]}kv{x[1]}")
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_decode_batch_independence(dtype, heads):
    kv = _kv()
    H, Hkv = heads
    D, max_T = 128, 2600
    lens = [700, 1, 2500]
    say(f"decode batch independence dtype={dtype} H={H} Hkv={Hkv} lens={lens}")
    hist_k = _rand((3, Hkv, max_T, D), dtype, 521)
    hist_v = _rand((3, Hkv, max_T, D), dtype, 522)
    q = _rand((3, H, 1, D), dtype, 523)

    def run(idx):
        c = kv.KVCache(1, len(idx), H, Hkv, D, max_T, TORCH_DT[dtype])
        c.k_view(0).copy_(to_dev(hist_k[idx], dtype))
        c.v_view(0).copy_(to_dev(hist_v[idx], dtype))
        c.set_lengths([lens[i] for i in idx])
        o = c.decode(0, to_dev(q[idx], dtype), out_dtype=torch.float32)
        torch.cuda.synchronize()
        bits = host_bits(o)
        c.close()
        return bits

    full = run([0, 1, 2])
    perm = run([2, 0, 1])
    for b in range(3):
        alone = run([b])
        assert np.array_equal(full[b], alone[0]), f"sequence {b}: batch of 3 != alone"
        assert np.array_equal(perm[[2, 0, 1].index(b)], alone[0]), f"sequence {b}: permuted batch != alone"


def test_cache_guard_bytes_untouched():
    """The cache payload placed inside a larger buffer (the caller-owned
    device_buf of kvattn_cache_alloc): prefill, append, decode, extend and a
    short extend leave the guard bytes on both sides as they were."""
    kv = _kv()
    L, B, H, Hkv, D, max_T, dtype = 2, 2, 4, 2, 128, 300, "f16"
    guard = 1 << 16
    nbytes = kv.cache_bytes(L, B, Hkv, D, max_T, TORCH_DT[dtype])
    big = torch.full((nbytes + 2 * guard,), 0x5A, dtype=torch.uint8, device="cuda")
    c = kv.KVCache.__new__(kv.KVCache)
    c.device = big.device
    c.layers, c.batch, c.q_heads, c.kv_heads = L, B, H, Hkv
    c.head_dim, c.max_T, c.dtype, c.nbytes = D, max_T, TORCH_DT[dtype], nbytes
    c._handle = ctypes.c_void_p()
    c._buf = big[guard:guard + nbytes]
    torch.cuda.synchronize()
    rc = kv.lib().kvattn_cache_alloc(ctypes.byref(c._handle), L, B, H, Hkv, D, max_T, 1,
                                     ctypes.c_void_p(c._buf.data_ptr()), nbytes)
    assert rc == 0
    say("guard bytes: prefill, append, decode, extend on both layers")
    T = 200
    for layer in range(L):
        s = 900 + 10 * layer
        c.prefill(layer, to_dev(_rand((B, H, T, D), dtype, s), dtype), to_dev(_rand((B, Hkv, T, D), dtype, s + 1), dtype),
                  to_dev(_rand((B, Hkv, T, D), dtype, s + 2), dtype))
        c.append(layer, to_dev(_rand((B, Hkv, 1, D), dtype, s + 3), dtype), to_dev(_rand((B, Hkv, 1, D), dtype, s + 4), dtype))
        c.decode(layer, to_dev(_rand((B, H, 1, D), dtype, s + 5), dtype))
        n = max_T - T - 1 - 4
        c.extend(layer, to_dev(_rand((B, H, n, D), dtype, s + 6), dtype), to_dev(_rand((B, Hkv, n, D), dtype, s + 7), dtype),
                 to_dev(_rand((B, Hkv, n, D), dtype, s + 8), dtype))
        c.extend(layer, to_dev(_rand((B, H, 4, D), dtype, s + 9), dtype), to_dev(_rand((B, Hkv, 4, D), dtype, s + 10), dtype),
                 to_dev(_rand((B, Hkv, 4, D), dtype, s + 11), dtype))
        assert c.lengths(layer) == [max_T] * B
    torch.cuda.synchronize()
    g = big.cpu().numpy()
    assert (g[:guard] == 0x5A).all() and (g[guard + nbytes:] == 0x5A).all(), "guard bytes written"
    assert not (g[guard:guard + nbytes] == 0x5A).all()
    c.close()
