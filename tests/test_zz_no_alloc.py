"""kvattn_decode_noalloc: the decode entry point that allocates nothing (collected last).

It runs the decode kernels of kvattn_decode with the split-K partials in the
library's fixed device array.  Its output must equal kvattn_decode's on the
same cache contents, lengths and query (same kernels, same split sizes), and
match the oracle within the usual tolerance, on two calls in a row, the
second one smaller (fewer sequences, shorter capacity and lengths), so the
second call runs over what the first left in the array.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_util import TORCH_DT, check_output, host_bits, say, to_dev

pytestmark = pytest.mark.gpu


def _rand(shape, dtype, seed):
    return si.round_to(np.random.default_rng(seed).standard_normal(shape), dtype)


# (dtype, B, H, Hkv, D, max_T, lengths): the first case has many splits per
# sequence; the second is smaller in every size
CALLS = [
    ("f16", 6, 8, 2, 128, 5000, [1, 385, 1024, 2049, 4999, 5000]),
    ("f16", 3, 8, 2, 128, 2500, [1, 1500, 2500]),
]


def _one_call(kv, dtype, B, H, Hkv, D, max_T, lens, seed):
    scale = float(np.float32(1 / np.sqrt(D)))
    tdt = TORCH_DT[dtype]
    hist_k = _rand((B, Hkv, max_T, D), dtype, seed)
    hist_v = _rand((B, Hkv, max_T, D), dtype, seed + 1)
    q = _rand((B, H, 1, D), dtype, seed + 2)
    # the existing entry point, on a library-owned cache
    c = kv.KVCache(1, B, H, Hkv, D, max_T, tdt)
    c.k_view(0).copy_(to_dev(hist_k, dtype))
    c.v_view(0).copy_(to_dev(hist_v, dtype))
    c.set_lengths(lens)
    qd = to_dev(q, dtype)
    ref_gpu32 = c.decode(0, qd, scale=scale, out_dtype=torch.float32)
    ref_gpun = c.decode(0, qd, scale=scale)
    torch.cuda.synchronize()
    # the no-alloc entry point, on caller-owned tensors of the same contents
    kc = to_dev(hist_k, dtype)
    vc = to_dev(hist_v, dtype)
    ld = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o32 = torch.full((B, H, 1, D), float("nan"), dtype=torch.float32, device="cuda")
    on = torch.full((B, H, 1, D), float("nan"), dtype=tdt, device="cuda")
    kv.decode_noalloc(kc, vc, ld, qd, o32, scale=scale)
    kv.decode_noalloc(kc, vc, ld, qd, on, scale=scale)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(o32), host_bits(ref_gpu32)), "no-alloc f32 output differs from kvattn_decode"
    assert np.array_equal(host_bits(on), host_bits(ref_gpun)), "no-alloc output differs from kvattn_decode"
    ref = oracle.decode_cached(si.to_f64(q[:, :, 0], dtype), si.to_f64(hist_k, dtype), si.to_f64(hist_v, dtype),
                               lens, scale)
    check_output(o32[:, :, 0], ref, dtype, "no-alloc decode o(f32)")
    check_output(on[:, :, 0], ref, dtype, f"no-alloc decode o({dtype})")
    c.close()


def test_noalloc_decode_matches_decode_twice_second_smaller():
    import kv_cached_causal_amd as kv
    for i, (dtype, B, H, Hkv, D, max_T, lens) in enumerate(CALLS):
        say(f"no-alloc decode call {i}: dtype={dtype} B={B} H={H} Hkv={Hkv} D={D} max_T={max_T} lens={lens}")
        _one_call(kv, dtype, B, H, Hkv, D, max_T, lens, 700 + 10 * i)


def test_noalloc_decode_rejects_a_shape_beyond_its_array():
    import kv_cached_causal_amd as kv
    # 4 * B * H * splits * (D + 2) bytes: B = 1024, H = 32, D = 128, 4096 keys in 2 splits: 34 MB > 16 MiB
    B, H, Hkv, D, max_T = 1024, 32, 8, 128, 4096
    lib = kv.lib()
    dummy = torch.zeros(16, dtype=torch.float16, device="cuda")
    lens = torch.ones(B, dtype=torch.int32, device="cuda")
    p = dummy.data_ptr()
    st = lib.kvattn_decode_noalloc(p, p, lens.data_ptr(), B, H, Hkv, D, max_T, 1, p, p, 0.125, 1, None)
    assert st == -3  # CAPACITY: rejected on the host, nothing enqueued
    assert b"scratch" in lib.kvattn_last_error()
