"""GPU parity of the sliding-window and attention-sink masks.

A layer's window W and sink S (kvattn_cache_set_window) restrict every query
at position i to keys j <= i with i - j < W or j < S.  Prefill, extend and
decode are compared with the CPU oracle (naive_windowed, extend, decode_cached
with the same W and S) on seeded inputs.  Decode must read only the visible
rows: every hidden cache row is poisoned with NaN, which would reach the
output if it were read.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_util import TORCH_DT, check_output, host_bits, say, to_dev

pytestmark = pytest.mark.gpu

# (window, sink): a window of one key, small ones with sinks, a window wider
# than a 64-key tile, a sink wider than a tile, a window wider than every length
MASKS = [(1, 0), (7, 2), (64, 4), (129, 70), (5000, 3)]


def _kv():
    import kv_cached_causal_amd as kv
    return kv


def _rand(shape, dtype, seed):
    return si.round_to(np.random.default_rng(seed).standard_normal(shape), dtype)


def test_set_window_validates_and_reports():
    kv = _kv()
    c = kv.KVCache(2, 1, 2, 1, 64, 16, torch.float16)
    assert c.window(0) == (0, 0)
    c.set_window(8, 2, layer=1)
    assert c.window(0) == (0, 0) and c.window(1) == (8, 2)
    c.set_window(0, 5)            # no window: the sink is dropped too
    assert c.window(0) == (0, 0) and c.window(1) == (0, 0)
    for bad in ((-1, 0), (4, -1)):
        with pytest.raises(kv.KVAttnError):
            c.set_window(*bad)
    with pytest.raises(kv.KVAttnError):
        c.set_window(4, 0, layer=2)
    c.close()


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("mask", MASKS, ids=lambda m: f"W{m[0]}S{m[1]}")
def test_prefill_window_matches_oracle(dtype, D, mask):
    kv = _kv()
    W, S = mask
    B, H, Hkv, T = 2, 4, 2, 300
    say(f"prefill window dtype={dtype} D={D} W={W} S={S} T={T}")
    seed = 7 * D + W + S
    q = _rand((B, H, T, D), dtype, seed)
    k = _rand((B, Hkv, T, D), dtype, seed + 1)
    v = _rand((B, Hkv, T, D), dtype, seed + 2)
    c = kv.KVCache(1, B, H, Hkv, D, T + 5, TORCH_DT[dtype])
    c.set_window(W, S)
    o = c.prefill(0, to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), out_dtype=torch.float32)
    torch.cuda.synchronize()
    f = lambda a: si.to_f64(a, dtype)
    ref = oracle.naive_windowed(f(q), f(k), f(v), 1.0 / np.sqrt(D), W, S)
    check_output(o, ref, dtype, "windowed prefill")
    # the whole prompt still goes to the cache, bit for bit
    assert np.array_equal(host_bits(c.k_view(0))[:, :, :T], k.view(host_bits(c.k_view(0)).dtype))
    assert np.array_equal(host_bits(c.v_view(0))[:, :, :T], v.view(host_bits(c.v_view(0)).dtype))
    assert c.lengths(0) == [T] * B
    c.close()


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("mask", MASKS, ids=lambda m: f"W{m[0]}S{m[1]}")
def test_extend_window_matches_oracle(dtype, mask):
    kv = _kv()
    W, S = mask
    B, H, Hkv, D, T = 3, 4, 1, 128, 70
    lengths = [0, 37, 200]
    max_T = max(lengths) + T + 2
    say(f"extend window dtype={dtype} W={W} S={S} T={T} lengths={lengths}")
    seed = 31 + W + S
    k_hist = _rand((B, Hkv, max_T, D), dtype, seed)
    v_hist = _rand((B, Hkv, max_T, D), dtype, seed + 1)
    q = _rand((B, H, T, D), dtype, seed + 2)
    k_new = np.stack([k_hist[b, :, L:L + T] for b, L in enumerate(lengths)])
    v_new = np.stack([v_hist[b, :, L:L + T] for b, L in enumerate(lengths)])
    c = kv.KVCache(1, B, H, Hkv, D, max_T, TORCH_DT[dtype])
    kview, vview = c.k_view(0), c.v_view(0)
    kview.fill_(float("nan"))     # rows at or past each length are never read
    vview.fill_(float("nan"))
    for b, L in enumerate(lengths):
        if L:
            kview[b, :, :L] = to_dev(k_hist[b, :, :L], dtype)
            vview[b, :, :L] = to_dev(v_hist[b, :, :L], dtype)
    c.set_lengths(lengths)
    c.set_window(W, S)
    o = c.extend(0, to_dev(q, dtype), to_dev(k_new, dtype), to_dev(v_new, dtype), out_dtype=torch.float32)
    torch.cuda.synchronize()
    f = lambda a: si.to_f64(a, dtype)
    ref = oracle.extend(f(q), f(k_hist), f(v_hist), lengths, 1.0 / np.sqrt(D), window=W, sink=S)
    check_output(o, ref, dtype, "windowed extend")
    assert c.lengths(0) == [L + T for L in lengths]
    c.close()


DECODE_LENS = [1, 5, 300, 385, 1100, 2000]


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("heads", [(4, 4), (8, 2), (4, 1)], ids=lambda x: f"H{x[0]}kv{x[1]}")
@pytest.mark.parametrize("mask", MASKS + [(400, 0), (1000, 16)], ids=lambda m: f"W{m[0]}S{m[1]}")
def test_decode_window_reads_only_visible_rows(dtype, heads, mask):
    kv = _kv()
    W, S = mask
    H, Hkv = heads
    D = 128
    B = len(DECODE_LENS)
    max_T = max(DECODE_LENS) + 3
    scale = float(np.float32(1 / np.sqrt(D)))
    say(f"decode window dtype={dtype} H={H} Hkv={Hkv} W={W} S={S} lens={DECODE_LENS}")
    hk = _rand((B, Hkv, max_T, D), dtype, 41 + W)
    hv = _rand((B, Hkv, max_T, D), dtype, 42 + S)
    q = _rand((B, H, 1, D), dtype, 43)
    # hidden rows (and rows past each length) hold NaN on both sides
    ck = si.to_f64(hk, dtype).copy()
    cv = si.to_f64(hv, dtype).copy()
    for b, L in enumerate(DECODE_LENS):
        hidden = np.ones(max_T, dtype=bool)
        hidden[oracle.visible_keys(L - 1, W, S)] = False
        ck[b, :, hidden] = np.nan
        cv[b, :, hidden] = np.nan
    c = kv.KVCache(1, B, H, Hkv, D, max_T, TORCH_DT[dtype])
    dev_dt = TORCH_DT[dtype]
    c.k_view(0).copy_(torch.from_numpy(ck).to(dev_dt).to("cuda"))
    c.v_view(0).copy_(torch.from_numpy(cv).to(dev_dt).to("cuda"))
    c.set_lengths(DECODE_LENS)
    c.set_window(W, S)
    o = c.decode(0, to_dev(q, dtype), scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.decode_cached(si.to_f64(q[:, :, 0], dtype), ck, cv, DECODE_LENS, scale, window=W, sink=S)
    assert np.isfinite(ref).all()
    check_output(o[:, :, 0], ref, dtype, "windowed decode")
    c.close()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_windowed_generation_matches_oracle(dtype):
    """Prefill a prompt under a window, then append + decode 6 tokens per
    sequence; each step's output is the oracle's for the same mask."""
    kv = _kv()
    W, S = 48, 4
    B, H, Hkv, D, P, N = 2, 8, 2, 64, 150, 6
    say(f"windowed generation dtype={dtype} W={W} S={S} P={P} N={N}")
    qs = _rand((B, H, P + N, D), dtype, 51)
    ks = _rand((B, Hkv, P + N, D), dtype, 52)
    vs = _rand((B, Hkv, P + N, D), dtype, 53)
    f = lambda a: si.to_f64(a, dtype)
    scale = 1.0 / np.sqrt(D)
    full = oracle.naive_windowed(f(qs), f(ks), f(vs), scale, W, S)
    c = kv.KVCache(1, B, H, Hkv, D, P + N, TORCH_DT[dtype])
    c.set_window(W, S, layer=0)
    o = c.prefill(0, to_dev(qs[:, :, :P], dtype), to_dev(ks[:, :, :P], dtype), to_dev(vs[:, :, :P], dtype),
                  out_dtype=torch.float32)
    check_output(o, full[:, :, :P], dtype, "windowed prompt")
    for t in range(P, P + N):
        c.append(0, to_dev(ks[:, :, t:t + 1], dtype), to_dev(vs[:, :, t:t + 1], dtype))
        od = c.decode(0, to_dev(qs[:, :, t:t + 1], dtype), scale=float(scale), out_dtype=torch.float32)
        torch.cuda.synchronize()
        check_output(od, full[:, :, t:t + 1], dtype, f"windowed decode at position {t}")
    c.close()
