"""GPU parity at the limits of the boundary: the longest contexts (where the
decode split size grows to keep at most 64 splits), sequences filled exactly
to capacity, one-token prompts, one-key decodes, a thousand short sequences
in one call and the largest block size of the paged cache.  Every case is
compared with the oracle on seeded inputs."""
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


@pytest.mark.parametrize("dtype,D", [("f16", 128), ("bf16", 64)])
def test_decode_at_131072_keys(dtype, D):
    """Capacity 131072: the split size is 2048 (grown from the head dim's
    default until a full sequence has at most 64 splits, the cap), so a full
    sequence has 64 splits.  One sequence exactly full, one not."""
    kv = _kv()
    B, H, Hkv, max_T = 2, 8, 2, 131072
    lens = [max_T, 65537]
    say(f"decode at {max_T} keys dtype={dtype} D={D}")
    k = _rand((B, Hkv, max_T, D), dtype, 1)
    v = _rand((B, Hkv, max_T, D), dtype, 2)
    q = _rand((B, H, 1, D), dtype, 3)
    c = kv.KVCache(1, B, H, Hkv, D, max_T, TORCH_DT[dtype])
    c.k_view(0).copy_(to_dev(k, dtype))
    c.v_view(0).copy_(to_dev(v, dtype))
    c.set_lengths(lens)
    o = c.decode(0, to_dev(q, dtype), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.decode_cached(si.to_f64(q[:, :, 0], dtype), si.to_f64(k, dtype), si.to_f64(v, dtype), lens,
                               float(np.float32(1 / np.sqrt(D))))
    check_output(o[:, :, 0], ref, dtype, "decode at capacity")
    with pytest.raises(kv.KVAttnError):   # sequence 0 is full
        c.append(0, to_dev(k[:, :, :1], dtype), to_dev(v[:, :, :1], dtype))
    c.close()
    free_gpu()


def test_extend_to_exact_capacity_then_full():
    kv = _kv()
    dtype, B, H, Hkv, D, max_T = "f16", 2, 4, 4, 64, 5000
    T = 10
    lens = [max_T - T, 0]
    say("extend to exactly max_T")
    kh = _rand((B, Hkv, max_T, D), dtype, 11)
    vh = _rand((B, Hkv, max_T, D), dtype, 12)
    q = _rand((B, H, T, D), dtype, 13)
    c = kv.KVCache(1, B, H, Hkv, D, max_T, TORCH_DT[dtype])
    c.k_view(0)[0, :, :lens[0]] = to_dev(kh[0, :, :lens[0]], dtype)
    c.v_view(0)[0, :, :lens[0]] = to_dev(vh[0, :, :lens[0]], dtype)
    c.set_lengths(lens)
    kn = np.stack([kh[b, :, L:L + T] for b, L in enumerate(lens)])
    vn = np.stack([vh[b, :, L:L + T] for b, L in enumerate(lens)])
    o = c.extend(0, to_dev(q, dtype), to_dev(kn, dtype), to_dev(vn, dtype), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.extend(si.to_f64(q, dtype), si.to_f64(kh, dtype), si.to_f64(vh, dtype), lens, 1 / np.sqrt(D))
    check_output(o, ref, dtype, "extend to capacity")
    assert c.lengths(0) == [max_T, T]
    with pytest.raises(kv.KVAttnError):
        c.extend(0, to_dev(q[:, :, :1], dtype), to_dev(kn[:, :, :1], dtype), to_dev(vn[:, :, :1], dtype))
    assert c.lengths(0) == [max_T, T]      # a refused call changes nothing
    c.close()


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("D", [32, 64, 128])
def test_one_token_prompt_and_one_key_decode(dtype, D):
    """T = 1: the only weight is exp(0) / exp(0), so the output is v_0; a decode
    at length 1 returns the appended v.  The kernels form that weight as
    exp2 of the rounding error of the scaled score (a few fp32 ulps from 1),
    and the bf16 prefill carries it as a hi + lo pair of bf16 values, so the
    output may sit a few fp32 ulps from v_0: the bound is 2^-16 relative,
    far inside the general tolerance, which is checked as well."""
    kv = _kv()
    B, H, Hkv = 3, 4, 2
    say(f"one-token prompt dtype={dtype} D={D}")
    q = _rand((B, H, 1, D), dtype, 21)
    k = _rand((B, Hkv, 1, D), dtype, 22)
    v = _rand((B, Hkv, 1, D), dtype, 23)
    c = kv.KVCache(1, B, H, Hkv, D, 4, TORCH_DT[dtype])
    o = c.prefill(0, to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), out_dtype=torch.float32)
    torch.cuda.synchronize()
    want = si.to_f64(np.repeat(v, H // Hkv, axis=1), dtype)

    def near_v(out, what):
        got = out.cpu().numpy().astype(np.float64)
        check_output(out, want, dtype, what)
        rel = np.abs(got - want) / np.maximum(np.abs(want), 1e-30)
        assert float(rel.max()) <= 2.0 ** -16, f"{what}: relative {float(rel.max()):.3e} from v_0"

    near_v(o, "one-token prompt")
    c.set_lengths([0, 0, 0])
    c.append(0, to_dev(k, dtype), to_dev(v, dtype))
    od = c.decode(0, to_dev(q, dtype), out_dtype=torch.float32)
    torch.cuda.synchronize()
    near_v(od, "one-key decode")
    c.close()


def test_a_thousand_short_sequences():
    """B = 1024 sequences of 1..40 keys, MQA (H = 4, Hkv = 1), D = 32, in one call."""
    kv = _kv()
    dtype, B, H, Hkv, D, max_T = "f16", 1024, 4, 1, 32, 40
    lens = np.random.default_rng(31).integers(1, max_T + 1, size=B).tolist()
    say("1024 short sequences")
    k = _rand((B, Hkv, max_T, D), dtype, 32)
    v = _rand((B, Hkv, max_T, D), dtype, 33)
    q = _rand((B, H, 1, D), dtype, 34)
    c = kv.KVCache(1, B, H, Hkv, D, max_T, TORCH_DT[dtype])
    c.k_view(0).copy_(to_dev(k, dtype))
    c.v_view(0).copy_(to_dev(v, dtype))
    c.set_lengths(lens)
    o = c.decode(0, to_dev(q, dtype), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.decode_cached(si.to_f64(q[:, :, 0], dtype), si.to_f64(k, dtype), si.to_f64(v, dtype), lens,
                               float(np.float32(1 / np.sqrt(D))))
    check_output(o[:, :, 0], ref, dtype, "1024 sequences")
    c.close()


def test_paged_largest_blocks():
    """4096-position blocks: one block per sequence, read through the table."""
    kv = _kv()
    dtype, B, H, Hkv, D, bs = "bf16", 2, 4, 2, 128, 4096
    lens = [4096, 1234]
    say("paged, 4096-position blocks")
    k = _rand((3, Hkv, bs, D), dtype, 41)
    v = _rand((3, Hkv, bs, D), dtype, 42)
    q = _rand((B, H, 1, D), dtype, 43)
    p = kv.PagedKVCache(1, B, 1, 3, bs, H, Hkv, D, TORCH_DT[dtype])
    p.k_view(0).copy_(to_dev(k, dtype))
    p.v_view(0).copy_(to_dev(v, dtype))
    p.set_blocks(0, [2])
    p.set_blocks(1, [0])
    p.set_lengths(lens)
    o = p.decode(0, to_dev(q, dtype), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ck = si.to_f64(np.stack([k[2], k[0]]), dtype)
    cv = si.to_f64(np.stack([v[2], v[0]]), dtype)
    ref = oracle.decode_cached(si.to_f64(q[:, :, 0], dtype), ck, cv, lens, float(np.float32(1 / np.sqrt(D))))
    check_output(o[:, :, 0], ref, dtype, "paged, one block per sequence")
    p.close()
