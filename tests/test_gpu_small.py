"""GPU parity on small shapes: several tiles, ragged tails, every dtype / head dim / head layout.

Every test calls the HIP path through the C ABI (the ctypes binding) and
compares with the CPU oracle on the same seeded inputs.
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


HEADS = [(4, 4), (4, 2), (4, 1)]   # MHA, GQA, MQA


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("heads", HEADS, ids=lambda x: f"H{x[0]}kv{x[1]}")
def test_append_is_bit_exact(dtype, D, heads):
    kv = _kv()
    H, Hkv = heads
    B, max_T, layers = 3, 40, 2
    say(f"append dtype={dtype} D={D} H={H} Hkv={Hkv}")
    c = kv.KVCache(layers, B, H, Hkv, D, max_T, TORCH_DT[dtype])
    c._buf.fill_(0xA5)
    c.set_lengths([0, 5, 39], layer=1)
    esz = si.ELEM_BYTES[dtype]
    utype = np.uint16 if esz == 2 else np.uint32
    rng = np.random.default_rng(7)
    # arbitrary bit patterns: subnormals, signed zeros, infinities and NaN payloads included
    kbits = rng.integers(0, np.iinfo(utype).max, size=(B, Hkv, 1, D), dtype=np.uint64, endpoint=True).astype(utype)
    vbits = rng.integers(0, np.iinfo(utype).max, size=(B, Hkv, 1, D), dtype=np.uint64, endpoint=True).astype(utype)
    kbits.flat[:4] = [0, 1 << (8 * esz - 1), 1, (1 << (8 * esz - 1)) | 1]
    tdt = TORCH_DT[dtype]
    idt = torch.int16 if esz == 2 else torch.int32
    k_new = torch.from_numpy(kbits.view(np.int16 if esz == 2 else np.int32)).cuda().view(tdt)
    v_new = torch.from_numpy(vbits.view(np.int16 if esz == 2 else np.int32)).cuda().view(tdt)
    before = host_bits(c._buf)
    c.append(1, k_new, v_new)
    torch.cuda.synchronize()
    after = host_bits(c._buf)
    assert c.lengths(1) == [1, 6, 40] and c.lengths(0) == [0, 0, 0]

    # expected image: canary everywhere except the appended rows
    exp = before.copy()
    img = exp.view(utype).reshape(layers, 2, B, Hkv, max_T, D)
    for b, pos in enumerate([0, 5, 39]):
        img[1, 0, b, :, pos] = kbits[b, :, 0]
        img[1, 1, b, :, pos] = vbits[b, :, 0]
    assert np.array_equal(after, exp), "append wrote something other than the new rows"
    del k_new, v_new, idt

    # a full sequence refuses further appends and nothing changes
    with pytest.raises(kv.KVAttnError) as e:
        c.append(1, torch.zeros((B, Hkv, 1, D), dtype=tdt, device="cuda"),
                 torch.zeros((B, Hkv, 1, D), dtype=tdt, device="cuda"))
    assert e.value.status == -3
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(c._buf), exp)
    assert c.lengths(1) == [1, 6, 40]
    c.close()


PREFILL_T = [1, 17, 64, 100, 129, 257]


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("heads", HEADS, ids=lambda x: f"H{x[0]}kv{x[1]}")
def test_prefill_matches_oracle(dtype, D, heads):
    kv = _kv()
    H, Hkv = heads
    B = 2
    max_T = max(PREFILL_T) + 3
    scale = float(np.float32(1 / np.sqrt(D)))
    for T in PREFILL_T:
        say(f"prefill dtype={dtype} D={D} H={H} Hkv={Hkv} T={T}")
        q = _rand((B, H, T, D), dtype, T)
        k = _rand((B, Hkv, T, D), dtype, T + 1)
        v = _rand((B, Hkv, T, D), dtype, T + 2)
        ref = oracle.naive_causal(si.to_f64(q, dtype), si.to_f64(k, dtype), si.to_f64(v, dtype), scale)
        c = kv.KVCache(1, B, H, Hkv, D, max_T, TORCH_DT[dtype])
        c._buf.fill_(0x5A)
        qd, kd, vd = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
        o32 = c.prefill(0, qd, kd, vd, scale=scale, out_dtype=torch.float32)
        check_output(o32, ref, dtype, f"T={T} o(f32)")
        assert c.lengths(0) == [T] * B
        # cache rows [0,T) hold the input bits; rows past T are untouched
        kb, vb = host_bits(c.k_view(0)), host_bits(c.v_view(0))
        assert np.array_equal(kb[:, :, :T], k.view(kb.dtype)) and np.array_equal(vb[:, :, :T], v.view(vb.dtype))
        canary = 0x5A5A if kb.dtype == np.uint16 else 0x5A5A5A5A
        assert (kb[:, :, T:] == canary).all() and (vb[:, :, T:] == canary).all()
        if dtype != "f32":
            c.set_lengths([0] * B)
            on = c.prefill(0, qd, kd, vd, scale=scale)
            check_output(on, ref, dtype, f"T={T} o({dtype})")
            # row 0 sees only key 0: the output is v_0 exactly
            onb = host_bits(on)
            for h in range(H):
                assert np.array_equal(onb[:, h, 0], v[:, h // (H // Hkv), 0].view(onb.dtype))
        c.close()


DECODE_LENS = [1, 7, 256, 257, 700, 1100]


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("heads", HEADS + [(8, 1), (12, 4), (6, 2), (10, 2), (12, 2), (14, 2), (16, 1)],
                         ids=lambda x: f"H{x[0]}kv{x[1]}")
def test_decode_matches_oracle(dtype, D, heads):
    """Ragged contexts across split boundaries; stale slots poisoned with NaN."""
    kv = _kv()
    H, Hkv = heads
    B = len(DECODE_LENS)
    max_T = max(DECODE_LENS) + 5
    scale = float(np.float32(1 / np.sqrt(D)))
    say(f"decode dtype={dtype} D={D} H={H} Hkv={Hkv} lens={DECODE_LENS}")
    c = kv.KVCache(1, B, H, Hkv, D, max_T, TORCH_DT[dtype])
    c.k_view(0).fill_(float("nan"))
    c.v_view(0).fill_(float("nan"))
    hist_k = _rand((B, Hkv, max_T, D), dtype, 11)
    hist_v = _rand((B, Hkv, max_T, D), dtype, 12)
    kview, vview = c.k_view(0), c.v_view(0)
    for b, L in enumerate(DECODE_LENS):
        kview[b, :, :L - 1] = to_dev(hist_k[b, :, :L - 1], dtype)
        vview[b, :, :L - 1] = to_dev(hist_v[b, :, :L - 1], dtype)
    c.set_lengths([L - 1 for L in DECODE_LENS])
    q = _rand((B, H, 1, D), dtype, 13)
    kn = _rand((B, Hkv, 1, D), dtype, 14)
    vn = _rand((B, Hkv, 1, D), dtype, 15)
    c.append(0, to_dev(kn, dtype), to_dev(vn, dtype))
    o32 = c.decode(0, to_dev(q, dtype), scale=scale, out_dtype=torch.float32)
    # oracle cache image
    ck = si.to_f64(hist_k, dtype).copy()
    cv = si.to_f64(hist_v, dtype).copy()
    for b, L in enumerate(DECODE_LENS):
        ck[b, :, L - 1] = si.to_f64(kn[b, :, 0], dtype)
        cv[b, :, L - 1] = si.to_f64(vn[b, :, 0], dtype)
    ref = oracle.decode_cached(si.to_f64(q[:, :, 0], dtype), ck, cv, DECODE_LENS, scale)
    check_output(o32[:, :, 0], ref, dtype, "decode o(f32)")
    if dtype != "f32":
        on = c.decode(0, to_dev(q, dtype), scale=scale)
        check_output(on[:, :, 0], ref, dtype, f"decode o({dtype})")
    # L = 1 sees only its appended row: output is v_new exactly
    b1 = DECODE_LENS.index(1)
    assert np.array_equal(host_bits(o32)[b1, :, 0].view(np.float32),
                          si.to_f64(vn[b1, [h // (H // Hkv) for h in range(H)], 0], dtype).astype(np.float32))
    c.close()


@pytest.mark.parametrize("heads", [(4, 4), (4, 1)], ids=lambda x: f"H{x[0]}kv{x[1]}")
def test_decode_split_workspace_across_calls(heads):
    """Successive decode calls whose split counts differ (many, one, many, a
    few) on two layers of one cache, sharing one split workspace, must each
    match the oracle, and a call repeated on the same inputs must give the
    same bits (the merge runs in split order, whatever order the splits
    finish in)."""
    kv = _kv()
    H, Hkv = heads
    B, D, dtype = 3, 64, "f16"
    max_T = 5000
    scale = float(np.float32(1 / np.sqrt(D)))
    hist_k = _rand((2, B, Hkv, max_T, D), dtype, 31)
    hist_v = _rand((2, B, Hkv, max_T, D), dtype, 32)
    c = kv.KVCache(2, B, H, Hkv, D, max_T, TORCH_DT[dtype])
    for layer in range(2):
        c.k_view(layer).copy_(to_dev(hist_k[layer], dtype))
        c.v_view(layer).copy_(to_dev(hist_v[layer], dtype))
    rounds = [[5000, 4097, 2999], [1, 7, 300], [4999, 5000, 1025], [385, 1024, 2048]]
    for r, lens in enumerate(rounds):
        for layer in range(2):
            say(f"split merge H={H} Hkv={Hkv} round={r} layer={layer} lens={lens}")
            c.set_lengths(lens, layer=layer)
            q = _rand((B, H, 1, D), dtype, 100 + 2 * r + layer)
            qd = to_dev(q, dtype)
            o1 = c.decode(layer, qd, scale=scale, out_dtype=torch.float32)
            o2 = c.decode(layer, qd, scale=scale, out_dtype=torch.float32)
            torch.cuda.synchronize()
            assert np.array_equal(host_bits(o1), host_bits(o2)), "repeated decode differs"
            ref = oracle.decode_cached(si.to_f64(q[:, :, 0], dtype), si.to_f64(hist_k[layer], dtype),
                                       si.to_f64(hist_v[layer], dtype), lens, scale)
            check_output(o1[:, :, 0], ref, dtype, f"decode round {r} layer {layer}")
    c.close()


def test_config1_end_to_end():
    """fp32, B=1, H=4, D=64: prefill 128 then 32 decode steps, every step checked
    against the cached oracle, the recompute oracle, and the GPU's own prefill row."""
    kv = _kv()
    w = si.WORKLOADS[1]
    say(f"fp32 workload end to end: {w.name}")
    T, S, dt = w.prompt, w.steps, w.dtype
    q, k, v = si.prefill_inputs(w, 0, T)
    steps = [si.decode_step_inputs(w, 0, s) for s in range(S)]
    c = kv.KVCache(1, w.batch, w.q_heads, w.kv_heads, w.head_dim, w.max_T, TORCH_DT[dt])
    o = c.prefill(0, to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), scale=w.scale)
    ref = oracle.naive_causal(si.to_f64(q, dt), si.to_f64(k, dt), si.to_f64(v, dt), w.scale)
    check_output(o, ref, dt, "prefill")
    model = oracle.CacheModel(1, w.batch, w.kv_heads, w.head_dim, w.max_T, np.float32)
    model.prefill(0, k, v)
    qh = np.concatenate([q] + [s[0] for s in steps], axis=2)
    kh = np.concatenate([k] + [s[1] for s in steps], axis=2)
    vh = np.concatenate([v] + [s[2] for s in steps], axis=2)
    outs = []
    for s, (qs, ks, vs) in enumerate(steps):
        c.append(0, to_dev(ks, dt), to_dev(vs, dt))
        model.append(0, ks, vs)
        od = c.decode(0, to_dev(qs, dt), scale=w.scale)
        cached = oracle.decode_cached(si.to_f64(qs[:, :, 0], dt), si.to_f64(model.k[0], dt),
                                      si.to_f64(model.v[0], dt), model.lengths[0], w.scale)
        P = T + s
        rec = oracle.decode_recompute(si.to_f64(qh[:, :, :P + 1], dt), si.to_f64(kh[:, :, :P + 1], dt),
                                      si.to_f64(vh[:, :, :P + 1], dt), w.scale)
        assert np.array_equal(cached, rec)
        check_output(od[:, :, 0], cached, dt, f"decode step {s}")
        outs.append(od)
    torch.cuda.synchronize()
    assert c.lengths(0) == [T + S]
    assert np.array_equal(host_bits(c.k_view(0))[:, :, :T + S], kh.view(np.uint32))
    assert np.array_equal(host_bits(c.v_view(0))[:, :, :T + S], vh.view(np.uint32))
    # each decode step against the matching row of a GPU causal prefill of the whole sequence
    c2 = kv.KVCache(1, w.batch, w.q_heads, w.kv_heads, w.head_dim, w.max_T, TORCH_DT[dt])
    full = c2.prefill(0, to_dev(qh, dt), to_dev(kh, dt), to_dev(vh, dt), scale=w.scale)
    fullh = full.cpu().numpy().astype(np.float64)
    for s, od in enumerate(outs):
        check_output(od[:, :, 0], fullh[:, :, T + s], dt, f"step {s} vs GPU prefill row")
    c.close()
    c2.close()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_bound_calls_match_regular_calls(dtype):
    """The pre-bound prefill/append/decode callables enqueue the same C calls: bit-identical outputs."""
    kv = _kv()
    B, H, Hkv, D, T = 2, 4, 2, 64, 77
    say(f"bound calls dtype={dtype}")
    q = to_dev(_rand((B, H, T + 1, D), dtype, 1), dtype)
    k = to_dev(_rand((B, Hkv, T + 1, D), dtype, 2), dtype)
    v = to_dev(_rand((B, Hkv, T + 1, D), dtype, 3), dtype)
    outs = []
    for bound in (False, True):
        c = kv.KVCache(1, B, H, Hkv, D, T + 1, TORCH_DT[dtype])
        qp, kp, vp = q[:, :, :T].contiguous(), k[:, :, :T].contiguous(), v[:, :, :T].contiguous()
        qd, kd, vd = q[:, :, T:].contiguous(), k[:, :, T:].contiguous(), v[:, :, T:].contiguous()
        op = torch.empty_like(qp)
        od = torch.empty_like(qd)
        if bound:
            c.bind_prefill(0, qp, kp, vp, op)()
            c.bind_append(0, kd, vd)()
            c.bind_decode(0, qd, od)()
        else:
            c.prefill(0, qp, kp, vp, out=op)
            c.append(0, kd, vd)
            c.decode(0, qd, out=od)
        torch.cuda.synchronize()
        outs.append((host_bits(op), host_bits(od), host_bits(c._buf)))
        c.close()
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_measurement_aids_run():
    """The plain kernels bench.py reads the device's ceilings with (a streaming
    read, an fp16 MFMA loop, an exp2 loop) launch and finish on small grids;
    their sinks stay untouched (they only write on an unlikely value)."""
    import ctypes
    kv = _kv()
    lib = kv.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    buf = torch.arange(1 << 18, dtype=torch.int32, device="cuda")
    sink_u = torch.zeros(64, dtype=torch.int32, device="cuda")
    sink_f = torch.zeros(64, dtype=torch.float32, device="cuda")
    say("measurement aids: stream read, MFMA loop, exp2 loop")
    assert lib.kvattn_measure_stream_read(ctypes.c_void_p(buf.data_ptr()), buf.numel() * 4, 64,
                                          ctypes.c_void_p(sink_u.data_ptr()), stream) == 0
    assert lib.kvattn_measure_mfma_f16(64, 50, ctypes.c_void_p(sink_f.data_ptr()), stream) == 0
    assert lib.kvattn_measure_exp2(64, 50, ctypes.c_void_p(sink_f.data_ptr()), stream) == 0
    torch.cuda.synchronize()
    assert int(sink_u.abs().sum()) == 0 and float(sink_f.abs().sum()) == 0.0
    assert lib.kvattn_measure_exp2_count(64, 50) == 64 * 256 * 50 * 32
    # the streaming write: word j of a 16-byte-word buffer holds j, j ^ 0x55555555, j + 1, ~j
    n_words = 3 * 64 * 256 * 4 + 37  # past a whole number of grid strides, with a ragged tail
    wbuf = torch.zeros(n_words * 4 + 4, dtype=torch.int32, device="cuda")
    say("measurement aid: stream write")
    assert lib.kvattn_measure_stream_write(ctypes.c_void_p(wbuf.data_ptr()), n_words * 16, 64, stream) == 0
    torch.cuda.synchronize()
    got = wbuf.cpu().numpy().view(np.uint32)
    j = np.arange(n_words, dtype=np.uint32)
    want = np.stack([j, j ^ np.uint32(0x55555555), j + np.uint32(1), ~j], axis=1).reshape(-1)
    assert np.array_equal(got[:4 * n_words], want) and got[4 * n_words:].tolist() == [0, 0, 0, 0]
