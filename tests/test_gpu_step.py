"""The fused decode step (kvattn_append_decode): append + decode in one launch.

The new K/V row of each sequence is stored into the cache bit for bit at
position len[b] and attended from the registers it was loaded into.  The
splits are merged inside the launch when the grid is small (the last
workgroup of a unit merges, the last of a sequence advances its length), else
by a second launch that also commits the lengths; both give the same bits.  Compared with the CPU oracle on seeded inputs:
small shapes over every dtype, head dim and head layout with lengths across
split boundaries (stale slots NaN-poisoned, including the new row's slot),
consecutive steps over several layers, windows, the host capacity check,
graph replays (bit-identical to eager steps; replays past capacity leave a
full sequence unchanged), and the two batched long-context workloads at full
size, where each sampled sequence's step is also compared with the matching
row of a GPU causal prefill of the same sequence.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_util import TORCH_DT, check_output, free_gpu, host_bits, host_f64, say, to_dev

pytestmark = pytest.mark.gpu


def _kv():
    import kv_cached_causal_amd as kv
    return kv


def _rand(shape, dtype, seed):
    return si.round_to(np.random.default_rng(seed).standard_normal(shape), dtype)


HEADS = [(4, 4), (4, 2), (4, 1), (8, 1), (12, 4), (6, 2), (10, 2), (14, 2), (16, 1)]
# lengths before the step (the query then sees len + 1 keys): empty, one key,
# and around the 384-, 768-, 1024- and 2048-key split sizes and their multiples
LENS_BEFORE = [0, 1, 383, 384, 767, 768, 1023, 1024, 1535, 2047, 2048]


def _poisoned_cache(kv, layers, B, H, Hkv, D, max_T, dtype):
    c = kv.KVCache(layers, B, H, Hkv, D, max_T, TORCH_DT[dtype])
    for l in range(layers):
        c.k_view(l).fill_(float("nan"))
        c.v_view(l).fill_(float("nan"))
    return c


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("heads", HEADS, ids=lambda x: f"H{x[0]}kv{x[1]}")
def test_step_matches_oracle_and_writes_the_row(dtype, D, heads):
    kv = _kv()
    H, Hkv = heads
    B = len(LENS_BEFORE)
    max_T = max(LENS_BEFORE) + 3
    scale = float(np.float32(1 / np.sqrt(D)))
    say(f"step dtype={dtype} D={D} H={H} Hkv={Hkv} lens_before={LENS_BEFORE}")
    c = _poisoned_cache(kv, 1, B, H, Hkv, D, max_T, dtype)
    hk = _rand((B, Hkv, max_T, D), dtype, 21)
    hv = _rand((B, Hkv, max_T, D), dtype, 22)
    kview, vview = c.k_view(0), c.v_view(0)
    for b, n in enumerate(LENS_BEFORE):
        if n:
            kview[b, :, :n] = to_dev(hk[b, :, :n], dtype)
            vview[b, :, :n] = to_dev(hv[b, :, :n], dtype)
    c.set_lengths(LENS_BEFORE)
    before = host_bits(c._buf)
    q = _rand((B, H, 1, D), dtype, 23)
    kn = _rand((B, Hkv, 1, D), dtype, 24)
    vn = _rand((B, Hkv, 1, D), dtype, 25)
    o32 = c.append_decode(0, to_dev(kn, dtype), to_dev(vn, dtype), to_dev(q, dtype), scale=scale,
                          out_dtype=torch.float32)
    torch.cuda.synchronize()
    after = host_bits(c._buf)
    lens = [n + 1 for n in LENS_BEFORE]
    assert c.lengths(0) == lens
    # cache image: only the new rows changed, bit for bit
    utype = np.uint32 if dtype == "f32" else np.uint16
    img = before.view(utype).reshape(2, B, Hkv, max_T, D).copy()
    kbits = kn.view(np.uint32 if dtype == "f32" else np.uint16)
    vbits = vn.view(np.uint32 if dtype == "f32" else np.uint16)
    for b, n in enumerate(LENS_BEFORE):
        img[0, b, :, n] = kbits[b, :, 0]
        img[1, b, :, n] = vbits[b, :, 0]
    assert np.array_equal(after.view(utype).reshape(img.shape), img), "cache bytes differ from the expected image"
    ck = si.to_f64(hk, dtype).copy()
    cv = si.to_f64(hv, dtype).copy()
    for b, n in enumerate(LENS_BEFORE):
        ck[b, :, n] = si.to_f64(kn[b, :, 0], dtype)
        cv[b, :, n] = si.to_f64(vn[b, :, 0], dtype)
    ref = oracle.decode_cached(si.to_f64(q[:, :, 0], dtype), ck, cv, lens, scale)
    check_output(o32[:, :, 0], ref, dtype, "step o(f32)")
    # the device length advanced: a plain decode now sees the same keys
    od = c.decode(0, to_dev(q, dtype), scale=scale, out_dtype=torch.float32)
    check_output(od[:, :, 0], ref, dtype, "decode after the step")
    # a sequence with no history sees only its new row: v_new exactly
    b0 = LENS_BEFORE.index(0)
    G = H // Hkv
    assert np.array_equal(host_bits(o32)[b0, :, 0].view(np.float32),
                          si.to_f64(vn[b0, [h // G for h in range(H)], 0], dtype).astype(np.float32))
    if dtype != "f32":
        c.set_lengths(LENS_BEFORE)
        on = c.append_decode(0, to_dev(kn, dtype), to_dev(vn, dtype), to_dev(q, dtype), scale=scale)
        check_output(on[:, :, 0], ref, dtype, f"step o({dtype})")
    c.close()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("heads", [(8, 8), (8, 2)], ids=lambda x: f"H{x[0]}kv{x[1]}")
def test_consecutive_steps_over_layers(dtype, heads):
    """Six steps over three layers of one cache (the split counters and the
    workspace shared by all layers), contexts crossing split boundaries
    during the run; every step against the oracle, the final cache bit for bit."""
    kv = _kv()
    H, Hkv = heads
    layers, B, D, steps = 3, 3, 128, 6
    start = [380, 1021, 2]
    max_T = max(start) + steps + 1
    scale = float(np.float32(1 / np.sqrt(D)))
    c = _poisoned_cache(kv, layers, B, H, Hkv, D, max_T, dtype)
    model = oracle.CacheModel(layers, B, Hkv, D, max_T, si.STORAGE[dtype])
    for l in range(layers):
        hk = _rand((B, Hkv, max(start), D), dtype, 300 + l)
        hv = _rand((B, Hkv, max(start), D), dtype, 310 + l)
        for b, n in enumerate(start):
            c.k_view(l)[b, :, :n] = to_dev(hk[b, :, :n], dtype)
            c.v_view(l)[b, :, :n] = to_dev(hv[b, :, :n], dtype)
            model.k[l, b, :, :n] = hk[b, :, :n]
            model.v[l, b, :, :n] = hv[b, :, :n]
        model.lengths[l] = np.array(start)
    c.set_lengths(start)
    for s in range(steps):
        for l in range(layers):
            say(f"consecutive steps dtype={dtype} H={H} Hkv={Hkv} step={s} layer={l}")
            q = _rand((B, H, 1, D), dtype, 400 + 10 * s + l)
            kn = _rand((B, Hkv, 1, D), dtype, 500 + 10 * s + l)
            vn = _rand((B, Hkv, 1, D), dtype, 600 + 10 * s + l)
            o = c.append_decode(l, to_dev(kn, dtype), to_dev(vn, dtype), to_dev(q, dtype), scale=scale,
                                out_dtype=torch.float32)
            model.append(l, kn, vn)
            Ls = model.lengths[l]
            ref = oracle.decode_cached(si.to_f64(q[:, :, 0], dtype), si.to_f64(model.k[l], dtype),
                                       si.to_f64(model.v[l], dtype), Ls, scale)
            check_output(o[:, :, 0], ref, dtype, f"step {s} layer {l}")
            assert c.lengths(l) == [int(x) for x in Ls]
    for l in range(layers):
        kb = host_bits(c.k_view(l))
        for b in range(B):
            n = int(model.lengths[l][b])
            assert np.array_equal(kb[b, :, :n], model.k[l, b, :, :n].view(kb.dtype))


@pytest.mark.parametrize("mask", [(64, 0), (400, 4), (1000, 16)], ids=lambda m: f"W{m[0]}S{m[1]}")
def test_step_under_a_window(mask):
    kv = _kv()
    W, S = mask
    dtype, H, Hkv, D = "f16", 8, 2, 128
    lens_before = [0, 4, 299, 384, 1099, 1999]
    B = len(lens_before)
    max_T = max(lens_before) + 2
    scale = float(np.float32(1 / np.sqrt(D)))
    say(f"windowed step W={W} S={S} lens_before={lens_before}")
    hk = _rand((B, Hkv, max_T, D), dtype, 71 + W)
    hv = _rand((B, Hkv, max_T, D), dtype, 72 + S)
    q, kn, vn = _rand((B, H, 1, D), dtype, 73), _rand((B, Hkv, 1, D), dtype, 74), _rand((B, Hkv, 1, D), dtype, 75)
    lens = [n + 1 for n in lens_before]
    ck = si.to_f64(hk, dtype).copy()
    cv = si.to_f64(hv, dtype).copy()
    for b, n in enumerate(lens_before):
        ck[b, :, n] = si.to_f64(kn[b, :, 0], dtype)
        cv[b, :, n] = si.to_f64(vn[b, :, 0], dtype)
        hidden = np.ones(max_T, dtype=bool)
        hidden[oracle.visible_keys(n, W, S)] = False
        hidden[n] = False
        ck[b, :, hidden] = np.nan
        cv[b, :, hidden] = np.nan
    c = kv.KVCache(1, B, H, Hkv, D, max_T, TORCH_DT[dtype])
    # the device cache holds NaN in every hidden row and in the new rows' slots
    dk, dv = ck.copy(), cv.copy()
    for b, n in enumerate(lens_before):
        dk[b, :, n] = np.nan
        dv[b, :, n] = np.nan
    c.k_view(0).copy_(torch.from_numpy(dk).to(torch.float16).to("cuda"))
    c.v_view(0).copy_(torch.from_numpy(dv).to(torch.float16).to("cuda"))
    c.set_lengths(lens_before)
    c.set_window(W, S)
    o = c.append_decode(0, to_dev(kn, dtype), to_dev(vn, dtype), to_dev(q, dtype), scale=scale,
                        out_dtype=torch.float32)
    ref = oracle.decode_cached(si.to_f64(q[:, :, 0], dtype), ck, cv, lens, scale, window=W, sink=S)
    assert np.isfinite(ref).all()
    check_output(o[:, :, 0], ref, dtype, "windowed step")
    c.close()


def test_step_capacity_is_checked_on_the_host():
    kv = _kv()
    B, H, Hkv, D, max_T = 2, 4, 2, 64, 10
    c = kv.KVCache(1, B, H, Hkv, D, max_T, torch.float16)
    c.set_lengths([10, 3])
    z = torch.zeros((B, Hkv, 1, D), dtype=torch.float16, device="cuda")
    q = torch.zeros((B, H, 1, D), dtype=torch.float16, device="cuda")
    before = host_bits(c._buf)
    with pytest.raises(kv.KVAttnError) as e:
        c.append_decode(0, z, z, q)
    assert e.value.status == -3
    torch.cuda.synchronize()
    assert c.lengths(0) == [10, 3]
    assert np.array_equal(host_bits(c._buf), before)
    c.close()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_graph_replayed_steps_equal_eager_and_stop_at_capacity(dtype):
    """One fused step of two layers captured in a HIP graph and replayed past
    the capacity of one sequence: every replay equals the eager step bit for
    bit while there is room; a sequence found full on the device is left as
    it is (cache, length and output rows), the others go on."""
    kv = _kv()
    layers, B, H, Hkv, D = 2, 3, 8, 2, 128
    start = [1020, 3000, 7]
    max_T = 3003  # sequence 1 has room for 3 steps
    steps = 5
    scale = float(np.float32(1 / np.sqrt(D)))
    hk = [_rand((B, Hkv, max_T, D), dtype, 800 + l) for l in range(layers)]
    hv = [_rand((B, Hkv, max_T, D), dtype, 810 + l) for l in range(layers)]
    kn, vn = to_dev(_rand((B, Hkv, 1, D), dtype, 820), dtype), to_dev(_rand((B, Hkv, 1, D), dtype, 821), dtype)
    qd = to_dev(_rand((B, H, 1, D), dtype, 822), dtype)
    od = torch.empty((B, H, 1, D), dtype=torch.float32, device="cuda")
    c = kv.KVCache(layers, B, H, Hkv, D, max_T, TORCH_DT[dtype])

    def reset():
        for l in range(layers):
            c.k_view(l).copy_(to_dev(hk[l], dtype))
            c.v_view(l).copy_(to_dev(hv[l], dtype))
        c.set_lengths(start)
        torch.cuda.synchronize()

    reset()
    eager = []
    for s in range(3):
        for l in range(layers):
            c.append_decode(l, kn, vn, qd, out=od, scale=scale, out_dtype=torch.float32)
        torch.cuda.synchronize()
        eager.append(host_bits(od))
    reset()
    od.fill_(float("nan"))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fns = [c.bind_append_decode(l, kn, vn, qd, od, scale=scale) for l in range(layers)]
        for f in fns:
            f()
    torch.cuda.synchronize()
    say(f"graph: {steps} replays of a fused step, sequence 1 has room for 3 ({dtype})")
    for i in range(steps):
        g.replay()
        scratch = torch.randn(1 << 16, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
        got = host_bits(od)
        if i < 3:
            assert np.array_equal(got, eager[i]), f"replay {i} differs from the eager step"
        else:
            # sequence 1 is full: its output rows keep the last written values;
            # the others advanced
            assert np.array_equal(got[1], prev[1]), f"replay {i}: the full sequence's output changed"
        prev = got
    kb = host_bits(c.k_view(layers - 1))
    expect = hk[layers - 1].view(kb.dtype)
    knb = host_bits(kn)
    # sequence 1: three appended rows, then the cache as it was; length at capacity
    assert np.array_equal(kb[1, :, :3000], expect[1, :, :3000])
    for t in range(3000, 3003):
        assert np.array_equal(kb[1, :, t], knb[1, :, 0])
    # sequences 0 and 2 took all five steps
    for b in (0, 2):
        for t in range(start[b], start[b] + steps):
            assert np.array_equal(kb[b, :, t], knb[b, :, 0])
        assert np.array_equal(kb[b, :, start[b] + steps:], expect[b, :, start[b] + steps:])
    del g
    c.close()


@pytest.mark.parametrize("cfg", [4, 5])
def test_batched_long_context_step(cfg):
    """The bf16 GQA 32/8 workload (B=16, context 4096) and the fp16 MHA
    workload (B=32, ragged contexts in [512, 4096], 1% heavy keys) through
    the fused step on layer 0 of the full 32-layer cache: every (b, h)
    against the oracle, the new rows bit for bit; then, for four sequences,
    the step's output against the last row of a GPU causal prefill over the
    same sequence with the step's query as its last query."""
    kv = _kv()
    w = si.WORKLOADS[cfg]
    dt = w.dtype
    ctx = si.decode_contexts(w)
    layer = 0
    c = kv.KVCache(w.layers, w.batch, w.q_heads, w.kv_heads, w.head_dim, w.max_T, TORCH_DT[dt])
    c.set_lengths([int(L) - 1 for L in ctx])
    kview, vview = c.k_view(layer), c.v_view(layer)
    kview.fill_(float("nan"))
    vview.fill_(float("nan"))
    ck = np.zeros((w.batch, w.kv_heads, int(ctx.max()), w.head_dim))
    cv = np.zeros_like(ck)
    hists = {}
    for b in range(w.batch):
        L = int(ctx[b])
        kh, vh = si.decode_history(w, layer, b, L)
        kview[b, :, :L - 1] = to_dev(kh, dt)
        vview[b, :, :L - 1] = to_dev(vh, dt)
        ck[b, :, :L - 1] = si.to_f64(kh, dt)
        cv[b, :, :L - 1] = si.to_f64(vh, dt)
        hists[b] = (kh, vh)
    q, kn, vn = si.decode_step_inputs(w, layer, 0, ctx)
    for b in range(w.batch):
        ck[b, :, int(ctx[b]) - 1] = si.to_f64(kn[b, :, 0], dt)
        cv[b, :, int(ctx[b]) - 1] = si.to_f64(vn[b, :, 0], dt)
    say(f"{w.name}: fused step, layer {layer}")
    o32 = c.append_decode(layer, to_dev(kn, dt), to_dev(vn, dt), to_dev(q, dt), scale=w.scale,
                          out_dtype=torch.float32)
    assert c.lengths(layer) == [int(L) for L in ctx]
    ref = oracle.decode_cached(si.to_f64(q[:, :, 0], dt), ck, cv, ctx, w.scale)
    check_output(o32[:, :, 0], ref, dt, "fused step (f32 out)")
    kb = host_bits(kview)
    for b in range(w.batch):
        assert np.array_equal(kb[b, :, int(ctx[b]) - 1], kn[b, :, 0].view(kb.dtype))
    o_step = host_f64(o32)
    del kview, vview
    c.close()
    free_gpu()
    # the step against the matching row of a GPU causal prefill of the whole sequence
    for b in sorted({0, int(np.argmax(ctx)), int(np.argmin(ctx)), w.batch - 1}):
        L = int(ctx[b])
        kh, vh = hists[b]
        kf = np.concatenate([kh, kn[b:b + 1, :, 0:1][0]], axis=1)[None]
        vf = np.concatenate([vh, vn[b:b + 1, :, 0:1][0]], axis=1)[None]
        qf = si.round_to(np.random.default_rng(900 + b).standard_normal((1, w.q_heads, L, w.head_dim)), dt)
        qf[0, :, L - 1] = q[b, :, 0]
        cp = kv.KVCache(1, 1, w.q_heads, w.kv_heads, w.head_dim, L, TORCH_DT[dt])
        full = host_f64(cp.prefill(0, to_dev(qf, dt), to_dev(kf, dt), to_dev(vf, dt), scale=w.scale,
                                   out_dtype=torch.float32))
        d = float(np.abs(full[0, :, L - 1] - o_step[b, :, 0]).max())
        say(f"  sequence {b} (L={L}): step vs GPU prefill row, max abs diff {d:.3e}")
        assert d <= 2e-3
        cp.close()
    free_gpu()


def test_in_kernel_and_separate_merge_give_the_same_bits():
    """One sequence stepped alone (88 workgroups: merged inside the decode
    launch) and as sequence 0 of a batch of three (264 workgroups: merged by the
    merge kernel) gives the same output bits, cache rows and lengths."""
    kv = _kv()
    dtype, D, H, max_T = "f16", 64, 8, 4000
    scale = float(np.float32(1 / np.sqrt(D)))
    lens = [3001, 2500, 3999 - 8]
    hk = _rand((3, H, max_T, D), dtype, 41)
    hv = _rand((3, H, max_T, D), dtype, 42)
    outs, caches = [], []
    for B in (1, 3):
        say(f"merge paths: B={B}, 11 splits x {H} heads")
        c = _poisoned_cache(kv, 1, B, H, H, D, max_T, dtype)
        for b in range(B):
            c.k_view(0)[b, :, :lens[b]] = to_dev(hk[b, :, :lens[b]], dtype)
            c.v_view(0)[b, :, :lens[b]] = to_dev(hv[b, :, :lens[b]], dtype)
        c.set_lengths(lens[:B])
        steps = []
        for t in range(3):
            q = _rand((3, H, 1, D), dtype, 50 + t)[:B]
            kn = _rand((3, H, 1, D), dtype, 60 + t)[:B]
            vn = _rand((3, H, 1, D), dtype, 70 + t)[:B]
            o = c.append_decode(0, to_dev(kn, dtype), to_dev(vn, dtype), to_dev(q, dtype), scale=scale,
                                out_dtype=torch.float32)
            steps.append(host_bits(o)[0].copy())
        torch.cuda.synchronize()
        assert c.lengths(0) == [n + 3 for n in lens[:B]]
        outs.append(steps)
        caches.append((host_bits(c.k_view(0))[0, :, :lens[0] + 3].copy(), host_bits(c.v_view(0))[0, :, :lens[0] + 3].copy()))
        if B == 1:
            # the first step also against the oracle
            q0 = _rand((3, H, 1, D), dtype, 50)[:1]
            kk = np.concatenate([hk[:1, :, :lens[0]], _rand((3, H, 1, D), dtype, 60)[:1]], axis=2)
            vv = np.concatenate([hv[:1, :, :lens[0]], _rand((3, H, 1, D), dtype, 70)[:1]], axis=2)
            ref = oracle.decode_cached(si.to_f64(q0[:, :, 0], dtype), si.to_f64(kk, dtype), si.to_f64(vv, dtype),
                                       [lens[0] + 1], scale)
            got = steps[0].view(np.float32).astype(np.float64).reshape(ref.shape)
            assert np.abs(got - ref).max() <= 2e-3
        c.close()
        free_gpu()
    for t in range(3):
        assert np.array_equal(outs[0][t], outs[1][t]), f"step {t}: merge paths differ"
    assert np.array_equal(caches[0][0], caches[1][0]) and np.array_equal(caches[0][1], caches[1][1])
