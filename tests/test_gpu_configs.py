"""GPU parity on the five workloads at their real sizes, through the C ABI.

Where the oracle cannot finish a whole workload in seconds, the outputs are
compared on samples the oracle computes one by one (whole layers of decode
steps, selected prompt rows for long prefills).  Every decode step is also
compared with the matching row of a GPU causal prefill over the same sequence.
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


def _prefill_rows_ref(q, k, v, dt, rows, scale, G):
    """Oracle prefill rows for selected query positions: (B, H, len(rows), D)."""
    qf, kf, vf = si.to_f64(q, dt), si.to_f64(k, dt), si.to_f64(v, dt)
    B, H, T, D = qf.shape
    out = np.empty((B, H, len(rows), D))
    for b in range(B):
        for h in range(H):
            g = h // G
            for n, i in enumerate(rows):
                out[b, h, n] = oracle.attend_row(qf[b, h, i], kf[b, g, :i + 1], vf[b, g, :i + 1], scale)
    return out


def _sample_rows(T, seed, extra=24):
    fixed = [0, 1, 2, 15, 16, 63, 64, 65, 127, 128, 129, 255, 256, T // 2, T - 2, T - 1]
    rnd = np.random.default_rng(seed).integers(0, T, size=extra).tolist()
    return sorted(set(r for r in fixed + rnd if 0 <= r < T))


def _run_prompt_then_decode(w, layers_full, layers_sampled, check_recompute_steps=()):
    kv = _kv()
    dt, T, S = w.dtype, w.prompt, w.steps
    c = kv.KVCache(w.layers, w.batch, w.q_heads, w.kv_heads, w.head_dim, w.max_T, TORCH_DT[dt])
    for layer in range(w.layers):
        say(f"{w.name}: prefill layer {layer}")
        q, k, v = si.prefill_inputs(w, layer, T)
        o = c.prefill(layer, to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), scale=w.scale,
                      out_dtype=torch.float32)
        if layer in layers_full:
            ref = oracle.naive_causal(si.to_f64(q, dt), si.to_f64(k, dt), si.to_f64(v, dt), w.scale)
            check_output(o, ref, dt, f"layer {layer} prefill (all rows)")
        elif layer in layers_sampled:
            rows = _sample_rows(T, layer)
            ref = _prefill_rows_ref(q, k, v, dt, rows, w.scale, w.group)
            check_output(o[:, :, rows], ref, dt, f"layer {layer} prefill ({len(rows)} sampled rows)")
        kb = host_bits(c.k_view(layer))[:, :, :T]
        assert np.array_equal(kb, k.view(kb.dtype)), "prefill cache write is not bit-exact"
        assert c.lengths(layer) == [T] * w.batch
    # decode: every step of every layer against the cached oracle
    model = oracle.CacheModel(w.layers, w.batch, w.kv_heads, w.head_dim, w.max_T, si.STORAGE[dt])
    hist = {}
    for layer in range(w.layers):
        q, k, v = si.prefill_inputs(w, layer, T)
        model.prefill(layer, k, v)
        hist[layer] = ([q], [k], [v])
    outs = {layer: [] for layer in range(w.layers)}
    for s in range(S):
        for layer in range(w.layers):
            qs, ks, vs = si.decode_step_inputs(w, layer, s)
            c.append(layer, to_dev(ks, dt), to_dev(vs, dt))
            od = c.decode(layer, to_dev(qs, dt), scale=w.scale, out_dtype=torch.float32)
            model.append(layer, ks, vs)
            L = model.lengths[layer]
            ref = oracle.decode_cached(si.to_f64(qs[:, :, 0], dt),
                                       si.to_f64(model.k[layer, :, :, :L.max()], dt),
                                       si.to_f64(model.v[layer, :, :, :L.max()], dt), L, w.scale)
            check_output(od[:, :, 0], ref, dt, f"layer {layer} decode step {s}")
            outs[layer].append(od)
            hist[layer][0].append(qs); hist[layer][1].append(ks); hist[layer][2].append(vs)
            if layer == 0 and s in check_recompute_steps:
                qh, kh, vh = (np.concatenate(x, axis=2) for x in hist[layer])
                rec = oracle.decode_recompute(si.to_f64(qh, dt), si.to_f64(kh, dt), si.to_f64(vh, dt), w.scale)
                assert np.array_equal(rec, ref), "cached and recompute oracles disagree"
    # native-dtype output of the last step
    qs, _, _ = si.decode_step_inputs(w, 0, S - 1)
    on = c.decode(0, to_dev(qs, dt), scale=w.scale)
    L = model.lengths[0]
    ref = oracle.decode_cached(si.to_f64(qs[:, :, 0], dt), si.to_f64(model.k[0], dt),
                               si.to_f64(model.v[0], dt), L, w.scale)
    check_output(on[:, :, 0], ref, dt, f"layer 0 last decode step, {dt} output")
    # cache image after everything
    for layer in range(w.layers):
        assert np.array_equal(host_bits(c.k_view(layer)), model.k[layer].view(host_bits(c.k_view(layer)).dtype))
    # every decode step of layer 0 against the GPU's own causal prefill of the whole sequence
    qh, kh, vh = (np.concatenate(x, axis=2) for x in hist[0])
    c2 = kv.KVCache(1, w.batch, w.q_heads, w.kv_heads, w.head_dim, w.max_T, TORCH_DT[dt])
    full = host_f64(c2.prefill(0, to_dev(qh, dt), to_dev(kh, dt), to_dev(vh, dt), scale=w.scale,
                               out_dtype=torch.float32))
    worst = 0.0
    for s, od in enumerate(outs[0]):
        d = np.abs(host_f64(od[:, :, 0]) - full[:, :, T + s]).max()
        worst = max(worst, float(d))
    say(f"  decode steps vs GPU prefill rows: max abs diff {worst:.3e}")
    assert worst <= 2e-3
    c.close()
    c2.close()
    free_gpu()


def test_config2_prompt2048_then_128_steps():
    w = si.WORKLOADS[2]
    _run_prompt_then_decode(w, layers_full=[0], layers_sampled=[], check_recompute_steps=(0,))


def test_config3_8_layers_prompt4096_then_128_steps():
    w = si.WORKLOADS[3]
    _run_prompt_then_decode(w, layers_full=[0], layers_sampled=list(range(1, 8)))


@pytest.mark.parametrize("cfg", [3, 5])
def test_long_prefill_8192(cfg):
    """B=1 causal prefill at T=8192 (8-layer H=16, D=32 workload; 32-layer H=32, D=128 workload,
    1% heavy keys), on layers 0 and 31 of the full cache; no T x T buffer."""
    kv = _kv()
    w = si.WORKLOADS[cfg]
    dt, T = w.dtype, w.extra_prefill_T
    layers = w.layers
    c = kv.KVCache(layers, 1, w.q_heads, w.kv_heads, w.head_dim, T, TORCH_DT[dt])
    for layer in sorted({0, layers - 1}):
        say(f"{w.name}: prefill T={T} layer {layer}")
        q, k, v = si.prefill_inputs(w, layer, T, batch=1, variant=1)
        qd, kd, vd = to_dev(q, dt), to_dev(k, dt), to_dev(v, dt)
        o = torch.empty(qd.shape, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        free_before = torch.cuda.mem_get_info()[0]
        c.prefill(layer, qd, kd, vd, out=o, scale=w.scale, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info()[0] >= free_before - (1 << 20), "prefill allocated device memory"
        rows = _sample_rows(T, 100 + layer, extra=32)
        ref = _prefill_rows_ref(q, k, v, dt, rows, w.scale, w.group)
        check_output(o[:, :, rows], ref, dt, f"layer {layer} ({len(rows)} sampled rows, f32 out)")
        c.set_lengths([0], layer=layer)
        on = c.prefill(layer, qd, kd, vd, scale=w.scale)
        check_output(on[:, :, rows], ref, dt, f"layer {layer} ({len(rows)} sampled rows, {dt} out)")
        kb = host_bits(c.k_view(layer))
        assert np.array_equal(kb, k.view(kb.dtype))
        assert np.array_equal(host_bits(c.v_view(layer)), v.view(kb.dtype))
        del qd, kd, vd, o, on
    c.close()
    free_gpu()


@pytest.mark.parametrize("cfg", [4, 5])
def test_batched_long_context_decode(cfg):
    """The bf16 GQA 32/8 workload (B=16, context 4096) and the fp16 MHA workload (B=32,
    ragged contexts in [512, 4096], 1% heavy keys): the full 32-layer cache, with
    layers 0 and 31 filled and checked over every (b, h); stale slots are NaN."""
    kv = _kv()
    w = si.WORKLOADS[cfg]
    dt = w.dtype
    ctx = si.decode_contexts(w)
    say(f"{w.name}: contexts min {ctx.min()} max {ctx.max()} sum {ctx.sum()}")
    c = kv.KVCache(w.layers, w.batch, w.q_heads, w.kv_heads, w.head_dim, w.max_T, TORCH_DT[dt])
    c.set_lengths([int(L) - 1 for L in ctx])
    for layer in (0, w.layers - 1):
        say(f"{w.name}: fill layer {layer}")
        kview, vview = c.k_view(layer), c.v_view(layer)
        kview.fill_(float("nan"))
        vview.fill_(float("nan"))
        ck = np.zeros((w.batch, w.kv_heads, int(ctx.max()), w.head_dim))
        cv = np.zeros_like(ck)
        for b in range(w.batch):
            L = int(ctx[b])
            kh, vh = si.decode_history(w, layer, b, L)
            kview[b, :, :L - 1] = to_dev(kh, dt)
            vview[b, :, :L - 1] = to_dev(vh, dt)
            ck[b, :, :L - 1] = si.to_f64(kh, dt)
            cv[b, :, :L - 1] = si.to_f64(vh, dt)
        q, kn, vn = si.decode_step_inputs(w, layer, 0, ctx)
        for b in range(w.batch):
            ck[b, :, int(ctx[b]) - 1] = si.to_f64(kn[b, :, 0], dt)
            cv[b, :, int(ctx[b]) - 1] = si.to_f64(vn[b, :, 0], dt)
        say(f"{w.name}: append + decode layer {layer}")
        c.append(layer, to_dev(kn, dt), to_dev(vn, dt))
        assert c.lengths(layer) == [int(L) for L in ctx]
        o32 = c.decode(layer, to_dev(q, dt), scale=w.scale, out_dtype=torch.float32)
        on = c.decode(layer, to_dev(q, dt), scale=w.scale)
        ref = oracle.decode_cached(si.to_f64(q[:, :, 0], dt), ck, cv, ctx, w.scale)
        check_output(o32[:, :, 0], ref, dt, f"layer {layer} decode (f32 out)")
        check_output(on[:, :, 0], ref, dt, f"layer {layer} decode ({dt} out)")
        # the appended rows landed at position L_b - 1, bit for bit
        kb = host_bits(kview)
        for b in range(w.batch):
            assert np.array_equal(kb[b, :, int(ctx[b]) - 1], kn[b, :, 0].view(kb.dtype))
        del kview, vview
    c.close()
    free_gpu()
