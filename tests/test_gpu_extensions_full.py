"""GPU parity of the extensions at the sizes bench.py times them.

On one layer of the batched ragged decode shape (fp16, 32 heads of D=128, batch 32,
contexts uniform in [512, 4096], 1% heavy keys): decode under a 1024-key
window with 4 sink positions, decode from a paged cache of 64-position blocks
drawn from a shuffled pool, and a 4-token verification (extend) after rolling
every sequence back by 4.  Every (sequence, head) output is compared with the
oracle.  Then the T=8192 prompt fed as four 2048-token chunks, on sampled
rows.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_util import TORCH_DT, check_output, free_gpu, say, to_dev

pytestmark = pytest.mark.gpu

W5 = si.WORKLOADS[5]


def _kv():
    import kv_cached_causal_amd as kv
    return kv


def test_window_paged_and_verify_at_config5_decode_shape():
    kv = _kv()
    w, dt = W5, W5.dtype
    ctx = si.decode_contexts(w)
    B, Hkv, D = w.batch, w.kv_heads, w.head_dim
    say(f"{w.name}: one layer, contexts sum {int(ctx.sum())}")
    c = kv.KVCache(1, B, w.q_heads, Hkv, D, w.max_T, TORCH_DT[dt])
    kview, vview = c.k_view(0), c.v_view(0)
    kview.zero_()
    vview.zero_()
    ck = np.zeros((B, Hkv, w.max_T, D))
    cv = np.zeros_like(ck)
    for b in range(B):
        L = int(ctx[b])
        kh, vh = si.decode_history(w, 0, b, L)
        kview[b, :, :L - 1] = to_dev(kh, dt)
        vview[b, :, :L - 1] = to_dev(vh, dt)
        ck[b, :, :L - 1] = si.to_f64(kh, dt)
        cv[b, :, :L - 1] = si.to_f64(vh, dt)
    q, kn, vn = si.decode_step_inputs(w, 0, 0, ctx)
    for b in range(B):
        ck[b, :, int(ctx[b]) - 1] = si.to_f64(kn[b, :, 0], dt)
        cv[b, :, int(ctx[b]) - 1] = si.to_f64(vn[b, :, 0], dt)
    c.set_lengths([int(L) - 1 for L in ctx])
    c.append(0, to_dev(kn, dt), to_dev(vn, dt))
    qd = to_dev(q, dt)
    qf = si.to_f64(q[:, :, 0], dt)

    say("window 1024 + sink 4")
    c.set_window(1024, 4)
    o = c.decode(0, qd, scale=w.scale, out_dtype=torch.float32)
    ref = oracle.decode_cached(qf, ck, cv, ctx, w.scale, window=1024, sink=4)
    check_output(o[:, :, 0], ref, dt, "windowed decode, every (b, h)")
    c.set_window(0, 0)
    full = c.decode(0, qd, scale=w.scale, out_dtype=torch.float32)
    check_output(full[:, :, 0], oracle.decode_cached(qf, ck, cv, ctx, w.scale), dt, "full decode, every (b, h)")

    say("paged: 64-position blocks from a shuffled pool")
    bs = 64
    nblk = [-(-int(L) // bs) for L in ctx]
    perm = np.random.default_rng(56).permutation(sum(nblk)).tolist()
    p = kv.PagedKVCache(1, B, w.max_T // bs, sum(nblk), bs, w.q_heads, Hkv, D, TORCH_DT[dt])
    pk, pv = p.k_view(0), p.v_view(0)
    off = 0
    for b, n in enumerate(nblk):
        ids = perm[off:off + n]
        off += n
        for j, blk in enumerate(ids):
            pk[blk] = kview[b, :, j * bs:(j + 1) * bs]
            pv[blk] = vview[b, :, j * bs:(j + 1) * bs]
        p.set_blocks(b, ids)
    p.set_lengths([int(L) for L in ctx])
    op = p.decode(0, qd, scale=w.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(op, full), "paged decode differs from the contiguous decode of the same rows"
    p.close()

    say("4-token verification after a rollback of 4")
    g = 4
    rng = np.random.default_rng(57)
    qv = si.round_to(rng.standard_normal((B, w.q_heads, g, D)), dt)
    kv_new = si.round_to(rng.standard_normal((B, Hkv, g, D)), dt)
    vv_new = si.round_to(rng.standard_normal((B, Hkv, g, D)), dt)
    base = [int(L) - g for L in ctx]
    c.set_lengths(base)
    ov = c.extend(0, to_dev(qv, dt), to_dev(kv_new, dt), to_dev(vv_new, dt), scale=w.scale,
                  out_dtype=torch.float32)
    torch.cuda.synchronize()
    for b in range(B):
        ck[b, :, base[b]:base[b] + g] = si.to_f64(kv_new[b], dt)
        cv[b, :, base[b]:base[b] + g] = si.to_f64(vv_new[b], dt)
    ref = oracle.extend(si.to_f64(qv, dt), ck, cv, base, w.scale)
    check_output(ov, ref, dt, "4-token verification, every (b, h, t)")
    assert c.lengths(0) == [int(L) for L in ctx]
    c.close()
    free_gpu()


def test_chunked_prefill_8192_in_four_chunks():
    kv = _kv()
    w, dt = W5, W5.dtype
    T, chunk = w.extra_prefill_T, 2048
    say(f"{w.name}: T={T} prompt in chunks of {chunk}")
    q, k, v = si.prefill_inputs(w, 0, T, batch=1, variant=1)
    c = kv.KVCache(1, 1, w.q_heads, w.kv_heads, w.head_dim, T, TORCH_DT[dt])
    outs = []
    for off in range(0, T, chunk):
        sl = slice(off, off + chunk)
        outs.append(c.extend(0, to_dev(np.ascontiguousarray(q[:, :, sl]), dt),
                             to_dev(np.ascontiguousarray(k[:, :, sl]), dt),
                             to_dev(np.ascontiguousarray(v[:, :, sl]), dt), scale=w.scale, out_dtype=torch.float32))
    o = torch.cat(outs, dim=2)
    torch.cuda.synchronize()
    fixed = [0, 1, 63, 64, 2047, 2048, 2049, 4095, 4096, 6143, 6144, T - 1]
    rows = sorted(set(fixed + np.random.default_rng(58).integers(0, T, size=20).tolist()))
    qf, kf, vf = si.to_f64(q, dt), si.to_f64(k, dt), si.to_f64(v, dt)
    ref = np.empty((1, w.q_heads, len(rows), w.head_dim))
    for h in range(w.q_heads):
        for n, i in enumerate(rows):
            ref[0, h, n] = oracle.attend_row(qf[0, h, i], kf[0, h, :i + 1], vf[0, h, :i + 1], w.scale)
    check_output(o[:, :, rows], ref, dt, f"chunked prefill ({len(rows)} sampled rows)")
    assert c.lengths(0) == [T]
    c.close()
    free_gpu()
