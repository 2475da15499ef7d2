"""Decode steps captured in a HIP graph (torch.cuda.CUDAGraph over the C ABI).

A decode step (append, then decode, for every layer) takes the lengths from
device memory, so one captured step replayed n times is n steps of
generation (inference chapter, section 9.3: each step appends one K/V row
and attends over the cache).  Checked here:

* every replay's output equals, bit for bit, the eager call sequence's output
  at the same step, with the program's own eager work and synchronisations
  between replays;
* replays past the cache's capacity, which the host-side capacity check
  cannot see (it runs once, at capture), leave the cache and the bytes around
  it as they were: the append kernel drops a position past max_T and leaves
  the length at max_T, and a decode then attends over all max_T rows.
"""
import ctypes

import numpy as np
import pytest
import torch

import synth_inputs as si
from gpu_util import TORCH_DT, check_output, host_bits, say, to_dev
from oracle import attention as oracle

pytestmark = pytest.mark.gpu


def _kv():
    import kv_cached_causal_amd as kv
    return kv


def _rand(shape, dtype, seed):
    return si.round_to(np.random.default_rng(seed).standard_normal(shape), dtype)


@pytest.mark.parametrize("heads", [(8, 8), (8, 2)], ids=lambda x: f"H{x[0]}kv{x[1]}")
@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_graph_replayed_steps_equal_eager(dtype, heads):
    kv = _kv()
    H, Hkv = heads
    L, B, D, T, steps = 2, 3, 64, 700, 6
    max_T = T + steps
    scale = float(np.float32(1 / np.sqrt(D)))
    say(f"graph replay dtype={dtype} H={H} Hkv={Hkv} L={L} B={B} T={T} steps={steps}")
    dev = lambda a: to_dev(a, dtype)
    qs = [dev(_rand((B, H, T, D), dtype, 40 + 3 * l)) for l in range(L)]
    ks = [dev(_rand((B, Hkv, T, D), dtype, 41 + 3 * l)) for l in range(L)]
    vs = [dev(_rand((B, Hkv, T, D), dtype, 42 + 3 * l)) for l in range(L)]
    kn, vn = dev(_rand((B, Hkv, 1, D), dtype, 50)), dev(_rand((B, Hkv, 1, D), dtype, 51))
    qd = dev(_rand((B, H, 1, D), dtype, 52))
    od = torch.empty((B, H, 1, D), dtype=torch.float32, device="cuda")
    c = kv.KVCache(L, B, H, Hkv, D, max_T, TORCH_DT[dtype])

    def prompt():
        c.set_lengths([0] * B)
        for l in range(L):
            c.prefill(l, qs[l], ks[l], vs[l], scale=scale)
        torch.cuda.synchronize()

    def step(app, dec):
        for l in range(L):
            app[l]()
            dec[l]()

    prompt()
    app = [c.bind_append(l, kn, vn) for l in range(L)]
    dec = [c.bind_decode(l, qd, od, scale=scale) for l in range(L)]
    eager = []
    for _ in range(steps):
        step(app, dec)
        torch.cuda.synchronize()
        eager.append(host_bits(od))
    # the first step's output is checked against the oracle too
    prompt()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gapp = [c.bind_append(l, kn, vn) for l in range(L)]
        gdec = [c.bind_decode(l, qd, od, scale=scale) for l in range(L)]
        step(gapp, gdec)
    torch.cuda.synchronize()
    for i in range(steps):
        g.replay()
        scratch = torch.randn(1 << 16, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
        assert np.array_equal(host_bits(od), eager[i]), f"replay {i} differs from the eager step"
    # last layer after the first step, against the oracle
    l = L - 1
    ck = np.concatenate([si.to_f64(host_bits_to_np(ks[l], dtype), dtype), si.to_f64(host_bits_to_np(kn, dtype), dtype)], axis=2)
    cv = np.concatenate([si.to_f64(host_bits_to_np(vs[l], dtype), dtype), si.to_f64(host_bits_to_np(vn, dtype), dtype)], axis=2)
    ref = oracle.decode_cached(si.to_f64(host_bits_to_np(qd, dtype)[:, :, 0], dtype), ck, cv, [T + 1] * B, scale)
    first = torch.from_numpy(eager[0].view(np.float32))
    check_output(first[:, :, 0], ref, dtype, "first step, last layer")
    del g
    c.close()


def host_bits_to_np(t: torch.Tensor, dtype: str) -> np.ndarray:
    """A device tensor back as the storage array synth_inputs uses for `dtype`."""
    b = host_bits(t)
    return b.view(np.float32) if dtype == "f32" else (b.view(np.float16) if dtype == "f16" else b)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_graph_replays_past_capacity_stay_inside_the_cache(dtype):
    kv = _kv()
    L, B, H, Hkv, D, T, room = 2, 2, 4, 2, 64, 50, 3
    max_T = T + room
    scale = float(np.float32(1 / np.sqrt(D)))
    guard = 1 << 16
    tdt = TORCH_DT[dtype]
    nbytes = kv.cache_bytes(L, B, Hkv, D, max_T, tdt)
    big = torch.full((nbytes + 2 * guard,), 0x5A, dtype=torch.uint8, device="cuda")
    c = kv.KVCache.__new__(kv.KVCache)
    c.device = big.device
    c.layers, c.batch, c.q_heads, c.kv_heads = L, B, H, Hkv
    c.head_dim, c.max_T, c.dtype, c.nbytes = D, max_T, tdt, nbytes
    c._handle = ctypes.c_void_p()
    c._buf = big[guard:guard + nbytes]
    torch.cuda.synchronize()
    rc = kv.lib().kvattn_cache_alloc(ctypes.byref(c._handle), L, B, H, Hkv, D, max_T, kv._DT[tdt],
                                     ctypes.c_void_p(c._buf.data_ptr()), nbytes)
    assert rc == 0
    q = [_rand((B, H, T, D), dtype, 60 + 3 * l) for l in range(L)]
    k = [_rand((B, Hkv, T, D), dtype, 61 + 3 * l) for l in range(L)]
    v = [_rand((B, Hkv, T, D), dtype, 62 + 3 * l) for l in range(L)]
    kn, vn, qd = _rand((B, Hkv, 1, D), dtype, 70), _rand((B, Hkv, 1, D), dtype, 71), _rand((B, H, 1, D), dtype, 72)
    kn_d, vn_d, qd_d = to_dev(kn, dtype), to_dev(vn, dtype), to_dev(qd, dtype)
    od = torch.empty((B, H, 1, D), dtype=torch.float32, device="cuda")
    for l in range(L):
        c.prefill(l, to_dev(q[l], dtype), to_dev(k[l], dtype), to_dev(v[l], dtype), scale=scale)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gapp = [c.bind_append(l, kn_d, vn_d) for l in range(L)]
        gdec = [c.bind_decode(l, qd_d, od, scale=scale) for l in range(L)]
        for l in range(L):
            gapp[l]()
            gdec[l]()
    torch.cuda.synchronize()
    n = room + 4
    say(f"graph: {n} replays of an append + decode step into {room} free positions ({dtype})")
    for _ in range(n):
        g.replay()
    torch.cuda.synchronize()
    gb = big.cpu().numpy()
    assert (gb[:guard] == 0x5A).all() and (gb[guard + nbytes:] == 0x5A).all(), "bytes outside the cache written"
    # every layer: the prompt rows, then `room` copies of the appended row, nothing else
    for l in range(L):
        kk = host_bits_to_np(c.k_view(l), dtype)
        vv = host_bits_to_np(c.v_view(l), dtype)
        assert np.array_equal(kk[:, :, :T], k[l]) and np.array_equal(vv[:, :, :T], v[l]), f"layer {l}: prompt rows changed"
        for t in range(T, max_T):
            assert np.array_equal(kk[:, :, t], kn[:, :, 0]) and np.array_equal(vv[:, :, t], vn[:, :, 0])
    # the last replay's decode saw all max_T rows
    l = L - 1
    ck = si.to_f64(np.concatenate([k[l]] + [kn] * room, axis=2), dtype)
    cv = si.to_f64(np.concatenate([v[l]] + [vn] * room, axis=2), dtype)
    ref = oracle.decode_cached(si.to_f64(qd[:, :, 0], dtype), ck, cv, [max_T] * B, scale)
    check_output(od[:, :, 0], ref, dtype, "decode at capacity")
    del g
    c.close()


def test_graph_paged_appends_stop_at_the_block_table_row():
    """Paged cache: replayed appends fill a slot up to the end of its block-table
    row (max_blocks blocks) and then leave the pool as it is; blocks of other
    slots and the unassigned block keep their contents."""
    kv = _kv()
    slots, max_blocks, num_blocks, bs, H, Hkv, D, dtype = 2, 2, 5, 16, 4, 2, 64, "f16"
    c = kv.PagedKVCache(1, slots, max_blocks, num_blocks, bs, H, Hkv, D, TORCH_DT[dtype])
    pk, pv = c.k_view(0), c.v_view(0)  # (num_blocks, Hkv, bs, D)
    pk.fill_(7.0)
    pv.fill_(-7.0)
    tables = [[3, 0], [1, 4]]  # block 2 belongs to no slot
    for s in range(slots):
        c.set_blocks(s, tables[s])
    start = [29, 31]  # capacity max_blocks * bs = 32 positions per slot
    c.set_lengths(start)
    kn, vn = _rand((slots, Hkv, 1, D), dtype, 80), _rand((slots, Hkv, 1, D), dtype, 81)
    kn_d, vn_d = to_dev(kn, dtype), to_dev(vn, dtype)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        c.append(0, kn_d, vn_d)
    torch.cuda.synchronize()
    say("paged graph: 5 replays of an append into 3 and 1 free positions")
    for _ in range(5):
        g.replay()
    torch.cuda.synchronize()
    ek = np.full(tuple(pk.shape), 7.0, dtype=np.float16)
    ev = np.full(tuple(pv.shape), -7.0, dtype=np.float16)
    for s in range(slots):
        for p in range(start[s], max_blocks * bs):
            blk = tables[s][p // bs]
            ek[blk, :, p % bs] = kn[s, :, 0]
            ev[blk, :, p % bs] = vn[s, :, 0]
    assert np.array_equal(host_bits(pk), ek.view(np.uint16)), "K pool differs from the expected appends"
    assert np.array_equal(host_bits(pv), ev.view(np.uint16)), "V pool differs from the expected appends"
    del g
    c.close()


def _guarded_cache(kv, L, B, H, Hkv, D, max_T, tdt, guard=1 << 16):
    """A cache whose payload sits between guard bytes of a larger device buffer."""
    nbytes = kv.cache_bytes(L, B, Hkv, D, max_T, tdt)
    big = torch.full((nbytes + 2 * guard,), 0x5A, dtype=torch.uint8, device="cuda")
    c = kv.KVCache.__new__(kv.KVCache)
    c.device = big.device
    c.layers, c.batch, c.q_heads, c.kv_heads = L, B, H, Hkv
    c.head_dim, c.max_T, c.dtype, c.nbytes = D, max_T, tdt, nbytes
    c._handle = ctypes.c_void_p()
    c._buf = big[guard:guard + nbytes]
    torch.cuda.synchronize()
    rc = kv.lib().kvattn_cache_alloc(ctypes.byref(c._handle), L, B, H, Hkv, D, max_T, kv._DT[tdt],
                                     ctypes.c_void_p(c._buf.data_ptr()), nbytes)
    assert rc == 0
    return c, big, guard, nbytes


@pytest.mark.parametrize("T", [4, 16], ids=["decode_form", "prefill_form"])
def test_graph_extends_past_capacity_leave_the_sequence_unchanged(T):
    """An extend of T rows captured once and replayed three times: sequence 0
    has room for two of them, sequence 1 for all three.  The third replay
    leaves sequence 0 as it is (no row copied, no output row written, length
    unchanged) and goes on for sequence 1; no byte outside the cache is
    written.  T = 4 runs on the decode kernels, T = 16 on the prefill ones."""
    kv = _kv()
    dtype, B, H, Hkv, D, max_T = "f16", 2, 4, 4, 64, 100
    start = [100 - 2 * T - 1, 10]
    scale = float(np.float32(1 / np.sqrt(D)))
    c, big, guard, nbytes = _guarded_cache(kv, 1, B, H, Hkv, D, max_T, torch.float16)
    hk = _rand((B, Hkv, max_T, D), dtype, 900)
    hv = _rand((B, Hkv, max_T, D), dtype, 901)
    c.k_view(0).copy_(to_dev(hk, dtype))
    c.v_view(0).copy_(to_dev(hv, dtype))
    c.set_lengths(start)
    q = _rand((B, H, T, D), dtype, 902)
    kn = _rand((B, Hkv, T, D), dtype, 903)
    vn = _rand((B, Hkv, T, D), dtype, 904)
    qd, knd, vnd = to_dev(q, dtype), to_dev(kn, dtype), to_dev(vn, dtype)
    od = torch.full((B, H, T, D), float("nan"), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        c.extend(0, qd, knd, vnd, out=od, scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    say(f"graph: 3 replays of a {T}-row extend, room for 2 in sequence 0")
    outs = []
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        outs.append(host_bits(od).copy())
    gb = big.cpu().numpy()
    assert (gb[:guard] == 0x5A).all() and (gb[guard + nbytes:] == 0x5A).all(), "bytes outside the cache written"
    # sequence 0: two extends written, then the cache as it was; its third output equals its second
    kk = host_bits(c.k_view(0)).view(np.uint16)
    exp0 = hk[0].view(np.uint16).copy()
    for r in range(2):
        exp0[:, start[0] + r * T:start[0] + (r + 1) * T] = kn[0].view(np.uint16)
    assert np.array_equal(kk[0], exp0), "sequence 0: cache differs from two extends"
    assert np.array_equal(outs[2][0], outs[1][0]), "sequence 0: the skipped extend wrote output rows"
    exp1 = hk[1].view(np.uint16).copy()
    for r in range(3):
        exp1[:, start[1] + r * T:start[1] + (r + 1) * T] = kn[1].view(np.uint16)
    assert np.array_equal(kk[1], exp1), "sequence 1: cache differs from three extends"
    # device lengths (the host copy saw one extend, at capture): a decode
    # reads them, and sees start + 2T and start + 3T keys
    lens = [start[0] + 2 * T, start[1] + 3 * T]
    qs = _rand((B, H, 1, D), dtype, 905)
    o = c.decode(0, to_dev(qs, dtype), scale=scale, out_dtype=torch.float32)
    ck = si.to_f64(np.stack([exp0.view(np.float16), exp1.view(np.float16)]), dtype)
    cv = si.to_f64(hv, dtype).copy()
    for r in range(2):
        cv[0, :, start[0] + r * T:start[0] + (r + 1) * T] = si.to_f64(vn[0], dtype)
    for r in range(3):
        cv[1, :, start[1] + r * T:start[1] + (r + 1) * T] = si.to_f64(vn[1], dtype)
    ref = oracle.decode_cached(si.to_f64(qs[:, :, 0], dtype), ck, cv, lens, scale)
    check_output(o[:, :, 0], ref, dtype, "decode after the replays")
    del g
    c.close()


def test_graph_paged_writes_stop_at_the_slot_blocks():
    """Paged cache whose slot 0 holds fewer blocks than a table row has room
    for: replayed appends and extends stop at the end of the slot's assigned
    blocks (the table entries past them are stale and point at another slot's
    block), leaving every other block as it was."""
    kv = _kv()
    slots, max_blocks, num_blocks, bs, H, Hkv, D, dtype = 2, 4, 6, 16, 4, 2, 64, "f16"
    c = kv.PagedKVCache(1, slots, max_blocks, num_blocks, bs, H, Hkv, D, TORCH_DT[dtype])
    pk, pv = c.k_view(0), c.v_view(0)
    pk.fill_(7.0)
    pv.fill_(-7.0)
    # slot 1 first takes 4 blocks, then gives its table row to slot 0's
    # neighbour: slot 0 keeps one block, and its table row past it still
    # names blocks of slot 1
    c.set_blocks(0, [2, 3, 4, 5])
    c.set_blocks(0, [2])
    c.set_blocks(1, [3, 4, 5, 0])
    start = [13, 0]
    c.set_lengths(start)
    kn, vn = _rand((slots, Hkv, 1, D), dtype, 910), _rand((slots, Hkv, 1, D), dtype, 911)
    kn_d, vn_d = to_dev(kn, dtype), to_dev(vn, dtype)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        c.append(0, kn_d, vn_d)
    torch.cuda.synchronize()
    say("paged graph: 6 replays of an append, slot 0 has room for 3")
    for _ in range(6):
        g.replay()
    torch.cuda.synchronize()
    ek = np.full(tuple(pk.shape), 7.0, dtype=np.float16)
    for p in range(13, 16):
        ek[2, :, p] = kn[0, :, 0]
    for p in range(6):
        ek[3, :, p] = kn[1, :, 0]
    assert np.array_equal(host_bits(pk), ek.view(np.uint16)), "K pool differs from the expected appends"
    # an extend of 8 rows captured at lengths (8, 6) and replayed twice: the
    # second replay finds slot 0 full and skips it, slot 1 advances
    T = 8
    q = to_dev(_rand((slots, H, T, D), dtype, 912), dtype)
    ke, ve = _rand((slots, Hkv, T, D), dtype, 913), _rand((slots, Hkv, T, D), dtype, 914)
    ked, ved = to_dev(ke, dtype), to_dev(ve, dtype)
    c.set_lengths([8, 6])
    torch.cuda.synchronize()
    g2 = torch.cuda.CUDAGraph()
    od = torch.empty((slots, H, T, D), dtype=torch.float16, device="cuda")
    with torch.cuda.graph(g2):
        c.extend(0, q, ked, ved, out=od)
    torch.cuda.synchronize()
    say("paged graph: 2 replays of an 8-row extend, slot 0 has room for 1")
    for _ in range(2):
        g2.replay()
    torch.cuda.synchronize()
    for p in range(8, 16):
        ek[2, :, p] = ke[0, :, p - 8]
    for p in range(6, 22):
        blk = [3, 4, 5, 0][p // bs]
        ek[blk, :, p % bs] = ke[1, :, (p - 6) % T]
    assert np.array_equal(host_bits(pk), ek.view(np.uint16)), "K pool differs after the extends"
    del g, g2
    c.close()
