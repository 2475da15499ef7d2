"""Benchmark of the KV-cached causal attention hot path on one MI355X.

One step = one pass of the whole path on the 32-layer, 32-head, D=128 fp16
workload with 1% of K rows scaled by 8:
  * prefill: a B=1 causal prefill of an 8192-token prompt through all 32
    layers (each layer writes its K/V into the cache), then
  * decode: one decode step of a batch of 32 sequences with ragged contexts
    drawn uniformly from [512, 4096], through all 32 layers (one fused call
    per layer appends the new K/V row and attends the whole cache).
Inputs are seeded synthetic N(0,1) tensors generated on the device and
resident in HBM before timing starts.  The same run also times a decode step
of the 32-layer bf16 GQA workload (32 query / 8 KV heads, batch 16, context
4096).

Printed: one JSON line.  `value` is the decode step's algorithmic HBM bytes
per second (K and V read once per KV head, plus q, o and the appended row);
the prefill's algorithmic TFLOP/s (4*B*H*D*T(T+1)/2 per layer) sits in
`prefill`.  Kernel durations come from HIP events on the launch stream: the
median over every timed launch, with p10 and p90.  `cpu_baseline` times the
CPU fp64 oracle on a bounded sample of the same workload (cached decode,
recompute-everything decode, naive prefill).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import statistics
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import synth_inputs as si  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix peak, TFLOP/s
METRIC = "decode attn HBM GB/s and prefill attn TFLOP/s (% of MI355X roofline)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--skip-gqa", action="store_true")
    p.add_argument("--only", choices=["prefill", "decode", "gqa", "prefill_d32", "small", "sweep"], default=None,
                   help="time one phase only (for profiling runs); prefill_d32: the 8-layer model's D=32 "
                        "prompts at T=4096 and T=8192; small: the three small workloads; sweep: B=1 fp16 "
                        "prefill per layer at T = 512 ... 16384 for 16 heads of D=32 and 32 heads of D=128")
    p.add_argument("--no-extras", action="store_true",
                   help="skip the windowed, paged and extend measurements (profiling runs: their launches "
                        "share kernel names with the headline ones)")
    p.add_argument("--calibrate", action="store_true",
                   help="also run a plain 4 GiB read and a plain 4 GiB write, whose FETCH_SIZE / WRITE_SIZE counter "
                        "readings calibrate the counters (for the --pmc runs that produce profiles/traffic.json)")
    p.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="read the counter_collection.csv files of a FETCH_SIZE and a WRITE_SIZE rocprofv3 run of "
                        "`bench.py --calibrate`, write profiles/traffic.json and exit (no GPU needed)")
    p.add_argument("--trace-summary", nargs=2, metavar=("TRACE_CSV", "WARMUP_FRACTION"),
                   help="summarise the kernel_trace.csv of a rocprofv3 --kernel-trace run: per library kernel, "
                        "the dispatches after the first WARMUP_FRACTION of them (the warmup steps); print and exit")
    return p.parse_args()


def kernel_source_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "kv_cached_causal_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# sources each measured kernel depends on (a traffic figure is dropped once any changes)
DECODE_SOURCES = ["decode.hip", "common.hpp", "kvattn.hip"]
PREFILL_SOURCES = ["prefill.hip", "common.hpp"]
CALIB_BYTES = 4 << 30
# kernels of each measured launch, by a substring of the demangled or mangled name
TRAFFIC_KERNELS = {
    "decode_ragged_b32": (DECODE_SOURCES, ["decode_kernel<kvattn::TagF16, 128, 1, 6, 1, 4, false, false, true, false>",
                                           "decode_merge_kernel<128, 1, true>"]),
    # 256 workgroups: the splits are merged inside the decode launch
    "decode_gqa_b16": (DECODE_SOURCES, ["decode_kernel<kvattn::TagBF16, 128, 4, 4, 1, 8, false, false, true, true>"]),
    "prefill_t8192": (PREFILL_SOURCES, ["prefill_pipe_kernelIDF16_Li128"]),
}


def _counter_medians(directory, counter):
    """Median counter value per kernel name over the dispatches of a rocprofv3 --pmc run."""
    import csv
    import glob
    vals = {}
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: float(np.median(v)) for k, v in vals.items()}


def write_traffic(fetch_dir, write_dir):
    """profiles/traffic.json: HBM bytes per launch from FETCH_SIZE and WRITE_SIZE (KiB per dispatch),
    each scaled by the reading for a plain read (write) of CALIB_BYTES bytes in the same run."""
    fetch = _counter_medians(fetch_dir, "FETCH_SIZE")
    write = _counter_medians(write_dir, "WRITE_SIZE")

    def pick(table, key):
        hits = [v for k, v in table.items() if key in k]
        if len(hits) != 1:
            raise SystemExit(f"expected one kernel matching {key!r}, found {len(hits)}")
        return hits[0]

    f_scale = CALIB_BYTES / 1024.0 / pick(fetch, "stream_read_kernel")
    w_scale = CALIB_BYTES / 1024.0 / pick(write, "stream_write_kernel")
    out = {"calibration": {"bytes": CALIB_BYTES, "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
                           "note": "FETCH_SIZE scaled by a plain streaming read, WRITE_SIZE by a plain streaming "
                                   "write, same run"}}
    for key, (sources, kernels) in TRAFFIC_KERNELS.items():
        fb = sum(pick(fetch, k) for k in kernels) * 1024.0 * f_scale
        wb = sum(pick(write, k) for k in kernels) * 1024.0 * w_scale
        out[key] = {"source_hash": kernel_source_hash(sources), "kernels": kernels,
                    "fetch_bytes_per_launch": int(fb), "write_bytes_per_launch": int(wb),
                    "bytes_per_launch": int(fb + wb)}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def measure_read_ceiling(kv, dev, nbytes=CALIB_BYTES, reps=10):
    """Streaming-read rate of this device (plain read kernel of the library), GB/s."""
    import ctypes
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(8192, dtype=torch.int32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    fn = kv.lib().kvattn_measure_stream_read

    def run():
        if fn(ctypes.c_void_p(buf.data_ptr()), nbytes, 8192, ctypes.c_void_p(sink.data_ptr()), stream) != 0:
            raise RuntimeError("kvattn_measure_stream_read failed")
    for _ in range(3):
        run()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        run()
    b.record()
    torch.cuda.synchronize()
    rate = nbytes / (a.elapsed_time(b) / reps * 1e-3) / 1e9
    del buf, sink
    torch.cuda.empty_cache()
    return rate


def measure_mfma_ceiling(kv, dev, workgroups=1024, iters=20000, reps=5):
    """fp16 MFMA rate of this device (plain matrix-core loop of the library), TFLOP/s."""
    import ctypes
    sink = torch.zeros(workgroups, dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    fn = kv.lib().kvattn_measure_mfma_f16

    def run():
        if fn(workgroups, iters, ctypes.c_void_p(sink.data_ptr()), stream) != 0:
            raise RuntimeError("kvattn_measure_mfma_f16 failed")
    for _ in range(3):
        run()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        run()
    b.record()
    torch.cuda.synchronize()
    flops = kv.lib().kvattn_measure_mfma_f16_flops(workgroups, iters)
    return flops / (a.elapsed_time(b) / reps * 1e-3) / 1e12


def measure_exp_ceiling(kv, dev, workgroups=4096, iters=5000, reps=5):
    """exp2 rate of this device (plain v_exp_f32 loop of the library), exponentials per second."""
    import ctypes
    sink = torch.zeros(workgroups, dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    fn = kv.lib().kvattn_measure_exp2

    def run():
        if fn(workgroups, iters, ctypes.c_void_p(sink.data_ptr()), stream) != 0:
            raise RuntimeError("kvattn_measure_exp2 failed")
    for _ in range(3):
        run()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        run()
    b.record()
    torch.cuda.synchronize()
    n = kv.lib().kvattn_measure_exp2_count(workgroups, iters)
    return n / (a.elapsed_time(b) / reps * 1e-3)


def small_head_prefill(kv, dev, mceil, eceil, reps=20, T=8192, H=16, D=32):
    """The 8-layer x 512-wide model's attention prefill at T (B=1, 16 heads of D=32, fp16; other
    head counts and dims for the sweep): per-launch time against the MFMA peak and against the
    exponential ceiling (one exp2 per unmasked score: at D=32 a score costs only 128 MFMA flops)."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(32)
    dt = torch.float16
    q = torch.randn((1, H, T, D), generator=gen, device=dev).to(dt)
    k = torch.randn((1, H, T, D), generator=gen, device=dev).to(dt)
    v = torch.randn((1, H, T, D), generator=gen, device=dev).to(dt)
    o = torch.empty_like(q)
    c = kv.KVCache(1, 1, H, H, D, T, dt, device=dev)
    call = c.bind_prefill(0, q, k, v, o, scale=D ** -0.5)
    times = []
    for i in range(reps + 3):
        c.set_lengths([0])
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        call()
        b.record()
        torch.cuda.synchronize()
        if i >= 3:
            times.append(a.elapsed_time(b))
    c.close()
    med = statistics.median(times) * 1e-3
    flops = 4.0 * H * D * T * (T + 1) / 2
    exps = H * T * (T + 1) / 2
    what = " (the 8L x 512d model's attention)" if (H, D) == (16, 32) else ""
    return {"workload": f"T={T} causal prefill, B=1, H={H}, D={D}, fp16{what}",
            "us_per_layer": round(med * 1e6, 1), "value": round(flops / med / 1e12, 1), "unit": "TFLOP/s",
            "frac_of_mfma_peak": round(flops / med / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
            "mfma_bound_us": round(flops / (mceil * 1e12) * 1e6, 1),
            "exp_bound_us": round(exps / eceil * 1e6, 1), "exps_per_layer": int(exps),
            "frac_of_exp_ceiling": round(exps / eceil / med, 4)}


def small_config_measurements(kv, dev):
    """The three small workloads, whole: prompt prefill of every layer, then every decode step
    (one fused append + decode call per layer), timed with HIP events around the prefills and around the steps
    (median of five runs).  Their caches (0.3-69 MB) stay in
    the 256 MB last-level cache and their launches take a few microseconds, so they are reported in
    microseconds per step (launch-bound), not as bandwidth."""
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
    out = {}
    for cfg in (1, 2, 3):
        w = si.WORKLOADS[cfg]
        dt = tdt[w.dtype]
        B, H, Hkv, D, T, L = w.batch, w.q_heads, w.kv_heads, w.head_dim, w.prompt, w.layers
        gen = torch.Generator(device=dev)
        gen.manual_seed(100 + cfg)
        rnd = lambda shape: torch.randn(shape, generator=gen, device=dev).to(dt)
        c = kv.KVCache(L, B, H, Hkv, D, w.max_T, dt, device=dev)
        # the bound calls hold raw pointers: keep the tensors alive alongside them
        ins = [(rnd((B, H, T, D)), rnd((B, Hkv, T, D)), rnd((B, Hkv, T, D)),
                torch.empty((B, H, T, D), dtype=dt, device=dev)) for _ in range(L)]
        pre = [c.bind_prefill(l, *ins[l], scale=w.scale) for l in range(L)]
        kn, vn, qd = rnd((B, Hkv, 1, D)), rnd((B, Hkv, 1, D)), rnd((B, H, 1, D))
        od = torch.empty((B, H, 1, D), dtype=dt, device=dev)
        dec = [c.bind_append_decode(l, kn, vn, qd, od, scale=w.scale) for l in range(L)]

        def run():
            # one event pair around all layers' prefills and one around all steps: an event
            # pair per launch adds its own gap to launches this short
            c.set_lengths([0] * B)
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record()
            for l in range(L):
                pre[l]()
            e[1].record()
            for _ in range(w.steps):
                for l in range(L):
                    dec[l]()
            e[2].record()
            torch.cuda.synchronize()
            return e[0].elapsed_time(e[1]) / L, e[1].elapsed_time(e[2]) / w.steps
        run()
        reps = [run() for _ in range(5)]
        c.close()
        pre_ms = statistics.median(r[0] for r in reps)
        step_ms = statistics.median(r[1] for r in reps)
        flops = 4.0 * B * H * D * T * (T + 1) / 2
        out[w.name] = {"prefill_us_per_layer": round(pre_ms * 1e3, 1),
                       "prefill_tflops": round(flops / (pre_ms * 1e-3) / 1e12, 2),
                       "decode_step_us": round(step_ms * 1e3, 1),
                       "decode_us_per_layer": round(step_ms * 1e3 / L, 2),
                       "decode_tok_s": round(B / (step_ms * 1e-3), 1),
                       "whole_run_ms": round(pre_ms * L + step_ms * w.steps, 3),
                       "note": f"{L} layer(s), B={B}, {H}/{Hkv} heads, D={D}, {w.dtype}: prompt {T} then "
                               f"{w.steps} steps; launch-bound, cache-resident"}
    return out


def calibration_kernels(kv, dev):
    """A plain read and a plain write of CALIB_BYTES each (run under --pmc to calibrate the HBM
    counters): the library's streaming kernels, 16-byte words per lane, coalesced."""
    import ctypes
    buf = torch.empty(CALIB_BYTES // 2, dtype=torch.float16, device=dev)
    sink = torch.zeros(8192, dtype=torch.int32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    for _ in range(3):
        if kv.lib().kvattn_measure_stream_write(ctypes.c_void_p(buf.data_ptr()), CALIB_BYTES, 8192, stream) != 0:
            raise RuntimeError("kvattn_measure_stream_write failed")
        if kv.lib().kvattn_measure_stream_read(ctypes.c_void_p(buf.data_ptr()), CALIB_BYTES, 8192,
                                               ctypes.c_void_p(sink.data_ptr()), stream) != 0:
            raise RuntimeError("kvattn_measure_stream_read failed")
    torch.cuda.synchronize()
    del buf, sink
    torch.cuda.empty_cache()


def traffic_from_profiles(kernel_key, src_hash):
    """HBM bytes per launch measured by rocprofv3 counters, if taken on this kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
        e = t[kernel_key]
        if e.get("source_hash") == src_hash:
            return e["bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        pass
    return None


def fill_normal_(t: torch.Tensor, gen: torch.Generator, chunk=1 << 26):
    flat = t.view(-1)
    for i in range(0, flat.numel(), chunk):
        n = min(chunk, flat.numel() - i)
        flat[i:i + n] = torch.randn(n, generator=gen, device=t.device, dtype=torch.float32).to(t.dtype)


def heavy_scale_(k_block: torch.Tensor, L, frac, gen: torch.Generator):
    """Scale 1% of each sequence's visible K rows by 8 (k_block: (B, Hkv, max_T, D))."""
    B, Hkv = k_block.shape[:2]
    for b in range(B):
        n = int(L[b])
        c = si.heavy_count(n, frac)
        for h in range(Hkv):
            rows = torch.randperm(n, generator=gen, device=k_block.device)[:c]
            k_block[b, h, rows] *= 8


class Timer:
    """Per-launch HIP event pairs on the current stream (the stream the library's calls are enqueued on)."""

    def __init__(self):
        self.pairs = []

    def start(self):
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def stop(self, s):
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.append((s, e))

    def times_ms(self):
        return [a.elapsed_time(b) for a, b in self.pairs]

    def mean_ms(self):
        return float(np.mean(self.times_ms())) if self.pairs else float("nan")

    def median_ms(self):
        return float(np.median(self.times_ms())) if self.pairs else float("nan")

    def spread(self):
        """Launch count, median, p10, p90 and mean of the per-launch times (ms)."""
        t = np.array(self.times_ms())
        return {"launches": int(t.size), "median_ms": round(float(np.median(t)), 5),
                "p10_ms": round(float(np.percentile(t, 10)), 5), "p90_ms": round(float(np.percentile(t, 90)), 5),
                "mean_ms": round(float(t.mean()), 5)}


def setup_decode(kv, w, dev, seed):
    ctx = si.decode_contexts(w)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    dt = {"f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    cache = kv.KVCache(w.layers, w.batch, w.q_heads, w.kv_heads, w.head_dim, w.max_T, dt, device=dev)
    for layer in range(w.layers):
        fill_normal_(cache.k_view(layer), gen)
        fill_normal_(cache.v_view(layer), gen)
        if w.heavy_frac > 0:
            heavy_scale_(cache.k_view(layer), ctx, w.heavy_frac, gen)
    qs = [torch.randn((w.batch, w.q_heads, 1, w.head_dim), generator=gen, device=dev).to(dt) for _ in range(w.layers)]
    kn = [torch.randn((w.batch, w.kv_heads, 1, w.head_dim), generator=gen, device=dev).to(dt) for _ in range(w.layers)]
    vn = [torch.randn((w.batch, w.kv_heads, 1, w.head_dim), generator=gen, device=dev).to(dt) for _ in range(w.layers)]
    outs = [torch.empty_like(q) for q in qs]
    appends = [cache.bind_append(l, kn[l], vn[l]) for l in range(w.layers)]
    decodes = [cache.bind_decode(l, qs[l], outs[l], scale=w.scale) for l in range(w.layers)]
    # the decode step as one call per layer: append + decode fused (kvattn_append_decode)
    steps = [cache.bind_append_decode(l, kn[l], vn[l], qs[l], outs[l], scale=w.scale) for l in range(w.layers)]
    e = 2
    bytes_kernel = int(2 * w.kv_heads * w.head_dim * e * int(ctx.sum())   # K and V once per KV head
                       + 2 * w.batch * w.q_heads * w.head_dim * e)         # q in, o out
    bytes_step_layer = bytes_kernel + 2 * w.batch * w.kv_heads * w.head_dim * e  # + appended row
    return dict(w=w, ctx=ctx, cache=cache, q=qs, kn=kn, vn=vn, o=outs, appends=appends, decodes=decodes,
                steps=steps, bytes_kernel=bytes_kernel, bytes_step_layer=bytes_step_layer,
                bytes_step=bytes_step_layer * w.layers)


def reset_decode(d):
    """Lengths back to the step's starting contexts (outside the timed region)."""
    d["cache"].set_lengths([int(L) - 1 for L in d["ctx"]])


def decode_step(d, timer=None):
    """One decode step of every layer: the fused append + decode call per layer (timed per launch)."""
    w = d["w"]
    for layer in range(w.layers):
        ev = timer.start() if timer else None
        d["steps"][layer]()
        if timer:
            timer.stop(ev)


def decode_step_two_calls(d, timer=None):
    """The same step as two calls per layer (kvattn_append, then kvattn_decode; the decode timed)."""
    w = d["w"]
    reset_decode(d)
    for layer in range(w.layers):
        d["appends"][layer]()
        ev = timer.start() if timer else None
        d["decodes"][layer]()
        if timer:
            timer.stop(ev)


def setup_prefill(kv, w, dev, seed):
    T = w.extra_prefill_T
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    dt = torch.float16
    cache = kv.KVCache(w.layers, 1, w.q_heads, w.kv_heads, w.head_dim, T, dt, device=dev)
    q, k, v, o = [], [], [], []
    for layer in range(w.layers):
        shape_q = (1, w.q_heads, T, w.head_dim)
        shape_kv = (1, w.kv_heads, T, w.head_dim)
        q.append(torch.randn(shape_q, generator=gen, device=dev).to(dt))
        kk = torch.randn(shape_kv, generator=gen, device=dev).to(dt)
        heavy_scale_(kk, [T], w.heavy_frac, gen)
        k.append(kk)
        v.append(torch.randn(shape_kv, generator=gen, device=dev).to(dt))
        o.append(torch.empty(shape_q, dtype=dt, device=dev))
    flops = 4.0 * 1 * w.q_heads * w.head_dim * T * (T + 1) / 2
    calls = [cache.bind_prefill(l, q[l], k[l], v[l], o[l], scale=w.scale) for l in range(w.layers)]
    return dict(w=w, T=T, cache=cache, q=q, k=k, v=v, o=o, calls=calls, flops_layer=flops)


def reset_prefill(p):
    p["cache"].set_lengths([0])


def prefill_step(p, timer=None):
    w = p["w"]
    for layer in range(w.layers):
        ev = timer.start() if timer else None
        p["calls"][layer]()
        if timer:
            timer.stop(ev)


def extend_measurements(kv, w, dec, pre, reps=3):
    """The extend path on the same workload: (a) the T=8192 prompt of 4 layers fed as four
    2048-token chunks (algorithmic flops as for one prefill), (b) a 4-token verification step
    on the ragged batch-32 decode cache (K/V of every sequence read once per query head, plus
    the 4 new rows), then rolled back."""
    out = {}
    T, layers, chunk = pre["T"], 4, 2048
    c = kv.KVCache(layers, 1, w.q_heads, w.kv_heads, w.head_dim, T, torch.float16, device=pre["q"][0].device)
    calls = []
    for l in range(layers):
        for off in range(0, T, chunk):
            sl = slice(off, off + chunk)
            q, k, v = (pre[n][l][:, :, sl].contiguous() for n in ("q", "k", "v"))
            calls.append((l, q, k, v, torch.empty_like(q)))

    def run_chunked():
        c.set_lengths([0])
        for l, q, k, v, o in calls:
            c.extend(l, q, k, v, out=o, scale=w.scale)
    run_chunked()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        run_chunked()
    b.record()
    torch.cuda.synchronize()
    ms_layer = a.elapsed_time(b) / reps / layers
    out["chunked_prefill"] = {"workload": f"T={T} in {T // chunk} chunks of {chunk}, H={w.q_heads}, D={w.head_dim}",
                              "us_per_layer": round(ms_layer * 1e3, 1),
                              "value": round(pre["flops_layer"] / (ms_layer * 1e-3) / 1e12, 1), "unit": "TFLOP/s"}
    c.close()
    del calls
    # verification of 4 draft positions per sequence on the decode cache, then rollback
    g = 4
    dc = dec["cache"]
    ctx = dec["ctx"]
    dev = dec["q"][0].device
    gen = torch.Generator(device=dev)
    gen.manual_seed(44)
    qv = torch.randn((w.batch, w.q_heads, g, w.head_dim), generator=gen, device=dev).to(torch.float16)
    kvn = torch.randn((w.batch, w.kv_heads, g, w.head_dim), generator=gen, device=dev).to(torch.float16)
    ov = torch.empty_like(qv)
    base = [int(L) - g for L in ctx]

    def run_verify():
        dc.set_lengths(base)
        for l in range(layers):
            dc.extend(l, qv, kvn, kvn, out=ov, scale=w.scale)
    run_verify()
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        run_verify()
    b.record()
    torch.cuda.synchronize()
    ms_layer = a.elapsed_time(b) / reps / layers
    e = 2
    nbytes = 2 * w.kv_heads * w.head_dim * e * int(ctx.sum()) + 2 * w.batch * w.q_heads * g * w.head_dim * e
    out["verify_4_tokens"] = {"workload": f"batch {w.batch}, contexts U[{w.ctx_lo},{w.ctx_hi}] (4 new each)",
                              "us_per_layer": round(ms_layer * 1e3, 1),
                              "value": round(nbytes / (ms_layer * 1e-3) / 1e9, 1), "unit": "GB/s"}
    return out


def window_measurements(kv, w, dec, full_us, window=1024, sink=4, reps=5):
    """Decode of the ragged batch-32 cache under a sliding window of `window` keys plus
    `sink` sink positions: only the visible rows are read (min(L, window + sink) per
    sequence), so the time per layer falls with the visible share of the contexts."""
    c, ctx = dec["cache"], dec["ctx"]
    vis = int(sum(min(int(L), window + sink) for L in ctx))
    c.set_lengths([int(L) for L in ctx])
    c.set_window(window, sink)

    def run():
        for d in dec["decodes"]:
            d()
    run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        run()
    b.record()
    torch.cuda.synchronize()
    c.set_window(0, 0)
    us = a.elapsed_time(b) * 1e3 / reps / w.layers
    e = 2
    nbytes = 2 * w.kv_heads * w.head_dim * e * vis + 2 * w.batch * w.q_heads * w.head_dim * e
    return {"workload": f"batch {w.batch}, contexts U[{w.ctx_lo},{w.ctx_hi}], window {window} + sink {sink}",
            "us_per_layer": round(us, 1), "visible_fraction": round(vis / int(ctx.sum()), 4),
            "value": round(nbytes / (us * 1e-6) / 1e9, 1), "unit": "GB/s",
            "speedup_vs_full_context": round(full_us / us, 2)}


def paged_measurements(kv, w, dec, full_us, block_size=64, layers=4, reps=5):
    """Decode of the ragged batch-32 contexts from a block-paged cache: each
    sequence holds ceil(L / block_size) blocks drawn from one shuffled pool (no
    capacity reserved beyond the blocks in use).  Same algorithmic bytes as the
    contiguous decode."""
    ctx = [int(L) for L in dec["ctx"]]
    nblk = [-(-L // block_size) for L in ctx]
    num_blocks = sum(nblk)
    dev = dec["q"][0].device
    dt = {"f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    c = kv.PagedKVCache(layers, w.batch, max(nblk), num_blocks, block_size, w.q_heads, w.kv_heads, w.head_dim,
                        dt, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(55)
    for layer in range(layers):
        fill_normal_(c.k_view(layer), gen)
        fill_normal_(c.v_view(layer), gen)
    perm = torch.randperm(num_blocks, generator=torch.Generator().manual_seed(56)).tolist()
    off = 0
    for s, n in enumerate(nblk):
        c.set_blocks(s, perm[off:off + n])
        off += n
    c.set_lengths(ctx)
    outs = [torch.empty_like(dec["q"][l]) for l in range(layers)]
    calls = [c.bind_decode(l, dec["q"][l], outs[l], scale=w.scale) for l in range(layers)]

    def run():
        for f in calls:
            f()
    run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        run()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / reps / layers
    out = {"workload": f"batch {w.batch}, contexts U[{w.ctx_lo},{w.ctx_hi}], {block_size}-position blocks, "
                       f"shuffled pool",
           "us_per_layer": round(us, 1),
           "value": round(dec["bytes_kernel"] / (us * 1e-6) / 1e9, 1), "unit": "GB/s",
           "vs_contiguous_time": round(us / full_us, 3),
           "pool_bytes_per_layer": c.nbytes // layers,
           "contiguous_bytes_per_layer": dec["cache"].nbytes // w.layers}
    c.close()
    return out


def decoder_measurements(kv, dev, prompt=4096, new_tokens=128):
    """The README's 8-layer, 512-wide, 16-head decoder (vocabulary 4096) with random
    weights: prompt of `prompt` tokens, then `new_tokens` greedy tokens, batch 1 (the
    README's KV-cache table) and batch 8.  Generation enqueues the steps back to back with
    the token kept on the device."""
    spec = si.TINYGPT
    flat = torch.from_numpy(si.pack_model_weights(spec, si.model_weights(spec))).to(dev)
    out = {"workload": f"{spec.layers}L x {spec.d_model}d, {spec.heads} heads, vocab {spec.vocab}, fp16 weights; "
                       f"prompt {prompt}, +{new_tokens} greedy tokens",
           "context": "llm-perf-lab README: 41.2 tok/s with KV cache after a 4096-token prompt "
                      "(RTX 3090, PyTorch eager, 128 new tokens)"}
    for batch in (1, 8):
        m = kv.Decoder(spec.layers, spec.d_model, spec.heads, spec.vocab, spec.max_T, spec.mlp_mult, batch, flat)
        tokens = torch.from_numpy(si.model_tokens(spec, batch, prompt)).to(dev)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        for rep in range(2):  # the first pass warms rocBLAS and the kernels
            m.reset()
            ev[0].record()
            _, nxt = m.prefill(tokens)
            ev[1].record()
            m.generate(new_tokens, nxt)
            ev[2].record()
            torch.cuda.synchronize()
        pre_ms, dec_ms = ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[2])
        m.reset()
        _, nxt = m.prefill(tokens)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(32):
            _, nxt = m.step(nxt)
        b.record()
        torch.cuda.synchronize()
        eager_ms = a.elapsed_time(b) / 32
        out[f"batch{batch}"] = {
            "prefill_ms": round(pre_ms, 3), "decode_ms_per_token": round(dec_ms / new_tokens, 4),
            "decode_tok_s": round(batch * new_tokens / (dec_ms * 1e-3), 1),
            "end_to_end_tok_s": round(batch * new_tokens / ((pre_ms + dec_ms) * 1e-3), 1),
            "eager_step_ms": round(eager_ms, 4)}
        m.close()
    return out


def prefill_memory_and_clock(kv, pre):
    """Peak device memory while the 32 prefills run (no T x T buffer: the prefill allocates
    nothing beyond its inputs, outputs and the cache), and the sustained shader clock of one
    prefill launch (workgroup 0's shader-clock and 100 MHz real-time counters)."""
    import ctypes
    reset_prefill(pre)
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    prefill_step(pre)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated()
    w, T = pre["w"], pre["T"]
    sample = torch.zeros(2, dtype=torch.int64, device=pre["q"][0].device)
    c = pre["cache"]
    c.set_lengths([0], layer=0)
    rc = kv.lib().kvattn_measure_prefill_clock(
        c._handle, 0, ctypes.c_void_p(pre["q"][0].data_ptr()), ctypes.c_void_p(pre["k"][0].data_ptr()),
        ctypes.c_void_p(pre["v"][0].data_ptr()), ctypes.c_void_p(pre["o"][0].data_ptr()), T, ctypes.c_float(w.scale),
        1, ctypes.c_void_p(sample.data_ptr()), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if rc != 0:
        raise RuntimeError(f"kvattn_measure_prefill_clock failed ({rc})")
    torch.cuda.synchronize()
    cyc, ticks = (int(x) for x in sample.cpu().tolist())
    clock = cyc / ticks * 0.1 if ticks > 0 else None
    return {"peak_bytes_during_prefill": int(peak), "allocated_before_bytes": int(base),
            "extra_bytes_during_prefill": int(peak - base),
            "tt_scores_fp32_bytes_per_layer": int(w.q_heads * T * T * 4),
            "sustained_clock_ghz": round(clock, 3) if clock else None}


def timed(fn, steps, warmup):
    for _ in range(warmup):
        fn(None)
    torch.cuda.synchronize()
    timer = Timer()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn(timer)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, timer.mean_ms()


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline():
    """The oracle, as it stands, on a bounded sample of the same workload: the cached decode
    (one layer-step of 8 sequences), the recompute-everything decode (one sequence, 4 heads:
    every row of the history recomputed, as the uncached generation loop does) and the naive
    prefill (2 heads at T=8192, materialising T x T)."""
    import oracle
    w = si.WORKLOADS[5]
    cores = len(os.sched_getaffinity(0))
    blas_threads, blas = None, None
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            blas_threads = max(i.get("num_threads", 0) for i in info)
            blas = info[0].get("internal_api")
    except Exception:
        pass
    ctx = si.decode_contexts(w)
    n_seq = 8
    log(f"cpu baseline: generating decode sample ({n_seq} sequences of layer 0)")
    ks, vs = [], []
    for b in range(n_seq):
        kh, vh = si.decode_history(w, 0, b, int(ctx[b]))
        ks.append(si.to_f64(kh, w.dtype))
        vs.append(si.to_f64(vh, w.dtype))
    q, kn, vn = si.decode_step_inputs(w, 0, 0, ctx)
    Lmax = int(ctx[:n_seq].max())
    ck = np.zeros((n_seq, w.kv_heads, Lmax, w.head_dim))
    cv = np.zeros_like(ck)
    for b in range(n_seq):
        L = int(ctx[b])
        ck[b, :, :L - 1] = ks[b]
        cv[b, :, :L - 1] = vs[b]
        ck[b, :, L - 1] = si.to_f64(kn[b, :, 0], w.dtype)
        cv[b, :, L - 1] = si.to_f64(vn[b, :, 0], w.dtype)
    qf = si.to_f64(q[:n_seq, :, 0], w.dtype)
    reps, t_dec = 0, 0.0
    t0 = time.perf_counter()
    while t_dec < 5.0:
        oracle.decode_cached(qf, ck, cv, ctx[:n_seq], w.scale)
        reps += 1
        t_dec = time.perf_counter() - t0
    dec_bytes = reps * (2 * w.kv_heads * w.head_dim * 2 * int(ctx[:n_seq].sum())
                        + 2 * n_seq * w.q_heads * w.head_dim * 2)
    cached_us_per_seq_head = t_dec / reps / (n_seq * w.q_heads) * 1e6
    # recompute-everything decode: sequence 0, 4 heads, every row of its L positions recomputed
    rh = 4
    L0 = int(ctx[0])
    qh = si.round_to(np.random.default_rng(55).standard_normal((1, rh, L0, w.head_dim)), w.dtype)
    qh[0, :, L0 - 1] = q[0, :rh, 0]
    log(f"cpu baseline: recompute decode of {rh} heads at context {L0}")
    t0 = time.perf_counter()
    rec = oracle.decode_recompute(si.to_f64(qh, w.dtype), ck[0:1, :rh, :L0], cv[0:1, :rh, :L0], w.scale)
    t_rec = time.perf_counter() - t0
    ref = oracle.decode_cached(qf[0:1, :rh], ck[0:1, :rh, :L0], cv[0:1, :rh, :L0], [L0], w.scale)
    if not np.array_equal(rec, ref):
        raise RuntimeError("cached and recompute oracles disagree")
    recompute_us_per_seq_head = t_rec / rh * 1e6
    cached_one = []
    for _ in range(20):
        t0 = time.perf_counter()
        oracle.decode_cached(qf[0:1, :rh], ck[0:1, :rh, :L0], cv[0:1, :rh, :L0], [L0], w.scale)
        cached_one.append(time.perf_counter() - t0)
    cached_one_us = statistics.median(cached_one) / rh * 1e6
    # prefill sample: whole heads of one layer at T = 8192, naive (materialises T x T)
    T = w.extra_prefill_T
    n_heads = 2
    log(f"cpu baseline: naive prefill of {n_heads} heads at T={T}")
    pq, pk, pv = si.prefill_inputs(w, 0, T, batch=1, variant=1)
    pq = si.to_f64(pq[:, :n_heads], w.dtype)
    pk = si.to_f64(pk[:, :n_heads], w.dtype)
    pv = si.to_f64(pv[:, :n_heads], w.dtype)
    t0 = time.perf_counter()
    oracle.naive_causal(pq, pk, pv, w.scale)
    t_pre = time.perf_counter() - t0
    pre_flops = 4.0 * n_heads * w.head_dim * T * (T + 1) / 2
    return {
        "value": round(dec_bytes / t_dec / 1e9, 4), "unit": "GB/s", "cores": int(cores), "kind": "oracle",
        "sample": (f"cached decode: layer 0 of the ragged batch-32 workload, first {n_seq} sequences x 32 heads "
                   f"(sum of contexts {int(ctx[:n_seq].sum())}), {reps} repetitions in {t_dec:.1f} s, fp64 NumPy; "
                   f"recompute decode: sequence 0 (context {L0}), {rh} heads, every history row recomputed, "
                   f"{t_rec:.1f} s; prefill: {n_heads} of 32 heads of one layer at T={T}, naive fp64 in {t_pre:.1f} s"),
        "cpu_model": cpu_model(), "blas": blas, "blas_threads": blas_threads,
        "prefill": {"value": round(pre_flops / t_pre / 1e12, 6), "unit": "TFLOP/s"},
        "decode_cached_us_per_seq_head": round(cached_us_per_seq_head, 2),
        "recompute_decode": {"context": L0, "us_per_seq_head_step": round(recompute_us_per_seq_head, 1),
                             "cached_us_per_seq_head_step": round(cached_one_us, 2),
                             "cache_speedup": round(recompute_us_per_seq_head / cached_one_us, 1)},
    }


def trace_summary(path, warm_frac):
    """Per library kernel of a rocprofv3 kernel trace: dispatch count, mean and
    median duration (us) over the dispatches after the first warm_frac of them."""
    import csv
    import statistics
    durs = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if "kvattn" in r["Kernel_Name"]:
                durs.setdefault(r["Kernel_Name"], []).append(
                    (int(r["Start_Timestamp"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    for name, v in durs.items():
        v.sort()
        timed = [d for _, d in v[int(len(v) * warm_frac):]]
        print(f"{name}\tdispatches={len(timed)}\tavg_us={statistics.mean(timed):.2f}\t"
              f"median_us={statistics.median(timed):.2f}")


def main():
    args = parse()
    if args.trace_summary:
        trace_summary(args.trace_summary[0], float(args.trace_summary[1]))
        return
    if args.traffic_from:
        write_traffic(*args.traffic_from)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import kv_cached_causal_amd as kv

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    if args.only == "sweep":
        mceil, eceil = MFMA_F16_PEAK_TFLOPS * 0.968, 18.9e12  # nominal, for the bound columns only
        rows = []
        for H, D in ((16, 32), (32, 128)):
            for T in (512, 1024, 2048, 4096, 8192, 16384):
                r = small_head_prefill(kv, dev, mceil, eceil, reps=args.steps, T=T, H=H, D=D)
                rows.append({"H": H, "D": D, "T": T, "us_per_layer": r["us_per_layer"], "tflops": r["value"],
                             "frac_of_mfma_peak": r["frac_of_mfma_peak"]})
                log(f"sweep H={H} D={D} T={T}: {r['us_per_layer']} us, {r['value']} TFLOP/s")
        print(json.dumps({"metric": METRIC, "n_gpus": 1, "steps": args.steps, "prefill_sweep": rows}), flush=True)
        return
    if args.only == "small":
        res = {"metric": METRIC, "n_gpus": 1, "small_configs": small_config_measurements(kv, dev)}
        print(json.dumps(res), flush=True)
        return
    if args.only == "prefill_d32":
        # the D=32 prompts alone (profiling runs): T=4096 (split query tiles) and T=8192
        mceil, eceil = MFMA_F16_PEAK_TFLOPS * 0.968, 18.9e12  # nominal, for the bound columns only
        res = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
               "prefill_d32_t4096": small_head_prefill(kv, dev, mceil, eceil, reps=args.steps, T=4096),
               "prefill_d32": small_head_prefill(kv, dev, mceil, eceil, reps=args.steps, T=8192)}
        res["value"], res["unit"] = res["prefill_d32"]["value"], "TFLOP/s"
        print(json.dumps(res), flush=True)
        return
    w5, w4 = si.WORKLOADS[5], si.WORKLOADS[4]
    res = {}

    # the GQA workload first, from a fresh allocation state: measured after the
    # 64 GiB workload in the same process it ran about 3.5 % slower
    gqa_out = None
    if not args.skip_gqa and args.only in (None, "gqa"):
        log("GQA bf16 decode workload (8 GiB cache)")
        g = setup_decode(kv, w4, dev, 4)
        for _ in range(args.warmup):
            reset_decode(g)
            decode_step(g)
        torch.cuda.synchronize()
        gsteps = []
        for _ in range(args.steps):
            reset_decode(g)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            decode_step(g)
            b.record()
            gsteps.append((a, b))
        tg = Timer()
        for _ in range(args.steps):
            reset_decode(g)
            decode_step(g, tg)
        torch.cuda.synchronize()
        step_ms = float(np.median([a.elapsed_time(b) for a, b in gsteps]))
        k_ms = tg.median_ms()
        achieved = g["bytes_step_layer"] / (k_ms * 1e-3) / 1e9
        gs = [a.elapsed_time(b) for a, b in gsteps]
        gqa_out = {"workload": w4.name, "value": round(g["bytes_step"] / (step_ms * 1e-3) / 1e9, 2),
                   "unit": "GB/s", "ms_per_step": round(step_ms, 4),
                   "ms_per_step_p10_p90": [round(float(np.percentile(gs, 10)), 4),
                                           round(float(np.percentile(gs, 90)), 4)],
                   "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                                "traffic": traffic_from_profiles("decode_gqa_b16", kernel_source_hash(DECODE_SOURCES)),
                                "algorithmic_bytes_per_launch": g["bytes_step_layer"],
                                "launch_ms": tg.spread()}}
        g["cache"].close()
        del g
        torch.cuda.empty_cache()

    dec = pre = None
    if args.only in (None, "decode"):
        log("setting up ragged batch-32 decode cache (64 GiB)")
        dec = setup_decode(kv, w5, dev, 5)
    if args.only in (None, "prefill"):
        log("setting up T=8192 prefill inputs")
        pre = setup_prefill(kv, w5, dev, 55)
    torch.cuda.synchronize()

    def step(timer):
        tp, td = (timer if timer else (None, None))
        if pre is not None:
            prefill_step(pre, tp)
        if dec is not None:
            decode_step(dec, td)

    def reset():
        if pre is not None:
            reset_prefill(pre)
        if dec is not None:
            reset_decode(dec)

    # warmup
    for _ in range(args.warmup):
        reset()
        step(None)
    torch.cuda.synchronize()
    # the timed steps: events at the phase boundaries only (an event pair per
    # launch would add its own gap between launches); the lengths are reset
    # between steps, outside the events
    marks = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        reset()
        e0 = torch.cuda.Event(enable_timing=True); e0.record()
        if pre is not None:
            prefill_step(pre)
        e1 = torch.cuda.Event(enable_timing=True); e1.record()
        if dec is not None:
            decode_step(dec)
        e2 = torch.cuda.Event(enable_timing=True); e2.record()
        marks.append((e0, e1, e2))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall / args.steps * 1e3
    # per-launch durations: the same steps again, an event pair around every launch
    tp, td = Timer(), Timer()
    for _ in range(args.steps):
        reset()
        if pre is not None:
            prefill_step(pre, tp)
        if dec is not None:
            decode_step(dec, td)
    torch.cuda.synchronize()
    pre_steps = [a.elapsed_time(b) for a, b, _ in marks]
    dec_steps = [b.elapsed_time(c) for _, b, c in marks]
    pre_ms = float(np.median(pre_steps))
    dec_ms = float(np.median(dec_steps))

    out = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f16", "data": "synthetic",
           "inputs": ("N(0,1) tensors drawn on the device (seeded torch generator) in HBM before timing, with the "
                      "shapes, dtype, ragged lengths and 1% x8 heavy K rows of the seeded host recipe the tests "
                      "and the CPU baseline use (the 64 GiB decode cache is not generated on the host)"),
           "timing": (f"{args.warmup} warmup steps, then {args.steps} timed steps of 32 layers per phase with HIP "
                      "events on the library's stream at the phase boundaries (phase and step figures: medians, "
                      "p10/p90 beside them; ms_per_step is the host wall clock of the timed steps, length resets "
                      "included), then the same steps again with an event pair around every launch (per-launch "
                      "medians, p10/p90: the roofline figures)")}
    dec_hash = kernel_source_hash(DECODE_SOURCES)
    pre_hash = kernel_source_hash(PREFILL_SOURCES)
    if gqa_out is not None:
        out["decode_gqa"] = gqa_out
        if args.only == "gqa":
            out["value"], out["unit"] = gqa_out["value"], "GB/s"
    if dec is not None:
        k_ms = td.median_ms()
        achieved = dec["bytes_step_layer"] / (k_ms * 1e-3) / 1e9
        out["value"] = round(dec["bytes_step"] / (dec_ms * 1e-3) / 1e9, 2)
        out["unit"] = "GB/s"
        out["roofline"] = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(achieved / HBM_PEAK_GBS, 4),
                           "traffic": traffic_from_profiles("decode_ragged_b32", dec_hash),
                           "kernel": "kvattn_append_decode per layer (fused append + split-K decode, and the "
                                     "merge kernel that commits the lengths)",
                           "algorithmic_bytes_per_launch": dec["bytes_step_layer"],
                           "launch_ms": td.spread()}
        out["decode"] = {"ms_per_step": round(dec_ms, 4),
                         "ms_per_step_p10_p90": [round(float(np.percentile(dec_steps, 10)), 4),
                                                 round(float(np.percentile(dec_steps, 90)), 4)],
                         "us_per_layer": round(dec_ms * 1e3 / w5.layers, 2),
                         "bytes_per_step": dec["bytes_step"], "sum_contexts": int(dec["ctx"].sum())}
    if pre is not None:
        k_ms = tp.median_ms()
        tf = pre["flops_layer"] / (k_ms * 1e-3) / 1e12
        out["prefill"] = {"value": round(pre["flops_layer"] * w5.layers / (pre_ms * 1e-3) / 1e12, 2),
                          "unit": "TFLOP/s", "ms_per_step": round(pre_ms, 4),
                          "ms_per_step_p10_p90": [round(float(np.percentile(pre_steps, 10)), 4),
                                                  round(float(np.percentile(pre_steps, 90)), 4)],
                          "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                                       "unit": "TFLOP/s", "frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
                                       "traffic": traffic_from_profiles("prefill_t8192", pre_hash),
                                       "kernel": "prefill_pipe_kernel<f16, D=128> (8 waves x 32 query rows, 64-key tiles, 32x32x16 MFMA)",
                                       "algorithmic_flops_per_launch": pre["flops_layer"],
                                       "launch_ms": tp.spread()}}
        out["prefill"].update(prefill_memory_and_clock(kv, pre))
        clk = out["prefill"]["sustained_clock_ghz"]
        if clk:
            # the dense peak scales with the clock (2.5 PFLOP/s at 2.4 GHz)
            out["prefill"]["roofline"]["frac_of_peak_at_sustained_clock"] = round(
                tf / (MFMA_F16_PEAK_TFLOPS * clk / 2.4), 4)
        if "value" not in out:
            out["value"], out["unit"] = out["prefill"]["value"], "TFLOP/s"
    out["config"] = {"workload": w5.name, "layers": w5.layers, "q_heads": w5.q_heads, "kv_heads": w5.kv_heads,
                     "head_dim": w5.head_dim, "decode_batch": w5.batch,
                     "decode_contexts": f"U[{w5.ctx_lo},{w5.ctx_hi}]", "heavy_k_rows": w5.heavy_frac,
                     "prefill_batch": 1, "prefill_T": w5.extra_prefill_T, "dtype": "f16"}
    out["device"] = {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                     "cus": props.multi_processor_count}
    if dec is not None and not args.no_extras:
        log("decode step as two calls (append, then decode)")
        t2 = Timer()
        for _ in range(3):
            decode_step_two_calls(dec)
        for _ in range(args.steps):
            decode_step_two_calls(dec, t2)
        torch.cuda.synchronize()
        out["decode_two_calls"] = {"decode_launch_ms": t2.spread(),
                                   "note": "kvattn_decode alone after a separate kvattn_append launch per layer"}
    if dec is not None and not args.no_extras:
        log("decode under a sliding window")
        out["decode_window"] = window_measurements(kv, w5, dec, out["roofline"]["launch_ms"]["median_ms"] * 1e3)
        log("decode from a paged cache")
        out["decode_paged"] = paged_measurements(kv, w5, dec, out["roofline"]["launch_ms"]["median_ms"] * 1e3)
    if dec is not None and pre is not None and not args.no_extras:
        log("extend: chunked prefill and 4-token verification")
        out["extend"] = extend_measurements(kv, w5, dec, pre)
    # free the big caches before the GQA workload
    if dec is not None:
        dec["cache"].close()
    if pre is not None:
        pre["cache"].close()
    dec = pre = None
    torch.cuda.empty_cache()

    if args.only is None and not args.no_extras:
        log("random-weight decoder: prompt 4096 + 128 greedy tokens")
        out["decoder"] = decoder_measurements(kv, dev)
    if args.only is None:
        ceil = measure_read_ceiling(kv, dev)
        out["hbm_read_ceiling"] = {"value": round(ceil, 1), "unit": "GB/s", "kernel": "kvattn_measure_stream_read",
                                   "bytes": CALIB_BYTES,
                                   "decode_frac_of_ceiling": round(out["roofline"]["achieved"] / ceil, 4)}
        mceil = measure_mfma_ceiling(kv, dev)
        out["mfma_f16_ceiling"] = {"value": round(mceil, 1), "unit": "TFLOP/s", "kernel": "kvattn_measure_mfma_f16",
                                   "prefill_frac_of_ceiling":
                                       round(out["prefill"]["roofline"]["achieved"] / mceil, 4)}
        eceil = measure_exp_ceiling(kv, dev)
        out["exp2_ceiling"] = {"value": round(eceil / 1e12, 3), "unit": "T exp2/s", "kernel": "kvattn_measure_exp2"}
        if not args.no_extras:
            log("small-head prefill (T=4096 and T=8192, 16 heads of D=32)")
            out["prefill_d32_t4096"] = small_head_prefill(kv, dev, mceil, eceil, T=4096)
            out["prefill_d32"] = small_head_prefill(kv, dev, mceil, eceil)
    if args.only is None and not args.no_extras:
        log("small workloads (configs 1-3), whole")
        out["small_configs"] = small_config_measurements(kv, dev)
    if args.calibrate:
        calibration_kernels(kv, dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
