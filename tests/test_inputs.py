"""Seeded input generation: determinism, rounding and workload recipes (no GPU)."""
import numpy as np
import torch

import synth_inputs as si


def test_streams_are_deterministic_and_independent():
    a = si.normal(2, 0, -1, si.Q, (2, 3, 4), "f16")
    b = si.normal(2, 0, -1, si.Q, (2, 3, 4), "f16")
    c = si.normal(2, 0, -1, si.K, (2, 3, 4), "f16")
    d = si.normal(2, 0, 0, si.Q, (2, 3, 4), "f16")
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    assert not np.array_equal(a, c) and not np.array_equal(a, d)


def test_bf16_rounding_is_rne_like_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32)
    x[:4] = [1.0 + 2**-8, 1.0 + 3 * 2**-8, -1.0 - 2**-8, 65504.0]   # exact ties
    ours = si.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    # the two ties round to even
    assert si.bf16_bits_to_f32(ours[:2]).tolist() == [1.0, 1.0 + 4 * 2**-8]


def test_f16_rounding_is_nearest():
    # numpy rounds float64 straight to float16 (no double rounding through float32)
    x = np.random.default_rng(1).standard_normal(100000)
    r = si.round_to(x, "f16")
    up = np.nextafter(r, np.float16(np.inf))
    dn = np.nextafter(r, np.float16(-np.inf))
    err = np.abs(x - r.astype(np.float64))
    assert (err <= np.abs(x - up.astype(np.float64))).all()
    assert (err <= np.abs(x - dn.astype(np.float64))).all()
    # agrees with torch's cast wherever float32 double rounding cannot interfere
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float16).numpy()
    assert (r.view(np.uint16) != ref.view(np.uint16)).sum() < 20


def test_widening_is_exact():
    x = si.normal(1, 0, -1, si.V, (1000,), "bf16")
    w = si.to_f64(x, "bf16")
    assert np.array_equal(si.round_to(w, "bf16"), x)


def test_heavy_rows_count_and_range():
    assert si.heavy_count(8192) == 82 and si.heavy_count(4096) == 41 and si.heavy_count(512) == 5
    rows = si.heavy_rows(5, 3, 0, 7, 2, 1000)
    assert len(rows) == 10 and len(set(rows.tolist())) == 10 and rows.max() < 1000
    k = si.normal(5, 3, -1, si.K, (1000, 8), "f16")
    k8 = si.scale_rows(k, rows, 8.0, "f16")
    assert np.array_equal(si.to_f64(k8[rows], "f16"), 8 * si.to_f64(k[rows], "f16"))
    keep = np.setdiff1d(np.arange(1000), rows)
    assert np.array_equal(k8[keep].view(np.uint16), k[keep].view(np.uint16))


def test_ragged_lengths_inclusive_range():
    L = si.ragged_lengths(5, 20000, 512, 4096)
    assert L.min() == 512 and L.max() == 4096
    w = si.WORKLOADS[5]
    Lb = si.decode_contexts(w)
    assert Lb.shape == (32,) and Lb.min() >= 512 and Lb.max() <= 4096


def test_workload_table():
    w4 = si.WORKLOADS[4]
    assert w4.group == 4 and w4.max_T == 4096
    assert si.WORKLOADS[1].scale == np.float32(1 / 8)
