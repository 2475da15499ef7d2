"""Helpers of the GPU parity tests: upload seeded inputs, compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import synth_inputs as si

TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
# fp16/bf16 outputs with fp32 accumulation on unit-variance inputs: max abs error bound
HALF_ATOL = 2e-3
# fp32: |gpu - ref| <= F32_ATOL + F32_RTOL * |ref|
F32_RTOL, F32_ATOL = 1e-4, 1e-5


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def host_f64(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return si.bf16_bits_to_f32(t.view(torch.int16).numpy().view(np.uint16)).astype(np.float64)
    return t.numpy().astype(np.float64)


def host_bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.element_size() == 2:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.element_size() == 4:
        return t.view(torch.int32).numpy().view(np.uint32)
    return t.numpy().view(np.uint8)


def _ordered16(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def check_output(gpu: torch.Tensor, ref: np.ndarray, in_dtype: str, what: str) -> float:
    """Compare a GPU output with the oracle at the tolerance its dtypes call for.

    fp32 inputs: allclose form with rtol 1e-4, atol 1e-5.  fp16/bf16 inputs with
    an fp32 output: max abs error <= 2e-3.  fp16/bf16 output: every element is
    within 2e-3 of the oracle or within one unit in the last place of the
    oracle rounded to the output dtype (the store's own rounding).
    Returns the max abs error.
    """
    g = host_f64(gpu)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - ref)
    mx = float(err.max()) if err.size else 0.0
    if in_dtype == "f32":
        bad = err > F32_ATOL + F32_RTOL * np.abs(ref)
        assert not bad.any(), f"{what}: {bad.sum()} elements outside rtol 1e-4 (max abs {mx:.3e})"
    elif gpu.dtype == torch.float32:
        assert mx <= HALF_ATOL, f"{what}: max abs error {mx:.3e} > {HALF_ATOL}"
    else:
        over = err > HALF_ATOL
        n_over = int(over.sum())
        if n_over:
            odt = "bf16" if gpu.dtype == torch.bfloat16 else "f16"
            r_bits = si.round_to(ref[over], odt).view(np.uint16)
            g_bits = host_bits(gpu)[over]
            ulps = np.abs(_ordered16(g_bits) - _ordered16(r_bits))
            assert ulps.max() <= 1, f"{what}: {n_over} elements over {HALF_ATOL}, max {ulps.max()} ulp"
            say(f"  {what}: {n_over} elements over {HALF_ATOL}, each within 1 ulp of the rounded oracle")
    say(f"  {what}: max abs err {mx:.3e}")
    return mx


def free_gpu():
    import gc
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
