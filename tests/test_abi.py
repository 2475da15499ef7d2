"""The C-ABI library loads, exports every declared symbol and validates on the host (no GPU)."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

import kv_cached_causal_amd as kv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"\b(kvattn_\w+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("kvattn_cache_alloc", "kvattn_prefill", "kvattn_append", "kvattn_decode",
                     "kvattn_cache_bytes", "kvattn_cache_free", "kvattn_cache_set_lengths"):
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = kv.lib()
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_signatures_cover_header():
    assert set(declared_functions()) == set(kv._SIGS)


def declared_arity():
    """Parameter count of every declared function, from the headers' text."""
    arity = {}
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        for name, params in re.findall(r"\b(kvattn_\w+)\s*\(([^;{]*?)\)\s*;", text, flags=re.S):
            params = params.strip()
            arity[name] = 0 if params in ("", "void") else params.count(",") + 1
    return arity


def test_binding_argument_counts_match_header():
    arity = declared_arity()
    assert set(arity) == set(declared_functions())
    wrong = {n: (len(kv._SIGS[n][1]), a) for n, a in arity.items() if len(kv._SIGS[n][1]) != a}
    assert not wrong, wrong


def test_cache_bytes_matches_worked_example():
    with open(os.path.join(ROOT, "tests", "golden", "kv_bytes_worked_example.json")) as f:
        gold = json.load(f)
    import torch
    for c in gold["cases"]:
        got = kv.cache_bytes(c["layers"], c["batch"], c["kv_heads"], c["head_dim"], c["seq_len"], torch.float16)
        assert got == c["exact_bytes"]


def test_cache_bytes_rejects_nonsense():
    lib = kv.lib()
    assert lib.kvattn_cache_bytes(0, 1, 1, 64, 16, 1) == 0
    assert lib.kvattn_cache_bytes(1, 1, 1, 64, -5, 1) == 0
    assert lib.kvattn_cache_bytes(1, 1, 1, 64, 16, 7) == 0
    # config sizes: 8 GiB GQA bf16, 64 GiB ragged fp16 decode cache
    assert lib.kvattn_cache_bytes(32, 16, 8, 128, 4096, 2) == 8 << 30
    assert lib.kvattn_cache_bytes(32, 32, 32, 128, 4096, 1) == 64 << 30


def _alloc(*args):
    h = ctypes.c_void_p()
    rc = kv.lib().kvattn_cache_alloc(ctypes.byref(h), *args)
    return rc, h


@pytest.mark.parametrize("args,status", [
    ((0, 1, 4, 4, 64, 16, 1, None, 0), -1),       # no layers
    ((1, 1, 4, 4, 64, 0, 1, None, 0), -1),        # no capacity
    ((1, 1, 4, 4, 48, 16, 1, None, 0), -2),       # unsupported head_dim
    ((1, 1, 6, 4, 64, 16, 1, None, 0), -2),       # H % Hkv != 0
    ((1, 1, 4, 4, 64, 16, 9, None, 0), -2),       # unknown dtype
    ((1, 1, 4, 4, 64, 16, 1, ctypes.c_void_p(256), 10), -5),   # adopted buffer too small
    ((1, 1, 4, 4, 64, 16, 1, ctypes.c_void_p(4), 1 << 20), -1),  # misaligned buffer
])
def test_alloc_validation_before_any_device_call(args, status):
    rc, h = _alloc(*args)
    assert rc == status and not h.value


def test_null_cache_is_rejected_everywhere():
    lib = kv.lib()
    p = ctypes.c_void_p(0)
    assert lib.kvattn_cache_free(None) == -1
    assert lib.kvattn_prefill(None, 0, p, p, p, p, 8, 0.1, 1, None) == -1
    assert lib.kvattn_append(None, 0, p, p, None) == -1
    assert lib.kvattn_decode(None, 0, p, p, 0.1, 1, None) == -1
    assert lib.kvattn_cache_set_lengths(None, 0, (ctypes.c_int32 * 1)(0), None) == -1
    assert lib.kvattn_cache_get_lengths(None, 0, (ctypes.c_int32 * 1)()) == -1
    k, v = ctypes.c_void_p(), ctypes.c_void_p()
    assert lib.kvattn_cache_kv_ptr(None, 0, ctypes.byref(k), ctypes.byref(v)) == -1
    assert lib.kvattn_cache_alloc(None, 1, 1, 1, 1, 64, 8, 1, None, 0) == -1


def test_status_strings():
    lib = kv.lib()
    for s in range(-6, 1):
        assert lib.kvattn_status_string(s)
    assert lib.kvattn_status_string(-99) == b"unknown status"


def test_measure_mfma_validates_on_host_and_counts_flops():
    lib = kv.lib()
    fake = ctypes.c_void_p(1 << 20)
    assert lib.kvattn_measure_mfma_f16(0, 10, fake, None) == -1
    assert lib.kvattn_measure_mfma_f16(8, 0, fake, None) == -1
    assert lib.kvattn_measure_mfma_f16(8, 10, None, None) == -1
    # 4 waves x 8 chains x 16*16*32 multiply-adds per round
    assert lib.kvattn_measure_mfma_f16_flops(3, 5) == 3 * 4 * 5 * 8 * 16 * 16 * 32 * 2
    assert lib.kvattn_measure_mfma_f16_flops(0, 5) == 0.0


def test_measure_exp2_validates_on_host_and_counts():
    lib = kv.lib()
    fake = ctypes.c_void_p(1 << 20)
    assert lib.kvattn_measure_exp2(0, 10, fake, None) == -1
    assert lib.kvattn_measure_exp2(8, 0, fake, None) == -1
    assert lib.kvattn_measure_exp2(8, 10, None, None) == -1
    # 256 threads x 32 chains per round
    assert lib.kvattn_measure_exp2_count(3, 5) == 3 * 256 * 5 * 32
    assert lib.kvattn_measure_exp2_count(0, 5) == 0.0


def test_measure_stream_read_validates_on_host():
    lib = kv.lib()
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails validation first
    assert lib.kvattn_measure_stream_read(None, 1 << 20, 64, fake, None) == -1
    assert lib.kvattn_measure_stream_read(fake, 0, 64, fake, None) == -1
    assert lib.kvattn_measure_stream_read(fake, 100, 64, fake, None) == -1      # not a multiple of 16
    assert lib.kvattn_measure_stream_read(ctypes.c_void_p((1 << 20) + 4), 1 << 20, 64, fake, None) == -1
    assert lib.kvattn_measure_stream_read(fake, 1 << 20, 0, fake, None) == -1
    assert lib.kvattn_measure_stream_read(fake, 1 << 20, 64, None, None) == -1


def test_measure_stream_write_validates_on_host():
    lib = kv.lib()
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails validation first
    assert lib.kvattn_measure_stream_write(None, 1 << 20, 64, None) == -1
    assert lib.kvattn_measure_stream_write(fake, 0, 64, None) == -1
    assert lib.kvattn_measure_stream_write(fake, 100, 64, None) == -1      # not a multiple of 16
    assert lib.kvattn_measure_stream_write(ctypes.c_void_p((1 << 20) + 4), 1 << 20, 64, None) == -1
    assert lib.kvattn_measure_stream_write(fake, 1 << 20, 0, None) == -1


def test_extend_rejects_null_cache_without_a_device():
    lib = kv.lib()
    assert lib.kvattn_extend(None, 0, None, None, None, None, 4, 0.1, 1, None) == -1


def test_window_calls_reject_null_cache_without_a_device():
    lib = kv.lib()
    assert lib.kvattn_cache_set_window(None, 0, 16, 4) == -1
    assert lib.kvattn_cache_set_window(None, -1, 0, 0) == -1
    w, s = ctypes.c_int(), ctypes.c_int()
    assert lib.kvattn_cache_get_window(None, 0, ctypes.byref(w), ctypes.byref(s)) == -1


def test_paged_bytes_is_the_capacity_formula():
    lib = kv.lib()
    # 32 layers, 512 blocks of 64 positions (= one 32768-position sequence), 8 KV heads, D=128, bf16
    assert lib.kvattn_paged_bytes(32, 512, 64, 8, 128, 2) == 2 * 32 * 8 * 128 * 32768 * 2
    assert lib.kvattn_paged_bytes(32, 512, 64, 8, 128, 2) == lib.kvattn_cache_bytes(32, 1, 8, 128, 32768, 2)
    assert lib.kvattn_paged_bytes(0, 512, 64, 8, 128, 2) == 0
    assert lib.kvattn_paged_bytes(1, 512, 64, 8, 128, 7) == 0


@pytest.mark.parametrize("args,status", [
    ((1, 2, 4, 8, 16, 4, 4, 64, 1), 0),          # valid shape (not allocated: null out)
    ((1, 2, 4, 8, 24, 4, 4, 64, 1), -2),         # block size not a power of two
    ((1, 2, 4, 8, 8, 4, 4, 64, 1), -2),          # block size below 16
    ((1, 2, 4, 8, 16, 4, 4, 48, 1), -2),         # head dim
    ((1, 2, 4, 8, 16, 6, 4, 64, 1), -2),         # H % Hkv
    ((0, 2, 4, 8, 16, 4, 4, 64, 1), -1),
    ((1, 2, 0, 8, 16, 4, 4, 64, 1), -1),
])
def test_paged_alloc_validation_before_any_device_call(args, status):
    lib = kv.lib()
    if status == 0:
        # a null out pointer is rejected first, so nothing touches the device
        assert lib.kvattn_paged_alloc(None, *args, None, 0) == -1
    else:
        out = ctypes.c_void_p()
        assert lib.kvattn_paged_alloc(ctypes.byref(out), *args, None, 0) == status
        assert not out.value


def test_paged_calls_reject_null_object_without_a_device():
    lib = kv.lib()
    p = ctypes.c_void_p(0)
    assert lib.kvattn_paged_free(None) == -1
    assert lib.kvattn_paged_prefill(None, 0, p, p, p, p, 8, 0.1, 1, None) == -1
    assert lib.kvattn_paged_append(None, 0, p, p, None) == -1
    assert lib.kvattn_paged_decode(None, 0, p, p, 0.1, 1, None) == -1
    assert lib.kvattn_paged_extend(None, 0, p, p, p, p, 4, 0.1, 1, None) == -1
    assert lib.kvattn_paged_set_window(None, 0, 64, 4) == -1
    w, sk = ctypes.c_int(), ctypes.c_int()
    assert lib.kvattn_paged_get_window(None, 0, ctypes.byref(w), ctypes.byref(sk)) == -1
    assert lib.kvattn_paged_set_blocks(None, 0, (ctypes.c_int32 * 1)(0), 1, None) == -1
    assert lib.kvattn_paged_set_lengths(None, 0, (ctypes.c_int32 * 1)(0), None) == -1
    assert lib.kvattn_paged_get_lengths(None, 0, (ctypes.c_int32 * 1)()) == -1
    k, v = ctypes.c_void_p(), ctypes.c_void_p()
    assert lib.kvattn_paged_kv_ptr(None, 0, ctypes.byref(k), ctypes.byref(v)) == -1


def test_model_weight_elems_matches_the_packing_order():
    import dataclasses
    import synth_inputs as si
    lib = kv.lib()
    for spec in (si.TINYGPT, dataclasses.replace(si.TINYGPT, layers=2, d_model=1024, heads=8, vocab=300, max_T=77)):
        n = sum(int(np.prod(shape)) for _, shape in si.model_weight_shapes(spec))
        assert lib.kvattn_model_weight_elems(spec.layers, spec.d_model, spec.vocab, spec.max_T, spec.mlp_mult) == n
    assert lib.kvattn_model_weight_elems(0, 512, 10, 10, 4) == 0


@pytest.mark.parametrize("args,status", [
    ((2, 512, 16, 100, 64, 4, 1), -1),   # null weights (checked first)
    ((2, 500, 10, 100, 64, 4, 1), -2),   # width not a multiple of 512
    ((2, 512, 5, 100, 64, 4, 1), -2),    # heads do not divide the width
    ((2, 512, 8, 100, 64, 4, 9), -2),    # batch above 8
    ((2, 2048, 16, 100, 64, 4, 1), -2),  # width above 1024
    ((2, 512, 2, 100, 64, 4, 1), -2),    # head dim 256
    ((0, 512, 16, 100, 64, 4, 1), -1),
])
def test_model_create_validation_before_any_device_call(args, status):
    lib = kv.lib()
    out = ctypes.c_void_p()
    weights = None if status == -1 and args[0] == 2 else ctypes.c_void_p(1 << 20)  # never dereferenced
    assert lib.kvattn_model_create(ctypes.byref(out), *args, weights) == status
    assert not out.value
    assert lib.kvattn_model_create(None, *args, weights) == -1


def test_model_calls_reject_null_model_without_a_device():
    lib = kv.lib()
    p = ctypes.c_void_p(0)
    assert lib.kvattn_model_free(None) == -1
    assert lib.kvattn_model_reset(None, None) == -1
    assert lib.kvattn_model_prefill(None, p, 4, p, p, None) == -1
    assert lib.kvattn_model_step(None, p, p, p, None) == -1
    assert lib.kvattn_model_generate(None, 4, p, p, None) == -1
    assert lib.kvattn_model_positions(None, (ctypes.c_int32 * 1)()) == -1


def test_noalloc_decode_validates_on_the_host():
    """kvattn_decode_noalloc checks its arguments, and the size of the split-K
    partials against its fixed array, before any device call (so this runs
    without a GPU): a shape that needs more than the array is CAPACITY, with
    the sizes in the error text."""
    lib = kv.lib()
    p = 0x1000  # never dereferenced: every case is rejected on the host
    # B = 1024, H = 32, D = 128, 4096 keys in 2 splits of 2048: 4*1024*32*2*130 B = 34 MB > 16 MiB
    assert lib.kvattn_decode_noalloc(p, p, p, 1024, 32, 8, 128, 4096, 1, p, p, 0.125, 1, None) == -3
    assert b"scratch" in lib.kvattn_last_error()
    assert kv.NOALLOC_SCRATCH_BYTES == 16 << 20
    assert lib.kvattn_decode_noalloc(None, p, p, 2, 4, 4, 64, 64, 1, p, p, 0.125, 1, None) == -1
    assert lib.kvattn_decode_noalloc(p, p, p, 2, 4, 3, 64, 64, 1, p, p, 0.125, 1, None) == -2
    assert lib.kvattn_decode_noalloc(p, p, p, 2, 4, 4, 48, 64, 1, p, p, 0.125, 1, None) == -2
    assert lib.kvattn_decode_noalloc(p, p, p, 2, 4, 4, 64, 64, 1, p, p, 0.125, 2, None) == -2
    assert lib.kvattn_decode_noalloc(p, p, p, 2, 4, 4, 64, 64, 1, p, p, -1.0, 1, None) == -1
    assert lib.kvattn_decode_noalloc(p, p, p, 0, 4, 4, 64, 64, 1, p, p, 0.125, 1, None) == -1


def test_library_links_no_vendor_blas():
    """Every kernel of the path, the decoder's prompt GEMMs included, is the
    library's own: libkvattn.so needs no BLAS library."""
    import subprocess
    out = subprocess.run(["ldd", kv.LIB_PATH], capture_output=True, text=True).stdout.lower()
    assert "libamdhip64" in out
    for vendor in ("rocblas", "hipblas", "hipblaslt", "miopen"):
        assert vendor not in out, f"libkvattn.so links {vendor}"
