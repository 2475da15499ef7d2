"""Python binding of libkvattn: exact causal KV-cached attention on MI355X.

Argument marshalling only: every step of prefill, append and decode runs in
the HIP kernels of ``libkvattn.so`` (built in-tree by
``kv_cached_causal_amd/build.py``).  PyTorch supplies device memory and the
stream.  If the library is missing this module raises at import time: there
is no CPU fallback.

Layouts are the (B, H, T, D) / (B, Hkv, T, D) contiguous tensors of the C ABI
(see ``include/kvattn.h``).
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = ["KVCache", "PagedKVCache", "Decoder", "KVAttnError", "cache_bytes", "paged_bytes", "decode_noalloc",
           "NOALLOC_SCRATCH_BYTES", "lib", "LIB_PATH"]

_HERE = os.path.dirname(os.path.abspath(__file__))
# KVATTN_LIB names another build of the library (for example a tuning variant)
LIB_PATH = os.environ.get("KVATTN_LIB") or os.path.join(_HERE, "libkvattn.so")

_DT = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
_ELEM = {torch.float32: 4, torch.float16: 2, torch.bfloat16: 2}

_STATUS = {
    0: "OK", -1: "INVALID_ARG", -2: "UNSUPPORTED", -3: "CAPACITY", -4: "STATE", -5: "OOM", -6: "HIP",
}

# the exported C symbols and their ctypes signatures
_SIGS = {
    "kvattn_cache_bytes": (ctypes.c_size_t, [ctypes.c_int] * 5 + [ctypes.c_int]),
    "kvattn_cache_alloc": (ctypes.c_int, [ctypes.POINTER(ctypes.c_void_p)] + [ctypes.c_int] * 7
                           + [ctypes.c_void_p, ctypes.c_size_t]),
    "kvattn_cache_free": (ctypes.c_int, [ctypes.c_void_p]),
    "kvattn_cache_kv_ptr": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int,
                                           ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_void_p)]),
    "kvattn_cache_set_lengths": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int,
                                                ctypes.POINTER(ctypes.c_int32), ctypes.c_void_p]),
    "kvattn_cache_get_lengths": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_int32)]),
    "kvattn_cache_set_window": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int]),
    "kvattn_cache_get_window": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                               ctypes.POINTER(ctypes.c_int)]),
    "kvattn_prefill": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int] + [ctypes.c_void_p] * 4
                       + [ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_void_p]),
    "kvattn_append": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p]),
    "kvattn_extend": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int] + [ctypes.c_void_p] * 4
                      + [ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_void_p]),
    "kvattn_decode": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_float, ctypes.c_int, ctypes.c_void_p]),
    "kvattn_append_decode": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int] + [ctypes.c_void_p] * 4
                             + [ctypes.c_float, ctypes.c_int, ctypes.c_void_p]),
    "kvattn_decode_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p] + [ctypes.c_int] * 6
                              + [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_int, ctypes.c_void_p]),
    "kvattn_paged_bytes": (ctypes.c_size_t, [ctypes.c_int] * 6),
    "kvattn_paged_alloc": (ctypes.c_int, [ctypes.POINTER(ctypes.c_void_p)] + [ctypes.c_int] * 9
                           + [ctypes.c_void_p, ctypes.c_size_t]),
    "kvattn_paged_free": (ctypes.c_int, [ctypes.c_void_p]),
    "kvattn_paged_kv_ptr": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int,
                                           ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_void_p)]),
    "kvattn_paged_set_blocks": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_int32),
                                               ctypes.c_int, ctypes.c_void_p]),
    "kvattn_paged_set_lengths": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int,
                                                ctypes.POINTER(ctypes.c_int32), ctypes.c_void_p]),
    "kvattn_paged_get_lengths": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_int32)]),
    "kvattn_paged_prefill": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int] + [ctypes.c_void_p] * 4
                             + [ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_void_p]),
    "kvattn_paged_append": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p]),
    "kvattn_paged_set_window": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int]),
    "kvattn_paged_get_window": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                               ctypes.POINTER(ctypes.c_int)]),
    "kvattn_paged_extend": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int] + [ctypes.c_void_p] * 4
                            + [ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_void_p]),
    "kvattn_paged_decode": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_float, ctypes.c_int, ctypes.c_void_p]),
    "kvattn_model_weight_elems": (ctypes.c_size_t, [ctypes.c_int] * 5),
    "kvattn_model_create": (ctypes.c_int, [ctypes.POINTER(ctypes.c_void_p)] + [ctypes.c_int] * 7 + [ctypes.c_void_p]),
    "kvattn_model_free": (ctypes.c_int, [ctypes.c_void_p]),
    "kvattn_model_reset": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p]),
    "kvattn_model_positions": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32)]),
    "kvattn_model_prefill": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p]),
    "kvattn_model_step": (ctypes.c_int, [ctypes.c_void_p] + [ctypes.c_void_p] * 4),
    "kvattn_model_generate": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int] + [ctypes.c_void_p] * 3),
    "kvattn_model_last_error": (ctypes.c_char_p, []),
    "kvattn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "kvattn_measure_mfma_f16": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]),
    "kvattn_measure_mfma_f16_flops": (ctypes.c_double, [ctypes.c_int, ctypes.c_int]),
    "kvattn_measure_exp2": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]),
    "kvattn_measure_exp2_count": (ctypes.c_double, [ctypes.c_int, ctypes.c_int]),
    "kvattn_measure_stream_read": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                                  ctypes.c_void_p]),
    "kvattn_measure_stream_write": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]),
    "kvattn_measure_prefill_clock": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int] + [ctypes.c_void_p] * 4
                                     + [ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_void_p,
                                        ctypes.c_void_p]),
    "kvattn_last_error": (ctypes.c_char_p, []),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libkvattn.so (once) and declare its signatures."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built: run `python kv_cached_causal_amd/build.py`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


lib()  # fail loudly at import when the native library is absent


class KVAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        detail = lib().kvattn_last_error().decode() if status == -6 else ""
        msg = f"{where}: {_STATUS.get(status, status)} ({lib().kvattn_status_string(status).decode()})"
        super().__init__(msg + (f" [{detail}]" if detail else ""))
        self.status = status


def _check(status: int, where: str) -> None:
    if status != 0:
        raise KVAttnError(status, where)


def cache_bytes(layers: int, batch: int, kv_heads: int, head_dim: int, max_T: int, dtype) -> int:
    """Cache payload bytes by the capacity formula (computed by the C library)."""
    return int(lib().kvattn_cache_bytes(layers, batch, kv_heads, head_dim, max_T, _DT[dtype]))


def _stream_ptr(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


class KVCache:
    """A preallocated per-layer KV cache on one GPU.

    Device memory for the payload is a PyTorch allocation handed to the C
    library (``buffer=True``), so that ``k_view``/``v_view`` can expose it as
    tensors; with ``buffer=False`` the library allocates it with hipMalloc.
    """

    def __init__(self, layers: int, batch: int, q_heads: int, kv_heads: int, head_dim: int,
                 max_T: int, dtype=torch.float16, device=None, buffer: bool = True):
        if dtype not in _DT:
            raise TypeError(f"unsupported dtype {dtype}")
        self.device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        self.layers, self.batch, self.q_heads, self.kv_heads = layers, batch, q_heads, kv_heads
        self.head_dim, self.max_T, self.dtype = head_dim, max_T, dtype
        self.nbytes = cache_bytes(layers, batch, kv_heads, head_dim, max_T, dtype)
        self._handle = ctypes.c_void_p()
        self._buf = None
        with torch.cuda.device(self.device):
            if buffer:
                if self.nbytes == 0:
                    raise KVAttnError(-1, "KVCache")
                self._buf = torch.empty(self.nbytes, dtype=torch.uint8, device=self.device)
                torch.cuda.synchronize(self.device)
                dev_ptr, dev_bytes = _ptr(self._buf), self.nbytes
            else:
                dev_ptr, dev_bytes = None, 0
            _check(lib().kvattn_cache_alloc(ctypes.byref(self._handle), layers, batch, q_heads, kv_heads,
                                            head_dim, max_T, _DT[dtype], dev_ptr, dev_bytes),
                   "kvattn_cache_alloc")

    # ------------------------------------------------------------------ views
    def _layer_ptrs(self, layer: int):
        k, v = ctypes.c_void_p(), ctypes.c_void_p()
        _check(lib().kvattn_cache_kv_ptr(self._handle, layer, ctypes.byref(k), ctypes.byref(v)),
               "kvattn_cache_kv_ptr")
        return k.value, v.value

    def _view(self, layer: int, which: int) -> torch.Tensor:
        if self._buf is None:
            raise RuntimeError("views need a PyTorch-allocated cache buffer")
        if not 0 <= layer < self.layers:
            raise IndexError(layer)
        block = self.nbytes // (2 * self.layers)
        off = (2 * layer + which) * block
        t = self._buf[off:off + block].view(self.dtype)
        return t.view(self.batch, self.kv_heads, self.max_T, self.head_dim)

    def k_view(self, layer: int) -> torch.Tensor:
        """Layer's K block (B, Hkv, max_T, D) as a tensor over the cache memory."""
        return self._view(layer, 0)

    def v_view(self, layer: int) -> torch.Tensor:
        return self._view(layer, 1)

    # ------------------------------------------------------------------ lengths
    def set_lengths(self, lengths, layer: int = -1) -> None:
        arr = (ctypes.c_int32 * self.batch)(*[int(x) for x in lengths])
        with torch.cuda.device(self.device):
            _check(lib().kvattn_cache_set_lengths(self._handle, layer, arr, _stream_ptr(self.device)),
                   "kvattn_cache_set_lengths")

    def lengths(self, layer: int) -> list:
        arr = (ctypes.c_int32 * self.batch)()
        _check(lib().kvattn_cache_get_lengths(self._handle, layer, arr), "kvattn_cache_get_lengths")
        return list(arr)

    # ------------------------------------------------------------------ masks
    def set_window(self, window: int, sink: int = 0, layer: int = -1) -> None:
        """Sliding window W (0: none) and sink S of one layer, or of all (-1)."""
        _check(lib().kvattn_cache_set_window(self._handle, layer, int(window), int(sink)),
               "kvattn_cache_set_window")

    def window(self, layer: int) -> tuple:
        w, s = ctypes.c_int(), ctypes.c_int()
        _check(lib().kvattn_cache_get_window(self._handle, layer, ctypes.byref(w), ctypes.byref(s)),
               "kvattn_cache_get_window")
        return w.value, s.value

    # ------------------------------------------------------------------ checks
    def _tensor(self, t: torch.Tensor, shape, name: str, dtype=None) -> None:
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a tensor")
        if t.device != self.device:
            raise ValueError(f"{name} is on {t.device}, cache on {self.device}")
        if t.dtype != (dtype or self.dtype):
            raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype or self.dtype}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")

    def _scale(self, scale):
        return float(1.0 / math.sqrt(self.head_dim)) if scale is None else float(scale)

    # ------------------------------------------------------------------ the path
    def prefill(self, layer: int, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                out: torch.Tensor | None = None, scale: float | None = None, out_dtype=None) -> torch.Tensor:
        """Causal attention over the prompt; copies k, v into cache rows [0, T)."""
        B, H, Hkv, D = self.batch, self.q_heads, self.kv_heads, self.head_dim
        T = q.shape[2] if q.dim() == 4 else -1
        self._tensor(q, (B, H, T, D), "q")
        self._tensor(k, (B, Hkv, T, D), "k")
        self._tensor(v, (B, Hkv, T, D), "v")
        od = out_dtype or self.dtype
        if out is None:
            out = torch.empty((B, H, T, D), dtype=od, device=self.device)
        self._tensor(out, (B, H, T, D), "out", od)
        with torch.cuda.device(self.device):
            _check(lib().kvattn_prefill(self._handle, layer, _ptr(q), _ptr(k), _ptr(v), _ptr(out), T,
                                        self._scale(scale), _DT[od], _stream_ptr(self.device)),
                   "kvattn_prefill")
        return out

    def extend(self, layer: int, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
               out: torch.Tensor | None = None, scale: float | None = None, out_dtype=None) -> torch.Tensor:
        """T new positions per sequence after its cached prefix (chunked prefill / multi-token verify)."""
        B, H, Hkv, D = self.batch, self.q_heads, self.kv_heads, self.head_dim
        T = q.shape[2] if q.dim() == 4 else -1
        self._tensor(q, (B, H, T, D), "q")
        self._tensor(k, (B, Hkv, T, D), "k")
        self._tensor(v, (B, Hkv, T, D), "v")
        od = out_dtype or self.dtype
        if out is None:
            out = torch.empty((B, H, T, D), dtype=od, device=self.device)
        self._tensor(out, (B, H, T, D), "out", od)
        with torch.cuda.device(self.device):
            _check(lib().kvattn_extend(self._handle, layer, _ptr(q), _ptr(k), _ptr(v), _ptr(out), T,
                                       self._scale(scale), _DT[od], _stream_ptr(self.device)),
                   "kvattn_extend")
        return out

    def append(self, layer: int, k_new: torch.Tensor, v_new: torch.Tensor) -> None:
        """Copy one K/V row per sequence to position len[b]; len[b] += 1."""
        shape = (self.batch, self.kv_heads, 1, self.head_dim)
        self._tensor(k_new, shape, "k_new")
        self._tensor(v_new, shape, "v_new")
        with torch.cuda.device(self.device):
            _check(lib().kvattn_append(self._handle, layer, _ptr(k_new), _ptr(v_new), _stream_ptr(self.device)),
                   "kvattn_append")

    def decode(self, layer: int, q: torch.Tensor, out: torch.Tensor | None = None,
               scale: float | None = None, out_dtype=None) -> torch.Tensor:
        """One query per (b, h) over the len[b] cached keys."""
        shape = (self.batch, self.q_heads, 1, self.head_dim)
        self._tensor(q, shape, "q")
        od = out_dtype or self.dtype
        if out is None:
            out = torch.empty(shape, dtype=od, device=self.device)
        self._tensor(out, shape, "out", od)
        with torch.cuda.device(self.device):
            _check(lib().kvattn_decode(self._handle, layer, _ptr(q), _ptr(out), self._scale(scale), _DT[od],
                                       _stream_ptr(self.device)),
                   "kvattn_decode")
        return out

    def append_decode(self, layer: int, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                      out: torch.Tensor | None = None, scale: float | None = None, out_dtype=None) -> torch.Tensor:
        """One decode step in one launch: append k_new/v_new at len[b], attend the
        len[b] + 1 keys with q, then len[b] += 1 (same result as append + decode)."""
        kv_shape = (self.batch, self.kv_heads, 1, self.head_dim)
        shape = (self.batch, self.q_heads, 1, self.head_dim)
        self._tensor(k_new, kv_shape, "k_new")
        self._tensor(v_new, kv_shape, "v_new")
        self._tensor(q, shape, "q")
        od = out_dtype or self.dtype
        if out is None:
            out = torch.empty(shape, dtype=od, device=self.device)
        self._tensor(out, shape, "out", od)
        with torch.cuda.device(self.device):
            _check(lib().kvattn_append_decode(self._handle, layer, _ptr(k_new), _ptr(v_new), _ptr(q), _ptr(out),
                                              self._scale(scale), _DT[od], _stream_ptr(self.device)),
                   "kvattn_append_decode")
        return out

    # ------------------------------------------------------------------ pre-bound calls
    # For launch-bound loops (many short kernels): the arguments are checked
    # and marshalled once, on the stream current at bind time, and the returned
    # callable only enqueues the C call.  The tensors must stay alive.
    def bind_prefill(self, layer: int, q, k, v, out, scale: float | None = None):
        B, H, Hkv, D = self.batch, self.q_heads, self.kv_heads, self.head_dim
        T = q.shape[2] if q.dim() == 4 else -1
        self._tensor(q, (B, H, T, D), "q")
        self._tensor(k, (B, Hkv, T, D), "k")
        self._tensor(v, (B, Hkv, T, D), "v")
        self._tensor(out, (B, H, T, D), "out", out.dtype)
        if out.dtype not in (self.dtype, torch.float32):
            raise TypeError(f"out has dtype {out.dtype}")
        fn = lib().kvattn_prefill
        args = (self._handle, layer, _ptr(q), _ptr(k), _ptr(v), _ptr(out), T, ctypes.c_float(self._scale(scale)),
                _DT[out.dtype], _stream_ptr(self.device))
        return lambda: _check(fn(*args), "kvattn_prefill")

    def bind_append(self, layer: int, k_new, v_new):
        shape = (self.batch, self.kv_heads, 1, self.head_dim)
        self._tensor(k_new, shape, "k_new")
        self._tensor(v_new, shape, "v_new")
        fn = lib().kvattn_append
        args = (self._handle, layer, _ptr(k_new), _ptr(v_new), _stream_ptr(self.device))
        return lambda: _check(fn(*args), "kvattn_append")

    def bind_decode(self, layer: int, q, out, scale: float | None = None):
        shape = (self.batch, self.q_heads, 1, self.head_dim)
        self._tensor(q, shape, "q")
        self._tensor(out, shape, "out", out.dtype)
        if out.dtype not in (self.dtype, torch.float32):
            raise TypeError(f"out has dtype {out.dtype}")
        fn = lib().kvattn_decode
        args = (self._handle, layer, _ptr(q), _ptr(out), ctypes.c_float(self._scale(scale)), _DT[out.dtype],
                _stream_ptr(self.device))
        return lambda: _check(fn(*args), "kvattn_decode")

    def bind_append_decode(self, layer: int, k_new, v_new, q, out, scale: float | None = None):
        kv_shape = (self.batch, self.kv_heads, 1, self.head_dim)
        shape = (self.batch, self.q_heads, 1, self.head_dim)
        self._tensor(k_new, kv_shape, "k_new")
        self._tensor(v_new, kv_shape, "v_new")
        self._tensor(q, shape, "q")
        self._tensor(out, shape, "out", out.dtype)
        if out.dtype not in (self.dtype, torch.float32):
            raise TypeError(f"out has dtype {out.dtype}")
        fn = lib().kvattn_append_decode
        args = (self._handle, layer, _ptr(k_new), _ptr(v_new), _ptr(q), _ptr(out), ctypes.c_float(self._scale(scale)),
                _DT[out.dtype], _stream_ptr(self.device))
        return lambda: _check(fn(*args), "kvattn_append_decode")

    # ------------------------------------------------------------------ lifetime
    def close(self) -> None:
        if self._handle and self._handle.value:
            _check(lib().kvattn_cache_free(self._handle), "kvattn_cache_free")
            self._handle = ctypes.c_void_p()
        self._buf = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


# bytes of the library's fixed split-K array used by decode_noalloc (KVATTN_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 16 << 20


def decode_noalloc(k_cache: torch.Tensor, v_cache: torch.Tensor, lengths: torch.Tensor, q: torch.Tensor,
                   out: torch.Tensor, scale: float | None = None) -> torch.Tensor:
    """kvattn_decode_noalloc: decode over a caller-owned cache, allocating nothing.

    k_cache, v_cache (B, Hkv, max_T, D) and q (B, H, 1, D) in one dtype; lengths a
    device int32 tensor [B]; out (B, H, 1, D) in that dtype or float32.  The
    split-K partials go to the library's fixed device array."""
    tensors = {"k_cache": k_cache, "v_cache": v_cache, "lengths": lengths, "q": q, "out": out}
    for name, t in tensors.items():
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
    if k_cache.dim() != 4 or k_cache.shape != v_cache.shape or k_cache.dtype != v_cache.dtype:
        raise ValueError("k_cache and v_cache must be (B, Hkv, max_T, D) of one dtype")
    B, Hkv, max_T, D = k_cache.shape
    if q.dim() != 4 or q.shape[0] != B or q.shape[2] != 1 or q.shape[3] != D or q.dtype != k_cache.dtype:
        raise ValueError("q must be (B, H, 1, D) in the cache dtype")
    if out.shape != q.shape or out.dtype not in (q.dtype, torch.float32):
        raise ValueError("out must have q's shape, in q's dtype or float32")
    if lengths.dtype != torch.int32 or tuple(lengths.shape) != (B,):
        raise ValueError("lengths must be an int32 tensor of shape (B,)")
    scale = float(1.0 / math.sqrt(D)) if scale is None else float(scale)
    st = lib().kvattn_decode_noalloc(_ptr(k_cache), _ptr(v_cache), _ptr(lengths), B, q.shape[1], Hkv, D, max_T,
                                     _DT[k_cache.dtype], _ptr(q), _ptr(out), scale, _DT[out.dtype],
                                     _stream_ptr(q.device))
    _check(st, "kvattn_decode_noalloc")
    return out


def paged_bytes(layers: int, num_blocks: int, block_size: int, kv_heads: int, head_dim: int, dtype) -> int:
    """Block-pool bytes of a paged cache (computed by the C library)."""
    return int(lib().kvattn_paged_bytes(layers, num_blocks, block_size, kv_heads, head_dim, _DT[dtype]))


class PagedKVCache:
    """A block-paged KV cache on one GPU: a pool of ``num_blocks`` blocks of
    ``block_size`` positions per layer and one block table per slot.

    The pool is a PyTorch allocation handed to the C library, exposed per
    layer by ``k_view``/``v_view`` as (num_blocks, Hkv, block_size, D).
    """

    def __init__(self, layers: int, slots: int, max_blocks: int, num_blocks: int, block_size: int,
                 q_heads: int, kv_heads: int, head_dim: int, dtype=torch.float16, device=None):
        if dtype not in _DT:
            raise TypeError(f"unsupported dtype {dtype}")
        self.device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        self.layers, self.slots, self.max_blocks, self.num_blocks = layers, slots, max_blocks, num_blocks
        self.block_size, self.q_heads, self.kv_heads, self.head_dim, self.dtype = (
            block_size, q_heads, kv_heads, head_dim, dtype)
        self.nbytes = paged_bytes(layers, num_blocks, block_size, kv_heads, head_dim, dtype)
        if self.nbytes == 0:
            raise KVAttnError(-1, "PagedKVCache")
        self._handle = ctypes.c_void_p()
        with torch.cuda.device(self.device):
            self._buf = torch.empty(self.nbytes, dtype=torch.uint8, device=self.device)
            torch.cuda.synchronize(self.device)
            _check(lib().kvattn_paged_alloc(ctypes.byref(self._handle), layers, slots, max_blocks, num_blocks,
                                            block_size, q_heads, kv_heads, head_dim, _DT[dtype], _ptr(self._buf),
                                            self.nbytes), "kvattn_paged_alloc")

    def _view(self, layer: int, which: int) -> torch.Tensor:
        if not 0 <= layer < self.layers:
            raise IndexError(layer)
        block = self.nbytes // (2 * self.layers)
        off = (2 * layer + which) * block
        t = self._buf[off:off + block].view(self.dtype)
        return t.view(self.num_blocks, self.kv_heads, self.block_size, self.head_dim)

    def k_view(self, layer: int) -> torch.Tensor:
        return self._view(layer, 0)

    def v_view(self, layer: int) -> torch.Tensor:
        return self._view(layer, 1)

    def set_blocks(self, slot: int, block_ids) -> None:
        ids = [int(x) for x in block_ids]
        arr = (ctypes.c_int32 * max(1, len(ids)))(*ids)
        with torch.cuda.device(self.device):
            _check(lib().kvattn_paged_set_blocks(self._handle, slot, arr, len(ids), _stream_ptr(self.device)),
                   "kvattn_paged_set_blocks")

    def set_lengths(self, lengths, layer: int = -1) -> None:
        arr = (ctypes.c_int32 * self.slots)(*[int(x) for x in lengths])
        with torch.cuda.device(self.device):
            _check(lib().kvattn_paged_set_lengths(self._handle, layer, arr, _stream_ptr(self.device)),
                   "kvattn_paged_set_lengths")

    def lengths(self, layer: int) -> list:
        arr = (ctypes.c_int32 * self.slots)()
        _check(lib().kvattn_paged_get_lengths(self._handle, layer, arr), "kvattn_paged_get_lengths")
        return list(arr)

    def set_window(self, window: int, sink: int = 0, layer: int = -1) -> None:
        """Sliding window W (0: none) and sink S of one layer, or of all (-1)."""
        _check(lib().kvattn_paged_set_window(self._handle, layer, int(window), int(sink)),
               "kvattn_paged_set_window")

    def window(self, layer: int) -> tuple:
        w, s = ctypes.c_int(), ctypes.c_int()
        _check(lib().kvattn_paged_get_window(self._handle, layer, ctypes.byref(w), ctypes.byref(s)),
               "kvattn_paged_get_window")
        return w.value, s.value

    def _tensor(self, t, shape, name, dtype=None):
        KVCache._tensor(self, t, shape, name, dtype)

    def _scale(self, scale):
        return float(1.0 / math.sqrt(self.head_dim)) if scale is None else float(scale)

    def prefill(self, layer: int, q, k, v, out=None, scale=None, out_dtype=None) -> torch.Tensor:
        S, H, Hkv, D = self.slots, self.q_heads, self.kv_heads, self.head_dim
        T = q.shape[2] if q.dim() == 4 else -1
        self._tensor(q, (S, H, T, D), "q")
        self._tensor(k, (S, Hkv, T, D), "k")
        self._tensor(v, (S, Hkv, T, D), "v")
        od = out_dtype or self.dtype
        if out is None:
            out = torch.empty((S, H, T, D), dtype=od, device=self.device)
        self._tensor(out, (S, H, T, D), "out", od)
        with torch.cuda.device(self.device):
            _check(lib().kvattn_paged_prefill(self._handle, layer, _ptr(q), _ptr(k), _ptr(v), _ptr(out), T,
                                              self._scale(scale), _DT[od], _stream_ptr(self.device)),
                   "kvattn_paged_prefill")
        return out

    def extend(self, layer: int, q, k, v, out=None, scale=None, out_dtype=None) -> torch.Tensor:
        """T new positions per slot after its cached prefix, read and written through the block tables."""
        S, H, Hkv, D = self.slots, self.q_heads, self.kv_heads, self.head_dim
        T = q.shape[2] if q.dim() == 4 else -1
        self._tensor(q, (S, H, T, D), "q")
        self._tensor(k, (S, Hkv, T, D), "k")
        self._tensor(v, (S, Hkv, T, D), "v")
        od = out_dtype or self.dtype
        if out is None:
            out = torch.empty((S, H, T, D), dtype=od, device=self.device)
        self._tensor(out, (S, H, T, D), "out", od)
        with torch.cuda.device(self.device):
            _check(lib().kvattn_paged_extend(self._handle, layer, _ptr(q), _ptr(k), _ptr(v), _ptr(out), T,
                                             self._scale(scale), _DT[od], _stream_ptr(self.device)),
                   "kvattn_paged_extend")
        return out

    def append(self, layer: int, k_new, v_new) -> None:
        shape = (self.slots, self.kv_heads, 1, self.head_dim)
        self._tensor(k_new, shape, "k_new")
        self._tensor(v_new, shape, "v_new")
        with torch.cuda.device(self.device):
            _check(lib().kvattn_paged_append(self._handle, layer, _ptr(k_new), _ptr(v_new),
                                             _stream_ptr(self.device)), "kvattn_paged_append")

    def decode(self, layer: int, q, out=None, scale=None, out_dtype=None) -> torch.Tensor:
        shape = (self.slots, self.q_heads, 1, self.head_dim)
        self._tensor(q, shape, "q")
        od = out_dtype or self.dtype
        if out is None:
            out = torch.empty(shape, dtype=od, device=self.device)
        self._tensor(out, shape, "out", od)
        with torch.cuda.device(self.device):
            _check(lib().kvattn_paged_decode(self._handle, layer, _ptr(q), _ptr(out), self._scale(scale), _DT[od],
                                             _stream_ptr(self.device)), "kvattn_paged_decode")
        return out

    def bind_decode(self, layer: int, q, out, scale=None):
        """Pre-bound decode call (arguments checked and marshalled once)."""
        shape = (self.slots, self.q_heads, 1, self.head_dim)
        self._tensor(q, shape, "q")
        self._tensor(out, shape, "out", out.dtype)
        fn = lib().kvattn_paged_decode
        args = (self._handle, layer, _ptr(q), _ptr(out), ctypes.c_float(self._scale(scale)), _DT[out.dtype],
                _stream_ptr(self.device))
        return lambda: _check(fn(*args), "kvattn_paged_decode")

    def close(self) -> None:
        if self._handle and self._handle.value:
            _check(lib().kvattn_paged_free(self._handle), "kvattn_paged_free")
            self._handle = ctypes.c_void_p()
        self._buf = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


class Decoder:
    """The random-weight decoder of kvattn_model.h on one GPU: packed fp16
    weights (a flat device tensor the caller keeps alive), ``batch`` sequences
    of up to ``max_T`` positions, greedy decoding."""

    def __init__(self, layers: int, d_model: int, heads: int, vocab: int, max_T: int, mlp_mult: int, batch: int,
                 weights: torch.Tensor):
        self.device = weights.device
        self.layers, self.d_model, self.heads, self.vocab = layers, d_model, heads, vocab
        self.max_T, self.mlp_mult, self.batch = max_T, mlp_mult, batch
        need = int(lib().kvattn_model_weight_elems(layers, d_model, vocab, max_T, mlp_mult))
        if weights.dtype != torch.float16 or weights.numel() != need or not weights.is_contiguous():
            raise ValueError(f"weights must be a contiguous fp16 tensor of {need} elements")
        self._weights = weights
        self._handle = ctypes.c_void_p()
        with torch.cuda.device(self.device):
            _check(lib().kvattn_model_create(ctypes.byref(self._handle), layers, d_model, heads, vocab, max_T,
                                             mlp_mult, batch, _ptr(weights)), "kvattn_model_create")

    def _ints(self, t: torch.Tensor, shape, name):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or t.device != self.device:
            raise TypeError(f"{name} must be an int32 tensor on {self.device}")
        if tuple(t.shape) != tuple(shape) or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous with shape {tuple(shape)}")

    def prefill(self, tokens: torch.Tensor):
        """Prompt (batch, T) int32 -> (logits of the last position (batch, vocab) fp32, greedy next (batch,))."""
        T = tokens.shape[1] if tokens.dim() == 2 else -1
        self._ints(tokens, (self.batch, T), "tokens")
        logits = torch.empty((self.batch, self.vocab), dtype=torch.float32, device=self.device)
        nxt = torch.empty((self.batch,), dtype=torch.int32, device=self.device)
        with torch.cuda.device(self.device):
            _check(lib().kvattn_model_prefill(self._handle, _ptr(tokens), T, _ptr(logits), _ptr(nxt),
                                              _stream_ptr(self.device)), "kvattn_model_prefill")
        return logits, nxt

    def step(self, tokens: torch.Tensor):
        """Feed tokens (batch,) int32 at the current positions -> (logits, greedy next)."""
        self._ints(tokens, (self.batch,), "tokens")
        logits = torch.empty((self.batch, self.vocab), dtype=torch.float32, device=self.device)
        nxt = torch.empty((self.batch,), dtype=torch.int32, device=self.device)
        with torch.cuda.device(self.device):
            _check(lib().kvattn_model_step(self._handle, _ptr(tokens), _ptr(logits), _ptr(nxt),
                                           _stream_ptr(self.device)), "kvattn_model_step")
        return logits, nxt

    def generate(self, n_steps: int, tokens: torch.Tensor) -> torch.Tensor:
        """Greedy: n_steps tokens per sequence from the current tokens (updated in place) -> (n_steps, batch)."""
        self._ints(tokens, (self.batch,), "tokens")
        out = torch.empty((n_steps, self.batch), dtype=torch.int32, device=self.device)
        with torch.cuda.device(self.device):
            _check(lib().kvattn_model_generate(self._handle, n_steps, _ptr(tokens), _ptr(out),
                                               _stream_ptr(self.device)), "kvattn_model_generate")
        return out

    def positions(self) -> list:
        arr = (ctypes.c_int32 * self.batch)()
        _check(lib().kvattn_model_positions(self._handle, arr), "kvattn_model_positions")
        return list(arr)

    def reset(self) -> None:
        with torch.cuda.device(self.device):
            _check(lib().kvattn_model_reset(self._handle, _stream_ptr(self.device)), "kvattn_model_reset")

    def close(self) -> None:
        if self._handle and self._handle.value:
            _check(lib().kvattn_model_free(self._handle), "kvattn_model_free")
            self._handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
