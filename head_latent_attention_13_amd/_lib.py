"""ctypes binding of libmla.so (argument marshalling only).

Every function here has the name of the C entry point it wraps, takes torch
tensors (device memory) or plain ints, passes their data pointers and the
current HIP stream to the library, and raises MLAError on a non-zero
status.  All computation happens in the HIP kernels of the library; there is
no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Dict, Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmla.so")

MLA_F32 = 0
MLA_BF16 = 1
MLA_WEIGHTS_MERGED = 0
MLA_WEIGHTS_FACTORED = 1

RAW_WEIGHT_NAMES = ("W_DQ", "W_UQ", "W_QR", "W_DKV", "W_KR", "W_UK", "W_UV", "W_O")


MLA_ROWS_DTYPE, MLA_ROWS_E4M3 = 0, 1


class MLAError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg} ({status})")
        self.status = status


class mla_dims(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("d_latent", ctypes.c_int32),
                ("d_q_latent", ctypes.c_int32), ("d_nope", ctypes.c_int32), ("d_rope", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("dtype", ctypes.c_int32), ("rope_base", ctypes.c_float),
                ("softmax_scale", ctypes.c_float), ("weight_form", ctypes.c_int32)]


class mla_raw_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in RAW_WEIGHT_NAMES]


class mla_cache(ctypes.Structure):
    _fields_ = [("pool", ctypes.c_void_p), ("page_table", ctypes.c_void_p), ("page_size", ctypes.c_int32),
                ("n_pages", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32), ("s_max", ctypes.c_int32),
                ("row_format", ctypes.c_int32), ("scales", ctypes.c_void_p)]


_lib = None

_SIGS = {
    "mla_status_str": (ctypes.c_char_p, [ctypes.c_int32]),
    "mla_last_error": (ctypes.c_char_p, []),
    "mla_version": (ctypes.c_char_p, []),
    "mla_absorbed_layout": (ctypes.c_int32, [ctypes.POINTER(mla_dims), ctypes.POINTER(ctypes.c_size_t),
                                             ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]),
    "mla_absorb_weights": (ctypes.c_int32, [ctypes.POINTER(mla_dims), ctypes.POINTER(mla_raw_weights),
                                            ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "mla_workspace_size": (ctypes.c_int32, [ctypes.POINTER(mla_dims), ctypes.c_int32, ctypes.c_int32,
                                            ctypes.POINTER(ctypes.c_size_t)]),
    "mla_workspace_check": (ctypes.c_int32, [ctypes.POINTER(mla_dims), ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_size_t]),
    "mla_prefill_workspace_check": (ctypes.c_int32, [ctypes.POINTER(mla_dims), ctypes.c_int32, ctypes.c_int32,
                                                     ctypes.c_int32, ctypes.c_size_t]),
    "mla_read_device_error": (ctypes.c_int32, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32), ctypes.c_void_p]),
    "mla_compress_append": (ctypes.c_int32, [ctypes.POINTER(mla_dims), ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.POINTER(mla_cache), ctypes.c_void_p, ctypes.c_size_t,
                                             ctypes.c_void_p]),
    "mla_cache_store_rows": (ctypes.c_int32, [ctypes.POINTER(mla_dims), ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(mla_cache),
                                              ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "mla_q_proj": (ctypes.c_int32, [ctypes.POINTER(mla_dims), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_size_t, ctypes.c_void_p]),
    "mla_attention": (ctypes.c_int32, [ctypes.POINTER(mla_dims), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.POINTER(mla_cache), ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "mla_attention_noalloc": (ctypes.c_int32, [ctypes.POINTER(mla_dims), ctypes.c_void_p, ctypes.c_void_p,
                                               ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(mla_cache),
                                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "mla_decode": (ctypes.c_int32, [ctypes.POINTER(mla_dims), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(mla_cache), ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "mla_out_proj": (ctypes.c_int32, [ctypes.POINTER(mla_dims), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "mla_prefill_workspace_size": (ctypes.c_int32, [ctypes.POINTER(mla_dims), ctypes.c_int32, ctypes.c_int32,
                                                    ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]),
    "mla_prefill_expanded": (ctypes.c_int32, [ctypes.POINTER(mla_dims), ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.POINTER(mla_cache), ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
}

EXPORTED = tuple(_SIGS)


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmla.so (once).  Raises if the library was not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build it first (python -m head_latent_attention_13_amd.build)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != 0:
        lib = load()
        raise MLAError(fn, status, lib.mla_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def make_dims(d_model, n_heads, d_latent, d_q_latent, d_nope, d_rope, d_v, dtype, rope_base=10000.0,
              softmax_scale=0.0, form="merged") -> mla_dims:
    dt = {"f32": MLA_F32, "bf16": MLA_BF16, MLA_F32: MLA_F32, MLA_BF16: MLA_BF16}[dtype]
    wf = {"merged": MLA_WEIGHTS_MERGED, "factored": MLA_WEIGHTS_FACTORED}[form]
    return mla_dims(d_model, n_heads, d_latent, d_q_latent, d_nope, d_rope, d_v, dt, rope_base, softmax_scale, wf)


@dataclass
class Cache:
    """Latent cache: contiguous pool [B, s_max, R] or paged pool [P, page_size, R].

    With ``scales`` set the rows are E4M3 codes (uint8 pool) and ``scales``
    holds one fp32 scale per row slot ([B, s_max] or [P, page_size])."""
    pool: torch.Tensor
    page_table: Optional[torch.Tensor] = None
    page_size: int = 0
    n_pages: int = 0
    max_pages_per_seq: int = 0
    s_max: int = 0
    scales: Optional[torch.Tensor] = None

    def c(self) -> mla_cache:
        return mla_cache(self.pool.data_ptr(), None if self.page_table is None else self.page_table.data_ptr(),
                         self.page_size, self.n_pages, self.max_pages_per_seq, self.s_max,
                         MLA_ROWS_DTYPE if self.scales is None else MLA_ROWS_E4M3,
                         None if self.scales is None else self.scales.data_ptr())


def mla_version() -> str:
    return load().mla_version().decode()


def mla_absorbed_layout(dims: mla_dims):
    offs = (ctypes.c_size_t * 4)()
    sizes = (ctypes.c_size_t * 4)()
    total = ctypes.c_size_t()
    _check("mla_absorbed_layout", load().mla_absorbed_layout(ctypes.byref(dims), offs, sizes, ctypes.byref(total)))
    return list(offs), list(sizes), total.value


def mla_absorb_weights(dims: mla_dims, raw: Dict[str, torch.Tensor], absorbed: torch.Tensor, stream=None):
    rw = mla_raw_weights(*[raw[n].data_ptr() for n in RAW_WEIGHT_NAMES])
    _check("mla_absorb_weights", load().mla_absorb_weights(ctypes.byref(dims), ctypes.byref(rw), _ptr(absorbed),
                                                           absorbed.numel() * absorbed.element_size(),
                                                           _stream(stream)))


def mla_workspace_size(dims: mla_dims, batch: int, n_q: int) -> int:
    n = ctypes.c_size_t()
    _check("mla_workspace_size", load().mla_workspace_size(ctypes.byref(dims), batch, n_q, ctypes.byref(n)))
    return n.value


def mla_workspace_check(dims: mla_dims, batch: int, n_q: int, ws_bytes: int) -> int:
    """Status (0 = fits) of the decode-path calls for batch x n_q rows on a
    workspace of ws_bytes (host only)."""
    return load().mla_workspace_check(ctypes.byref(dims), batch, n_q, ws_bytes)


def mla_prefill_workspace_check(dims: mla_dims, batch: int, n_q: int, s_max: int, ws_bytes: int) -> int:
    """Status (0 = fits) of mla_prefill_expanded for these sizes on a
    workspace of ws_bytes (host only)."""
    return load().mla_prefill_workspace_check(ctypes.byref(dims), batch, n_q, s_max, ws_bytes)


def mla_read_device_error(workspace: torch.Tensor, stream=None) -> int:
    f = ctypes.c_int32()
    _check("mla_read_device_error", load().mla_read_device_error(_ptr(workspace), ctypes.byref(f), _stream(stream)))
    return f.value


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def mla_compress_append(dims, absorbed, x, pos, batch, n_q, cache: Cache, workspace, stream=None):
    cc = cache.c()
    _check("mla_compress_append", load().mla_compress_append(
        ctypes.byref(dims), _ptr(absorbed), _ptr(x), _ptr(pos), batch, n_q, ctypes.byref(cc), _ptr(workspace),
        _nbytes(workspace), _stream(stream)))


def mla_cache_store_rows(dims, rows, pos, batch, n_q, cache: Cache, workspace, stream=None):
    cc = cache.c()
    _check("mla_cache_store_rows", load().mla_cache_store_rows(ctypes.byref(dims), _ptr(rows), _ptr(pos), batch, n_q,
                                                               ctypes.byref(cc), _ptr(workspace), _nbytes(workspace),
                                                               _stream(stream)))


def mla_q_proj(dims, absorbed, x, kv_len, batch, n_q, q, workspace, stream=None):
    _check("mla_q_proj", load().mla_q_proj(ctypes.byref(dims), _ptr(absorbed), _ptr(x), _ptr(kv_len), batch, n_q,
                                           _ptr(q), _ptr(workspace), _nbytes(workspace), _stream(stream)))


def mla_attention(dims, q, kv_len, batch, n_q, cache: Cache, o_lat, lse, workspace, stream=None):
    cc = cache.c()
    _check("mla_attention", load().mla_attention(ctypes.byref(dims), _ptr(q), _ptr(kv_len), batch, n_q,
                                                 ctypes.byref(cc), _ptr(o_lat), _ptr(lse), _ptr(workspace),
                                                 _nbytes(workspace), _stream(stream)))


def mla_attention_noalloc(dims, q, kv_len, batch, n_q, cache: Cache, o_lat, lse, dev_err=None, stream=None):
    cc = cache.c()
    _check("mla_attention_noalloc", load().mla_attention_noalloc(ctypes.byref(dims), _ptr(q), _ptr(kv_len), batch,
                                                                 n_q, ctypes.byref(cc), _ptr(o_lat), _ptr(lse),
                                                                 _ptr(dev_err), _stream(stream)))


def mla_decode(dims, absorbed, x, kv_len, batch, n_q, cache: Cache, o_lat, lse, workspace, stream=None):
    cc = cache.c()
    _check("mla_decode", load().mla_decode(ctypes.byref(dims), _ptr(absorbed), _ptr(x), _ptr(kv_len), batch, n_q,
                                           ctypes.byref(cc), _ptr(o_lat), _ptr(lse), _ptr(workspace),
                                           _nbytes(workspace), _stream(stream)))


def mla_prefill_workspace_size(dims: mla_dims, batch: int, n_q: int, s_max: int) -> int:
    n = ctypes.c_size_t()
    _check("mla_prefill_workspace_size",
           load().mla_prefill_workspace_size(ctypes.byref(dims), batch, n_q, s_max, ctypes.byref(n)))
    return n.value


def mla_prefill_expanded(dims, absorbed, x, kv_len, batch, n_q, cache: Cache, y, lse, workspace, stream=None):
    cc = cache.c()
    _check("mla_prefill_expanded", load().mla_prefill_expanded(
        ctypes.byref(dims), _ptr(absorbed), _ptr(x), _ptr(kv_len), batch, n_q, ctypes.byref(cc), _ptr(y), _ptr(lse),
        _ptr(workspace), _nbytes(workspace), _stream(stream)))


def mla_out_proj(dims, absorbed, o_lat, n_tok, y, workspace, stream=None):
    _check("mla_out_proj", load().mla_out_proj(ctypes.byref(dims), _ptr(absorbed), _ptr(o_lat), n_tok, _ptr(y),
                                               _ptr(workspace), _nbytes(workspace), _stream(stream)))
