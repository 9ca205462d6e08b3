"""ctypes binding of libkvq (include/kvq.h): same entry points, argument marshalling only.

Device buffers may be given as torch tensors (their ``data_ptr()`` is passed;
they must be contiguous) or as raw integer addresses.  ``stream`` is a raw
hipStream_t address, a ``torch.cuda.Stream``, or None for torch's current
stream when torch has a GPU (else the null stream).  Every non-OK status
raises ``KvqError`` carrying ``kvq_last_error()``.

The library must have been built (``python -m rotated_int2_kv_centering_amd.build``);
loading raises ImportError otherwise.  There is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

# kvq_status
KVQ_OK, KVQ_EINVAL, KVQ_EUNSUPPORTED, KVQ_ENOSPACE, KVQ_EHIP = 0, 1, 2, 3, 4
# kvq_dtype
KVQ_BF16, KVQ_F32, KVQ_F32_ROTATED = 0, 1, 2
# kvq_rotation
KVQ_ROT_DENSE, KVQ_ROT_HADAMARD = 0, 1
# kvq_pt_policy
KVQ_PT_CONTIGUOUS, KVQ_PT_PERMUTED, KVQ_PT_INTERLEAVED, KVQ_PT_VALIDATE = 0, 1, 2, 3

HEAD_DIM, GROUP_SIZE, PAGE_SIZE = 128, 32, 16
STATUS_NAMES = {0: "KVQ_OK", 1: "KVQ_EINVAL", 2: "KVQ_EUNSUPPORTED", 3: "KVQ_ENOSPACE", 4: "KVQ_EHIP"}


class KvqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class kvq_cache(ctypes.Structure):
    _fields_ = [("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32), ("pool", ctypes.c_void_p),
                ("clip_ratio", ctypes.c_float), ("rotation", ctypes.c_int32), ("key_bits", ctypes.c_int32),
                ("val_bits", ctypes.c_int32)]


class kvq_window(ctypes.Structure):
    _fields_ = [("sinks", ctypes.c_int32), ("recent", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("buf", ctypes.c_void_p), ("mu", ctypes.c_void_p)]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libkvq.so once and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libkvq.so not built at {path}; run python -m rotated_int2_kv_centering_amd.build")
    lib = ctypes.CDLL(path)
    P, I32, U64, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_size_t, ctypes.c_float
    CP = ctypes.POINTER(kvq_cache)
    WP = ctypes.POINTER(kvq_window)
    lib.kvq_pool_bytes.argtypes = [CP]
    lib.kvq_pool_bytes.restype = SZ
    lib.kvq_quant_append.argtypes = [CP, P, P, I32, I32, P, P, P, P, P, P]
    lib.kvq_quant_append.restype = I32
    lib.kvq_quant_append_err.argtypes = [CP, P, P, I32, I32, P, P, P, P, P, P, P]
    lib.kvq_quant_append_err.restype = I32
    lib.kvq_output_error_workspace_bytes.argtypes = [I32, I32, I32, I32, I32]
    lib.kvq_output_error_workspace_bytes.restype = SZ
    lib.kvq_output_error.argtypes = [CP, P, I32, I32, I32, P, I32, P, I32, P, P, I32, P, P, P, P, F, P, I32, I32, P, P,
                                     P, P, P, SZ, P]
    lib.kvq_output_error.restype = I32
    lib.kvq_decode_workspace_bytes.argtypes = [I32, I32, I32, I32, I32]
    lib.kvq_decode_workspace_bytes.restype = SZ
    lib.kvq_decode_attn.argtypes = [CP, P, I32, I32, I32, P, I32, P, I32, P, P, F, P, I32, P, SZ, I32, WP, P]
    lib.kvq_decode_attn.restype = I32
    lib.kvq_decode_attn_noalloc.argtypes = [CP, P, I32, I32, I32, P, I32, P, I32, P, P, F, P, I32, I32, WP, P]
    lib.kvq_decode_attn_noalloc.restype = I32
    lib.kvq_decode_attn_traced.argtypes = [CP, P, I32, I32, I32, P, I32, P, I32, P, P, F, P, I32, P, SZ, I32, WP, P,
                                           P, P]
    lib.kvq_decode_attn_traced.restype = I32
    lib.kvq_decode_step.argtypes = [CP, P, P, I32, P, P, I32, I32, I32, P, I32, P, I32, P, P, F, P, I32, P, SZ, I32,
                                    WP, P, P, P]
    lib.kvq_decode_step.restype = I32
    lib.kvq_window_bytes.argtypes = [WP, I32]
    lib.kvq_window_bytes.restype = SZ
    lib.kvq_window_fill.argtypes = [WP, I32, P, P, I32, I32, P, P, P, P]
    lib.kvq_window_fill.restype = I32
    lib.kvq_page_table.argtypes = [I32, U64, P, I32, I32, I32, I32, P, P]
    lib.kvq_page_table.restype = I32
    lib.kvq_last_error.argtypes = []
    lib.kvq_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


# ------------------------------------------------------------- marshalling
def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        if hasattr(x, "is_contiguous") and not x.is_contiguous():
            raise ValueError("tensor arguments must be contiguous")
        return int(x.data_ptr())
    if isinstance(x, np.ndarray):
        if not x.flags["C_CONTIGUOUS"]:
            raise ValueError("array arguments must be C-contiguous")
        return int(x.ctypes.data)
    raise TypeError(f"cannot pass {type(x).__name__} as a pointer")


def _stream(stream) -> Optional[int]:
    if stream is None:
        try:
            import torch
            if torch.cuda.is_available():
                return int(torch.cuda.current_stream().cuda_stream)
        except ImportError:
            pass
        return None
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _check(status: int) -> None:
    if status != KVQ_OK:
        raise KvqError(status, load().kvq_last_error().decode(errors="replace"))


def make_cache(num_kv_heads: int, num_pages: int, pool=None, head_dim: int = HEAD_DIM, group_size: int = GROUP_SIZE,
               page_size: int = PAGE_SIZE, clip_ratio: float = 0.0, rotation: int = 0, key_bits: int = 2,
               val_bits: int = 2) -> kvq_cache:
    return kvq_cache(num_kv_heads, head_dim, group_size, page_size, num_pages, _ptr(pool), clip_ratio, rotation,
                     key_bits, val_bits)


def make_window(sinks: int, recent: int, batch: int, buf=None, mu=None) -> kvq_window:
    return kvq_window(sinks, recent, batch, _ptr(buf), _ptr(mu))


def _win(window):
    return ctypes.byref(window) if window is not None else None


# --------------------------------------------------------------- the calls
def kvq_pool_bytes(cache: kvq_cache) -> int:
    return int(load().kvq_pool_bytes(ctypes.byref(cache)))


def kvq_quant_append(cache: kvq_cache, k, v, in_dtype: int, n_tokens: int, slots, mu, r_k, r_v, rot_out=None,
                     stream=None) -> None:
    _check(load().kvq_quant_append(ctypes.byref(cache), _ptr(k), _ptr(v), in_dtype, n_tokens, _ptr(slots), _ptr(mu),
                                   _ptr(r_k), _ptr(r_v), _ptr(rot_out), _stream(stream)))


def kvq_quant_append_err(cache: kvq_cache, k, v, in_dtype: int, n_tokens: int, slots, mu, r_k, r_v, rot_out=None,
                         sq_err=None, stream=None) -> None:
    _check(load().kvq_quant_append_err(ctypes.byref(cache), _ptr(k), _ptr(v), in_dtype, n_tokens, _ptr(slots),
                                       _ptr(mu), _ptr(r_k), _ptr(r_v), _ptr(rot_out), _ptr(sq_err), _stream(stream)))


def kvq_output_error_workspace_bytes(batch: int, num_q_heads: int, num_kv_heads: int, max_seq_len: int,
                                     d_model: int) -> int:
    return int(load().kvq_output_error_workspace_bytes(batch, num_q_heads, num_kv_heads, max_seq_len, d_model))


def kvq_output_error(cache: kvq_cache, q, q_dtype: int, batch: int, num_q_heads: int, page_table, max_pages: int,
                     seq_lens, max_seq_len: int, k, v, kv_dtype: int, row_offsets, sq_err, r_k, r_v, sm_scale: float,
                     w_o, w_dtype: int, d_model: int, dy_k, dy_v, e_out, e_rec, workspace, workspace_bytes: int,
                     stream=None) -> None:
    _check(load().kvq_output_error(ctypes.byref(cache), _ptr(q), q_dtype, batch, num_q_heads, _ptr(page_table),
                                   max_pages, _ptr(seq_lens), max_seq_len, _ptr(k), _ptr(v), kv_dtype,
                                   _ptr(row_offsets), _ptr(sq_err), _ptr(r_k), _ptr(r_v), float(sm_scale), _ptr(w_o),
                                   w_dtype, d_model, _ptr(dy_k), _ptr(dy_v), _ptr(e_out), _ptr(e_rec),
                                   _ptr(workspace), int(workspace_bytes), _stream(stream)))


def kvq_decode_workspace_bytes(batch: int, num_q_heads: int, num_kv_heads: int, max_seq_len: int,
                               num_splits: int = 0) -> int:
    return int(load().kvq_decode_workspace_bytes(batch, num_q_heads, num_kv_heads, max_seq_len, num_splits))


def kvq_decode_attn(cache: kvq_cache, q, q_dtype: int, batch: int, num_q_heads: int, page_table, max_pages: int,
                    seq_lens, max_seq_len: int, r_k, r_v, sm_scale: float, out, out_dtype: int, workspace,
                    workspace_bytes: int, num_splits: int = 0, window=None, stream=None) -> None:
    _check(load().kvq_decode_attn(ctypes.byref(cache), _ptr(q), q_dtype, batch, num_q_heads, _ptr(page_table),
                                  max_pages, _ptr(seq_lens), max_seq_len, _ptr(r_k), _ptr(r_v), float(sm_scale),
                                  _ptr(out), out_dtype, _ptr(workspace), int(workspace_bytes), num_splits,
                                  _win(window), _stream(stream)))


def kvq_decode_attn_noalloc(cache: kvq_cache, q, q_dtype: int, batch: int, num_q_heads: int, page_table,
                            max_pages: int, seq_lens, max_seq_len: int, r_k, r_v, sm_scale: float, out,
                            out_dtype: int, num_splits: int = 0, window=None, stream=None) -> None:
    _check(load().kvq_decode_attn_noalloc(ctypes.byref(cache), _ptr(q), q_dtype, batch, num_q_heads,
                                          _ptr(page_table), max_pages, _ptr(seq_lens), max_seq_len, _ptr(r_k),
                                          _ptr(r_v), float(sm_scale), _ptr(out), out_dtype, num_splits, _win(window),
                                          _stream(stream)))


def kvq_decode_attn_traced(cache: kvq_cache, q, q_dtype: int, batch: int, num_q_heads: int, page_table,
                           max_pages: int, seq_lens, max_seq_len: int, r_k, r_v, sm_scale: float, out, out_dtype: int,
                           workspace, workspace_bytes: int, num_splits: int = 0, window=None, stream=None,
                           ev_begin=None, ev_end=None) -> None:
    """``ev_begin``/``ev_end`` are raw hipEvent_t addresses (or None)."""
    _check(load().kvq_decode_attn_traced(ctypes.byref(cache), _ptr(q), q_dtype, batch, num_q_heads, _ptr(page_table),
                                         max_pages, _ptr(seq_lens), max_seq_len, _ptr(r_k), _ptr(r_v),
                                         float(sm_scale), _ptr(out), out_dtype, _ptr(workspace), int(workspace_bytes),
                                         num_splits, _win(window), _stream(stream), ev_begin, ev_end))


def kvq_decode_step(cache: kvq_cache, k_new, v_new, kv_dtype: int, mu, q, q_dtype: int, batch: int,
                    num_q_heads: int, page_table, max_pages: int, seq_lens, max_seq_len: int, r_k, r_v,
                    sm_scale: float, out, out_dtype: int, workspace, workspace_bytes: int, num_splits: int = 0,
                    window=None, stream=None, ev_begin=None, ev_end=None) -> None:
    """Append the newest token of every sequence (position seq_lens[b] - 1), then decode."""
    _check(load().kvq_decode_step(ctypes.byref(cache), _ptr(k_new), _ptr(v_new), kv_dtype, _ptr(mu), _ptr(q), q_dtype,
                                  batch, num_q_heads, _ptr(page_table), max_pages, _ptr(seq_lens), max_seq_len,
                                  _ptr(r_k), _ptr(r_v), float(sm_scale), _ptr(out), out_dtype, _ptr(workspace),
                                  int(workspace_bytes), num_splits, _win(window), _stream(stream), ev_begin, ev_end))


def kvq_window_bytes(window, num_kv_heads: int) -> int:
    return int(load().kvq_window_bytes(_win(window), num_kv_heads))


def kvq_window_fill(window, num_kv_heads: int, k, v, in_dtype: int, n_tokens: int, seq_ids, positions, seq_lens,
                    stream=None) -> None:
    _check(load().kvq_window_fill(_win(window), num_kv_heads, _ptr(k), _ptr(v), in_dtype, n_tokens, _ptr(seq_ids),
                                  _ptr(positions), _ptr(seq_lens), _stream(stream)))


def kvq_page_table(policy: int, seed: int, seq_lens, page_size: int, num_pages: int, max_pages: int, table=None):
    """Host helper; returns (table int32 [batch][max_pages], slots int32 [batch]).

    Under KVQ_PT_VALIDATE ``table`` must be given; it is only read.
    """
    seq = np.ascontiguousarray(seq_lens, dtype=np.int32)
    batch = int(seq.shape[0])
    if table is None:
        table = np.full((batch, max_pages), -1, dtype=np.int32)
    else:
        table = np.ascontiguousarray(table, dtype=np.int32)
    slots = np.empty(batch, dtype=np.int32)
    _check(load().kvq_page_table(policy, seed, _ptr(seq) if batch else None, batch, page_size, num_pages, max_pages,
                                 _ptr(table) if table.size else None, _ptr(slots) if batch else None))
    return table, slots


def kvq_last_error() -> str:
    return load().kvq_last_error().decode(errors="replace")
