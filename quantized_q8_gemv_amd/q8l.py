"""ctypes binding of libq8l.so: the C ABI in include/q8l.h, same names.

This layer only marshals arguments. Every step of the forward pass runs in
the library's HIP kernels; PyTorch is used for device memory and streams. If
the library is missing, loading fails loudly -- there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
import re
from typing import List, Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libq8l.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "q8l.h")

Q8L_OK = 0
Q8L_E_INVALID_ARG = 1
Q8L_E_MISSING_TENSOR = 2
Q8L_E_SHAPE = 3
Q8L_E_POS_RANGE = 4
Q8L_E_POS_MISMATCH = 5
Q8L_E_KV_FULL = 6
Q8L_E_NOT_FINALIZED = 7
Q8L_E_HIP = 8
Q8L_E_FORMAT = 9
Q8L_E_MISSING_KEY = 10
Q8L_E_IO = 11
Q8L_E_RANGE = 12
STATUS_NAMES = {0: "OK", 1: "E_INVALID_ARG", 2: "E_MISSING_TENSOR", 3: "E_SHAPE",
                4: "E_POS_RANGE", 5: "E_POS_MISMATCH", 6: "E_KV_FULL",
                7: "E_NOT_FINALIZED", 8: "E_HIP", 9: "E_FORMAT", 10: "E_MISSING_KEY", 11: "E_IO",
                12: "E_RANGE"}

Q8L_F32 = 0
Q8L_Q8_0 = 1
Q8L_Q4_K = 2
Q8L_Q6_K = 3
Q8L_Q5_0 = 4

Q8L_ROPE_NORM = 0
Q8L_ROPE_NEOX = 1


class q8l_config(ctypes.Structure):
    _fields_ = [("n_layer", ctypes.c_int32), ("n_embd", ctypes.c_int32),
                ("n_head", ctypes.c_int32), ("n_head_kv", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("n_ff", ctypes.c_int32),
                ("n_vocab", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
                ("rms_eps", ctypes.c_double), ("rope_theta", ctypes.c_double),
                ("tied_output", ctypes.c_int32), ("rope_type", ctypes.c_int32)]


class Q8LError(RuntimeError):
    def __init__(self, status: int, message: str = ""):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")


_lib: Optional[ctypes.CDLL] = None

_P = ctypes.c_void_p
_SIGS = {
    "q8l_version": ([], ctypes.c_char_p),
    "q8l_workspace_bytes": ([ctypes.POINTER(q8l_config)], ctypes.c_size_t),
    "q8l_create": ([ctypes.POINTER(q8l_config), ctypes.POINTER(_P)], ctypes.c_int),
    "q8l_bind_tensor": ([_P, ctypes.c_char_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, _P,
                         ctypes.c_size_t], ctypes.c_int),
    "q8l_bind_workspace": ([_P, _P, ctypes.c_size_t], ctypes.c_int),
    "q8l_finalize": ([_P, _P], ctypes.c_int),
    "q8l_forward": ([_P, _P, ctypes.c_int32, ctypes.c_int32, _P, _P, _P], ctypes.c_int),
    "q8l_generate": ([_P, _P, ctypes.c_int32, ctypes.c_int32, _P, _P, _P], ctypes.c_int),
    "q8l_clear_kv_cache": ([_P], ctypes.c_int),
    "q8l_cache_len": ([_P], ctypes.c_int32),
    "q8l_last_error": ([_P], ctypes.c_char_p),
    "q8l_destroy": ([_P], None),
    "q8l_op_matmul_q8_0": ([_P, ctypes.c_int64, ctypes.c_int64, _P, ctypes.c_int64, _P,
                            ctypes.c_double, ctypes.c_int32, _P, _P], ctypes.c_int),
    "q8l_op_matmul_q5_0": ([_P, ctypes.c_int64, ctypes.c_int64, _P, ctypes.c_int64, ctypes.c_int32, _P, _P],
                           ctypes.c_int),
    "q8l_op_matmul_kq": ([_P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, _P, ctypes.c_int64,
                          ctypes.c_int32, _P, _P], ctypes.c_int),
    "q8l_op_attention": ([_P, _P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                          ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P, ctypes.c_size_t,
                          _P], ctypes.c_int),
    "q8l_op_attention_workspace": ([ctypes.c_int32] * 5, ctypes.c_size_t),
    "q8l_op_attention_noalloc": ([_P, _P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                  ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P], ctypes.c_int),
    "q8l_op_argmax": ([_P, ctypes.c_int64, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "q8l_time_decode_kernels": ([_P, ctypes.c_int32, _P, _P], ctypes.c_int),
    "q8l_gguf_open": ([ctypes.c_char_p, ctypes.POINTER(_P)], ctypes.c_int),
    "q8l_gguf_open_error": ([], ctypes.c_char_p),
    "q8l_gguf_last_error": ([_P], ctypes.c_char_p),
    "q8l_gguf_close": ([_P], None),
    "q8l_gguf_version": ([_P], ctypes.c_uint32),
    "q8l_gguf_n_kv": ([_P], ctypes.c_int64),
    "q8l_gguf_n_tensors": ([_P], ctypes.c_int64),
    "q8l_gguf_data_offset": ([_P], ctypes.c_uint64),
    "q8l_gguf_file_size": ([_P], ctypes.c_uint64),
    "q8l_gguf_get_number": ([_P, ctypes.c_char_p, ctypes.POINTER(ctypes.c_double)], ctypes.c_int),
    "q8l_gguf_get_string": ([_P, ctypes.c_char_p, ctypes.c_char_p, ctypes.c_size_t], ctypes.c_int),
    "q8l_gguf_config": ([_P, ctypes.c_int32, ctypes.POINTER(q8l_config)], ctypes.c_int),
    "q8l_gguf_find_tensor": ([_P, ctypes.c_char_p], ctypes.c_int64),
    "q8l_gguf_tensor_info": ([_P, ctypes.c_int64, ctypes.POINTER(ctypes.c_char_p),
                              ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64),
                              ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_uint64),
                              ctypes.POINTER(ctypes.c_uint64)], ctypes.c_int),
    "q8l_gguf_read_tensor": ([_P, ctypes.c_int64, _P, ctypes.c_size_t], ctypes.c_int),
    "q8l_gguf_tensor_file_type": ([_P, ctypes.c_int64], ctypes.c_int32),
}


def header_functions() -> List[str]:
    """Names of the functions include/q8l.h declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q8l_[a-z0-9_]+)\s*\(", text)))


def lib() -> ctypes.CDLL:
    """Load libq8l.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m quantized_q8_gemv_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _ptr(x) -> Optional[int]:
    """Device/host address of a torch tensor, an int, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    return x.ctypes.data  # numpy array (host memory)


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---- the C ABI, one Python function per C function --------------------------

def q8l_version() -> str:
    return lib().q8l_version().decode()


def q8l_workspace_bytes(cfg: q8l_config) -> int:
    return int(lib().q8l_workspace_bytes(ctypes.byref(cfg)))


def q8l_create(cfg: q8l_config) -> int:
    h = _P()
    st = lib().q8l_create(ctypes.byref(cfg), ctypes.byref(h))
    if st != Q8L_OK:
        raise Q8LError(st, "invalid config")
    return h.value


def q8l_bind_tensor(m: int, name: str, dtype: int, rows: int, cols: int, dev_ptr, nbytes: int) -> int:
    return lib().q8l_bind_tensor(m, name.encode(), dtype, rows, cols, _ptr(dev_ptr), nbytes)


def q8l_bind_workspace(m: int, dev_ptr, nbytes: int) -> int:
    return lib().q8l_bind_workspace(m, _ptr(dev_ptr), nbytes)


def q8l_finalize(m: int, stream=None) -> int:
    return lib().q8l_finalize(m, _stream(stream))


def q8l_forward(m: int, tokens_host, n_tokens: int, index_pos: int, logits_dev, argmax_dev=None,
                stream=None) -> int:
    return lib().q8l_forward(m, _ptr(tokens_host), n_tokens, index_pos, _ptr(logits_dev), _ptr(argmax_dev),
                             _stream(stream))


def q8l_generate(m: int, token_dev, index_pos: int, n_steps: int, ids_dev, logits_dev=None,
                 stream=None) -> int:
    return lib().q8l_generate(m, _ptr(token_dev), index_pos, n_steps, _ptr(ids_dev), _ptr(logits_dev),
                              _stream(stream))


def q8l_clear_kv_cache(m: int) -> int:
    return lib().q8l_clear_kv_cache(m)


def q8l_cache_len(m: int) -> int:
    return int(lib().q8l_cache_len(m))


def q8l_last_error(m: int) -> str:
    return lib().q8l_last_error(m).decode()


def q8l_destroy(m: int) -> None:
    lib().q8l_destroy(m)


def q8l_op_matmul_q8_0(W, N: int, K: int, X, T: int, norm_w, eps: float, accumulate: int, Y,
                       stream=None) -> int:
    return lib().q8l_op_matmul_q8_0(_ptr(W), N, K, _ptr(X), T, _ptr(norm_w), eps, accumulate,
                                    _ptr(Y), _stream(stream))


def q8l_op_matmul_q5_0(W, N: int, K: int, X, T: int, accumulate: int, Y, stream=None) -> int:
    return lib().q8l_op_matmul_q5_0(_ptr(W), N, K, _ptr(X), T, accumulate, _ptr(Y), _stream(stream))


def q8l_op_matmul_kq(W, dtype: int, N: int, K: int, X, T: int, accumulate: int, Y, stream=None) -> int:
    return lib().q8l_op_matmul_kq(_ptr(W), dtype, N, K, _ptr(X), T, accumulate, _ptr(Y), _stream(stream))


def q8l_op_attention(Q, K, V, T: int, kv_len: int, kv_stride: int, n_head: int, n_head_kv: int,
                     hd: int, O, workspace, workspace_bytes: int, stream=None) -> int:
    return lib().q8l_op_attention(_ptr(Q), _ptr(K), _ptr(V), T, kv_len, kv_stride, n_head, n_head_kv,
                                  hd, _ptr(O), _ptr(workspace), workspace_bytes, _stream(stream))


def q8l_op_attention_workspace(T: int, kv_len: int, n_head: int, n_head_kv: int, hd: int) -> int:
    return int(lib().q8l_op_attention_workspace(T, kv_len, n_head, n_head_kv, hd))


def q8l_op_attention_noalloc(Q, K, V, T: int, kv_len: int, kv_stride: int, n_head: int, n_head_kv: int,
                             hd: int, O, stream=None) -> int:
    return lib().q8l_op_attention_noalloc(_ptr(Q), _ptr(K), _ptr(V), T, kv_len, kv_stride, n_head, n_head_kv,
                                          hd, _ptr(O), _stream(stream))


def q8l_op_argmax(x, n: int, out, workspace, workspace_bytes: int, stream=None) -> int:
    return lib().q8l_op_argmax(_ptr(x), n, _ptr(out), _ptr(workspace), workspace_bytes,
                               _stream(stream))


def q8l_time_decode_kernels(m: int, reps: int, ms_out, stream=None) -> int:
    return lib().q8l_time_decode_kernels(m, reps, _ptr(ms_out), _stream(stream))


# ---- GGUF model files (host side) ----

def q8l_gguf_open(path: str) -> int:
    """Open and parse a GGUF file; raises Q8LError with the reader's message."""
    h = _P()
    st = lib().q8l_gguf_open(path.encode(), ctypes.byref(h))
    if st != Q8L_OK:
        raise Q8LError(st, lib().q8l_gguf_open_error().decode())
    return h.value


def q8l_gguf_open_error() -> str:
    return lib().q8l_gguf_open_error().decode()


def q8l_gguf_last_error(g: int) -> str:
    return lib().q8l_gguf_last_error(g).decode()


def q8l_gguf_close(g: int) -> None:
    lib().q8l_gguf_close(g)


def q8l_gguf_version(g: int) -> int:
    return int(lib().q8l_gguf_version(g))


def q8l_gguf_n_kv(g: int) -> int:
    return int(lib().q8l_gguf_n_kv(g))


def q8l_gguf_n_tensors(g: int) -> int:
    return int(lib().q8l_gguf_n_tensors(g))


def q8l_gguf_data_offset(g: int) -> int:
    return int(lib().q8l_gguf_data_offset(g))


def q8l_gguf_file_size(g: int) -> int:
    return int(lib().q8l_gguf_file_size(g))


def q8l_gguf_get_number(g: int, key: str):
    """(status, value)"""
    v = ctypes.c_double()
    st = lib().q8l_gguf_get_number(g, key.encode(), ctypes.byref(v))
    return st, v.value


def q8l_gguf_get_string(g: int, key: str, size: int = 4096):
    """(status, value)"""
    buf = ctypes.create_string_buffer(size)
    st = lib().q8l_gguf_get_string(g, key.encode(), buf, size)
    return st, buf.value.decode(errors="replace")


def q8l_gguf_config(g: int, max_seq_len: int = 4096):
    """(status, q8l_config)"""
    cfg = q8l_config()
    st = lib().q8l_gguf_config(g, max_seq_len, ctypes.byref(cfg))
    return st, cfg


def q8l_gguf_find_tensor(g: int, name: str) -> int:
    return int(lib().q8l_gguf_find_tensor(g, name.encode()))


def q8l_gguf_tensor_info(g: int, index: int):
    """(status, dict(name, dtype, rows, cols, offset, nbytes))"""
    name = ctypes.c_char_p()
    dt, rows, cols = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int64()
    off, nb = ctypes.c_uint64(), ctypes.c_uint64()
    st = lib().q8l_gguf_tensor_info(g, index, ctypes.byref(name), ctypes.byref(dt), ctypes.byref(rows),
                                    ctypes.byref(cols), ctypes.byref(off), ctypes.byref(nb))
    info = dict(name=(name.value or b"").decode(), dtype=dt.value, rows=rows.value, cols=cols.value,
                offset=off.value, nbytes=nb.value)
    return st, info


def q8l_gguf_read_tensor(g: int, index: int, host_dst, nbytes: int) -> int:
    return lib().q8l_gguf_read_tensor(g, index, _ptr(host_dst), nbytes)


def q8l_gguf_tensor_file_type(g: int, index: int) -> int:
    return int(lib().q8l_gguf_tensor_file_type(g, index))


def config_from(shape_fields: dict) -> q8l_config:
    return q8l_config(**shape_fields)
