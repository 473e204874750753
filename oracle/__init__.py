"""CPU oracle for the quantized Llama forward pass -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package. It shares no code with the GPU library
(``quantized_q8_gemv_amd``) and never imports it.

Two independent implementations live here:
  * ``q8_oracle.c`` (loaded through ctypes as ``OracleModel`` and the component
    functions below): the plain f64 forward used for parity;
  * ``np_reference.py``: a separate NumPy f64 implementation written the way
    the pages describe candle's non-fused attention branch, used only as a
    brute-force cross-check on small shapes.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "q8_oracle.c")
LIB = os.path.join(HERE, "libq8oracle.so")

# Status codes (same meaning as the library's boundary).
OK, E_INVALID_ARG, E_MISSING_TENSOR, E_SHAPE, E_POS_RANGE, E_POS_MISMATCH, E_KV_FULL = range(7)
STATUS_NAMES = {OK: "OK", E_INVALID_ARG: "E_INVALID_ARG", E_MISSING_TENSOR: "E_MISSING_TENSOR",
                E_SHAPE: "E_SHAPE", E_POS_RANGE: "E_POS_RANGE",
                E_POS_MISMATCH: "E_POS_MISMATCH", E_KV_FULL: "E_KV_FULL"}


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (plain -O2, OpenMP, no FP contraction)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
               "-std=c11", "-Wall", "-o", LIB + ".tmp", SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(LIB + ".tmp", LIB)
    return LIB


class _Config(ctypes.Structure):
    _fields_ = [("n_layer", ctypes.c_int32), ("n_embd", ctypes.c_int32),
                ("n_head", ctypes.c_int32), ("n_head_kv", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("n_ff", ctypes.c_int32),
                ("n_vocab", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
                ("rms_eps", ctypes.c_double), ("rope_theta", ctypes.c_double),
                ("tied_output", ctypes.c_int32), ("rope_neox", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build(force=True)
        L = ctypes.CDLL(LIB)
        P, D, I64, I32 = ctypes.c_void_p, ctypes.c_double, ctypes.c_int64, ctypes.c_int32
        L.orc_f16_to_f64.argtypes = [ctypes.c_uint16]; L.orc_f16_to_f64.restype = D
        L.orc_dequant_row.argtypes = [P, I64, P]; L.orc_dequant_row.restype = None
        L.orc_dequant_q4_0_row.argtypes = [P, I64, P]; L.orc_dequant_q4_0_row.restype = None
        L.orc_dequant_q5_0_row.argtypes = [P, I64, P]; L.orc_dequant_q5_0_row.restype = None
        L.orc_dequant_q4_k_row.argtypes = [P, I64, P]; L.orc_dequant_q4_k_row.restype = None
        L.orc_dequant_q6_k_row.argtypes = [P, I64, P]; L.orc_dequant_q6_k_row.restype = None
        L.orc_matmul_q8.argtypes = [P, I64, I64, P, I64, P]; L.orc_matmul_q8.restype = None
        L.orc_matmul_fmt.argtypes = [P, ctypes.c_int32, I64, I64, P, I64, P]
        L.orc_matmul_fmt.restype = None
        L.orc_rmsnorm.argtypes = [P, P, I64, D, P]; L.orc_rmsnorm.restype = None
        L.orc_rope_angle.argtypes = [I64, I64, I64, D]; L.orc_rope_angle.restype = D
        L.orc_rope_i.argtypes = [P, I64, I64, D]; L.orc_rope_i.restype = None
        L.orc_rope_neox.argtypes = [P, I64, I64, D]; L.orc_rope_neox.restype = None
        L.orc_silu.argtypes = [D]; L.orc_silu.restype = D
        L.orc_attend.argtypes = [P, P, P, I64, I64, I64, P]; L.orc_attend.restype = None
        L.orc_create.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(ctypes.c_void_p)]
        L.orc_create.restype = P
        L.orc_create_fmt.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(ctypes.c_void_p), P, P]
        L.orc_create_fmt.restype = P
        L.orc_create_fmt7.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(ctypes.c_void_p), P]
        L.orc_create_fmt7.restype = P
        L.orc_destroy.argtypes = [P]; L.orc_destroy.restype = None
        L.orc_clear_kv_cache.argtypes = [P]; L.orc_clear_kv_cache.restype = None
        L.orc_cache_len.argtypes = [P]; L.orc_cache_len.restype = I32
        L.orc_counts.argtypes = [P, P]; L.orc_counts.restype = None
        L.orc_forward.argtypes = [P, P, I32, I32, P, P]; L.orc_forward.restype = ctypes.c_int
        L.orc_argmax.argtypes = [P, I64]; L.orc_argmax.restype = I64
        L.orc_read_cache.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, I64, P]
        L.orc_read_cache.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> ctypes.c_void_p:
    return ctypes.c_void_p(a.ctypes.data)


# ---- component functions (each mirrors one C function) --------------------

def f16_to_f64(bits: int) -> float:
    return lib().orc_f16_to_f64(bits & 0xFFFF)


def dequant_q8_0(raw: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Decode a Q8_0 matrix [rows, cols] from its raw block bytes."""
    raw = np.ascontiguousarray(raw, dtype=np.uint8).reshape(rows, cols // 32 * 34)
    out = np.empty((rows, cols), dtype=np.float64)
    for r in range(rows):
        lib().orc_dequant_row(_ptr(raw[r]), cols, _ptr(out[r]))
    return out


def dequant_q4_0(raw: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Decode a Q4_0 matrix [rows, cols] (18 bytes per 32 weights)."""
    raw = np.ascontiguousarray(raw, dtype=np.uint8).reshape(rows, cols // 32 * 18)
    out = np.empty((rows, cols), dtype=np.float64)
    for r in range(rows):
        lib().orc_dequant_q4_0_row(_ptr(raw[r]), cols, _ptr(out[r]))
    return out


def dequant_q5_0(raw: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Decode a Q5_0 matrix [rows, cols] (22 bytes per 32 weights)."""
    raw = np.ascontiguousarray(raw, dtype=np.uint8).reshape(rows, cols // 32 * 22)
    out = np.empty((rows, cols), dtype=np.float64)
    for r in range(rows):
        lib().orc_dequant_q5_0_row(_ptr(raw[r]), cols, _ptr(out[r]))
    return out


# Block formats of the 256-weight "K" family (bytes per 256 weights) and the
# oracle's format codes for the matrices' block formats.
K_BLOCK_BYTES = {"q4_k": 144, "q6_k": 210}
FMT_CODES = {"q8_0": 0, "q4_k": 1, "q6_k": 2, "q5_0": 3}
LAYER_MATRICES = ("attn_q", "attn_k", "attn_v", "attn_output", "ffn_gate", "ffn_up", "ffn_down")


def dequant_q4_k(raw: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Decode a Q4_K matrix [rows, cols] (144 bytes per 256 weights)."""
    raw = np.ascontiguousarray(raw, dtype=np.uint8).reshape(rows, cols // 256 * 144)
    out = np.empty((rows, cols), dtype=np.float64)
    for r in range(rows):
        lib().orc_dequant_q4_k_row(_ptr(raw[r]), cols, _ptr(out[r]))
    return out


def dequant_q6_k(raw: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Decode a Q6_K matrix [rows, cols] (210 bytes per 256 weights)."""
    raw = np.ascontiguousarray(raw, dtype=np.uint8).reshape(rows, cols // 256 * 210)
    out = np.empty((rows, cols), dtype=np.float64)
    for r in range(rows):
        lib().orc_dequant_q6_k_row(_ptr(raw[r]), cols, _ptr(out[r]))
    return out


def matmul_fmt(raw: np.ndarray, fmt: str, rows: int, cols: int, x: np.ndarray) -> np.ndarray:
    """Y[t] = W @ X[t] for W [rows, cols] in block format ``fmt`` ('q8_0', 'q5_0', 'q4_k', 'q6_k')."""
    raw = np.ascontiguousarray(raw, dtype=np.uint8)
    X = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float64)
    Y = np.empty((X.shape[0], rows), dtype=np.float64)
    lib().orc_matmul_fmt(_ptr(raw), FMT_CODES[fmt], rows, cols, _ptr(X), X.shape[0], _ptr(Y))
    return Y


def matmul_q8(raw: np.ndarray, rows: int, cols: int, x: np.ndarray) -> np.ndarray:
    """Y[t] = W @ X[t] for Q8_0 W [rows, cols] and X [T, cols] (f64)."""
    raw = np.ascontiguousarray(raw, dtype=np.uint8)
    X = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float64)
    Y = np.empty((X.shape[0], rows), dtype=np.float64)
    lib().orc_matmul_q8(_ptr(raw), rows, cols, _ptr(X), X.shape[0], _ptr(Y))
    return Y


def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    w = np.ascontiguousarray(w, dtype=np.float32)
    y = np.empty_like(x)
    lib().orc_rmsnorm(_ptr(x), _ptr(w), x.size, eps, _ptr(y))
    return y


def rope_angle(p: int, j: int, hd: int, theta: float) -> float:
    return lib().orc_rope_angle(p, j, hd, theta)


def rope_i(v: np.ndarray, p: int, theta: float) -> np.ndarray:
    out = np.ascontiguousarray(v, dtype=np.float64).copy()
    lib().orc_rope_i(_ptr(out), out.size, p, theta)
    return out


def rope_neox(v: np.ndarray, p: int, theta: float) -> np.ndarray:
    out = np.ascontiguousarray(v, dtype=np.float64).copy()
    lib().orc_rope_neox(_ptr(out), out.size, p, theta)
    return out


def silu(z: float) -> float:
    return lib().orc_silu(z)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, last_visible: Optional[int] = None) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.float64)
    K = np.ascontiguousarray(K, dtype=np.float64)
    V = np.ascontiguousarray(V, dtype=np.float64)
    n, hd = K.shape
    o = np.empty(hd, dtype=np.float64)
    lv = n - 1 if last_visible is None else last_visible
    lib().orc_attend(_ptr(q), _ptr(K), _ptr(V), n, hd, lv, _ptr(o))
    return o


def argmax(v: np.ndarray) -> int:
    v = np.ascontiguousarray(v, dtype=np.float32)
    return int(lib().orc_argmax(_ptr(v), v.size))


# ---- whole model -------------------------------------------------------------

class OracleModel:
    """The f64 CPU forward with its KV cache; takes a ``synth.Model``."""

    def __init__(self, model, max_seq_len: Optional[int] = None):
        s = model.shape
        self.shape = s
        self.cfg = _Config(s.n_layer, s.n_embd, s.n_head, s.n_head_kv, s.head_dim, s.n_ff,
                           s.n_vocab, max_seq_len or s.max_seq_len, s.rms_eps, s.rope_theta,
                           int(s.tied_output), int(getattr(s, "rope_neox", False)))
        self._arrays = [np.ascontiguousarray(t.data) for t in model.tensors]
        ptrs = (ctypes.c_void_p * len(self._arrays))(*[a.ctypes.data for a in self._arrays])
        self._ptrs = ptrs
        fmts = np.array([[FMT_CODES[model[f"blk.{l}.{r}.weight"].dtype] for r in LAYER_MATRICES]
                         for l in range(s.n_layer)], dtype=np.int32)
        self._fmts = fmts
        h = lib().orc_create_fmt7(ctypes.byref(self.cfg), ptrs, _ptr(fmts))
        if not h:
            raise ValueError("oracle rejected the model configuration")
        self._h = h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            lib().orc_destroy(h)
            self._h = None

    @property
    def n_vocab(self) -> int:
        return self.cfg.n_vocab

    def forward(self, tokens: Sequence[int], index_pos: int) -> Tuple[int, Optional[np.ndarray], Optional[np.ndarray]]:
        """Returns (status, f32 logits, f64 logits); logits are None on error."""
        t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64).astype(np.uint32))
        lg = np.empty(self.n_vocab, dtype=np.float32)
        lg64 = np.empty(self.n_vocab, dtype=np.float64)
        st = lib().orc_forward(self._h, _ptr(t) if t.size else None, int(t.size), int(index_pos),
                               _ptr(lg), _ptr(lg64))
        if st != OK:
            return st, None, None
        return st, lg, lg64

    def clear_kv_cache(self) -> None:
        lib().orc_clear_kv_cache(self._h)

    @property
    def cache_len(self) -> int:
        return int(lib().orc_cache_len(self._h))

    def counts(self) -> Tuple[int, int, int]:
        """(matmul calls, rmsnorm calls, rope applications) in the last forward."""
        out = np.zeros(3, dtype=np.int64)
        lib().orc_counts(self._h, _ptr(out))
        return int(out[0]), int(out[1]), int(out[2])

    def read_cache(self, kind: str, layer: int, group: int, pos: int) -> np.ndarray:
        out = np.empty(self.shape.head_dim, dtype=np.float64)
        st = lib().orc_read_cache(self._h, 1 if kind == "v" else 0, layer, group, pos, _ptr(out))
        if st != OK:
            raise IndexError("cache position out of range")
        return out

    def generate(self, prompt: Sequence[int], steps: int):
        """Prefill at position 0, then ``steps`` greedy decode steps.

        Returns (ids, logits per step): ids[0] is picked from the prefill.
        """
        st, lg, _ = self.forward(prompt, 0)
        if st != OK:
            raise RuntimeError(STATUS_NAMES[st])
        ids, all_logits = [argmax(lg)], [lg]
        pos = len(prompt)
        for k in range(steps):
            st, lg, _ = self.forward([ids[-1]], pos + k)
            if st != OK:
                raise RuntimeError(STATUS_NAMES[st])
            ids.append(argmax(lg))
            all_logits.append(lg)
        return ids, all_logits
