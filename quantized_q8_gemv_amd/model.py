"""Q8Model: place a model's tensors in device memory and drive the library.

Argument marshalling only: the forward pass runs in libq8l.so's kernels.
"""

from __future__ import annotations

import ctypes
import os
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

from . import q8l as C


class Q8Model:
    """A model bound to the library.

    ``config`` is a dict of q8l_config fields; ``tensors`` yields objects with
    ``name``, ``dtype`` ('q8_0', 'q5_0', 'q4_k', 'q6_k' or 'f32'), ``rows``, ``cols``
    and ``data`` (a host numpy array of the raw bytes / f32 values).
    """

    def __init__(self, config: dict, tensors: Iterable, device: str = "cuda:0", stream=None):
        import torch

        self.torch = torch
        self.device = torch.device(device)
        self.cfg = C.q8l_config(**config)
        self.n_vocab = self.cfg.n_vocab
        nbytes = C.q8l_workspace_bytes(self.cfg)
        if nbytes == 0:
            raise C.Q8LError(C.Q8L_E_INVALID_ARG, "invalid config")
        self.handle = C.q8l_create(self.cfg)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self.buffers = {}
        for t in tensors:
            arr = np.ascontiguousarray(t.data)
            dev = torch.from_numpy(arr.view(np.uint8).reshape(-1)).to(self.device)
            self.buffers[t.name] = dev
            dt = _DTYPES[t.dtype]
            self._check(C.q8l_bind_tensor(self.handle, t.name, dt, t.rows, t.cols, dev, dev.numel()))
        self._check(C.q8l_bind_workspace(self.handle, self.workspace, nbytes))
        self._check(C.q8l_finalize(self.handle, stream))
        self.logits = torch.empty(self.n_vocab, dtype=torch.float32, device=self.device)
        self.argmax = torch.zeros(1, dtype=torch.int32, device=self.device)

    @classmethod
    def from_gguf(cls, path: str, device: str = "cuda:0", max_seq_len: int = 4096, stream=None) -> "Q8Model":
        """Build a model from a GGUF file: config from its llama.* keys, then
        each required tensor read by name and bound (C ABI q8l_gguf_*)."""
        g = C.q8l_gguf_open(path)
        try:
            st, cfg = C.q8l_gguf_config(g, max_seq_len)
            if st != C.Q8L_OK:
                raise C.Q8LError(st, C.q8l_gguf_last_error(g))
            fields = {name: getattr(cfg, name) for name, _ in C.q8l_config._fields_}
            names = ["token_embd.weight"]
            for i in range(cfg.n_layer):
                names += [f"blk.{i}.{t}.weight" for t in ("attn_norm", "attn_q", "attn_k", "attn_v",
                                                           "attn_output", "ffn_norm", "ffn_gate", "ffn_up",
                                                           "ffn_down")]
            names.append("output_norm.weight")
            if not cfg.tied_output:
                names.append("output.weight")
            return cls(fields, _gguf_tensors(g, names), device=device, stream=stream)
        finally:
            C.q8l_gguf_close(g)

    def _check(self, st: int) -> None:
        if st != C.Q8L_OK:
            raise C.Q8LError(st, C.q8l_last_error(self.handle))

    def forward_async(self, tokens: Sequence[int], index_pos: int, stream=None, argmax_out=None) -> int:
        """Enqueue forward(tokens, index_pos); returns the status (no raise).

        ``argmax_out`` (default: the device tensor ``self.argmax``) may be the
        device address of pinned host memory (``host_mapped_u32``): the last
        kernel then writes the greedy id straight to the host."""
        if isinstance(tokens, np.ndarray) and tokens.dtype == np.uint32 and tokens.flags.c_contiguous:
            toks = tokens
        else:
            toks = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64).astype(np.uint32))
        return C.q8l_forward(self.handle, toks, int(toks.size), int(index_pos), self.logits,
                             self.argmax if argmax_out is None else argmax_out, stream)

    def forward(self, tokens: Sequence[int], index_pos: int, stream=None) -> Tuple[np.ndarray, int]:
        """Run forward and wait; returns (f32 logits on the host, argmax)."""
        self._check(self.forward_async(tokens, index_pos, stream))
        self.torch.cuda.synchronize(self.device)
        return self.logits.cpu().numpy(), int(self.argmax.item())

    def generate_async(self, token_dev, index_pos: int, n_steps: int, ids_dev, stream=None) -> int:
        return C.q8l_generate(self.handle, token_dev, int(index_pos), int(n_steps), ids_dev,
                              self.logits, stream)

    def clear_kv_cache(self) -> None:
        self._check(C.q8l_clear_kv_cache(self.handle))

    @property
    def cache_len(self) -> int:
        return C.q8l_cache_len(self.handle)

    def close(self) -> None:
        if getattr(self, "handle", None):
            C.q8l_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _loaded_hip_runtime() -> str:
    """Path of the HIP runtime this process has already loaded (torch's, which
    libq8l.so shares): opening that same file returns the loaded library
    instead of starting a second runtime under another soname."""
    C.lib()  # libq8l.so links the runtime: it is mapped from here on
    with open("/proc/self/maps") as f:
        for line in f:
            path = line.split()[-1] if line.strip() else ""
            if os.path.basename(path).startswith("libamdhip64.so"):
                return path
    raise RuntimeError("no HIP runtime (libamdhip64.so) is loaded in this process")


def host_mapped_u32():
    """A pinned host int32 tensor of one element and its device address.

    The device writes it directly (pinned host memory is mapped into the
    device's address space), so reading a per-token result needs only a stream
    synchronisation, no copy."""
    import torch

    t = torch.zeros(1, dtype=torch.int32, pin_memory=True)
    hip = ctypes.CDLL(_loaded_hip_runtime())
    dptr = ctypes.c_void_p()
    err = hip.hipHostGetDevicePointer(ctypes.byref(dptr), ctypes.c_void_p(t.data_ptr()), 0)
    if err != 0 or not dptr.value:
        raise RuntimeError(f"hipHostGetDevicePointer failed ({err})")
    return t, int(dptr.value)


_DTYPES = {"f32": C.Q8L_F32, "q8_0": C.Q8L_Q8_0, "q4_k": C.Q8L_Q4_K, "q6_k": C.Q8L_Q6_K, "q5_0": C.Q8L_Q5_0}
_DTYPE_NAMES = {v: k for k, v in _DTYPES.items()}


class _FileTensor:
    __slots__ = ("name", "dtype", "rows", "cols", "data")


def _gguf_tensors(g: int, names):
    """Yield the named tensors of an open GGUF file one at a time (absent names
    are skipped: finalize then reports the first missing one)."""
    for name in names:
        idx = C.q8l_gguf_find_tensor(g, name)
        if idx < 0:
            continue
        st, info = C.q8l_gguf_tensor_info(g, idx)
        if st != C.Q8L_OK:
            raise C.Q8LError(st, C.q8l_gguf_last_error(g))
        buf = np.empty(info["nbytes"], dtype=np.uint8)
        st = C.q8l_gguf_read_tensor(g, idx, buf, info["nbytes"])
        if st != C.Q8L_OK:
            raise C.Q8LError(st, C.q8l_gguf_last_error(g))
        t = _FileTensor()
        t.name, t.rows, t.cols, t.data = name, info["rows"], info["cols"], buf
        t.dtype = _DTYPE_NAMES[info["dtype"]]
        yield t
