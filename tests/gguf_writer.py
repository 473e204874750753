"""Write GGUF model files for the loader tests.

Written from the public GGUF specification (version 3, little-endian), on
its own: it shares nothing with the library's reader. A file is: magic
"GGUF", u32 version, u64 tensor count, u64 metadata count; metadata entries
(string key, u32 type, value); tensor entries (string name, u32 dimension
count, u64 dimensions innermost first, u32 type, u64 offset into the data
region); padding to the alignment; the tensor data, each tensor at an offset
that is a multiple of the alignment. Strings are a u64 byte length and the
bytes.
"""

from __future__ import annotations

import struct
from typing import List, Sequence, Tuple

import numpy as np

MAGIC = b"GGUF"
U8, I8, U16, I16, U32, I32, F32, BOOL, STRING, ARRAY, U64, I64, F64 = range(13)
_SCALAR = {U8: "<B", I8: "<b", U16: "<H", I16: "<h", U32: "<I", I32: "<i", F32: "<f",
           BOOL: "<?", U64: "<Q", I64: "<q", F64: "<d"}
TYPE_F32, TYPE_F16, TYPE_Q8_0 = 0, 1, 8

KV = Tuple[str, int, object]            # (key, type, value); arrays: (key, ARRAY, (elem_type, values))
TensorEntry = Tuple[str, int, Sequence[int], bytes]   # (name, type, dims innermost first, data)


def _string(s: str) -> bytes:
    b = s.encode()
    return struct.pack("<Q", len(b)) + b


def _value(t: int, v) -> bytes:
    if t == STRING:
        return _string(v)
    if t == ARRAY:
        et, vals = v
        out = [struct.pack("<IQ", et, len(vals))]
        if et == STRING:
            out += [_string(x) for x in vals]
        elif isinstance(vals, np.ndarray):
            out.append(vals.astype(np.dtype(_SCALAR[et])).tobytes())
        else:
            out += [struct.pack(_SCALAR[et], x) for x in vals]
        return b"".join(out)
    return struct.pack(_SCALAR[t], v)


def header_bytes(kv: Sequence[KV], tensors: Sequence[TensorEntry], alignment: int = 32,
                 version: int = 3) -> Tuple[bytes, List[int]]:
    """The bytes before the data region (unpadded) and each tensor's offset."""
    parts = [MAGIC, struct.pack("<IQQ", version, len(tensors), len(kv))]
    for key, t, v in kv:
        parts += [_string(key), struct.pack("<I", t), _value(t, v)]
    offsets, off = [], 0
    for name, ttype, dims, data in tensors:
        off = (off + alignment - 1) // alignment * alignment
        offsets.append(off)
        parts += [_string(name), struct.pack("<I", len(dims)), struct.pack(f"<{len(dims)}Q", *dims),
                  struct.pack("<IQ", ttype, off)]
        off += len(data)
    return b"".join(parts), offsets


def write(path: str, kv: Sequence[KV], tensors: Sequence[TensorEntry], alignment: int = 32,
          version: int = 3) -> int:
    """Write the file; returns the data region's offset."""
    head, offsets = header_bytes(kv, tensors, alignment, version)
    data_off = (len(head) + alignment - 1) // alignment * alignment
    with open(path, "wb") as f:
        f.write(head)
        f.write(b"\0" * (data_off - len(head)))
        pos = 0
        for (name, ttype, dims, data), off in zip(tensors, offsets):
            f.write(b"\0" * (off - pos))
            f.write(data)
            pos = off + len(data)
    return data_off


def llama_kv(shape, arch: str = "llama", rope_dim=None) -> List[KV]:
    """The llama.* hyper-parameter keys of a synth.ModelShape."""
    return [
        ("general.architecture", STRING, arch),
        ("llama.block_count", U32, shape.n_layer),
        ("llama.context_length", U32, shape.max_seq_len),
        ("llama.embedding_length", U32, shape.n_embd),
        ("llama.feed_forward_length", U32, shape.n_ff),
        ("llama.attention.head_count", U32, shape.n_head),
        ("llama.attention.head_count_kv", U32, shape.n_head_kv),
        ("llama.rope.freq_base", F32, shape.rope_theta),
        ("llama.attention.layer_norm_rms_epsilon", F32, shape.rms_eps),
        ("llama.rope.dimension_count", U32, shape.head_dim if rope_dim is None else rope_dim),
    ]


def model_tensors(model) -> List[TensorEntry]:
    """A synth.Model's tensors as file entries (GGUF dims: columns first)."""
    out = []
    for t in model.tensors:
        data = np.ascontiguousarray(t.data).tobytes()
        if t.dtype in ("q8_0", "q5_0", "q4_k", "q6_k"):
            ty = {"q8_0": TYPE_Q8_0, "q5_0": TYPE_Q5_0, "q4_k": TYPE_Q4_K, "q6_k": TYPE_Q6_K}[t.dtype]
            out.append((t.name, ty, [t.cols, t.rows], data))
        else:
            out.append((t.name, TYPE_F32, [t.cols] if t.rows == 1 else [t.cols, t.rows], data))
    return out


# ---- 32-weight integer block formats (public GGUF block definitions) ----
# Q4_0: f16 d, 16 bytes; weight i < 16 = low nibble of byte i, i + 16 = high
# nibble; value d * (nibble - 8). Q5_0: f16 d, u32 fifth bits (bit i for weight
# i), 16 bytes of nibbles as in Q4_0; value d * ((nibble | bit << 4) - 16).
TYPE_Q4_0, TYPE_Q5_0 = 2, 6
TYPE_Q4_K, TYPE_Q6_K = 12, 14


def random_blocks(rng: np.random.Generator, rows: int, cols: int, fmt: str) -> np.ndarray:
    """Random Q4_0 / Q5_0 bytes [rows, cols/32 * block] with synth-style f16 scales."""
    nb = cols // 32
    d = (np.abs(rng.standard_normal((rows, nb))) * 0.02 / 15).astype(np.float16)
    body = 16 if fmt == "q4_0" else 20
    rest = rng.integers(0, 256, (rows, nb, body), dtype=np.uint8)
    return np.concatenate([d.view(np.uint8).reshape(rows, nb, 2), rest], axis=2).reshape(rows, -1)


def to_q8_0(raw: np.ndarray, rows: int, cols: int, fmt: str) -> np.ndarray:
    """The same values as Q8_0 blocks (same scale, int8 = the block's integer)."""
    nb = cols // 32
    size = 18 if fmt == "q4_0" else 22
    b = raw.reshape(rows, nb, size)
    qs = b[:, :, size - 16:]
    lo, hi = (qs & 0x0F).astype(np.int16), (qs >> 4).astype(np.int16)
    if fmt == "q4_0":
        vals = np.concatenate([lo - 8, hi - 8], axis=2)
    else:
        qh = b[:, :, 2:6].copy().view("<u4")[..., 0]
        bits = (qh[..., None] >> np.arange(32, dtype=np.uint32)) & 1
        vals = np.concatenate([lo, hi], axis=2) + (bits.astype(np.int16) << 4) - 16
    out = np.concatenate([b[:, :, :2], vals.astype(np.int8).view(np.uint8)], axis=2)
    return out.reshape(rows, nb * 34)
