"""Seeded synthetic inputs for the quantized Llama forward pass.

This module only draws random numbers and lays them out as the model's input
files would hold them: model shapes, random-init weights in the Q8_0 block
format (an f16 little-endian scale followed by 32 signed 8-bit values, 34
bytes per 32 weights), f32 RMSNorm weights, and prompt token ids. It holds
none of the forward pass's arithmetic and imports neither the oracle nor the
GPU library; both take their inputs from here.

Model and workload shapes follow the pages' model, SmolLM2-135M-Instruct in
Q8_0 ("量化 llama 的一次前向" intro: 30 layers, hidden 576, 9 query heads,
3 KV heads, head_dim 64, vocab 49152; "生成一个 token", section 建模型: 272
tensors, no ``output.weight`` so the output layer is the embedding), plus a
tiny model of the same widths and a larger GQA Llama shape.

Random-init recipe (the pages publish no weights we can use):
  * ``rng = numpy.random.default_rng(seed)`` (PCG64), one stream per model;
  * tensors are drawn in canonical order: ``token_embd``, then per layer
    ``attn_norm, attn_q, attn_k, attn_v, attn_output, ffn_norm, ffn_gate,
    ffn_up, ffn_down``, then ``output_norm``, then ``output`` when untied;
  * a Q8_0 tensor of n weights draws its n/32 scales first as
    ``standard_normal``, scale = f16(|z| * 0.02 / 127) (about 30 % of them are
    f16 subnormals), then its n values as ``integers(-127, 128, int8)``;
  * a norm weight draws ``normal(1, 0.1, H)`` and is stored as f32;
  * prompt ids are ``default_rng(prompt_seed).integers(0, V, T)`` as uint32.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, Iterator, List, Optional, Tuple

import numpy as np

QK8_0 = 32             # weights per Q8_0 block
Q8_0_BLOCK_BYTES = 34  # 2-byte f16 scale + 32 int8

LAYER_TENSORS = ("attn_norm", "attn_q", "attn_k", "attn_v", "attn_output",
                 "ffn_norm", "ffn_gate", "ffn_up", "ffn_down")


@dataclasses.dataclass(frozen=True)
class ModelShape:
    """Hyper-parameters of one Llama-shaped model (the ``llama.*`` keys)."""
    name: str
    n_layer: int
    n_embd: int
    n_head: int
    n_head_kv: int
    head_dim: int
    n_ff: int
    n_vocab: int
    tied_output: bool = True
    max_seq_len: int = 4096
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0
    rope_neox: bool = False   # rope pairs (j, j + hd/2) instead of (2j, 2j + 1)

    @property
    def q_dim(self) -> int:
        return self.n_head * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_head_kv * self.head_dim

    def tensor_specs(self) -> List[Tuple[str, str, int, int]]:
        """(name, dtype, rows, cols) in canonical order; dtype 'q8_0' or 'f32'.

        Weight matrices are [out, in] with ``in`` contiguous; norm weights are
        given as rows=1, cols=H.
        """
        H, F, V = self.n_embd, self.n_ff, self.n_vocab
        specs = [("token_embd.weight", "q8_0", V, H)]
        for i in range(self.n_layer):
            p = f"blk.{i}."
            specs += [
                (p + "attn_norm.weight", "f32", 1, H),
                (p + "attn_q.weight", "q8_0", self.q_dim, H),
                (p + "attn_k.weight", "q8_0", self.kv_dim, H),
                (p + "attn_v.weight", "q8_0", self.kv_dim, H),
                (p + "attn_output.weight", "q8_0", H, self.q_dim),
                (p + "ffn_norm.weight", "f32", 1, H),
                (p + "ffn_gate.weight", "q8_0", F, H),
                (p + "ffn_up.weight", "q8_0", F, H),
                (p + "ffn_down.weight", "q8_0", H, F),
            ]
        specs.append(("output_norm.weight", "f32", 1, H))
        if not self.tied_output:
            specs.append(("output.weight", "q8_0", V, H))
        return specs

    def tensor_nbytes(self, dtype: str, rows: int, cols: int) -> int:
        if dtype == "q8_0":
            return rows * cols // QK8_0 * Q8_0_BLOCK_BYTES
        return rows * cols * 4

    def total_bytes(self) -> int:
        return sum(self.tensor_nbytes(d, r, c) for _, d, r, c in self.tensor_specs())


# The five model/workload shapes. C2-C4 share the 135M-shaped model.
TINY = ModelShape("tiny", n_layer=4, n_embd=576, n_head=9, n_head_kv=3, head_dim=64,
                  n_ff=1536, n_vocab=4096)
SMOL135M = ModelShape("smollm2-135m", n_layer=30, n_embd=576, n_head=9, n_head_kv=3,
                      head_dim=64, n_ff=1536, n_vocab=49152)
BIG_GQA = ModelShape("llama-7b-gqa", n_layer=32, n_embd=4096, n_head=32, n_head_kv=8,
                     head_dim=128, n_ff=14336, n_vocab=32000, tied_output=False)


@dataclasses.dataclass(frozen=True)
class Workload:
    """A generation run: prompt prefill at position 0, then greedy decode."""
    name: str
    model: ModelShape
    prompt_len: int
    decode_steps: int
    reps: int = 1
    seed: int = 0          # weight stream
    prompt_seed: int = 1   # prompt-id stream


WORKLOADS: Dict[str, Workload] = {
    "C1": Workload("tiny-13+20", TINY, 13, 20),
    "C2": Workload("smollm2-135m-q8_0 13+20", SMOL135M, 13, 20),
    "C3": Workload("smollm2-135m-q8_0 203+128 x10", SMOL135M, 203, 128, reps=10),
    "C4": Workload("smollm2-135m-q8_0 4000+96 long-context", SMOL135M, 4000, 96),
    "C5": Workload("llama-7b-gqa-q8_0 512+128", BIG_GQA, 512, 128),
}


def micro_shape(n_layer=2, n_embd=64, n_head=4, n_head_kv=2, head_dim=16, n_ff=128,
                n_vocab=50, tied_output=True, max_seq_len=64, name="micro",
                rope_neox=False) -> ModelShape:
    """Small shapes for brute-force and edge-case tests."""
    return ModelShape(name, n_layer=n_layer, n_embd=n_embd, n_head=n_head,
                      n_head_kv=n_head_kv, head_dim=head_dim, n_ff=n_ff, n_vocab=n_vocab,
                      tied_output=tied_output, max_seq_len=max_seq_len, rope_neox=rope_neox)


def draw_q8_0(rng: np.random.Generator, rows: int, cols: int,
              scale_std: float = 0.02) -> Tuple[np.ndarray, np.ndarray]:
    """Draw one Q8_0 tensor's parts: f16 scales [rows, cols/32] and int8 [rows, cols]."""
    if cols % QK8_0:
        raise ValueError(f"Q8_0 rows must hold whole 32-weight blocks, got cols={cols}")
    nb = rows * cols // QK8_0
    z = rng.standard_normal(nb)
    scales = (np.abs(z) * (scale_std / 127.0)).astype(np.float16)
    q = rng.integers(-127, 128, size=rows * cols, dtype=np.int8)
    return scales.reshape(rows, cols // QK8_0), q.reshape(rows, cols)


def pack_q8_0(scales: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Lay out Q8_0 blocks: per block the f16 scale (little-endian) then 32 int8.

    ``scales`` is [rows, cols/32] float16 and ``q`` is [rows, cols] int8; the
    result is [rows, cols/32*34] uint8 with blocks along each row.
    """
    rows, cols = q.shape
    nb = cols // QK8_0
    out = np.empty((rows, nb, Q8_0_BLOCK_BYTES), dtype=np.uint8)
    out[:, :, 0:2] = np.ascontiguousarray(scales, dtype="<f2").view(np.uint8).reshape(rows, nb, 2)
    out[:, :, 2:] = np.ascontiguousarray(q).view(np.uint8).reshape(rows, nb, QK8_0)
    return out.reshape(rows, nb * Q8_0_BLOCK_BYTES)


@dataclasses.dataclass
class Tensor:
    name: str
    dtype: str          # 'q8_0', 'q5_0', 'q4_k', 'q6_k' or 'f32'
    rows: int
    cols: int
    data: np.ndarray    # block formats: uint8 [rows, row bytes]; f32: float32 [cols]

    @property
    def nbytes(self) -> int:
        return int(self.data.nbytes)


class Model:
    """A random-init model: shape plus tensors in canonical order."""

    def __init__(self, shape: ModelShape, tensors: List[Tensor]):
        self.shape = shape
        self.tensors = tensors
        self.by_name = {t.name: t for t in tensors}

    def __getitem__(self, name: str) -> Tensor:
        return self.by_name[name]

    def __iter__(self) -> Iterator[Tensor]:
        return iter(self.tensors)

    @property
    def total_bytes(self) -> int:
        return sum(t.nbytes for t in self.tensors)

    def replace(self, name: str, data: np.ndarray) -> "Model":
        """A copy of the model with one tensor's bytes replaced (same shape)."""
        old = self.by_name[name]
        if data.shape != old.data.shape or data.dtype != old.data.dtype:
            raise ValueError(f"{name}: expected {old.data.shape} {old.data.dtype}")
        ts = [Tensor(t.name, t.dtype, t.rows, t.cols, data if t.name == name else t.data)
              for t in self.tensors]
        return Model(self.shape, ts)


def random_model(shape: ModelShape, seed: int = 0, keep_parts: bool = False) -> Model:
    """Draw a model by the recipe in this module's docstring.

    With ``keep_parts`` each Q8_0 tensor also carries its unpacked ``scales``
    and ``q`` arrays as attributes (for tests of the block layout).
    """
    rng = np.random.default_rng(seed)
    tensors = []
    for name, dtype, rows, cols in shape.tensor_specs():
        if dtype == "q8_0":
            scales, q = draw_q8_0(rng, rows, cols)
            t = Tensor(name, dtype, rows, cols, pack_q8_0(scales, q))
            if keep_parts:
                t.scales, t.q = scales, q  # type: ignore[attr-defined]
        else:
            w = rng.normal(1.0, 0.1, size=cols).astype(np.float32)
            t = Tensor(name, dtype, rows, cols, w)
        tensors.append(t)
    return Model(shape, tensors)


# ---- 256-weight "K" block formats (public GGUF block definitions) ----------
# Q4_K, 144 bytes: f16 d, f16 dmin, 12 bytes of packed 6-bit scales and mins,
# 128 bytes of 4-bit values. Q6_K, 210 bytes: 128 bytes of low 4 bits, 64 of
# high 2 bits, 16 int8 scales, f16 d. Only their byte layout is drawn here.
K_BLOCK_BYTES = {"q4_k": 144, "q6_k": 210}


def draw_k_quant(rng: np.random.Generator, rows: int, cols: int, fmt: str,
                 scale_std: float = 0.02) -> np.ndarray:
    """Random Q4_K / Q6_K bytes [rows, cols/256 * block]: uniform random
    value, scale and min bytes; f16 super-block scales |z| * scale_std / (63*15)
    (Q4_K d), / (63*4) (Q4_K dmin), / (127*32) (Q6_K d), so weights stay near
    the Q8_0 draw's magnitude."""
    if cols % 256:
        raise ValueError(f"{fmt} rows must hold whole 256-weight blocks, got cols={cols}")
    nb = cols // 256
    size = K_BLOCK_BYTES[fmt]
    body = rng.integers(0, 256, size=(rows, nb, size), dtype=np.uint8)
    f16 = lambda div: (np.abs(rng.standard_normal((rows, nb))) * (scale_std / div)).astype("<f2").view(np.uint8)
    if fmt == "q4_k":
        body[:, :, 0:2] = f16(63 * 15).reshape(rows, nb, 2)
        body[:, :, 2:4] = f16(63 * 4).reshape(rows, nb, 2)
    elif fmt == "q6_k":
        body[:, :, 208:210] = f16(127 * 32).reshape(rows, nb, 2)
    else:
        raise ValueError(fmt)
    return body.reshape(rows, nb * size)


# ---- Q5_0 (public GGUF block definition) ------------------------------------
# 22 bytes per 32 weights: f16 d, a little-endian 32-bit word of fifth bits,
# 16 bytes of nibbles (low nibbles weights 0..15, high nibbles 16..31).
Q5_0_BLOCK_BYTES = 22


def draw_q5_0(rng: np.random.Generator, rows: int, cols: int, scale_std: float = 0.02) -> np.ndarray:
    """Random Q5_0 bytes [rows, cols/32 * 22]: f16 scales |z| * scale_std / 15
    (weights near the Q8_0 draw's magnitude), uniform random fifth-bit words
    and nibble bytes."""
    if cols % QK8_0:
        raise ValueError(f"Q5_0 rows must hold whole 32-weight blocks, got cols={cols}")
    nb = cols // QK8_0
    body = rng.integers(0, 256, size=(rows, nb, Q5_0_BLOCK_BYTES), dtype=np.uint8)
    d = (np.abs(rng.standard_normal((rows, nb))) * (scale_std / 15.0)).astype("<f2")
    body[:, :, 0:2] = d.view(np.uint8).reshape(rows, nb, 2)
    return body.reshape(rows, nb * Q5_0_BLOCK_BYTES)


def with_formats(model: Model, want: Dict[str, str], seed: int = 7) -> Model:
    """A copy of ``model`` whose tensors named in ``want`` are redrawn in the
    given block format ('q5_0', 'q4_k', 'q6_k'; 'q8_0' keeps the original),
    drawn in canonical tensor order from one stream."""
    rng = np.random.default_rng(seed)
    ts = []
    for t in model.tensors:
        f = want.get(t.name, "q8_0")
        if t.dtype == "q8_0" and f == "q5_0":
            ts.append(Tensor(t.name, f, t.rows, t.cols, draw_q5_0(rng, t.rows, t.cols)))
        elif t.dtype == "q8_0" and f != "q8_0":
            ts.append(Tensor(t.name, f, t.rows, t.cols, draw_k_quant(rng, t.rows, t.cols, f)))
        else:
            ts.append(t)
    return Model(model.shape, ts)


def with_k_quants(model: Model, o_fmts, d_fmts, seed: int = 7) -> Model:
    """A copy of ``model`` whose per-layer attn_output / ffn_down matrices are
    redrawn in the given formats ('q8_0' keeps the original tensor)."""
    want = {}
    for l in range(model.shape.n_layer):
        want[f"blk.{l}.attn_output.weight"] = o_fmts[l]
        want[f"blk.{l}.ffn_down.weight"] = d_fmts[l]
    return with_formats(model, want, seed)


# Per-layer formats of the seven projections, in the order q, k, v, o, gate,
# up, down.
LAYER_ROLES = ("attn_q", "attn_k", "attn_v", "attn_output", "ffn_gate", "ffn_up", "ffn_down")


def random_model_formats(shape: ModelShape, seed: int, fmts) -> Model:
    """A model drawn with each projection directly in its block format
    (``fmts[l]`` = seven formats for layer l, q .. down): Q8_0 tensors and
    norms as in ``random_model``, Q5_0 / K-format tensors by ``draw_q5_0`` /
    ``draw_k_quant``, all from one stream in canonical order. (Not the same
    values as ``with_layer_formats``, which redraws on top of a Q8_0 model.)"""
    rng = np.random.default_rng(seed)
    want = {}
    for l in range(shape.n_layer):
        for role, f in zip(LAYER_ROLES, fmts[l]):
            want[f"blk.{l}.{role}.weight"] = f
    tensors = []
    for name, dtype, rows, cols in shape.tensor_specs():
        f = want.get(name, dtype)
        if f == "q8_0":
            tensors.append(Tensor(name, f, rows, cols, pack_q8_0(*draw_q8_0(rng, rows, cols))))
        elif f == "q5_0":
            tensors.append(Tensor(name, f, rows, cols, draw_q5_0(rng, rows, cols)))
        elif f in K_BLOCK_BYTES:
            tensors.append(Tensor(name, f, rows, cols, draw_k_quant(rng, rows, cols, f)))
        else:
            tensors.append(Tensor(name, f, rows, cols, rng.normal(1.0, 0.1, size=cols).astype(np.float32)))
    return Model(shape, tensors)


def with_layer_formats(model: Model, fmts, seed: int = 7) -> Model:
    """``fmts[l]`` = seven formats for layer l (q, k, v, o, gate, up, down)."""
    want = {}
    for l in range(model.shape.n_layer):
        for role, f in zip(LAYER_ROLES, fmts[l]):
            want[f"blk.{l}.{role}.weight"] = f
    return with_formats(model, want, seed)


def prompt_ids(n_vocab: int, length: int, seed: int = 1) -> np.ndarray:
    """Uniform-random prompt token ids in [0, V) as uint32."""
    return np.random.default_rng(seed).integers(0, n_vocab, size=length).astype(np.uint32)


def workload_inputs(key: str, keep_parts: bool = False) -> Tuple[Workload, Model, np.ndarray]:
    w = WORKLOADS[key]
    m = random_model(w.model, w.seed, keep_parts=keep_parts)
    return w, m, prompt_ids(w.model.n_vocab, w.prompt_len, w.prompt_seed)


def shape_fields(shape: ModelShape) -> Dict[str, object]:
    """The hyper-parameters as a flat dict (for config structs on either side)."""
    return dict(n_layer=shape.n_layer, n_embd=shape.n_embd, n_head=shape.n_head,
                n_head_kv=shape.n_head_kv, head_dim=shape.head_dim, n_ff=shape.n_ff,
                n_vocab=shape.n_vocab, max_seq_len=shape.max_seq_len,
                rms_eps=shape.rms_eps, rope_theta=shape.rope_theta,
                tied_output=int(shape.tied_output), rope_type=int(shape.rope_neox))


__all__ = ["QK8_0", "Q8_0_BLOCK_BYTES", "LAYER_TENSORS", "ModelShape", "TINY", "SMOL135M",
           "BIG_GQA", "Workload", "WORKLOADS", "micro_shape", "draw_q8_0", "pack_q8_0",
           "Tensor", "Model", "random_model", "K_BLOCK_BYTES", "draw_k_quant", "with_k_quants", "Q5_0_BLOCK_BYTES", "draw_q5_0",
           "with_formats", "LAYER_ROLES", "with_layer_formats", "random_model_formats", "prompt_ids", "workload_inputs", "shape_fields"]

