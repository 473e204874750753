"""An independent NumPy f64 forward -- TEST INFRASTRUCTURE ONLY (brute force).

A second implementation of the same forward pass, written separately from
``q8_oracle.c`` and structured the way the pages describe candle's non-fused
attention branch ("生成一个 token", section "prefill 和 decode：同一个 forward，
不同的路"; "量化 llama 的一次前向", sections "forward：mask 什么时候建" and
"forward_attn：自己拼 KV"):
  * whole weight matrices decoded at once with NumPy's own f16 conversion;
  * the KV cache grown by concatenation along the sequence axis, dropped when
    index_pos == 0;
  * KV heads repeated to the query-head count by concatenating along the
    sequence axis and reshaping (each KV head's copies end up adjacent);
  * a u8 mask table of shape (T, index_pos + T), built only when T > 1, whose
    first index_pos columns are open and whose last T columns are a causal
    triangle; masked scores replaced by -inf; softmax over the last axis.
It is slow and only meant for small shapes. It keeps candle's lack of a
counter check: callers must pass consistent positions.
"""

from __future__ import annotations

from typing import List, Optional, Tuple

import numpy as np


def decode_q8_0(raw: np.ndarray, rows: int, cols: int) -> np.ndarray:
    blocks = np.ascontiguousarray(raw, dtype=np.uint8).reshape(rows, cols // 32, 34)
    d = blocks[:, :, 0:2].copy().view("<f2").astype(np.float64)        # [rows, nb, 1]
    q = blocks[:, :, 2:].copy().view(np.int8).astype(np.float64)        # [rows, nb, 32]
    return (d * q).reshape(rows, cols)


def build_causal_mask(seq_len: int, index_pos: int) -> np.ndarray:
    """u8 [seq_len, index_pos + seq_len], 1 = may not attend."""
    kv_len = index_pos + seq_len
    m = np.zeros((seq_len, kv_len), dtype=np.uint8)
    for i in range(seq_len):
        for j in range(seq_len):
            if j > i:
                m[i, index_pos + j] = 1
    return m


def repeat_kv(x: np.ndarray, n_rep: int) -> np.ndarray:
    """x [n_kv, S, hd] -> [n_kv * n_rep, S, hd] by cat on the sequence axis + reshape."""
    if n_rep == 1:
        return x
    n_kv, s, hd = x.shape
    return np.concatenate([x] * n_rep, axis=1).reshape(n_kv * n_rep, s, hd)


class NumpyLlama:
    def __init__(self, model):
        s = self.s = model.shape
        self.emb = decode_q8_0(model["token_embd.weight"].data, s.n_vocab, s.n_embd)
        self.layers = []
        for i in range(s.n_layer):
            p = f"blk.{i}."
            dq = lambda n, r, c: decode_q8_0(model[p + n].data, r, c)
            self.layers.append(dict(
                attn_norm=model[p + "attn_norm.weight"].data.astype(np.float64),
                wq=dq("attn_q.weight", s.q_dim, s.n_embd),
                wk=dq("attn_k.weight", s.kv_dim, s.n_embd),
                wv=dq("attn_v.weight", s.kv_dim, s.n_embd),
                wo=dq("attn_output.weight", s.n_embd, s.q_dim),
                ffn_norm=model[p + "ffn_norm.weight"].data.astype(np.float64),
                wg=dq("ffn_gate.weight", s.n_ff, s.n_embd),
                wu=dq("ffn_up.weight", s.n_ff, s.n_embd),
                wd=dq("ffn_down.weight", s.n_embd, s.n_ff)))
        self.norm = model["output_norm.weight"].data.astype(np.float64)
        if s.tied_output:
            self.out = self.emb
        else:
            self.out = decode_q8_0(model["output.weight"].data, s.n_vocab, s.n_embd)
        half = np.arange(0, s.head_dim, 2, dtype=np.float64) / s.head_dim
        inv = (1.0 / np.power(s.rope_theta, half)).astype(np.float32)
        pos = np.arange(s.max_seq_len, dtype=np.float32).reshape(-1, 1)
        ang = (pos * inv.reshape(1, -1)).astype(np.float32).astype(np.float64)
        self.cos, self.sin = np.cos(ang), np.sin(ang)
        self.cache: List[Optional[Tuple[np.ndarray, np.ndarray]]] = [None] * s.n_layer

    def clear_kv_cache(self):
        self.cache = [None] * self.s.n_layer

    def _rms(self, x, w):
        return x / np.sqrt((x * x).mean(axis=-1, keepdims=True) + self.s.rms_eps) * w

    def _rope(self, x, index_pos):
        # x [heads, T, hd]; pairs (2j, 2j+1), or with rope_neox the two halves
        # rotated against each other (dimension j with j + hd/2)
        T = x.shape[1]
        c = self.cos[index_pos:index_pos + T][None]
        s = self.sin[index_pos:index_pos + T][None]
        if getattr(self.s, "rope_neox", False):
            x1, x2 = np.split(x, 2, axis=-1)
            return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)
        a, b = x[..., 0::2], x[..., 1::2]
        out = np.empty_like(x)
        out[..., 0::2] = a * c - b * s
        out[..., 1::2] = a * s + b * c
        return out

    def forward(self, tokens, index_pos: int) -> np.ndarray:
        s = self.s
        T = len(tokens)
        if index_pos + T > s.max_seq_len:
            raise IndexError("narrow: index_pos + seq_len beyond the rope table")
        mask = build_causal_mask(T, index_pos) if T > 1 else None
        x = self.emb[np.asarray(tokens, dtype=np.int64)]
        for li, L in enumerate(self.layers):
            res = x
            h = self._rms(x, L["attn_norm"])
            q = (h @ L["wq"].T).reshape(T, s.n_head, s.head_dim).transpose(1, 0, 2)
            k = (h @ L["wk"].T).reshape(T, s.n_head_kv, s.head_dim).transpose(1, 0, 2)
            v = (h @ L["wv"].T).reshape(T, s.n_head_kv, s.head_dim).transpose(1, 0, 2)
            q = self._rope(q, index_pos)
            k = self._rope(k, index_pos)
            if index_pos != 0 and self.cache[li] is not None:
                k = np.concatenate([self.cache[li][0], k], axis=1)
                v = np.concatenate([self.cache[li][1], v], axis=1)
            self.cache[li] = (k, v)
            kk = repeat_kv(k, s.n_head // s.n_head_kv)
            vv = repeat_kv(v, s.n_head // s.n_head_kv)
            att = q @ kk.transpose(0, 2, 1) / np.sqrt(s.head_dim)
            if mask is not None:
                if mask.shape != att.shape[1:]:
                    raise ValueError(f"cannot broadcast {list(mask.shape)} to {[1] + list(att.shape)}")
                att = np.where(mask[None].astype(bool), -np.inf, att)
            att = att - att.max(axis=-1, keepdims=True)
            att = np.exp(att)
            att = att / att.sum(axis=-1, keepdims=True)
            y = (att @ vv).transpose(1, 0, 2).reshape(T, s.q_dim)
            x = y @ L["wo"].T + res
            res = x
            h = self._rms(x, L["ffn_norm"])
            g = h @ L["wg"].T
            u = h @ L["wu"].T
            x = ((g / (1.0 + np.exp(-g))) * u) @ L["wd"].T + res
        y = self._rms(x, self.norm)[T - 1]
        return y @ self.out.T
