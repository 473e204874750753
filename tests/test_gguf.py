"""The GGUF reader (C ABI q8l_gguf_*, host only) on files written by
tests/gguf_writer.py, which follows the public format independently.

Pins from the pages ("生成一个 token", section "读 GGUF"): the SmolLM2-135M Q8_0
file holds 37 metadata keys and 272 tensors, its data region starts at byte
1,785,952 and the file is 144,811,360 bytes long; the model is built from the
llama.* keys ("量化 llama 的一次前向", section "from_gguf") whose absence fails
with "cannot find {key} in metadata"; no output.weight means the output layer
is the embedding ("建模型：按名字取张量"); general.architecture picks the rope
pairing ("RoPE：两种约定，按架构名选").
"""

import os

import numpy as np
import pytest

import gguf_writer as W
import synth

C = pytest.importorskip("quantized_q8_gemv_amd.q8l")


@pytest.fixture(scope="module")
def lib():
    C.lib()
    return C


def _tiny_file(tmp_path, shape=synth.TINY, arch="llama", seed=0, drop_keys=(), extra_kv=(), alignment=32):
    m = synth.random_model(shape, seed)
    kv = [e for e in W.llama_kv(shape, arch) if e[0] not in drop_keys] + list(extra_kv)
    if alignment != 32:
        kv.append(("general.alignment", W.U32, alignment))
    path = str(tmp_path / f"{shape.name}-{arch}.gguf")
    off = W.write(path, kv, W.model_tensors(m), alignment=alignment)
    return path, m, kv, off


def test_directory_and_config_of_a_tiny_model(lib, tmp_path):
    path, m, kv, off = _tiny_file(tmp_path)
    g = C.q8l_gguf_open(path)
    try:
        assert C.q8l_gguf_version(g) == 3
        assert C.q8l_gguf_n_kv(g) == len(kv)
        assert C.q8l_gguf_n_tensors(g) == len(m.tensors)
        assert C.q8l_gguf_data_offset(g) == off
        assert C.q8l_gguf_file_size(g) == os.path.getsize(path)
        st, cfg = C.q8l_gguf_config(g, 4096)
        assert st == C.Q8L_OK
        s = synth.TINY
        assert (cfg.n_layer, cfg.n_embd, cfg.n_head, cfg.n_head_kv, cfg.head_dim, cfg.n_ff, cfg.n_vocab) == \
            (s.n_layer, s.n_embd, s.n_head, s.n_head_kv, s.head_dim, s.n_ff, s.n_vocab)
        assert cfg.max_seq_len == 4096 and cfg.tied_output == 1 and cfg.rope_type == C.Q8L_ROPE_NORM
        assert cfg.rope_theta == 10000.0
        assert cfg.rms_eps == pytest.approx(1e-5, rel=1e-6)       # stored as f32 in the file
        st, name = C.q8l_gguf_get_string(g, "general.architecture")
        assert st == C.Q8L_OK and name == "llama"
        # every tensor: name, type, shape, size, and its bytes by name
        for t in m.tensors:
            idx = C.q8l_gguf_find_tensor(g, t.name)
            assert idx >= 0
            st, info = C.q8l_gguf_tensor_info(g, idx)
            assert st == C.Q8L_OK
            assert info["name"] == t.name
            assert info["dtype"] == (C.Q8L_Q8_0 if t.dtype == "q8_0" else C.Q8L_F32)
            assert (info["rows"], info["cols"]) == (t.rows, t.cols)
            raw = np.ascontiguousarray(t.data).view(np.uint8).reshape(-1)
            assert info["nbytes"] == raw.size
            assert info["offset"] % 32 == 0
            buf = np.empty(raw.size, dtype=np.uint8)
            assert C.q8l_gguf_read_tensor(g, idx, buf, raw.size) == C.Q8L_OK
            assert np.array_equal(buf, raw)
        assert C.q8l_gguf_find_tensor(g, "output.weight") == -1
    finally:
        C.q8l_gguf_close(g)


def test_pages_directory_figures_for_the_135m_file(lib, tmp_path, golden_printed):
    """A 135M-shaped file with the pages' 37 keys (a synthetic tokenizer block
    sized so the data starts where theirs does) and the 272 tensors: the reader
    reports the printed data offset, and the file size comes out as printed."""
    s = synth.SMOL135M
    tensors = [(name, W.TYPE_Q8_0 if dt == "q8_0" else W.TYPE_F32,
                [c, r] if dt == "q8_0" or r > 1 else [c],
                bytes(s.tensor_nbytes(dt, r, c))) for name, dt, r, c in s.tensor_specs()]
    assert len(tensors) == golden_printed["gguf_tensor_count"] == 272
    kv = W.llama_kv(s) + [
        ("general.name", W.STRING, "synthetic 135M-shaped"),
        ("general.file_type", W.U32, 7),
        ("llama.vocab_size", W.U32, s.n_vocab),
        ("tokenizer.ggml.model", W.STRING, "gpt2"),
        ("tokenizer.ggml.tokens", W.ARRAY, (W.STRING, [f"t{i}" for i in range(s.n_vocab)])),
        ("tokenizer.ggml.token_type", W.ARRAY, (W.I32, np.ones(s.n_vocab, dtype=np.int32))),
        ("tokenizer.ggml.merges", W.ARRAY, (W.STRING, [f"m{i}" for i in range(48900)])),
    ]
    kv += [(f"general.synthetic_{i}", W.U32, i) for i in range(37 - len(kv) - 1)]
    # the last key: a byte array sized so that the data region starts at the printed offset
    target = golden_printed["gguf_data_offset"]
    head, _ = W.header_bytes(kv + [("general.pad", W.ARRAY, (W.U8, np.zeros(0, np.uint8)))], tensors)
    kv.append(("general.pad", W.ARRAY, (W.U8, np.zeros(target - len(head), np.uint8))))
    assert len(kv) == golden_printed["gguf_metadata_keys"] == 37
    path = str(tmp_path / "smol135m.gguf")
    off = W.write(path, kv, tensors)
    assert off == target
    g = C.q8l_gguf_open(path)
    try:
        assert C.q8l_gguf_n_kv(g) == 37
        assert C.q8l_gguf_n_tensors(g) == 272
        assert C.q8l_gguf_data_offset(g) == golden_printed["gguf_data_offset"]
        assert C.q8l_gguf_file_size(g) == golden_printed["gguf_file_bytes"] == 144_811_360
        st, cfg = C.q8l_gguf_config(g, 4096)
        assert st == C.Q8L_OK
        assert (cfg.n_layer, cfg.n_embd, cfg.n_head, cfg.n_head_kv, cfg.head_dim, cfg.n_vocab) == \
            (30, 576, 9, 3, 64, 49152)
        assert cfg.tied_output == 1
        total = 0
        for i in range(272):
            st, info = C.q8l_gguf_tensor_info(g, i)
            assert st == C.Q8L_OK
            total += info["nbytes"]
        assert total == golden_printed["gguf_file_bytes"] - golden_printed["gguf_data_offset"]
    finally:
        C.q8l_gguf_close(g)


@pytest.mark.parametrize("key", ["llama.attention.head_count", "llama.attention.head_count_kv",
                                 "llama.block_count", "llama.embedding_length",
                                 "llama.feed_forward_length", "llama.rope.dimension_count",
                                 "llama.attention.layer_norm_rms_epsilon"])
def test_missing_llama_key_is_named(lib, tmp_path, key):
    path, *_ = _tiny_file(tmp_path, drop_keys=(key,))
    g = C.q8l_gguf_open(path)
    try:
        st, _ = C.q8l_gguf_config(g, 4096)
        assert st == C.Q8L_E_MISSING_KEY
        assert C.q8l_gguf_last_error(g) == f"cannot find {key} in metadata"
    finally:
        C.q8l_gguf_close(g)


def test_optional_freq_base_defaults_to_10000(lib, tmp_path):
    path, *_ = _tiny_file(tmp_path, drop_keys=("llama.rope.freq_base",))
    g = C.q8l_gguf_open(path)
    try:
        st, cfg = C.q8l_gguf_config(g, 4096)
        assert st == C.Q8L_OK and cfg.rope_theta == 10000.0
    finally:
        C.q8l_gguf_close(g)


def test_untied_file_has_output_layer(lib, tmp_path):
    s = synth.micro_shape(n_embd=128, n_head=4, n_head_kv=2, head_dim=32, n_vocab=64, tied_output=False,
                          name="untied")
    path, m, *_ = _tiny_file(tmp_path, shape=s)
    g = C.q8l_gguf_open(path)
    try:
        st, cfg = C.q8l_gguf_config(g, 64)
        assert st == C.Q8L_OK and cfg.tied_output == 0
        assert C.q8l_gguf_find_tensor(g, "output.weight") >= 0
    finally:
        C.q8l_gguf_close(g)


@pytest.mark.parametrize("arch,rope", [("llama", 0), ("qwen2", 1), ("qwen", 1), ("falcon", 1),
                                       ("phi3", 1), ("stablelm", 1), ("gptneox", 1), ("mistral", 0)])
def test_architecture_selects_rope_pairing(lib, tmp_path, arch, rope):
    path, *_ = _tiny_file(tmp_path, arch=arch)
    g = C.q8l_gguf_open(path)
    try:
        st, cfg = C.q8l_gguf_config(g, 4096)
        assert st == C.Q8L_OK and cfg.rope_type == rope
    finally:
        C.q8l_gguf_close(g)


def test_alignment_key_is_honoured(lib, tmp_path):
    path, m, kv, off = _tiny_file(tmp_path, alignment=256)
    g = C.q8l_gguf_open(path)
    try:
        assert C.q8l_gguf_data_offset(g) == off and off % 256 == 0
        for i in range(C.q8l_gguf_n_tensors(g)):
            st, info = C.q8l_gguf_tensor_info(g, i)
            assert st == C.Q8L_OK and (info["offset"] - off) % 256 == 0
        idx = C.q8l_gguf_find_tensor(g, "blk.1.ffn_down.weight")
        t = m["blk.1.ffn_down.weight"]
        raw = np.ascontiguousarray(t.data).view(np.uint8).reshape(-1)
        buf = np.empty(raw.size, np.uint8)
        assert C.q8l_gguf_read_tensor(g, idx, buf, raw.size) == C.Q8L_OK
        assert np.array_equal(buf, raw)
    finally:
        C.q8l_gguf_close(g)


def test_malformed_files_are_rejected(lib, tmp_path):
    path, *_ = _tiny_file(tmp_path)
    data = open(path, "rb").read()
    cases = {
        "bad magic": b"GGUX" + data[4:],
        "version 1": data[:4] + (1).to_bytes(4, "little") + data[8:],
        "truncated header": data[:20],
        "truncated directory": data[:3000],
        "huge counts": data[:8] + (1 << 60).to_bytes(8, "little") + data[16:],
    }
    for what, blob in cases.items():
        p = str(tmp_path / "bad.gguf")
        open(p, "wb").write(blob)
        with pytest.raises(C.Q8LError) as e:
            C.q8l_gguf_open(p)
        assert e.value.status == C.Q8L_E_FORMAT, what
    # a file cut inside the data region: the directory is fine, a tensor ends past the end
    p = str(tmp_path / "cut.gguf")
    open(p, "wb").write(data[:-100])
    with pytest.raises(C.Q8LError) as e:
        C.q8l_gguf_open(p)
    assert e.value.status == C.Q8L_E_FORMAT
    with pytest.raises(C.Q8LError) as e:
        C.q8l_gguf_open(str(tmp_path / "absent.gguf"))
    assert e.value.status == C.Q8L_E_IO


def test_unsupported_tensor_type_is_reported_by_name(lib, tmp_path):
    m = synth.random_model(synth.TINY, 0)
    tensors = W.model_tensors(m)
    name, _, dims, data = tensors[1]                      # blk.0.attn_norm.weight as F16
    tensors[1] = (name, W.TYPE_F16, dims, data[: len(data) // 2])
    path = str(tmp_path / "f16.gguf")
    W.write(path, W.llama_kv(synth.TINY), tensors)
    g = C.q8l_gguf_open(path)
    try:
        idx = C.q8l_gguf_find_tensor(g, name)
        st, info = C.q8l_gguf_tensor_info(g, idx)
        assert st == C.Q8L_E_FORMAT and info["dtype"] == -1
        assert name in C.q8l_gguf_last_error(g)
        assert C.q8l_gguf_read_tensor(g, idx, np.empty(8, np.uint8), 8) == C.Q8L_E_FORMAT
    finally:
        C.q8l_gguf_close(g)


@pytest.mark.parametrize("fmt,ftype,name", [("q5_0", W.TYPE_Q5_0, "output.weight"),
                                            ("q4_0", W.TYPE_Q4_0, "blk.0.ffn_down.weight"),
                                            ("q4_0", W.TYPE_Q4_0, "token_embd.weight")])
def test_q4_0_and_q5_0_tensors_read_as_exact_q8_0(lib, tmp_path, fmt, ftype, name):
    """Q4_0 anywhere, and Q5_0 outside the layers' projections, are read as
    Q8_0 blocks with the same scale and the block's integers."""
    import oracle
    rng = np.random.default_rng(9)
    rows, cols = 40, 1536
    raw = W.random_blocks(rng, rows, cols, fmt)
    path = str(tmp_path / f"{fmt}.gguf")
    W.write(path, W.llama_kv(synth.TINY), [(name, ftype, [cols, rows], raw.tobytes())])
    g = C.q8l_gguf_open(path)
    try:
        assert C.q8l_gguf_tensor_file_type(g, 0) == ftype
        st, info = C.q8l_gguf_tensor_info(g, 0)
        assert st == C.Q8L_OK and info["dtype"] == C.Q8L_Q8_0
        assert info["nbytes"] == rows * cols // 32 * 34
        buf = np.empty(info["nbytes"], np.uint8)
        assert C.q8l_gguf_read_tensor(g, 0, buf, buf.size) == C.Q8L_OK
    finally:
        C.q8l_gguf_close(g)
    # the reader's blocks equal the test's own conversion byte for byte ...
    assert np.array_equal(buf.reshape(rows, -1), W.to_q8_0(raw, rows, cols, fmt))
    # ... and decode to the oracle's values of the original format exactly
    ref = oracle.dequant_q5_0(raw, rows, cols) if fmt == "q5_0" else oracle.dequant_q4_0(raw, rows, cols)
    assert np.array_equal(oracle.dequant_q8_0(buf, rows, cols), ref)


@pytest.mark.parametrize("role", ["attn_q", "attn_k", "attn_v", "attn_output", "ffn_gate", "ffn_up",
                                  "ffn_down"])
def test_q5_0_projections_read_as_they_are(lib, tmp_path, role):
    """Rows of 2048 weights and more: the 22-byte blocks as they are."""
    rng = np.random.default_rng(13)
    rows, cols = 24, 2048
    raw = W.random_blocks(rng, rows, cols, "q5_0")
    other = W.random_blocks(rng, 3, 64, "q5_0")          # 44-byte rows: a tensor not 16-byte sized
    name = f"blk.2.{role}.weight"
    path = str(tmp_path / "q5.gguf")
    W.write(path, W.llama_kv(synth.TINY), [("blk.1.attn_q.weight", W.TYPE_Q5_0, [64, 3], other.tobytes()),
                                           (name, W.TYPE_Q5_0, [cols, rows], raw.tobytes())])
    g = C.q8l_gguf_open(path)
    try:
        idx = C.q8l_gguf_find_tensor(g, name)
        st, info = C.q8l_gguf_tensor_info(g, idx)
        assert st == C.Q8L_OK and info["dtype"] == C.Q8L_Q5_0
        assert info["nbytes"] == rows * cols // 32 * 22 and (info["rows"], info["cols"]) == (rows, cols)
        buf = np.empty(info["nbytes"], np.uint8)
        assert C.q8l_gguf_read_tensor(g, idx, buf, buf.size) == C.Q8L_OK
        assert np.array_equal(buf, raw.reshape(-1))
    finally:
        C.q8l_gguf_close(g)


@pytest.mark.parametrize("cols", [576, 1536, 2016])
def test_q5_0_projections_of_short_rows_read_as_exact_q8_0(lib, tmp_path, cols):
    """Rows under 2048 weights (the wave-per-row decode kernels' lengths) are
    read as Q8_0: the same values, each block's scale and integer."""
    import oracle
    rng = np.random.default_rng(cols)
    rows = 5
    raw = W.random_blocks(rng, rows, cols, "q5_0")
    name = "blk.0.ffn_up.weight"
    path = str(tmp_path / "q5s.gguf")
    W.write(path, W.llama_kv(synth.TINY), [(name, W.TYPE_Q5_0, [cols, rows], raw.tobytes())])
    g = C.q8l_gguf_open(path)
    try:
        idx = C.q8l_gguf_find_tensor(g, name)
        st, info = C.q8l_gguf_tensor_info(g, idx)
        assert st == C.Q8L_OK and info["dtype"] == C.Q8L_Q8_0 and info["nbytes"] == rows * cols // 32 * 34
        buf = np.empty(info["nbytes"], np.uint8)
        assert C.q8l_gguf_read_tensor(g, idx, buf, buf.size) == C.Q8L_OK
        assert np.array_equal(oracle.dequant_q8_0(buf, rows, cols), oracle.dequant_q5_0(raw, rows, cols))
    finally:
        C.q8l_gguf_close(g)


@pytest.mark.parametrize("fmt,ftype,size", [("q4_k", W.TYPE_Q4_K, 144), ("q6_k", W.TYPE_Q6_K, 210)])
def test_k_format_tensors_read_as_they_are(lib, tmp_path, fmt, ftype, size):
    rng = np.random.default_rng(12)
    rows, cols = 24, 1536                                 # an odd row count of 210-byte blocks too
    raw = synth.draw_k_quant(rng, rows, cols, fmt)
    other = synth.draw_k_quant(rng, 3, 512, fmt)
    path = str(tmp_path / f"{fmt}.gguf")
    W.write(path, W.llama_kv(synth.TINY), [("blk.0.ffn_down.weight", ftype, [cols, rows], raw.tobytes()),
                                           ("blk.1.ffn_down.weight", ftype, [512, 3], other.tobytes())])
    g = C.q8l_gguf_open(path)
    try:
        for idx, (arr, r, c) in enumerate(((raw, rows, cols), (other, 3, 512))):
            assert C.q8l_gguf_tensor_file_type(g, idx) == ftype
            st, info = C.q8l_gguf_tensor_info(g, idx)
            want = C.Q8L_Q4_K if fmt == "q4_k" else C.Q8L_Q6_K
            assert st == C.Q8L_OK and info["dtype"] == want
            assert (info["rows"], info["cols"], info["nbytes"]) == (r, c, r * c // 256 * size)
            buf = np.empty(info["nbytes"], np.uint8)
            assert C.q8l_gguf_read_tensor(g, idx, buf, buf.size) == C.Q8L_OK
            assert np.array_equal(buf, arr.reshape(-1))
    finally:
        C.q8l_gguf_close(g)


def test_k_format_rows_must_hold_whole_blocks(lib, tmp_path):
    path = str(tmp_path / "ragged.gguf")
    W.write(path, W.llama_kv(synth.TINY), [("blk.0.ffn_down.weight", W.TYPE_Q4_K, [576, 2], bytes(576 * 2 // 256 * 144))])
    with pytest.raises(C.Q8LError) as e:
        C.q8l_gguf_open(path)
    assert e.value.status == C.Q8L_E_FORMAT
