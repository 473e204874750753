"""A model built from a GGUF file (Q8Model.from_gguf over the C ABI reader)
runs the same forward as the same tensors bound directly, and matches the
oracle; the architecture key selects the rope pairing end to end."""

import numpy as np
import pytest

import gguf_writer as W
import oracle
import synth
from helpers import compare_generation, gpu_model, log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _write(tmp_path, m, arch="llama", drop=()):
    path = str(tmp_path / f"{m.shape.name}-{arch}.gguf")
    tensors = [t for t in W.model_tensors(m) if t[0] not in drop]
    W.write(path, W.llama_kv(m.shape, arch), tensors)
    return path


def test_gguf_model_equals_direct_binding(tmp_path):
    from quantized_q8_gemv_amd.model import Q8Model
    w, m, prompt = synth.workload_inputs("C1")
    path = _write(tmp_path, m)
    log(f"gguf tiny: {path}")
    a, b = Q8Model.from_gguf(path), gpu_model(m)
    la, ia = a.forward(prompt, 0)
    lb, ib = b.forward(prompt, 0)
    assert np.array_equal(la, lb) and ia == ib
    tok = ia
    for k in range(5):
        la, ia = a.forward([tok], len(prompt) + k)
        lb, ib = b.forward([tok], len(prompt) + k)
        assert np.array_equal(la, lb) and ia == ib
        tok = ia
    ids, err, ties = compare_generation(Q8Model.from_gguf(path), oracle.OracleModel(m), prompt, 8, "gguf tiny 13+8")
    assert ties <= 1


def test_gguf_neox_architecture_runs_the_neox_forward(tmp_path):
    from quantized_q8_gemv_amd.model import Q8Model
    s = synth.ModelShape("tiny-neox", n_layer=4, n_embd=576, n_head=9, n_head_kv=3, head_dim=64,
                         n_ff=1536, n_vocab=4096, rope_neox=True)
    m = synth.random_model(s, 0)
    path = _write(tmp_path, m, arch="qwen2")
    gm = Q8Model.from_gguf(path)
    assert gm.cfg.rope_type == 1
    prompt = synth.prompt_ids(s.n_vocab, 13, 1)
    ids, err, ties = compare_generation(gm, oracle.OracleModel(m), prompt, 6, "gguf qwen2-arch neox 13+6")
    log(f"gguf neox: max abs err {err:.3g}")
    assert ties <= 1


def test_gguf_missing_tensor_is_named(tmp_path):
    from quantized_q8_gemv_amd import q8l as C
    from quantized_q8_gemv_amd.model import Q8Model
    w, m, prompt = synth.workload_inputs("C1")
    path = _write(tmp_path, m, drop=("blk.2.attn_v.weight",))
    with pytest.raises(C.Q8LError) as e:
        Q8Model.from_gguf(path)
    assert e.value.status == C.Q8L_E_MISSING_TENSOR
    assert "cannot find blk.2.attn_v.weight" in str(e.value)


def test_gguf_mixed_block_formats_match_the_oracle(tmp_path):
    """A file in the mix the pages' Q4_K_M file shows for rows of 576 (Q5_0
    projections, some v in Q8_0) plus Q4_0 down projections: read as exact
    Q8_0 and compared with the oracle on the test's own conversion."""
    from quantized_q8_gemv_amd.model import Q8Model
    w, m, prompt = synth.workload_inputs("C1")
    s = m.shape
    rng = np.random.default_rng(17)
    file_tensors, oracle_model = [], m
    for name, ftype, dims, data in W.model_tensors(m):
        kind = name.split(".")[-2] if name.startswith("blk.") else ""
        layer = int(name.split(".")[1]) if name.startswith("blk.") else -1
        fmt = None
        if kind in ("attn_q", "attn_k", "attn_output", "ffn_gate", "ffn_up") or (kind == "attn_v" and layer % 2):
            fmt = "q5_0"
        elif kind == "ffn_down":
            fmt = "q4_0"
        if fmt is None:
            file_tensors.append((name, ftype, dims, data))
            continue
        cols, rows = dims
        raw = W.random_blocks(rng, rows, cols, fmt)
        file_tensors.append((name, W.TYPE_Q5_0 if fmt == "q5_0" else W.TYPE_Q4_0, dims, raw.tobytes()))
        oracle_model = oracle_model.replace(name, W.to_q8_0(raw, rows, cols, fmt))
    path = str(tmp_path / "mixed.gguf")
    W.write(path, W.llama_kv(s), file_tensors)
    ids, err, ties = compare_generation(Q8Model.from_gguf(path), oracle.OracleModel(oracle_model), prompt, 8,
                                        "gguf mixed q5_0/q4_0/q8_0 13+8")
    log(f"gguf mixed formats: max abs err {err:.3g}")
    assert ties <= 1
