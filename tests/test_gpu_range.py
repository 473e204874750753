"""Prefill activations far from 1 in magnitude, against the oracle.

The matrix-core prefill holds activations as f16 pairs (hi + lo, 22 bits).
The normalised rows are scaled per token by a power of two, and the gate/up
output per token and 32-wide block when a value would reach 2^15, so those
pairs keep their bits at any magnitude; q, k, v and the attention output are
range-checked, an out-of-range prefill being reported by the next call.
"""

import numpy as np
import pytest

import oracle
import synth
from helpers import assert_logits_close, compare_generation, gpu_model, log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


def scaled_norms(model, factor, which=("attn_norm", "ffn_norm"), layers=None):
    """A copy of the model with the given norm weights multiplied by `factor`."""
    L = model.shape.n_layer
    for l in (range(L) if layers is None else layers):
        for n in which:
            name = f"blk.{l}.{n}.weight"
            model = model.replace(name, (model[name].data * np.float32(factor)).astype(np.float32))
    return model


def scaled_q8_0(model, name, factor):
    """A copy with every f16 block scale of a Q8_0 tensor multiplied by `factor`
    (a power of two, so the scales stay exact)."""
    t = model[name]
    raw = t.data.copy().reshape(t.rows, -1, 34)
    d = (raw[:, :, 0:2].copy().view("<f2").astype(np.float32) * np.float32(factor)).astype("<f2")
    assert np.isfinite(d).all()
    raw[:, :, 0:2] = d.view(np.uint8)
    return model.replace(name, raw.reshape(t.data.shape))


def test_large_norm_weights_prefill_matches_oracle():
    """Norm weights x4096: the normalised rows reach ~1e5 (past the f16 range)
    and SiLU(gate)*up ~1e6; a 13-token prefill (matrix cores) and 3 decode
    steps against the oracle."""
    w, m, prompt = synth.workload_inputs("C1")
    m = scaled_norms(m, 4096.0)
    ids, err, ties = compare_generation(gpu_model(m), oracle.OracleModel(m), prompt, 3, "norms x4096")
    log(f"norms x4096: max abs err {err:.3g}, near ties {ties}")
    assert ties <= 1


def test_tiny_norm_weights_prefill_matches_oracle():
    """Norm weights x2^-20 in every other layer, that layer's q/k/v and
    gate/up block scales x2^20: normalised rows of ~1e-6 (whose f16 pairs
    would be subnormal or zero without the per-row scaling) feeding products
    of the usual size."""
    w, m, prompt = synth.workload_inputs("C1")
    layers = range(0, m.shape.n_layer, 2)
    m = scaled_norms(m, 2.0 ** -20, layers=layers)
    for l in layers:
        for t in ("attn_q", "attn_k", "attn_v", "ffn_gate", "ffn_up"):
            m = scaled_q8_0(m, f"blk.{l}.{t}.weight", 2.0 ** 20)
    prompt = synth.prompt_ids(m.shape.n_vocab, 40, 3)
    gm, om = gpu_model(m), oracle.OracleModel(m)
    ids, err, ties = compare_generation(gm, om, prompt, 3, "norms x2^-20")
    log(f"norms x2^-20: max abs err {err:.3g}, near ties {ties}")
    assert ties <= 1


def test_large_activations_prefill_equals_decode_chain():
    """With norm weights x4096 the prefill (f16 pairs on the matrix cores)
    gives the logits of the same tokens fed one at a time (f32 GEMVs)."""
    w, m, prompt = synth.workload_inputs("C1")
    m = scaled_norms(m, 4096.0)
    gm = gpu_model(m)
    toks = synth.prompt_ids(m.shape.n_vocab, 64, 5)
    full, _ = gm.forward(toks, 0)
    for i, t in enumerate(toks):
        step, _ = gm.forward([t], i)
    assert_logits_close(full, step, "norms x4096: prefill 64 vs 64 single-token steps")


def test_out_of_range_qkv_is_reported_by_the_next_call():
    """q/k/v of ~1e6 cannot be split into f16 pairs: the prefill still runs,
    the next call returns Q8L_E_RANGE once and changes nothing, and the model
    works after it."""
    from quantized_q8_gemv_amd import q8l as C
    w, m, prompt = synth.workload_inputs("C1")
    m = scaled_q8_0(scaled_norms(m, 4096.0, which=("attn_norm",), layers=[1]), "blk.1.attn_k.weight", 1024.0)
    gm = gpu_model(m)
    assert gm.forward_async(prompt, 0) == C.Q8L_OK
    torch.cuda.synchronize()
    assert gm.cache_len == 13
    st = gm.forward_async([5], 13)
    assert st == C.Q8L_E_RANGE, C.q8l_last_error(gm.handle)
    assert gm.cache_len == 13
    log("out-of-range report: " + C.q8l_last_error(gm.handle))
    # decode (f32 throughout) is unaffected, and the report is not repeated
    assert gm.forward_async([5], 13) == C.Q8L_OK
    torch.cuda.synchronize()
    assert gm.cache_len == 14
