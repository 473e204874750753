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


@pytest.mark.parametrize("neox,plen", [(False, 13), (False, 4), (True, 13), (True, 4)])
def test_out_of_range_qkv_is_reported_by_the_next_call(neox, plen):
    """q/k/v of ~1e6 cannot be split into f16 pairs: the prefill still runs,
    the next call returns Q8L_E_RANGE once and changes nothing, and the model
    works after it. Prompts of 13 (matrix-core q/k/v, range checked in its
    epilogue) and 4 tokens (the multi-token GEMV's epilogue); with NEOX rope
    the rotation kernel checks q and k."""
    from quantized_q8_gemv_amd import q8l as C
    if neox:
        s = synth.ModelShape("tiny-neox", n_layer=4, n_embd=576, n_head=9, n_head_kv=3, head_dim=64,
                             n_ff=1536, n_vocab=4096, rope_neox=True)
        m = synth.random_model(s, 0)
    else:
        w, m, _ = synth.workload_inputs("C1")
    prompt = synth.prompt_ids(m.shape.n_vocab, plen, 1)
    m = scaled_q8_0(scaled_norms(m, 4096.0, which=("attn_norm",), layers=[1]), "blk.1.attn_k.weight", 1024.0)
    gm = gpu_model(m)
    assert gm.forward_async(prompt, 0) == C.Q8L_OK
    torch.cuda.synchronize()
    assert gm.cache_len == plen
    st = gm.forward_async([5], plen)
    assert st == C.Q8L_E_RANGE, C.q8l_last_error(gm.handle)
    assert gm.cache_len == plen
    log(f"out-of-range report (neox={neox}, {plen} tokens): " + C.q8l_last_error(gm.handle))
    # decode (f32 throughout) is unaffected, and the report is not repeated
    assert gm.forward_async([5], plen) == C.Q8L_OK
    torch.cuda.synchronize()
    assert gm.cache_len == plen + 1


def scaled_q8_0_rows(model, name, rows, factor):
    """A copy where the f16 block scales of the given rows of a Q8_0 tensor
    are multiplied by `factor` (a power of two)."""
    t = model[name]
    raw = t.data.copy().reshape(t.rows, -1, 34)
    for r in rows:
        d = (raw[r, :, 0:2].copy().view("<f2").astype(np.float32) * np.float32(factor)).astype("<f2")
        assert np.isfinite(d).all()
        raw[r, :, 0:2] = d.view(np.uint8)
    return model.replace(name, raw.reshape(t.data.shape))


def test_cache_written_by_decode_is_checked_before_a_prefill_reads_it():
    """A decode step writes its key in f32, unchecked; a later prefill that
    appends to the cache reads that key as an f16 pair, so the positions
    decode steps wrote are range-checked first. One token's embedding is
    replaced by the direction that maximises layer 0's first key row, and
    that rope pair of rows is scaled by a power of two so that this token's
    rotated key at position 13 passes 2^15 while every other token's stays
    below 2^14: decoding it and then prefilling 3 more tokens makes the next
    call return Q8L_E_RANGE. The same calls with an ordinary token in its
    place all return Q8L_OK."""
    from quantized_q8_gemv_amd import q8l as C
    w, m, _ = synth.workload_inputs("C1")
    sh = m.shape
    H, V = sh.n_embd, sh.n_vocab
    Wk = oracle.dequant_q8_0(m["blk.0.attn_k.weight"].data, sh.kv_dim, H)
    nw = m["blk.0.attn_norm.weight"].data.astype(np.float64)
    star = 7
    v = (Wk[0] * nw).reshape(-1, 32)
    d = (np.abs(v).max(axis=1) / 127.0).astype(np.float16)
    q = np.clip(np.round(v / d.astype(np.float64)[:, None]), -127, 127).astype(np.int8)
    emb = m["token_embd.weight"].data.copy()
    emb[star] = synth.pack_q8_0(d[None, :], q.reshape(1, H))[0]
    m = m.replace("token_embd.weight", emb)
    # layer-0 keys of every token (before rope): rmsnorm(embedding) * attn_norm times W_k
    E = oracle.dequant_q8_0(m["token_embd.weight"].data, V, H)
    u = E / np.sqrt((E * E).mean(axis=1, keepdims=True) + sh.rms_eps) * nw
    K = u @ Wk[:2].T
    pair = np.sqrt(K[:, 0] ** 2 + K[:, 1] ** 2)          # rope keeps the pair's norm
    others = np.delete(np.arange(V), star)
    e = int(np.floor(np.log2(2.0 ** 14 / pair[others].max())))
    th = 13.0   # position 13, pair 0: angle 13 * theta^0
    rot = max(abs(K[star, 0] * np.cos(th) - K[star, 1] * np.sin(th)),
              abs(K[star, 0] * np.sin(th) + K[star, 1] * np.cos(th)))
    assert rot * 2.0 ** e >= 1.1 * 2.0 ** 15, "the chosen token's key does not stand out"
    m = scaled_q8_0_rows(m, "blk.0.attn_k.weight", [0, 1], 2.0 ** e)
    prompt = [t for t in synth.prompt_ids(V, 16, 3) if t != star][:13]
    gm = gpu_model(m)

    def run(tok):
        sts = [gm.forward_async(prompt, 0)]                # (index 0 drops the cache)
        sts.append(gm.forward_async([tok], 13))            # decode: writes tok's key unchecked
        sts.append(gm.forward_async([prompt[0]], 14))      # decode: reads it in f32
        sts.append(gm.forward_async(prompt[1:4], 15))      # prefill: reads it as an f16 pair
        torch.cuda.synchronize()
        sts.append(gm.forward_async([prompt[5]], 18))
        torch.cuda.synchronize()
        return sts

    assert run(prompt[6]) == [C.Q8L_OK] * 5
    sts = run(star)
    log(f"decode-written key, rows x2^{e}: statuses {sts}")
    assert sts[:4] == [C.Q8L_OK] * 4 and sts[4] == C.Q8L_E_RANGE
