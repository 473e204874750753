"""Pins of the CPU oracle to values and facts it does not compute itself.

Each test checks the oracle against something fixed outside it: numbers the
pages print (tests/golden/), closed forms, invariants of the forward pass that
follow from the pages' description, library routines for special cases, or a
brute-force NumPy implementation built the way the pages describe candle's
non-fused attention branch.
"""

import math

import numpy as np
import pytest

import oracle
import synth
from oracle.np_reference import NumpyLlama, build_causal_mask, repeat_kv


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


# ---------------------------------------------------------------- sizes / layout

def test_model_bytes_match_printed_file(golden_printed):
    """Tensor bytes of the 135M shape = file size - data offset (Q8_0 = 34 B per 32)."""
    g = golden_printed
    s = synth.SMOL135M
    specs = s.tensor_specs()
    assert len(specs) == g["gguf_tensor_count"] == 30 * 9 + 2
    assert s.total_bytes() == g["gguf_file_bytes"] - g["gguf_data_offset"]
    q8 = sum(s.tensor_nbytes(d, r, c) for _, d, r, c in specs if d == "q8_0")
    assert round(q8 / 2**20, 1) == g["q8_0_weight_mib"]
    params = sum(r * c for _, _, r, c in specs)
    assert int(params * 4 / 2**20) == g["f32_weight_mib"]
    assert "output.weight" not in {n for n, *_ in specs}


def test_generator_draws_the_stated_distributions():
    m = synth.random_model(synth.micro_shape(n_vocab=512, n_embd=256), 0, keep_parts=True)
    t = m["token_embd.weight"]
    assert t.q.min() >= -127 and t.q.max() <= 127
    s = t.scales.astype(np.float64)
    assert (s >= 0).all()
    assert 0.25 < (s < 2.0**-14).mean() < 0.35     # f16 subnormal share
    w = m["blk.0.attn_norm.weight"].data
    assert w.dtype == np.float32 and abs(w.mean() - 1.0) < 0.05


def test_f16_decode_matches_library_for_every_bit_pattern():
    bits = np.arange(65536, dtype=np.uint32)
    ref = bits.astype(np.uint16).view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(b)) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))
    assert np.isnan(got[np.isnan(ref)]).all()
    assert oracle.f16_to_f64(0x0001) == 2.0**-24
    assert oracle.f16_to_f64(0x7BFF) == 65504.0


def test_dequant_hand_block():
    blk = np.zeros(34, dtype=np.uint8)
    blk[0:2] = [0x00, 0x3C]                                   # f16 1.0
    blk[2:] = np.arange(-16, 16, dtype=np.int8).view(np.uint8)
    assert np.array_equal(oracle.dequant_q8_0(blk, 1, 32)[0], np.arange(-16, 16))
    blk[0:2] = [0x01, 0x00]                                   # smallest subnormal
    blk[2:] = 127
    assert np.all(oracle.dequant_q8_0(blk, 1, 32)[0] == 127 * 2.0**-24)
    blk[0:2] = 0                                              # d = 0
    assert np.all(oracle.dequant_q8_0(blk, 1, 32)[0] == 0)


def test_dequant_agrees_with_drawn_parts():
    rng = np.random.default_rng(5)
    scales, q = synth.draw_q8_0(rng, 7, 96)
    raw = synth.pack_q8_0(scales, q)
    ref = np.repeat(scales.astype(np.float64), 32, axis=1) * q
    assert np.array_equal(oracle.dequant_q8_0(raw, 7, 96), ref)


# ---------------------------------------------------------------- GEMV

def test_matmul_single_nonzero_block():
    rows, cols = 5, 128
    raw = np.zeros((rows, cols // 32 * 34), dtype=np.uint8)
    r, b = 3, 2
    raw[r, b * 34:b * 34 + 2] = [0x00, 0x38]                  # f16 0.5
    qv = np.arange(1, 33, dtype=np.int8)
    raw[r, b * 34 + 2:b * 34 + 34] = qv.view(np.uint8)
    x = np.linspace(-1, 1, cols)
    y = oracle.matmul_q8(raw, rows, cols, x)[0]
    expect = np.zeros(rows)
    expect[r] = 0.5 * np.dot(qv.astype(np.float64), x[32 * b:32 * b + 32])
    assert np.allclose(y, expect, rtol=1e-15, atol=0)
    assert np.count_nonzero(y) == 1


def test_matmul_matches_library_matmul():
    rng = np.random.default_rng(11)
    scales, q = synth.draw_q8_0(rng, 33, 192)
    raw = synth.pack_q8_0(scales, q)
    X = rng.standard_normal((4, 192))
    W = np.repeat(scales.astype(np.float64), 32, axis=1) * q
    got = oracle.matmul_q8(raw, 33, 192, X)
    assert np.allclose(got, X @ W.T, rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------- norm / rope / silu / attention

def test_rmsnorm_constant_input_closed_form():
    H, eps, c = 64, 1e-5, 0.37
    w = np.random.default_rng(2).normal(1, 0.1, H).astype(np.float32)
    y = oracle.rmsnorm(np.full(H, c), w, eps)
    assert np.allclose(y, c / math.sqrt(c * c + eps) * w.astype(np.float64), rtol=1e-14)


def test_rope_pairs_adjacent_dims_and_rotates_counterclockwise():
    hd, theta = 64, 10000.0
    for p in (0, 1, 7, 100):
        e0 = np.zeros(hd); e0[0] = 1.0
        r = oracle.rope_i(e0, p, theta)
        assert r[0] == pytest.approx(math.cos(p), abs=1e-15)
        assert r[1] == pytest.approx(math.sin(p), abs=1e-15)
        assert np.all(r[2:] == 0)
        e2 = np.zeros(hd); e2[2] = 1.0                       # pair j = 1
        r = oracle.rope_i(e2, p, theta)
        ang = float(np.float32(p) * np.float32(theta ** (-2.0 / hd)))
        assert r[2] == pytest.approx(math.cos(ang), abs=1e-15)
        assert r[3] == pytest.approx(math.sin(ang), abs=1e-15)
        assert np.count_nonzero(r) <= 2


def test_rope_angle_table_first_column_is_the_position():
    for p in (0, 1, 33, 4095):
        assert oracle.rope_angle(p, 0, 64, 10000.0) == float(p)


def test_rope_identity_at_zero_and_norm_preserving():
    v = np.random.default_rng(3).standard_normal(64)
    assert np.array_equal(oracle.rope_i(v, 0, 1e4), v)
    r = oracle.rope_i(v, 1234, 1e4)
    assert np.allclose(np.hypot(r[0::2], r[1::2]), np.hypot(v[0::2], v[1::2]), rtol=1e-14)


def test_rope_scores_depend_on_relative_position_only():
    rng = np.random.default_rng(4)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    base = oracle.rope_i(q, 9, 1e4) @ oracle.rope_i(k, 4, 1e4)
    for shift in (1, 3, 20):
        s = oracle.rope_i(q, 9 + shift, 1e4) @ oracle.rope_i(k, 4 + shift, 1e4)
        assert s == pytest.approx(base, rel=1e-5)


# NEOX pairing ("量化 llama 的一次前向", section "RoPE：两种约定，按架构名选": dimension
# j is paired with j + hd/2; the angles are the same table's).

def test_rope_neox_pairs_half_apart():
    hd, theta = 64, 10000.0
    for p in (0, 1, 7, 100):
        for j in (0, 1, 31):
            e = np.zeros(hd); e[j] = 1.0
            r = oracle.rope_neox(e, p, theta)
            ang = float(np.float32(p) * np.float32(theta ** (-2.0 * j / hd)))
            assert r[j] == pytest.approx(math.cos(ang), abs=1e-15)
            assert r[j + hd // 2] == pytest.approx(math.sin(ang), abs=1e-15)
            assert np.count_nonzero(r) <= 2


def test_rope_neox_is_interleaved_rope_under_the_half_permutation():
    # Placing dimension j at 2j and j + hd/2 at 2j + 1 turns the NEOX rotation
    # into the interleaved one: neox(v) = P^-1 rope_i(P v).
    hd = 64
    perm = np.empty(hd, dtype=np.int64)
    perm[0::2] = np.arange(hd // 2)
    perm[1::2] = np.arange(hd // 2) + hd // 2
    v = np.random.default_rng(11).standard_normal(hd)
    for p in (0, 5, 4095):
        inter = oracle.rope_i(v[perm], p, 1e4)
        back = np.empty(hd); back[perm] = inter
        assert np.allclose(oracle.rope_neox(v, p, 1e4), back, rtol=0, atol=1e-15)


def test_rope_neox_identity_norms_and_relative_position():
    rng = np.random.default_rng(12)
    v = rng.standard_normal(64)
    assert np.array_equal(oracle.rope_neox(v, 0, 1e4), v)
    r = oracle.rope_neox(v, 777, 1e4)
    assert np.allclose(np.hypot(r[:32], r[32:]), np.hypot(v[:32], v[32:]), rtol=1e-14)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    base = oracle.rope_neox(q, 9, 1e4) @ oracle.rope_neox(k, 4, 1e4)
    for shift in (1, 3, 20):
        s = oracle.rope_neox(q, 9 + shift, 1e4) @ oracle.rope_neox(k, 4 + shift, 1e4)
        assert s == pytest.approx(base, rel=1e-5)


def test_rope_convention_changes_the_forward():
    a = synth.micro_shape(name="i")
    b = synth.micro_shape(name="neox", rope_neox=True)
    ma, mb = synth.random_model(a, 5), synth.random_model(b, 5)
    toks = synth.prompt_ids(a.n_vocab, 6, 2)
    _, _, la = oracle.OracleModel(ma).forward(toks, 0)
    _, _, lb = oracle.OracleModel(mb).forward(toks, 0)
    assert not np.allclose(la, lb)
    # position 0 only: rope is the identity there, so one token agrees exactly
    _, _, la1 = oracle.OracleModel(ma).forward(toks[:1], 0)
    _, _, lb1 = oracle.OracleModel(mb).forward(toks[:1], 0)
    assert np.array_equal(la1, lb1)


def test_silu_identities():
    assert oracle.silu(0.0) == 0.0
    for z in (-3.0, -0.5, 0.25, 2.0):
        assert oracle.silu(z) - oracle.silu(-z) == pytest.approx(z, rel=1e-14)
    assert oracle.silu(40.0) == pytest.approx(40.0, rel=1e-15)


def test_attention_special_cases():
    rng = np.random.default_rng(6)
    hd = 16
    K, V = rng.standard_normal((5, hd)), rng.standard_normal((5, hd))
    q = rng.standard_normal(hd)
    assert np.allclose(oracle.attend(q, K[:1], V[:1]), V[0], rtol=1e-15)       # one key: o = v
    assert np.allclose(oracle.attend(np.zeros(hd), K, V), V.mean(axis=0), rtol=1e-14)
    assert np.allclose(oracle.attend(q, K, V, last_visible=0), V[0], rtol=1e-15)
    perm = rng.permutation(5)
    assert np.allclose(oracle.attend(q, K[perm], V[perm]), oracle.attend(q, K, V), rtol=1e-13)


def test_attention_two_keys_hand_values():
    hd = 4
    q = np.array([1.0, 0, 0, 0])
    K = np.array([[2.0, 0, 0, 0], [0, 0, 0, 0]])            # scores 2/sqrt(4) = 1 and 0
    V = np.array([[1.0, 0, 0, 0], [0, 1.0, 0, 0]])
    w0 = math.e / (math.e + 1.0)
    assert np.allclose(oracle.attend(q, K, V), [w0, 1 - w0, 0, 0], rtol=1e-15)


# ---------------------------------------------------------------- NumPy brute-force reference pins

def test_np_reference_mask_and_repeat_kv_match_printed_shapes(golden_printed):
    g = golden_printed
    m = build_causal_mask(5, 5)
    assert m.shape == g["misuse_mask_shape"]
    m = build_causal_mask(13, 33)
    assert m.shape == g["clear_mask_shape"]
    assert m[:, :33].sum() == 0 and np.array_equal(m[:, 33:], np.triu(np.ones((13, 13), np.uint8), 1))
    x = np.arange(3 * 2 * 1).reshape(3, 2, 1).astype(float)
    r = repeat_kv(x, 3)
    assert r.shape == (9, 2, 1)
    assert [int(r[h, 0, 0]) for h in range(9)] == [0, 0, 0, 2, 2, 2, 4, 4, 4]


def test_np_reference_fails_like_the_pages_on_misuse(golden_printed):
    g = golden_printed
    s = synth.micro_shape(n_head=9, n_head_kv=3, head_dim=32, n_embd=64)
    n = NumpyLlama(synth.random_model(s, 0))
    toks = synth.prompt_ids(s.n_vocab, 13, 1)
    n.forward(toks[:8], 0)
    with pytest.raises(ValueError) as e:
        n.forward(toks[8:], 5)
    assert str(list(g["misuse_mask_shape"])) in str(e.value)
    assert str(list(g["misuse_scores_shape"])) in str(e.value)


# ---------------------------------------------------------------- whole forward

MICRO_SHAPES = [
    synth.micro_shape(),
    synth.micro_shape(n_head=4, n_head_kv=1, name="mqa"),
    synth.micro_shape(n_head=4, n_head_kv=4, name="mha"),
    synth.micro_shape(n_layer=1, n_embd=96, n_head=6, n_head_kv=3, head_dim=16, n_ff=96,
                      n_vocab=37, tied_output=False, name="odd-untied"),
    synth.micro_shape(name="neox", rope_neox=True),
    synth.micro_shape(n_head=4, n_head_kv=1, name="mqa-neox", rope_neox=True),
]


@pytest.mark.parametrize("shape", MICRO_SHAPES, ids=lambda s: s.name)
def test_brute_force_numpy_agrees(shape):
    m = synth.random_model(shape, 3)
    o, n = oracle.OracleModel(m), NumpyLlama(m)
    toks = synth.prompt_ids(shape.n_vocab, 12, 7)
    # prefill 8, chunked prefill 3 at p=8, then decode steps
    for chunk, p in ((toks[:8], 0), (toks[8:11], 8), (toks[11:12], 11), ([5], 12), ([1], 13)):
        st, _, lg64 = o.forward(chunk, p)
        assert st == oracle.OK
        ref = n.forward(chunk, p)
        assert np.allclose(lg64, ref, rtol=1e-11, atol=1e-13)
    # decode misuse (T = 1, stale counter) follows candle: not an error
    st, _, lg64 = o.forward([2], 3)
    assert st == oracle.OK
    assert np.allclose(lg64, n.forward([2], 3), rtol=1e-11, atol=1e-13)


def test_brute_force_tiny_config():
    w, m, prompt = synth.workload_inputs("C1")
    o, n = oracle.OracleModel(m), NumpyLlama(m)
    st, _, lg64 = o.forward(prompt, 0)
    assert np.allclose(lg64, n.forward(prompt, 0), rtol=1e-11, atol=1e-13)
    for k in range(3):
        tok = int(np.argmax(lg64))
        st, _, lg64 = o.forward([tok], len(prompt) + k)
        assert np.allclose(lg64, n.forward([tok], len(prompt) + k), rtol=1e-11, atol=1e-13)


@pytest.fixture(scope="module")
def micro():
    s = synth.micro_shape(n_layer=2, n_head=4, n_head_kv=2, max_seq_len=64)
    return s, synth.random_model(s, 1)


def test_prefill_equals_token_by_token_decode(micro):
    """T == 1 needs no mask: feeding tokens one at a time = one causal prefill."""
    s, m = micro
    toks = synth.prompt_ids(s.n_vocab, 10, 2)
    a = oracle.OracleModel(m)
    _, _, full = a.forward(toks, 0)
    b = oracle.OracleModel(m)
    for i, t in enumerate(toks):
        _, _, step = b.forward([t], i)
    assert np.allclose(full, step, rtol=1e-12, atol=1e-14)


def test_chunked_prefill_equals_single(micro):
    s, m = micro
    toks = synth.prompt_ids(s.n_vocab, 13, 3)
    a = oracle.OracleModel(m)
    _, _, one = a.forward(toks, 0)
    b = oracle.OracleModel(m)
    assert b.forward(toks[:8], 0)[0] == oracle.OK
    st, _, two = b.forward(toks[8:], 8)
    assert st == oracle.OK and np.allclose(one, two, rtol=1e-12, atol=1e-14)
    c = oracle.OracleModel(m)
    c.forward(toks[:8], 0)
    assert c.forward(toks[8:], 5)[0] == oracle.E_POS_MISMATCH
    assert c.cache_len == 8                       # nothing changed


def test_index_pos_zero_drops_cache_exactly(micro):
    s, m = micro
    p1, p2 = synth.prompt_ids(s.n_vocab, 9, 4), synth.prompt_ids(s.n_vocab, 7, 5)
    fresh = oracle.OracleModel(m)
    _, ref, _ = fresh.forward(p2, 0)
    a = oracle.OracleModel(m)
    a.forward(p1, 0)
    a.forward([3], 9)
    _, got, _ = a.forward(p2, 0)
    assert np.array_equal(got, ref)
    assert a.cache_len == 7


def test_clear_then_stale_counter(micro):
    s, m = micro
    p1 = synth.prompt_ids(s.n_vocab, 9, 4)
    a = oracle.OracleModel(m)
    a.forward(p1, 0)
    a.clear_kv_cache()
    assert a.cache_len == 0
    assert a.forward(p1, 9)[0] == oracle.E_POS_MISMATCH      # T > 1 with a stale counter
    assert a.cache_len == 0
    # one token after a clear sees only itself: q and k share the rotation
    _, at_p, _ = a.forward([7], 9)
    b = oracle.OracleModel(m)
    _, at_0, _ = b.forward([7], 0)
    assert np.allclose(at_p, at_0, rtol=1e-12, atol=1e-14)


def test_index_pos_zero_every_step_sees_one_token(micro):
    s, m = micro
    a = oracle.OracleModel(m)
    a.forward(synth.prompt_ids(s.n_vocab, 5, 6), 0)
    for t in (4, 9, 2):
        _, got, _ = a.forward([t], 0)
        _, ref, _ = oracle.OracleModel(m).forward([t], 0)
        assert np.array_equal(got, ref)


def test_position_bounds(golden_printed):
    s = synth.micro_shape(max_seq_len=golden_printed["rope_table_rows"])
    m = synth.random_model(s, 2)
    a = oracle.OracleModel(m)
    assert a.forward([1], golden_printed["rope_error_index_pos"])[0] == oracle.E_POS_RANGE
    assert a.forward([1], s.max_seq_len - 1)[0] == oracle.OK
    assert a.forward([1, 2], s.max_seq_len - 1)[0] == oracle.E_POS_RANGE


def test_error_codes_and_kv_full():
    s = synth.micro_shape(max_seq_len=16)
    m = synth.random_model(s, 2)
    a = oracle.OracleModel(m)
    assert a.forward([], 0)[0] == oracle.E_INVALID_ARG
    assert a.forward([s.n_vocab], 0)[0] == oracle.E_INVALID_ARG
    assert a.forward([1], -1)[0] == oracle.E_INVALID_ARG
    assert a.forward(list(range(16)), 0)[0] == oracle.OK
    assert a.cache_len == 16
    assert a.forward([1], 3)[0] == oracle.E_KV_FULL          # T == 1 misuse into a full cache
    assert a.cache_len == 16


def test_call_counts_match_printed_spans(golden_printed):
    g = golden_printed
    s = synth.micro_shape(n_layer=30)
    a = oracle.OracleModel(synth.random_model(s, 0))
    for toks, p in ((synth.prompt_ids(s.n_vocab, 13, 1), 0), ([3], 13)):
        a.forward(toks, p)
        assert a.counts() == (g["qmatmul_calls"], g["rms_norm_calls"], g["rope_calls"])


def test_only_last_position_logits(micro):
    s, m = micro
    _, lg, _ = oracle.OracleModel(m).forward(synth.prompt_ids(s.n_vocab, 13, 1), 0)
    assert lg.shape == (s.n_vocab,)


def test_untied_with_copied_embedding_equals_tied():
    s_t = synth.micro_shape(tied_output=True)
    s_u = synth.micro_shape(tied_output=False)
    mt = synth.random_model(s_t, 8)
    mu = synth.random_model(s_u, 8)
    mu = mu.replace("output.weight", mt["token_embd.weight"].data.copy())
    for name in (t.name for t in mt.tensors):
        mu = mu.replace(name, mt[name].data)
    toks = synth.prompt_ids(s_t.n_vocab, 6, 1)
    _, a, _ = oracle.OracleModel(mt).forward(toks, 0)
    _, b, _ = oracle.OracleModel(mu).forward(toks, 0)
    assert np.array_equal(a, b)


def test_zero_gate_or_down_removes_the_mlp(micro):
    s, m = micro
    toks = synth.prompt_ids(s.n_vocab, 6, 1)
    outs = []
    for which in ("ffn_gate", "ffn_up", "ffn_down"):
        mm = m
        for l in range(s.n_layer):
            name = f"blk.{l}.{which}.weight"
            raw = mm[name].data.copy().reshape(-1, 34)
            raw[:, 0:2] = 0                                    # every block scale = 0
            mm = mm.replace(name, raw.reshape(mm[name].data.shape))
        outs.append(oracle.OracleModel(mm).forward(toks, 0)[1])
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])
    assert not np.array_equal(outs[0], oracle.OracleModel(m).forward(toks, 0)[1])


def test_argmax_lowest_index_on_ties():
    assert oracle.argmax(np.array([1.0, 3.0, 3.0, 2.0], np.float32)) == 1
    assert oracle.argmax(np.array([5.0], np.float32)) == 0


# ---------------------------------------------------------------- other block formats

def test_q4_k_m_table_pins_the_block_sizes(golden_printed):
    """The pages' Q4_K_M file of the 135M model ("速度", section "CPU GGUF"): 166
    Q5_0 tensors hold 51.2 MiB, 16 Q4K 7.6, 14 Q6K 9.7, 15 Q8_0 30.3, 61 F32 0.1.
    With 22 bytes per 32 weights (Q5_0), 144 and 210 per 256 (Q4K, Q6K) and the
    reading that rows of 576 (not a multiple of 256) fall back to Q5_0 or Q8_0:
    q, k, o, gate, up and 16 of the v projections in Q5_0; token_embd and the
    other 14 v in Q8_0; ffn_down (rows of 1536) in Q4K (16) and Q6K (14)."""
    s = synth.SMOL135M
    H, F, KV = s.n_embd, s.n_ff, s.kv_dim
    b = lambda rows, cols, per, size: rows * cols // per * size
    q5 = 30 * (b(s.q_dim, H, 32, 22) + b(KV, H, 32, 22) + b(H, s.q_dim, 32, 22) + 2 * b(F, H, 32, 22)) \
        + 16 * b(KV, H, 32, 22)
    q8 = b(s.n_vocab, H, 32, 34) + 14 * b(KV, H, 32, 34)
    q4k, q6k = 16 * b(H, F, 256, 144), 14 * b(H, F, 256, 210)
    f32 = 61 * H * 4
    mib = lambda x: round(x / 2 ** 20, 1)
    assert (166, mib(q5)) == golden_printed["q4km_q5_0"]
    assert (15, mib(q8)) == golden_printed["q4km_q8_0"]
    assert (16, mib(q4k)) == golden_printed["q4km_q4k"]
    assert (14, mib(q6k)) == golden_printed["q4km_q6k"]
    assert (61, mib(f32)) == golden_printed["q4km_f32"]
    # and 30 x 9 + 2 = 272 tensors in all
    assert 166 + 15 + 16 + 14 + 61 == golden_printed["gguf_tensor_count"]


def test_q4_0_and_q5_0_hand_blocks():
    d = np.float16(0.5).view(np.uint16)
    # Q4_0: byte i = (high << 4) | low; weights i and i + 16
    qs = np.array([(15 << 4) | 0] + [(8 << 4) | 9] * 15, dtype=np.uint8)
    blk = np.concatenate([np.array([d & 0xff, d >> 8], dtype=np.uint8), qs])
    w = oracle.dequant_q4_0(blk, 1, 32)[0]
    assert w[0] == 0.5 * -8 and w[16] == 0.5 * 7
    assert np.all(w[1:16] == 0.5) and np.all(w[17:] == 0.0)
    # Q5_0: fifth bits for weights 0 and 17 only
    qh = (1 << 0) | (1 << 17)
    qs = np.zeros(16, dtype=np.uint8)
    qs[1] = (3 << 4) | 2
    blk = np.concatenate([np.array([d & 0xff, d >> 8], dtype=np.uint8),
                          np.frombuffer(np.uint32(qh).tobytes(), dtype=np.uint8), qs])
    w = oracle.dequant_q5_0(blk, 1, 32)[0]
    assert w[0] == 0.5 * (16 - 16) and w[16] == 0.5 * -16
    assert w[1] == 0.5 * (2 - 16) and w[17] == 0.5 * (3 + 16 - 16)
    assert np.all(w[2:16] == 0.5 * -16) and np.all(w[18:] == 0.5 * -16)


def test_q4_0_and_q5_0_values_are_q8_0_values():
    """Both formats hold d * (small integer) per 32-weight block: the same
    values as a Q8_0 block with the same d and int8 = the integer (the basis
    of loading them on the Q8_0 path)."""
    rng = np.random.default_rng(21)
    rows, cols = 3, 128
    d = synth.draw_q8_0(rng, rows, cols)[0]           # f16 scales [rows, cols/32]
    q5 = rng.integers(0, 256, (rows, cols // 32, 20), dtype=np.uint8)
    raw5 = np.concatenate([d.view(np.uint8).reshape(rows, cols // 32, 2), q5], axis=2).reshape(rows, -1)
    w5 = oracle.dequant_q5_0(raw5, rows, cols)
    ints = np.rint(w5 / np.repeat(d.astype(np.float64), 32, axis=1), where=np.repeat(d != 0, 32, axis=1),
                   out=np.zeros_like(w5))
    assert ints.min() >= -16 and ints.max() <= 15
    q8 = synth.pack_q8_0(d, ints.astype(np.int8))
    nz = np.repeat(d != 0, 32, axis=1)
    assert np.array_equal(oracle.dequant_q8_0(q8, rows, cols)[nz], w5[nz])


# ---- 256-weight "K" formats. The pages fix only their block sizes (the
# Q4_K_M table above); the bit layouts follow the public GGUF block
# definitions. Blocks are built here by packing chosen integers (the inverse
# of decoding, written separately), and the K formats are tied to the Q8_0
# decoding (pinned by the pages' printed values) where their values coincide.

def _f16_bytes(v: float) -> list:
    b = int(np.float16(v).view(np.uint16))
    return [b & 0xFF, b >> 8]


def _pack_q4_k(d: float, dmin: float, s, m, q) -> np.ndarray:
    """One Q4_K block from 8 scales, 8 mins (0..63) and 256 values (0..15):
    scale/min j < 4 in the low 6 bits of bytes j / j + 4; j >= 4 split into
    low nibbles in byte j + 4 (scale low, min high) and top two bits in the
    top of bytes j - 4 (scale) and j (min). Values of sub-blocks 2c and 2c+1
    share bytes 32c..32c+31 (low / high nibble)."""
    sc = [0] * 12
    for j in range(4):
        sc[j] = (s[j] & 63) | ((s[j + 4] >> 4) << 6)
        sc[j + 4] = (m[j] & 63) | ((m[j + 4] >> 4) << 6)
        sc[j + 8] = (s[j + 4] & 15) | ((m[j + 4] & 15) << 4)
    qs = [0] * 128
    for c in range(4):
        for l in range(32):
            qs[32 * c + l] = q[64 * c + l] | (q[64 * c + 32 + l] << 4)
    return np.array(_f16_bytes(d) + _f16_bytes(dmin) + sc + qs, dtype=np.uint8)


def _pack_q6_k(d: float, sc, q) -> np.ndarray:
    """One Q6_K block from 16 int8 scales and 256 values (0..63, stored +32):
    in half h, value 32k + l keeps its low 4 bits in byte 64h + l + 32(k odd)
    (low nibble for k < 2, high for k >= 2) and its top 2 bits at bit 2k of
    byte 128 + 32h + l."""
    ql = [0] * 128
    qh = [0] * 64
    for h in range(2):
        for k in range(4):
            for l in range(32):
                v = q[128 * h + 32 * k + l]
                i = 64 * h + l + 32 * (k & 1)
                ql[i] |= (v & 15) << (4 * (k >= 2))
                qh[32 * h + l] |= (v >> 4) << (2 * k)
    scb = [int(np.int8(x).view(np.uint8)) for x in sc]
    return np.array(ql + qh + scb + _f16_bytes(d), dtype=np.uint8)


def test_q4_k_hand_block():
    s = [1, 2, 3, 4, 17, 33, 49, 63]          # >= 16 uses the split top bits
    m = [0, 1, 2, 63, 20, 40, 60, 5]
    q = [(7 * i + 3) % 16 for i in range(256)]
    d, dmin = 0.25, 0.125
    blk = _pack_q4_k(d, dmin, s, m, q)
    assert blk.size == 144
    w = oracle.dequant_q4_k(blk, 1, 256)[0]
    want = np.array([d * s[i // 32] * q[i] - dmin * m[i // 32] for i in range(256)])
    assert np.array_equal(w, want)


def test_q6_k_hand_block():
    sc = [1, -2, 3, -4, 5, 127, -128, 8, 9, -10, 11, 12, -13, 14, 15, 100]
    q = [(11 * i + 5) % 64 for i in range(256)]
    d = 0.5
    blk = _pack_q6_k(d, sc, q)
    assert blk.size == 210
    w = oracle.dequant_q6_k(blk, 1, 256)[0]
    want = np.array([d * sc[i // 16] * (q[i] - 32) for i in range(256)])
    assert np.array_equal(w, want)


def test_k_formats_equal_q8_0_where_values_coincide():
    """Q4_K with dmin = 0 holds (d * s_j) * q per 32 weights, Q6_K with equal
    scales in each 32 holds (d * sc) * (q - 32): Q8_0 blocks with those f16
    scales and int8 values hold the same numbers (d = 2^-10, so d * s is an
    exact f16)."""
    rng = np.random.default_rng(31)
    rows, cols = 3, 512
    nb = cols // 256
    q4 = [[], [], []]
    q8_scales = np.zeros((rows, cols // 32), np.float16)
    q8_vals = np.zeros((rows, cols), np.int8)
    q6 = [[], [], []]
    q8b_scales = np.zeros((rows, cols // 32), np.float16)
    q8b_vals = np.zeros((rows, cols), np.int8)
    d = 2.0 ** -10
    for r in range(rows):
        for b in range(nb):
            s = rng.integers(0, 64, 8)
            q = rng.integers(0, 16, 256)
            q4[r].append(_pack_q4_k(d, 0.0, s.tolist(), [int(x) for x in rng.integers(0, 64, 8)], q.tolist()))
            q8_scales[r, 8 * b:8 * b + 8] = (d * s).astype(np.float16)
            q8_vals[r, 256 * b:256 * b + 256] = q
            s6 = np.repeat(rng.integers(-128, 128, 8), 2)
            v6 = rng.integers(0, 64, 256)
            q6[r].append(_pack_q6_k(d, s6.tolist(), v6.tolist()))
            q8b_scales[r, 8 * b:8 * b + 8] = (d * s6[::2]).astype(np.float16)
            q8b_vals[r, 256 * b:256 * b + 256] = v6 - 32
    raw4 = np.stack([np.concatenate(x) for x in q4])
    raw6 = np.stack([np.concatenate(x) for x in q6])
    ref4 = oracle.dequant_q8_0(synth.pack_q8_0(q8_scales, q8_vals), rows, cols)
    ref6 = oracle.dequant_q8_0(synth.pack_q8_0(q8b_scales, q8b_vals), rows, cols)
    assert np.array_equal(oracle.dequant_q4_k(raw4, rows, cols), ref4)
    assert np.array_equal(oracle.dequant_q6_k(raw6, rows, cols), ref6)
    # and the matrix products through the per-format entry
    x = rng.standard_normal((2, cols))
    assert np.array_equal(oracle.matmul_fmt(raw4, "q4_k", rows, cols, x),
                          oracle.matmul_fmt(synth.pack_q8_0(q8_scales, q8_vals), "q8_0", rows, cols, x))
    np.testing.assert_allclose(oracle.matmul_fmt(raw6, "q6_k", rows, cols, x), (ref6 @ x.T).T,
                               rtol=1e-13, atol=1e-15)


def test_k_quant_model_matches_its_q8_0_twin():
    """A model whose o and down projections are K-quant matrices with
    Q8_0-representable values gives bitwise the logits of the same model with
    those matrices stored as Q8_0 (the per-layer format plumbing)."""
    shape = synth.micro_shape(n_layer=2, n_embd=64, n_head=4, n_head_kv=2, head_dim=64, n_ff=256)
    base = synth.random_model(shape, 3)
    rng = np.random.default_rng(5)
    d = 2.0 ** -12
    k_ts, q8_ts = {}, {}
    for l in range(shape.n_layer):
        for name, rows, cols, fmt in ((f"blk.{l}.attn_output.weight", shape.n_embd, shape.q_dim, "q6_k"),
                                      (f"blk.{l}.ffn_down.weight", shape.n_embd, shape.n_ff, "q4_k")):
            blocks, scales, vals = [], np.zeros((rows, cols // 32), np.float16), np.zeros((rows, cols), np.int8)
            for r in range(rows):
                row = []
                for b in range(cols // 256):
                    if fmt == "q4_k":
                        s, q = rng.integers(0, 64, 8), rng.integers(0, 16, 256)
                        row.append(_pack_q4_k(d, 0.0, s.tolist(), [0] * 8, q.tolist()))
                        scales[r, 8 * b:8 * b + 8], vals[r, 256 * b:256 * b + 256] = d * s, q
                    else:
                        s, v = np.repeat(rng.integers(-128, 128, 8), 2), rng.integers(0, 64, 256)
                        row.append(_pack_q6_k(d, s.tolist(), v.tolist()))
                        scales[r, 8 * b:8 * b + 8], vals[r, 256 * b:256 * b + 256] = d * s[::2], v - 32
                blocks.append(np.concatenate(row))
            k_ts[name] = synth.Tensor(name, fmt, rows, cols, np.stack(blocks))
            q8_ts[name] = synth.Tensor(name, "q8_0", rows, cols, synth.pack_q8_0(scales, vals))
    mk = synth.Model(shape, [k_ts.get(t.name, t) for t in base.tensors])
    mq = synth.Model(shape, [q8_ts.get(t.name, t) for t in base.tensors])
    toks = synth.prompt_ids(shape.n_vocab, 7, seed=2)
    a = oracle.OracleModel(mk).forward(toks, 0)[2]
    b = oracle.OracleModel(mq).forward(toks, 0)[2]
    assert np.array_equal(a, b)


def test_k_quant_oracle_rejects_rows_without_whole_blocks():
    shape = synth.micro_shape(n_ff=128)          # 128 is not a multiple of 256
    m = synth.random_model(shape, 0)
    ts = [synth.Tensor(t.name, "q4_k", t.rows, t.cols, np.zeros((t.rows, 72), np.uint8))
          if t.name == "blk.0.ffn_down.weight" else t for t in m.tensors]
    with pytest.raises(ValueError):
        oracle.OracleModel(synth.Model(shape, ts))


# ---- Q5_0 on every projection. The values are tied to Q8_0 as above: a
# Q5_0 block holds d * (integer in [-16, 15]), the same numbers as a Q8_0
# block with that d and those integers (unpacked here from the bit layout,
# independently of the oracle's decoder).

def _q5_0_integers(raw: np.ndarray, rows: int, cols: int):
    """f16 scales [rows, cols/32] and integers [rows, cols] of Q5_0 bytes."""
    blk = np.ascontiguousarray(raw, dtype=np.uint8).reshape(rows, cols // 32, 22)
    d = blk[:, :, 0:2].copy().view("<f2").reshape(rows, cols // 32)
    qh = blk[:, :, 2:6].copy().view("<u4").reshape(rows, cols // 32).astype(np.int64)
    qs = blk[:, :, 6:22].astype(np.int64)
    lo = (qs & 15) | (((qh[:, :, None] >> np.arange(16)) & 1) << 4)
    hi = (qs >> 4) | (((qh[:, :, None] >> (np.arange(16) + 16)) & 1) << 4)
    ints = np.concatenate([lo, hi], axis=2) - 16
    return d, ints.reshape(rows, cols).astype(np.int8)


def test_q5_0_matmul_equals_its_q8_0_twin():
    rng = np.random.default_rng(41)
    rows, cols = 5, 192
    raw = synth.draw_q5_0(rng, rows, cols)
    d, ints = _q5_0_integers(raw, rows, cols)
    assert ints.min() == -16 and ints.max() == 15
    twin = synth.pack_q8_0(d, ints)
    x = rng.standard_normal((3, cols))
    assert np.array_equal(oracle.dequant_q5_0(raw, rows, cols), oracle.dequant_q8_0(twin, rows, cols))
    assert np.array_equal(oracle.matmul_fmt(raw, "q5_0", rows, cols, x),
                          oracle.matmul_fmt(twin, "q8_0", rows, cols, x))


@pytest.mark.parametrize("pattern", ["all_q5_0", "mixed"])
def test_q5_0_model_matches_its_q8_0_twin(pattern):
    """Every projection of a layer may be Q5_0: the logits equal bitwise those
    of the model with the same matrices stored as Q8_0 (each matrix's format
    reaches that matrix: a mixed pattern differs per layer and per role)."""
    shape = synth.micro_shape(n_layer=2, n_embd=64, n_head=4, n_head_kv=2, head_dim=16, n_ff=128)
    base = synth.random_model(shape, 3)
    if pattern == "all_q5_0":
        fmts = [["q5_0"] * 7 for _ in range(shape.n_layer)]
    else:
        fmts = [["q5_0", "q8_0", "q5_0", "q8_0", "q5_0", "q5_0", "q8_0"],
                ["q8_0", "q5_0", "q8_0", "q5_0", "q8_0", "q8_0", "q5_0"]]
    m5 = synth.with_layer_formats(base, fmts, seed=9)
    twins = []
    for t in m5.tensors:
        if t.dtype == "q5_0":
            d, ints = _q5_0_integers(t.data, t.rows, t.cols)
            twins.append(synth.Tensor(t.name, "q8_0", t.rows, t.cols, synth.pack_q8_0(d, ints)))
        else:
            twins.append(t)
    mq = synth.Model(shape, twins)
    assert sum(t.dtype == "q5_0" for t in m5.tensors) == sum(f == "q5_0" for r in fmts for f in r)
    toks = synth.prompt_ids(shape.n_vocab, 6, seed=2)
    a = oracle.OracleModel(m5).forward(toks, 0)[2]
    b = oracle.OracleModel(mq).forward(toks, 0)[2]
    assert np.array_equal(a, b)
    # and the Q5_0 matrices matter: the base model's logits differ
    assert not np.array_equal(a, oracle.OracleModel(base).forward(toks, 0)[2])


def test_k_formats_only_for_o_and_down():
    shape = synth.micro_shape(n_embd=256, n_ff=256)
    m = synth.random_model(shape, 0)
    bad = synth.with_formats(m, {"blk.0.attn_q.weight": "q4_k"})
    with pytest.raises(ValueError):
        oracle.OracleModel(bad)
