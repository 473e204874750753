"""Host-side checks of libq8l.so that need no GPU: it loads, exports every
function include/q8l.h declares, and rejects bad configs, bindings and
positions before touching the device."""

import ctypes

import pytest

import synth
from quantized_q8_gemv_amd import q8l as C


def test_library_exports_every_declared_function():
    lib = C.lib()
    names = C.header_functions()
    assert len(names) >= 16
    for n in names:
        assert hasattr(lib, n), n
    assert "gfx950" in C.q8l_version()


def cfg_of(shape):
    return C.config_from(synth.shape_fields(shape))


def test_workspace_bytes_cover_the_kv_arena():
    s = synth.SMOL135M
    ws = C.q8l_workspace_bytes(cfg_of(s))
    kv = s.n_layer * 2 * s.n_head_kv * s.max_seq_len * s.head_dim * 4
    assert kv == 188_743_680
    assert ws > kv
    assert C.q8l_workspace_bytes(cfg_of(synth.BIG_GQA)) > 32 * 2 * 8 * 4096 * 128 * 4


@pytest.mark.parametrize("field,value", [("n_head_kv", 2), ("head_dim", 6), ("n_embd", 96),
                                         ("n_layer", 0), ("head_dim", 256), ("rope_theta", 0.0),
                                         ("rope_type", 2), ("rope_type", -1)])
def test_invalid_configs_rejected(field, value):
    f = synth.shape_fields(synth.TINY)
    f[field] = value
    cfg = C.config_from(f)
    assert C.q8l_workspace_bytes(cfg) == 0
    with pytest.raises(C.Q8LError):
        C.q8l_create(cfg)


FAKE = 1 << 20  # a 16-byte aligned address; never dereferenced by these checks


@pytest.fixture
def tiny_handle():
    h = C.q8l_create(cfg_of(synth.TINY))
    yield h
    C.q8l_destroy(h)


def test_bind_checks(tiny_handle):
    h = tiny_handle
    s = synth.TINY
    nb = s.n_vocab * s.n_embd // 32 * 34
    assert C.q8l_bind_tensor(h, "token_embd.weight", C.Q8L_Q8_0, s.n_vocab, s.n_embd, FAKE, nb) == C.Q8L_OK
    assert C.q8l_bind_tensor(h, "token_embd.weight", C.Q8L_Q8_0, s.n_vocab, s.n_embd, FAKE, nb + 1) == C.Q8L_E_SHAPE
    assert C.q8l_bind_tensor(h, "token_embd.weight", C.Q8L_F32, s.n_vocab, s.n_embd, FAKE, nb) == C.Q8L_E_SHAPE
    assert C.q8l_bind_tensor(h, "blk.0.attn_q.weight", C.Q8L_Q8_0, 576, 576, FAKE + 4, 576 * 18 * 34) == C.Q8L_E_INVALID_ARG
    assert C.q8l_bind_tensor(h, "blk.4.attn_q.weight", C.Q8L_Q8_0, 576, 576, FAKE, 576 * 18 * 34) == C.Q8L_E_INVALID_ARG
    assert C.q8l_bind_tensor(h, "blk.0.attn_qq.weight", C.Q8L_Q8_0, 576, 576, FAKE, 576 * 18 * 34) == C.Q8L_E_INVALID_ARG
    assert C.q8l_bind_tensor(h, "output.weight", C.Q8L_Q8_0, s.n_vocab, s.n_embd, FAKE, nb) == C.Q8L_E_INVALID_ARG
    assert C.q8l_bind_tensor(h, "blk.3.ffn_down.weight", C.Q8L_Q8_0, 576, 1536, FAKE, 576 * 48 * 34) == C.Q8L_OK
    assert C.q8l_bind_tensor(h, "blk.3.ffn_norm.weight", C.Q8L_F32, 1, 576, FAKE, 576 * 4) == C.Q8L_OK


def test_bind_accepts_k_formats_only_for_o_and_down(tiny_handle):
    """Q4_K / Q6_K bind for ffn_down (1536 = 6 blocks of 256 per row) with the
    block sizes 144 / 210; not for other roles, nor for attn_output at the
    135M shape (576 is not a multiple of 256)."""
    h = tiny_handle
    q4, q6 = 576 * 6 * 144, 576 * 6 * 210
    assert C.q8l_bind_tensor(h, "blk.1.ffn_down.weight", C.Q8L_Q4_K, 576, 1536, FAKE, q4) == C.Q8L_OK
    assert C.q8l_bind_tensor(h, "blk.2.ffn_down.weight", C.Q8L_Q6_K, 576, 1536, FAKE, q6) == C.Q8L_OK
    assert C.q8l_bind_tensor(h, "blk.2.ffn_down.weight", C.Q8L_Q6_K, 576, 1536, FAKE, q4) == C.Q8L_E_SHAPE
    assert C.q8l_bind_tensor(h, "blk.2.ffn_down.weight", C.Q8L_Q4_K, 576, 1536, FAKE, q6) == C.Q8L_E_SHAPE
    assert "497664 bytes" in C.q8l_last_error(h)
    assert C.q8l_bind_tensor(h, "blk.2.ffn_down.weight", C.Q8L_F32, 576, 1536, FAKE, q6) == C.Q8L_E_SHAPE
    assert "Q8_0, Q5_0, Q4_K or Q6_K" in C.q8l_last_error(h)
    assert C.q8l_bind_tensor(h, "blk.0.ffn_gate.weight", C.Q8L_Q4_K, 1536, 576, FAKE, 1536 * 576 // 256 * 144) \
        == C.Q8L_E_SHAPE
    assert C.q8l_bind_tensor(h, "blk.0.attn_output.weight", C.Q8L_Q4_K, 576, 576, FAKE, 576 * 576 // 256 * 144) \
        == C.Q8L_E_SHAPE
    assert C.q8l_bind_tensor(h, "blk.0.attn_norm.weight", C.Q8L_Q6_K, 1, 576, FAKE, 576 * 4) == C.Q8L_E_SHAPE


def test_k_format_op_rejects_bad_arguments_before_device_work():
    X, Y = FAKE, FAKE
    ok = dict(W=FAKE, dtype=C.Q8L_Q4_K, N=576, K=1536, X=X, T=1, accumulate=0, Y=Y)
    for bad in (dict(dtype=C.Q8L_Q8_0), dict(dtype=7), dict(K=1535), dict(K=128), dict(N=0), dict(T=0),
                dict(W=FAKE + 4), dict(X=FAKE + 8), dict(W=None), dict(Y=None)):
        a = {**ok, **bad}
        assert C.q8l_op_matmul_kq(a["W"], a["dtype"], a["N"], a["K"], a["X"], a["T"], a["accumulate"],
                                  a["Y"], stream=0) == C.Q8L_E_INVALID_ARG, bad


def test_bind_accepts_q5_0_for_every_projection(tiny_handle):
    """Q5_0 (22 bytes per 32 weights) binds for the seven projections of a
    layer, not for the embedding, the norms or the output matrix."""
    h = tiny_handle
    s = synth.TINY
    q5 = lambda r, c: r * c // 32 * 22
    for role, r, c in (("attn_q", s.q_dim, 576), ("attn_k", s.kv_dim, 576), ("attn_v", s.kv_dim, 576),
                       ("attn_output", 576, s.q_dim), ("ffn_gate", 1536, 576), ("ffn_up", 1536, 576),
                       ("ffn_down", 576, 1536)):
        assert C.q8l_bind_tensor(h, f"blk.1.{role}.weight", C.Q8L_Q5_0, r, c, FAKE, q5(r, c)) == C.Q8L_OK, role
    assert C.q8l_bind_tensor(h, "blk.1.ffn_down.weight", C.Q8L_Q5_0, 576, 1536, FAKE, q5(576, 1536) + 22) \
        == C.Q8L_E_SHAPE
    assert "expected Q5_0 [576, 1536] (608256 bytes)" in C.q8l_last_error(h)
    assert C.q8l_bind_tensor(h, "token_embd.weight", C.Q8L_Q5_0, s.n_vocab, 576, FAKE, q5(s.n_vocab, 576)) \
        == C.Q8L_E_SHAPE
    assert C.q8l_bind_tensor(h, "blk.0.attn_norm.weight", C.Q8L_Q5_0, 1, 576, FAKE, 576 * 4) == C.Q8L_E_SHAPE


def test_q5_0_op_rejects_bad_arguments_before_device_work():
    ok = dict(W=FAKE, N=576, K=576, X=FAKE, T=1, accumulate=0, Y=FAKE)
    for bad in (dict(K=96), dict(K=0), dict(N=0), dict(T=0), dict(T=(1 << 20) + 1), dict(W=FAKE + 4),
                dict(X=FAKE + 8), dict(W=None), dict(X=None), dict(Y=None)):
        a = {**ok, **bad}
        assert C.q8l_op_matmul_q5_0(a["W"], a["N"], a["K"], a["X"], a["T"], a["accumulate"], a["Y"],
                                    stream=0) == C.Q8L_E_INVALID_ARG, bad


def test_finalize_names_the_first_missing_tensor(tiny_handle):
    h = tiny_handle
    s = synth.TINY
    for name, dt, r, c in s.tensor_specs():
        if name == "blk.2.ffn_up.weight":
            continue
        nbytes = s.tensor_nbytes(dt, r, c)
        st = C.q8l_bind_tensor(h, name, C.Q8L_Q8_0 if dt == "q8_0" else C.Q8L_F32, r, c, FAKE, nbytes)
        assert st == C.Q8L_OK, (name, C.q8l_last_error(h))
    assert C.q8l_finalize(h, 0) == C.Q8L_E_MISSING_TENSOR
    assert "cannot find blk.2.ffn_up.weight" in C.q8l_last_error(h)


def test_tensor_count_required_at_the_135m_shape(golden_printed):
    assert len(synth.SMOL135M.tensor_specs()) == golden_printed["gguf_tensor_count"]


def test_forward_argument_and_position_checks_precede_device_work(tiny_handle):
    h = tiny_handle
    s = synth.TINY
    toks = (ctypes.c_uint32 * 13)(*range(13))
    bad = (ctypes.c_uint32 * 1)(s.n_vocab)
    lib = C.lib()
    fwd = lambda t, n, p: lib.q8l_forward(h, ctypes.cast(t, ctypes.c_void_p), n, p, FAKE, None, None)
    assert fwd(toks, 0, 0) == C.Q8L_E_INVALID_ARG
    assert fwd(bad, 1, 0) == C.Q8L_E_INVALID_ARG
    assert fwd(toks, 1, -1) == C.Q8L_E_INVALID_ARG
    assert fwd(toks, 1, s.max_seq_len) == C.Q8L_E_POS_RANGE
    assert fwd(toks, 2, s.max_seq_len - 1) == C.Q8L_E_POS_RANGE
    assert fwd(toks, 5, 5) == C.Q8L_E_POS_MISMATCH      # nothing cached yet
    assert C.q8l_cache_len(h) == 0
    assert fwd(toks, 13, 0) == C.Q8L_E_NOT_FINALIZED
    assert C.q8l_cache_len(h) == 0
    assert C.q8l_clear_kv_cache(h) == C.Q8L_OK


def test_rope_types_accepted():
    for rt in (C.Q8L_ROPE_NORM, C.Q8L_ROPE_NEOX):
        f = synth.shape_fields(synth.TINY)
        f["rope_type"] = rt
        assert C.q8l_workspace_bytes(C.config_from(f)) > 0


def test_attention_op_rejects_misaligned_operands():
    ok = [FAKE, FAKE, FAKE]
    for i in range(3):
        ptrs = list(ok)
        ptrs[i] = FAKE + 4
        assert C.q8l_op_attention(ptrs[0], ptrs[1], ptrs[2], 1, 16, 16, 4, 2, 64, FAKE, FAKE, 1 << 20,
                                  stream=0) == C.Q8L_E_INVALID_ARG
