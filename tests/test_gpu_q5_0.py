"""Q5_0 matrices on the GPU against the oracle.

The pages' 4-bit file of the 135M model stores most of its 576-wide
projections as Q5_0 ("速度", section "CPU GGUF"); the library binds them as
they are (22 bytes per 32 weights) for every projection of a layer. Covered
here: the single-op entry at the 135M projection shapes for 1 to 203 tokens
(the wave GEMV, the multi-token GEMV and the MFMA GEMM), ragged rows, the
chunk-outer GEMV of long rows (K = 11008, 14336, 17152) and 7B-sized matrices
on sampled rows; whole models whose layers mix Q5_0 and Q8_0 per matrix at
the 135M widths (prompts through the GEMM, the small multi-token path, and a
cache past one attention split) and at the 7B-class widths; the captured
decode graphs; and GGUF files in the pages' 4-bit mix at both widths, every
block format read as it is.

Op tolerance: |gpu - oracle| <= 1e-4 * sqrt(K) * rms(w_row) * rms(x_t), as for
the K formats (f32 accumulation and the f16 hi + lo activation split stay
near 1e-6 of the output's typical size; a wrong bit, nibble or scale is of
order one).
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


def _run_op(N, K, T, accumulate, seed, sample_rows=None):
    from quantized_q8_gemv_amd import q8l as C
    rng = np.random.default_rng(seed)
    raw = synth.draw_q5_0(rng, N, K)
    X = rng.standard_normal((T, K)).astype(np.float32)
    Y0 = rng.standard_normal((T, N)).astype(np.float32)
    dev = torch.device("cuda:0")
    Wd = torch.from_numpy(raw.reshape(-1)).to(dev)
    Xd = torch.from_numpy(X).to(dev)
    Yd = torch.from_numpy(Y0).to(dev)
    log(f"q5_0 op N={N} K={K} T={T} acc={accumulate}")
    assert C.q8l_op_matmul_q5_0(Wd, N, K, Xd, T, accumulate, Yd) == C.Q8L_OK
    torch.cuda.synchronize()
    Y = Yd.cpu().numpy().astype(np.float64)
    rows = np.arange(N) if sample_rows is None else np.sort(rng.choice(N, sample_rows, replace=False))
    sub = raw[rows]
    ref = oracle.matmul_fmt(sub, "q5_0", len(rows), K, X.astype(np.float64))      # [T, rows]
    if accumulate:
        ref = ref + Y0[:, rows]
    w = oracle.dequant_q5_0(sub, len(rows), K)
    scale = np.sqrt(K) * np.sqrt((w ** 2).mean(axis=1))[None, :] * \
        np.sqrt((X.astype(np.float64) ** 2).mean(axis=1))[:, None]
    err = np.abs(Y[:, rows] - ref)
    bound = 1e-4 * scale + (1e-6 * np.abs(Y0[:, rows]) if accumulate else 0.0)
    assert np.isfinite(Y).all()
    bad = err > bound
    assert not bad.any(), f"N={N} K={K} T={T}: {int(bad.sum())} outputs off, worst {float((err / scale).max()):.3g}"
    return float((err / scale).max())


@pytest.mark.parametrize("N,K", [(576, 576), (1536, 576), (576, 1536)])
@pytest.mark.parametrize("T", [1, 2, 7, 16, 17, 203])
def test_projection_shapes_of_the_135m_model(N, K, T):
    rel = _run_op(N, K, T, 1, seed=N + K + T)
    log(f"  worst error / scale {rel:.3g}")


@pytest.mark.parametrize("N,K,T,acc", [(100, 512, 1, 1), (100, 512, 33, 0), (64, 11008, 1, 0),
                                       (64, 11008, 6, 1), (64, 14336, 1, 1), (40, 17152, 1, 1),
                                       (1, 64, 1, 0), (1, 64, 5, 1), (3, 64, 40, 0), (257, 128, 1, 1)])
def test_ragged_and_chunked_shapes(N, K, T, acc):
    _run_op(N, K, T, acc, seed=N + K + T)


@pytest.mark.parametrize("N,K,T", [(4096, 4096, 1), (4096, 4096, 64), (14336, 4096, 1), (4096, 14336, 1),
                                   (4096, 14336, 24)])
def test_7b_sized_matrices_sampled_rows(N, K, T):
    """All rows computed, 96 sampled rows checked against the oracle."""
    _run_op(N, K, T, 1, seed=N // 64 + K // 64 + T, sample_rows=96)


# Per-layer formats of q, k, v, o, gate, up, down. Layer 1 keeps v and down
# in Q8_0 (as the pages' 4-bit file keeps some v projections), layer 2 its q
# and o (its attention and o-projection then run as one kernel), layer 3 its
# gate / up pair.
MIX = [["q5_0"] * 7,
       ["q5_0", "q5_0", "q8_0", "q5_0", "q5_0", "q5_0", "q8_0"],
       ["q8_0", "q5_0", "q5_0", "q8_0", "q5_0", "q5_0", "q5_0"],
       ["q5_0", "q8_0", "q8_0", "q5_0", "q8_0", "q8_0", "q5_0"]]


@pytest.fixture(scope="module")
def mixed():
    w, m, _ = synth.workload_inputs("C1")
    return synth.with_layer_formats(m, MIX, seed=11)


@pytest.mark.parametrize("plen", [13, 4, 70])
def test_135m_width_model_with_q5_0_layers_matches_the_oracle(mixed, plen):
    """13 tokens run the MFMA GEMM, 4 the multi-token GEMV, 70 put the cache
    past one attention split (decode merges splits before the o-projection);
    greedy decode steps follow."""
    m = mixed
    assert sum(t.dtype == "q5_0" for t in m.tensors) == sum(f == "q5_0" for r in MIX for f in r)
    prompt = synth.prompt_ids(m.shape.n_vocab, plen, 3)
    ids, err, ties = compare_generation(gpu_model(m), oracle.OracleModel(m), prompt, 8, f"q5_0 mix {plen}+8")
    log(f"q5_0 mix {plen}+8: max abs err {err:.3g}, near ties {ties}")
    assert ties <= 1


def test_all_q5_0_neox_model_matches_the_oracle():
    s = synth.ModelShape("tiny-neox", n_layer=2, n_embd=576, n_head=9, n_head_kv=3, head_dim=64,
                         n_ff=1536, n_vocab=4096, rope_neox=True)
    m = synth.with_layer_formats(synth.random_model(s, 4), [["q5_0"] * 7] * 2, seed=12)
    prompt = synth.prompt_ids(s.n_vocab, 21, 5)
    ids, err, ties = compare_generation(gpu_model(m), oracle.OracleModel(m), prompt, 6, "q5_0 neox 21+6")
    log(f"q5_0 neox 21+6: max abs err {err:.3g}")
    assert ties <= 1


def test_generate_with_q5_0_layers_equals_stepwise_forward(mixed):
    """The captured decode graphs (on-device greedy loop) give the same ids
    as step-by-step forward calls."""
    from quantized_q8_gemv_amd import q8l as C
    m = mixed
    prompt = synth.prompt_ids(m.shape.n_vocab, 9, 6)
    a = gpu_model(m)
    _, tok = a.forward(prompt, 0)
    want = []
    for k in range(12):
        _, tok = a.forward([tok], len(prompt) + k)
        want.append(tok)
    b = gpu_model(m)
    _, first = b.forward(prompt, 0)
    dev = torch.device("cuda:0")
    tok_dev = torch.tensor([first], dtype=torch.int32, device=dev)
    ids_dev = torch.zeros(12, dtype=torch.int32, device=dev)
    assert b.generate_async(tok_dev, len(prompt), 12, ids_dev) == C.Q8L_OK
    torch.cuda.synchronize()
    assert ids_dev.cpu().tolist() == want


def test_7b_width_q5_0_model_two_layers():
    """hidden 4096, 32/8 heads, head_dim 128, FFN 14336 (the down rows take
    the chunk-outer GEMV), vocab 32000 untied; every projection Q5_0 in layer
    0, a mix in layer 1."""
    s = synth.ModelShape("7b-width-2layer", n_layer=2, n_embd=4096, n_head=32, n_head_kv=8,
                         head_dim=128, n_ff=14336, n_vocab=32000, tied_output=False)
    m = synth.with_layer_formats(synth.random_model(s, 6), [["q5_0"] * 7, MIX[2]], seed=13)
    prompt = synth.prompt_ids(s.n_vocab, 40, 7)
    gm = gpu_model(m)
    ids, err, ties = compare_generation(gm, oracle.OracleModel(m), prompt, 4, "7b-width q5_0 40+4")
    log(f"7b-width q5_0: max abs err {err:.3g}")
    assert ties <= 1
    # the 40-token prefill (MFMA path) equals the same tokens fed one by one (GEMV path)
    full, _ = gm.forward(prompt, 0)
    for i, t in enumerate(prompt):
        step, _ = gm.forward([t], i)
    assert_logits_close(step, full, "7b-width q5_0: prefill 40 vs 40 single-token steps")


def _q4_k_m_layer(l):
    """The pages' 4-bit file of the 135M model, per layer ("速度", section
    "CPU GGUF"): q, k, o, gate and up in Q5_0, v in Q5_0 in every other layer
    (Q8_0 otherwise), down in Q4_K and Q6_K in alternate layers."""
    return ["q5_0", "q5_0", "q5_0" if l % 2 else "q8_0", "q5_0", "q5_0", "q5_0", "q4_k" if l % 2 == 0 else "q6_k"]


@pytest.mark.parametrize("width", ["135m", "7b"])
def test_gguf_in_the_pages_4bit_mix_read_natively(tmp_path, width):
    """A GGUF file in the pages' 4-bit mix read by Q8Model.from_gguf: K
    formats streamed as they are, Q5_0 as it is in rows of 2048 weights and
    more (the 7B-class widths) and as the same values in Q8_0 in shorter ones
    (the 135M widths), against the oracle on the same blocks. At the 135M
    widths (4 layers) and the 7B-class ones (2 layers, hidden 4096, FFN 14336,
    untied vocab 32000)."""
    import gguf_writer as W
    from quantized_q8_gemv_amd import q8l as C
    from quantized_q8_gemv_amd.model import Q8Model
    if width == "135m":
        s, plen = synth.TINY, 13
    else:
        s = synth.ModelShape("7b-width-2layer", n_layer=2, n_embd=4096, n_head=32, n_head_kv=8,
                             head_dim=128, n_ff=14336, n_vocab=32000, tied_output=False)
        plen = 24
    m = synth.random_model_formats(s, 21, [_q4_k_m_layer(l) for l in range(s.n_layer)])
    path = str(tmp_path / f"q4_k_m-{width}.gguf")
    W.write(path, W.llama_kv(s), W.model_tensors(m))
    g = C.q8l_gguf_open(path)
    try:
        for t in m.tensors:
            st, info = C.q8l_gguf_tensor_info(g, C.q8l_gguf_find_tensor(g, t.name))
            q5 = C.Q8L_Q5_0 if t.cols >= 2048 else C.Q8L_Q8_0
            want = {"q8_0": C.Q8L_Q8_0, "q5_0": q5, "q4_k": C.Q8L_Q4_K, "q6_k": C.Q8L_Q6_K,
                    "f32": C.Q8L_F32}[t.dtype]
            nbytes = t.rows * t.cols // 32 * 34 if (t.dtype == "q5_0" and q5 == C.Q8L_Q8_0) else t.nbytes
            assert st == C.Q8L_OK and info["dtype"] == want and info["nbytes"] == nbytes, t.name
    finally:
        C.q8l_gguf_close(g)
    prompt = synth.prompt_ids(s.n_vocab, plen, 8)
    ids, err, ties = compare_generation(Q8Model.from_gguf(path), oracle.OracleModel(m), prompt, 6,
                                        f"gguf 4-bit mix {width} {plen}+6")
    log(f"gguf 4-bit mix {width}: max abs err {err:.3g}")
    assert ties <= 1
