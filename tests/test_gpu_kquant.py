"""Q4_K / Q6_K matrices on the GPU against the oracle.

The pages' 4-bit file stores the 1536-wide down projections of the 135M model
as Q4K and Q6K ("速度", section "CPU GGUF") and times the product on that
shape, [203, 1536] x [1536, 576] and [1, 1536] x [1536, 576]. Covered here:
the single-op entry (one token: the GEMV; several: the MFMA GEMM) at that
shape, at ragged and misaligned shapes (an odd number of 210-byte blocks per
row starts every other row 2-byte aligned) and with two activation chunks;
whole models whose o and down projections mix Q8_0, Q4_K and Q6_K; and a
GGUF file in the pages' Q4_K_M mix read by Q8Model.from_gguf.

Op tolerance: |gpu - oracle| <= 1e-4 * sqrt(K) * rms(w_row) * rms(x_t), a
ten-thousandth of the output's typical size (f32 accumulation and the f16
hi + lo activation split stay near 1e-6 of it; a wrong index or scale is of
order one).
"""

import numpy as np
import pytest

import gguf_writer as W
import oracle
import synth
from helpers import compare_generation, gpu_model, log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _dequant(raw, fmt, rows, cols):
    return oracle.dequant_q4_k(raw, rows, cols) if fmt == "q4_k" else oracle.dequant_q6_k(raw, rows, cols)


def _run_op(fmt, N, K, T, accumulate, seed, sample_rows=None):
    from quantized_q8_gemv_amd import q8l as C
    rng = np.random.default_rng(seed)
    raw = synth.draw_k_quant(rng, N, K, fmt)
    X = rng.standard_normal((T, K)).astype(np.float32)
    Y0 = rng.standard_normal((T, N)).astype(np.float32)
    dev = torch.device("cuda:0")
    Wd = torch.from_numpy(raw.reshape(-1)).to(dev)
    Xd = torch.from_numpy(X).to(dev)
    Yd = torch.from_numpy(Y0).to(dev)
    log(f"k-format op {fmt} N={N} K={K} T={T} acc={accumulate}")
    dt = C.Q8L_Q4_K if fmt == "q4_k" else C.Q8L_Q6_K
    assert C.q8l_op_matmul_kq(Wd, dt, N, K, Xd, T, accumulate, Yd) == C.Q8L_OK
    torch.cuda.synchronize()
    Y = Yd.cpu().numpy().astype(np.float64)
    rows = np.arange(N) if sample_rows is None else np.sort(rng.choice(N, sample_rows, replace=False))
    sub = raw[rows]
    ref = oracle.matmul_fmt(sub, fmt, len(rows), K, X.astype(np.float64))      # [T, rows]
    if accumulate:
        ref = ref + Y0[:, rows]
    w = _dequant(sub, fmt, len(rows), K)
    scale = np.sqrt(K) * np.sqrt((w ** 2).mean(axis=1))[None, :] * np.sqrt((X.astype(np.float64) ** 2).mean(axis=1))[:, None]
    err = np.abs(Y[:, rows] - ref)
    bound = 1e-4 * scale + (1e-6 * np.abs(Y0[:, rows]) if accumulate else 0.0)
    assert np.isfinite(Y).all()
    bad = err > bound
    assert not bad.any(), f"{fmt} N={N} K={K} T={T}: {int(bad.sum())} outputs off, worst {float((err / scale).max()):.3g}"
    return float((err / scale).max())


@pytest.mark.parametrize("fmt", ["q4_k", "q6_k"])
@pytest.mark.parametrize("T", [1, 2, 7, 203])
def test_down_projection_shape_of_the_pages(fmt, T):
    rel = _run_op(fmt, 576, 1536, T, 0, seed=T)
    log(f"  worst error / scale {rel:.3g}")


@pytest.mark.parametrize("fmt", ["q4_k", "q6_k"])
@pytest.mark.parametrize("N,K,T,acc", [(100, 512, 1, 1), (100, 512, 33, 1), (64, 11008, 1, 0),
                                       (64, 11008, 6, 1), (40, 17152, 1, 1), (40, 17152, 3, 0),
                                       (1, 256, 1, 0), (1, 256, 5, 1)])
def test_ragged_misaligned_and_chunked_shapes(fmt, N, K, T, acc):
    _run_op(fmt, N, K, T, acc, seed=N + K + T)


@pytest.mark.parametrize("fmt", ["q4_k", "q6_k"])
@pytest.mark.parametrize("T", [1, 64])
def test_large_down_projection_sampled_rows(fmt, T):
    """A 7B-sized down projection (4096 x 11008): all rows computed, 96 sampled
    rows checked against the oracle."""
    _run_op(fmt, 4096, 11008, T, 1, seed=5 + T, sample_rows=96)


def _kquant_shape(name="kq-micro"):
    # q_dim 256 and n_ff 512: whole 256-weight blocks for both K-format roles
    return synth.ModelShape(name, n_layer=3, n_embd=256, n_head=4, n_head_kv=2, head_dim=64, n_ff=512,
                            n_vocab=300, max_seq_len=128)


@pytest.mark.parametrize("prompt_len", [9, 4])
def test_model_with_k_format_layers_matches_the_oracle(prompt_len):
    """Per-layer formats o = (Q4_K, Q6_K, Q8_0), down = (Q6_K, Q8_0, Q4_K);
    a prompt of 9 tokens runs the MFMA GEMM path, 4 the small multi-token one,
    then greedy decode steps run the GEMV."""
    s = _kquant_shape()
    m = synth.with_k_quants(synth.random_model(s, 0), ["q4_k", "q6_k", "q8_0"], ["q6_k", "q8_0", "q4_k"])
    prompt = synth.prompt_ids(s.n_vocab, prompt_len, 3)
    ids, err, ties = compare_generation(gpu_model(m), oracle.OracleModel(m), prompt, 8,
                                        f"k-format model {prompt_len}+8")
    log(f"k-format model: max abs err {err:.3g}")
    assert ties <= 1


def test_generate_with_k_format_layers_equals_stepwise_forward():
    """The captured decode graphs (on-device greedy loop) give the same ids as
    step-by-step forward calls when layers hold K-format matrices."""
    s = _kquant_shape()
    m = synth.with_k_quants(synth.random_model(s, 1), ["q6_k", "q4_k", "q4_k"], ["q4_k", "q6_k", "q6_k"])
    prompt = synth.prompt_ids(s.n_vocab, 7, 4)
    a = gpu_model(m)
    _, tok = a.forward(prompt, 0)
    want = []
    for k in range(10):
        _, tok = a.forward([tok], len(prompt) + k)
        want.append(tok)
    b = gpu_model(m)
    _, first = b.forward(prompt, 0)
    dev = torch.device("cuda:0")
    tok_dev = torch.tensor([first], dtype=torch.int32, device=dev)
    ids_dev = torch.zeros(10, dtype=torch.int32, device=dev)
    from quantized_q8_gemv_amd import q8l as C
    assert b.generate_async(tok_dev, len(prompt), 10, ids_dev) == C.Q8L_OK
    torch.cuda.synchronize()
    assert ids_dev.cpu().tolist() == want


def test_gguf_in_the_pages_q4_k_m_mix_matches_the_oracle(tmp_path):
    """The pages' Q4_K_M file of the 135M model (tensor table in "速度",
    section "CPU GGUF"): rows of 576 in Q5_0 (q, k, o, gate, up and half of
    v) or Q8_0 (token_embd, the other v), the 1536-wide down projections in
    Q4_K and Q6_K. On the 4-layer model of the same widths: Q5_0 is read as
    exact Q8_0, the K formats as they are."""
    from quantized_q8_gemv_amd.model import Q8Model
    w, m, prompt = synth.workload_inputs("C1")
    s = m.shape
    rng = np.random.default_rng(23)
    file_tensors, om_tensors = [], []
    for t, (name, ftype, dims, data) in zip(m.tensors, W.model_tensors(m)):
        kind = name.split(".")[-2] if name.startswith("blk.") else ""
        layer = int(name.split(".")[1]) if name.startswith("blk.") else -1
        if kind in ("attn_q", "attn_k", "attn_output", "ffn_gate", "ffn_up") or (kind == "attn_v" and layer % 2):
            cols, rows = dims
            raw = W.random_blocks(rng, rows, cols, "q5_0")
            file_tensors.append((name, W.TYPE_Q5_0, dims, raw.tobytes()))
            om_tensors.append(synth.Tensor(name, "q8_0", rows, cols, W.to_q8_0(raw, rows, cols, "q5_0")))
        elif kind == "ffn_down":
            fmt = "q4_k" if layer % 2 == 0 else "q6_k"
            cols, rows = dims
            raw = synth.draw_k_quant(rng, rows, cols, fmt)
            file_tensors.append((name, W.TYPE_Q4_K if fmt == "q4_k" else W.TYPE_Q6_K, dims, raw.tobytes()))
            om_tensors.append(synth.Tensor(name, fmt, rows, cols, raw))
        else:
            file_tensors.append((name, ftype, dims, data))
            om_tensors.append(t)
    path = str(tmp_path / "q4_k_m-mix.gguf")
    W.write(path, W.llama_kv(s), file_tensors)
    om = oracle.OracleModel(synth.Model(s, om_tensors))
    ids, err, ties = compare_generation(Q8Model.from_gguf(path), om, prompt, 8, "gguf Q4_K_M mix 13+8")
    log(f"gguf Q4_K_M mix: max abs err {err:.3g}")
    assert ties <= 1


def test_k_format_o_projection_after_a_multi_split_merge():
    """A 70-token prompt puts the cache past one 64-key split, so decode runs
    the split merge before the K-format o-projection GEMV."""
    s = _kquant_shape()
    m = synth.with_k_quants(synth.random_model(s, 2), ["q4_k", "q6_k", "q4_k"], ["q8_0", "q4_k", "q6_k"])
    prompt = synth.prompt_ids(s.n_vocab, 70, 9)
    ids, err, ties = compare_generation(gpu_model(m), oracle.OracleModel(m), prompt, 6,
                                        "k-format model 70+6")
    log(f"k-format model 70+6: max abs err {err:.3g}")
    assert ties <= 1
