"""GPU parity of the single-op entry points (Q8_0 matmul, attention, argmax)
against the CPU oracle, at the model shapes and ragged edge cases."""

import numpy as np
import pytest

import oracle
import synth
from helpers import log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def C():
    from quantized_q8_gemv_amd import q8l
    q8l.lib()
    oracle.build(force=False)
    return q8l


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def gemv_bound(W, X):
    """Per-output error bound for f32 accumulation: 1e-5 * sum |w x| (+ tiny)."""
    return 1e-5 * (np.abs(X) @ np.abs(W).T) + 1e-7


SHAPES = [(576, 576), (192, 576), (1536, 576), (576, 1536), (49152, 576),
          (4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336), (32000, 4096),
          (37, 64), (1001, 192), (3, 128), (130, 320),
          # 172 block pairs per row: chunks of 64, 64 and a ragged 44
          (301, 11008), (4096, 11008)]


@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("T", [1, 13, 100])
def test_matmul_q8_0_matches_oracle(C, N, K, T):
    log(f"matmul N={N} K={K} T={T}")
    rng = np.random.default_rng(N * 7 + K + T)
    scales, q = synth.draw_q8_0(rng, N, K)
    raw = synth.pack_q8_0(scales, q)
    X = rng.standard_normal((T, K)).astype(np.float32)
    Y = torch.zeros((T, N), dtype=torch.float32, device="cuda:0")
    assert C.q8l_op_matmul_q8_0(dev(raw), N, K, dev(X), T, None, 0.0, 0, Y) == C.Q8L_OK
    torch.cuda.synchronize()
    ref = oracle.matmul_q8(raw, N, K, X.astype(np.float64))
    W = oracle.dequant_q8_0(raw, N, K)
    err = np.abs(Y.cpu().numpy() - ref)
    assert (err <= gemv_bound(W, X.astype(np.float64))).all(), err.max()


@pytest.mark.parametrize("T", [1, 5, 16, 17, 40])
def test_matmul_norm_prologue_and_accumulate(C, T):
    N, K, eps = 768, 576, 1e-5
    rng = np.random.default_rng(T)
    scales, q = synth.draw_q8_0(rng, N, K)
    raw = synth.pack_q8_0(scales, q)
    X = (rng.standard_normal((T, K)) * 0.02).astype(np.float32)
    w = rng.normal(1, 0.1, K).astype(np.float32)
    Y0 = rng.standard_normal((T, N)).astype(np.float32)
    Y = dev(Y0)
    assert C.q8l_op_matmul_q8_0(dev(raw), N, K, dev(X), T, dev(w), eps, 1, Y) == C.Q8L_OK
    torch.cuda.synchronize()
    U = np.stack([oracle.rmsnorm(X[t].astype(np.float64), w, eps) for t in range(T)])
    ref = Y0.astype(np.float64) + oracle.matmul_q8(raw, N, K, U)
    W = oracle.dequant_q8_0(raw, N, K)
    err = np.abs(Y.cpu().numpy() - ref)
    assert (err <= gemv_bound(W, U) + 1e-6 * np.abs(Y0)).all(), err.max()


def test_matmul_subnormal_and_zero_scales(C):
    N, K = 64, 256
    rng = np.random.default_rng(3)
    scales, q = synth.draw_q8_0(rng, N, K)
    scales[: N // 2] = np.float16(2.0 ** -24) * rng.integers(1, 1023, (N // 2, K // 32))
    scales[N // 2:, ::2] = 0
    raw = synth.pack_q8_0(scales, q)
    X = rng.standard_normal((1, K)).astype(np.float32)
    Y = torch.zeros((1, N), dtype=torch.float32, device="cuda:0")
    assert C.q8l_op_matmul_q8_0(dev(raw), N, K, dev(X), 1, None, 0.0, 0, Y) == C.Q8L_OK
    torch.cuda.synchronize()
    ref = oracle.matmul_q8(raw, N, K, X.astype(np.float64))[0]
    got = Y.cpu().numpy()[0]
    assert np.all(got[: N // 2] != 0)                   # subnormal scales were not flushed
    W = oracle.dequant_q8_0(raw, N, K)
    assert (np.abs(got - ref) <= gemv_bound(W, X.astype(np.float64))[0]).all()


def test_matmul_rejects_bad_arguments(C):
    x = torch.zeros(64, device="cuda:0")
    w = torch.zeros(34 * 2, dtype=torch.uint8, device="cuda:0")
    assert C.q8l_op_matmul_q8_0(w, 1, 96, x, 1, None, 0.0, 0, x) == C.Q8L_E_INVALID_ARG   # K % 64
    assert C.q8l_op_matmul_q8_0(w, 0, 64, x, 1, None, 0.0, 0, x) == C.Q8L_E_INVALID_ARG


def attention_ref(Q, K, V, T, kv_len, nh, nkv, hd):
    G = nh // nkv
    O = np.zeros((T, nh, hd))
    prefix = kv_len - T
    for h in range(nh):
        g = h // G
        for i in range(T):
            last = prefix + i if T > 1 else kv_len - 1
            O[i, h] = oracle.attend(Q[i, h], K[g, :kv_len], V[g, :kv_len], last)
    return O


@pytest.mark.parametrize("nh,nkv,hd", [(9, 3, 64), (32, 8, 128), (4, 4, 16)])
@pytest.mark.parametrize("T,kv_len", [(1, 1), (1, 33), (1, 64), (1, 65), (1, 331), (1, 4096),
                                      (2, 2), (13, 13), (5, 46), (203, 203), (37, 300)])
def test_attention_matches_oracle(C, nh, nkv, hd, T, kv_len):
    log(f"attention nh={nh} nkv={nkv} hd={hd} T={T} kv={kv_len}")
    rng = np.random.default_rng(nh * 1000 + T * 10 + kv_len)
    stride = kv_len + 3
    Q = rng.standard_normal((T, nh, hd)).astype(np.float32)
    K = rng.standard_normal((nkv, stride, hd)).astype(np.float32)
    V = rng.standard_normal((nkv, stride, hd)).astype(np.float32)
    O = torch.zeros((T, nh, hd), dtype=torch.float32, device="cuda:0")
    wsb = C.q8l_op_attention_workspace(T, kv_len, nh, nkv, hd)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda:0")
    st = C.q8l_op_attention(dev(Q), dev(K), dev(V), T, kv_len, stride, nh, nkv, hd, O, ws, wsb)
    assert st == C.Q8L_OK
    torch.cuda.synchronize()
    ref = attention_ref(Q.astype(np.float64), K.astype(np.float64), V.astype(np.float64), T,
                        kv_len, nh, nkv, hd)
    err = np.abs(O.cpu().numpy() - ref)
    assert err.max() <= 2e-5 * max(1.0, np.abs(ref).max()), err.max()


@pytest.mark.parametrize("n", [1, 7, 4096, 4097, 49152, 32000])
def test_argmax_lowest_index_on_ties(C, n):
    rng = np.random.default_rng(n)
    x = rng.standard_normal(n).astype(np.float32)
    if n > 10:
        x[[3, n // 2, n - 1]] = x.max() + 1.0               # a three-way tie
    out = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    wsb = 256 + 8 * ((n + 4095) // 4096)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda:0")
    assert C.q8l_op_argmax(dev(x), n, out, ws, wsb) == C.Q8L_OK
    torch.cuda.synchronize()
    assert int(out.item()) == oracle.argmax(x)
