"""The attention entry point that allocates nothing (q8l_op_attention_noalloc)
against q8l_op_attention, whose kernels it shares, through the C ABI.

The no-allocation variant keeps the single-query split partials in a static
device array shared by every call on the device; two calls in a row, the
second smaller, must each give exactly (bitwise) what the workspace entry
point gives on the same inputs, and sizes beyond the array are refused."""

import numpy as np
import pytest

from helpers import log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _inputs(rng, T, kv_len, kv_stride, nh, nkv, hd, dev):
    q = torch.from_numpy(rng.standard_normal((T, nh, hd)).astype(np.float32)).to(dev)
    k = torch.from_numpy(rng.standard_normal((nkv, kv_stride, hd)).astype(np.float32)).to(dev)
    v = torch.from_numpy(rng.standard_normal((nkv, kv_stride, hd)).astype(np.float32)).to(dev)
    return q, k, v


def _with_workspace(C, q, k, v, T, kv_len, kv_stride, nh, nkv, hd, dev):
    o = torch.full((T, nh, hd), float("nan"), dtype=torch.float32, device=dev)
    wsb = C.q8l_op_attention_workspace(T, kv_len, nh, nkv, hd)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    assert C.q8l_op_attention(q, k, v, T, kv_len, kv_stride, nh, nkv, hd, o, ws, wsb) == C.Q8L_OK
    return o


def _no_alloc(C, q, k, v, T, kv_len, kv_stride, nh, nkv, hd, dev):
    o = torch.full((T, nh, hd), float("nan"), dtype=torch.float32, device=dev)
    assert C.q8l_op_attention_noalloc(q, k, v, T, kv_len, kv_stride, nh, nkv, hd, o) == C.Q8L_OK
    return o


@pytest.mark.parametrize("shape", [
    # (kv_len first call, kv_len second call, kv_stride, n_head, n_head_kv, head_dim)
    (4096, 1000, 4096, 32, 8, 128),   # 7B-class heads: 128 then 32 splits
    (3000, 65, 4096, 9, 3, 64),       # 135M-shaped heads: 47 then 2 splits
])
def test_no_alloc_attention_equals_workspace_entry(shape):
    from quantized_q8_gemv_amd import q8l as C
    kv1, kv2, stride, nh, nkv, hd = shape
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(31)
    for kv in (kv1, kv2):   # the second call is smaller and reuses the array's leftovers
        q, k, v = _inputs(rng, 1, kv, stride, nh, nkv, hd, dev)
        ref = _with_workspace(C, q, k, v, 1, kv, stride, nh, nkv, hd, dev)
        got = _no_alloc(C, q, k, v, 1, kv, stride, nh, nkv, hd, dev)
        torch.cuda.synchronize()
        a, b = got.cpu().numpy(), ref.cpu().numpy()
        log(f"no-alloc attention kv {kv}, {nh}/{nkv} heads of {hd}: max |diff| {np.abs(a - b).max():.3g}")
        assert np.isfinite(a).all()
        assert np.array_equal(a, b)


def test_no_alloc_attention_prefill_and_limits():
    from quantized_q8_gemv_amd import q8l as C
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(32)
    T, kv, stride, nh, nkv, hd = 40, 100, 128, 8, 2, 64
    q, k, v = _inputs(rng, T, kv, stride, nh, nkv, hd, dev)
    ref = _with_workspace(C, q, k, v, T, kv, stride, nh, nkv, hd, dev)
    got = _no_alloc(C, q, k, v, T, kv, stride, nh, nkv, hd, dev)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), ref.cpu().numpy())
    # partials beyond the static array: 64 heads of 128 over 20000 keys (~20 MB) are refused
    # (buffers sized for the request, so nothing could read past them even if it ran)
    qb = torch.zeros(64 * 128, dtype=torch.float32, device=dev)
    ob = torch.empty(64 * 128, dtype=torch.float32, device=dev)
    kb = torch.zeros(8 * 20000 * 128, dtype=torch.float32, device=dev)
    assert C.q8l_op_attention_noalloc(qb, kb, kb, 1, 20000, 20000, 64, 8, 128, ob) == C.Q8L_E_INVALID_ARG
    assert C.q8l_op_attention_noalloc(None, kb, kb, 1, 10, 10, 8, 2, 64, ob) == C.Q8L_E_INVALID_ARG
