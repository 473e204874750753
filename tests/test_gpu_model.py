"""End-to-end GPU parity of the forward pass against the CPU oracle, and the
index_pos / KV-cache contract, through the C ABI (Q8Model only marshals)."""

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


@pytest.fixture(scope="module")
def tiny():
    w, m, prompt = synth.workload_inputs("C1")
    return m, prompt, gpu_model(m)


def test_tiny_generation_matches_oracle(tiny):
    m, prompt, gm = tiny
    ids, err, ties = compare_generation(gm, oracle.OracleModel(m), prompt, 20, "tiny 13+20")
    log(f"tiny: max abs err {err:.3g}, near ties {ties}, ids {ids[:8]}...")
    assert ties <= 1


def test_135m_generation_matches_oracle():
    w, m, prompt = synth.workload_inputs("C2")
    gm = gpu_model(m)
    ids, err, ties = compare_generation(gm, oracle.OracleModel(m), prompt, 20, "135m 13+20")
    log(f"135m 13+20: max abs err {err:.3g}, near ties {ties}")
    assert ties <= 1


def test_135m_203_prompt_128_steps():
    w, m, prompt = synth.workload_inputs("C3")
    gm = gpu_model(m)
    ids, err, ties = compare_generation(gm, oracle.OracleModel(m), prompt, 128, "135m 203+128")
    log(f"135m 203+128: max abs err {err:.3g}, near ties {ties}")
    assert ties <= 2


@pytest.mark.parametrize("plen", [4, 13, 203])
def test_neox_rope_generation_matches_oracle(plen):
    """The NEOX pairing (j, j + hd/2): prompts through the multi-token GEMV
    (4 tokens) and the GEMM path (13, 203), then decode."""
    s = synth.ModelShape("tiny-neox", n_layer=4, n_embd=576, n_head=9, n_head_kv=3, head_dim=64,
                         n_ff=1536, n_vocab=4096, rope_neox=True)
    m = synth.random_model(s, 0)
    prompt = synth.prompt_ids(s.n_vocab, plen, 1)
    ids, err, ties = compare_generation(gpu_model(m), oracle.OracleModel(m), prompt, 8, f"neox {plen}+8")
    log(f"neox {plen}+8: max abs err {err:.3g}, near ties {ties}")
    assert ties <= 1


@pytest.mark.parametrize("n_embd,n_head,n_head_kv,n_vocab", [(1536, 24, 8, 1001), (1984, 31, 31, 999),
                                                             (256, 4, 2, 777)])
def test_output_layer_of_short_rows(n_embd, n_head, n_head_kv, n_vocab):
    """Output rows of 24, 31 and 4 pairs: the output layer takes 64 / P rows
    per wave (2, 2 and 16; 48, 62 and 64 lanes busy) with a vocabulary that
    leaves a partial last group; logits and greedy ids against the oracle."""
    s = synth.micro_shape(n_layer=1, n_embd=n_embd, n_head=n_head, n_head_kv=n_head_kv, head_dim=64,
                          n_ff=512, n_vocab=n_vocab, name=f"w{n_embd}")
    m = synth.random_model(s, n_embd)
    prompt = synth.prompt_ids(n_vocab, 5, 2)
    ids, err, ties = compare_generation(gpu_model(m), oracle.OracleModel(m), prompt, 4, f"width {n_embd} 5+4")
    log(f"width {n_embd}, vocab {n_vocab}: max abs err {err:.3g}, near ties {ties}")
    assert ties <= 1


def test_neox_rope_head_dim_128():
    s = synth.ModelShape("neox-hd128", n_layer=2, n_embd=1024, n_head=8, n_head_kv=2, head_dim=128,
                         n_ff=1024, n_vocab=2048, rope_neox=True)
    m = synth.random_model(s, 4)
    prompt = synth.prompt_ids(s.n_vocab, 40, 3)
    ids, err, ties = compare_generation(gpu_model(m), oracle.OracleModel(m), prompt, 6, "neox hd128 40+6")
    assert ties <= 1


def test_chunked_prefill_and_reset(tiny):
    m, prompt, gm = tiny
    gm.clear_kv_cache()
    one, _ = gm.forward(prompt, 0)
    gm.forward(prompt[:8], 0)
    two, _ = gm.forward(prompt[8:], 8)
    assert_logits_close(two, one, "chunked vs single")
    # index_pos == 0 drops the cache: identical to a fresh prefill (bitwise)
    gm.forward([5], 13)
    again, _ = gm.forward(prompt, 0)
    assert np.array_equal(again, one)
    assert gm.cache_len == 13


def test_position_errors_leave_state_unchanged(tiny):
    from quantized_q8_gemv_amd import q8l as C
    m, prompt, gm = tiny
    gm.forward(prompt[:8], 0)
    assert gm.forward_async(prompt[8:], 5) == C.Q8L_E_POS_MISMATCH
    assert gm.cache_len == 8
    two, _ = gm.forward(prompt[8:], 8)                     # the right counter still works
    om = oracle.OracleModel(m)
    om.forward(prompt[:8], 0)
    _, ref, _ = om.forward(prompt[8:], 8)
    assert_logits_close(two, ref, "after a rejected call")
    gm.clear_kv_cache()
    assert gm.forward_async(prompt, 33) == C.Q8L_E_POS_MISMATCH
    assert gm.forward_async([1], m.shape.max_seq_len) == C.Q8L_E_POS_RANGE
    assert gm.cache_len == 0


def test_single_token_misuse_matches_oracle(tiny):
    """T == 1 with a stale counter is not an error; both sides compute the same thing."""
    m, prompt, gm = tiny
    om = oracle.OracleModel(m)
    gm.forward(prompt, 0)
    om.forward(prompt, 0)
    for tok, p in ((7, 113), (9, 10), (3, 0), (4, 1)):
        g, _ = gm.forward([tok], p)
        st, ref, _ = om.forward([tok], p)
        assert st == oracle.OK
        assert_logits_close(g, ref, f"misuse p={p}")
        assert gm.cache_len == om.cache_len


def test_kv_full():
    from quantized_q8_gemv_amd import q8l as C
    s = synth.micro_shape(n_layer=1, n_embd=64, n_head=4, n_head_kv=2, head_dim=16, n_ff=128,
                          n_vocab=64, max_seq_len=16)
    m = synth.random_model(s, 2)
    gm = gpu_model(m)
    om = oracle.OracleModel(m)
    toks = list(range(16))
    g, _ = gm.forward(toks, 0)
    _, ref, _ = om.forward(toks, 0)
    assert_logits_close(g, ref, "full cache")
    assert gm.forward_async([1], 3) == C.Q8L_E_KV_FULL
    assert gm.cache_len == 16


def test_decode_is_deterministic(tiny):
    m, prompt, gm = tiny
    runs = []
    for _ in range(2):
        gm.forward(prompt, 0)
        outs = [gm.forward([i + 1], 13 + i)[0] for i in range(5)]
        runs.append(np.stack(outs))
    assert np.array_equal(runs[0], runs[1])


def test_device_generation_equals_host_loop(tiny):
    m, prompt, gm = tiny
    lg, first = gm.forward(prompt, 0)
    host_ids, host_last = [first], None
    for k in range(12):
        host_last, nxt = gm.forward([host_ids[-1]], 13 + k)
        host_ids.append(nxt)
    gm.forward(prompt, 0)
    tok = torch.tensor([first], dtype=torch.int32, device="cuda:0")
    ids = torch.zeros(12, dtype=torch.int32, device="cuda:0")
    from quantized_q8_gemv_amd import q8l as C
    assert gm.generate_async(tok, 13, 12, ids) == C.Q8L_OK
    torch.cuda.synchronize()
    assert ids.cpu().numpy().tolist() == host_ids[1:]
    assert np.array_equal(gm.logits.cpu().numpy(), host_last)
    assert gm.cache_len == 25


def test_long_context_prefill_and_decode_to_the_table_end():
    """4000-token prefill + decode to position 4095 at the 135M widths (2 layers)."""
    from quantized_q8_gemv_amd import q8l as C
    s = synth.ModelShape("135m-width-2layer", n_layer=2, n_embd=576, n_head=9, n_head_kv=3,
                         head_dim=64, n_ff=1536, n_vocab=49152)
    m = synth.random_model(s, 4)
    prompt = synth.prompt_ids(s.n_vocab, 4000, 5)
    gm = gpu_model(m)
    om = oracle.OracleModel(m)
    log("long context: prefill 4000")
    g, gid = gm.forward(prompt, 0)
    _, ref, _ = om.forward(prompt, 0)
    assert_logits_close(g, ref, "prefill 4000")
    tok = oracle.argmax(ref)
    for p in range(4000, 4096):
        g, _ = gm.forward([tok], p)
        _, ref, _ = om.forward([tok], p)
        assert_logits_close(g, ref, f"decode at {p}")
        tok = oracle.argmax(ref)
    assert gm.cache_len == 4096
    assert gm.forward_async([tok], 4096) == C.Q8L_E_POS_RANGE


@pytest.mark.parametrize("plen", [200, 1023, 1100])
def test_long_prompt_head_dim_128(plen):
    """Prefill attention with the key ranges of long query blocks split over
    workgroups and merged (1023 and 1100 tokens: 16 and 18 key blocks of 64
    in ranges of 4 and 5; 200 tokens: no split), head size 128, 4 query heads
    per KV head, then decode steps."""
    s = synth.micro_shape(n_layer=1, n_embd=512, n_head=4, n_head_kv=1, head_dim=128, n_ff=512,
                          n_vocab=1000, max_seq_len=1200, name="hd128-long")
    m = synth.random_model(s, plen)
    prompt = synth.prompt_ids(s.n_vocab, plen, 9)
    ids, err, ties = compare_generation(gpu_model(m), oracle.OracleModel(m), prompt, 3, f"hd128 {plen}+3")
    log(f"hd128 {plen}+3: max abs err {err:.3g}, near ties {ties}")
    assert ties <= 1


@pytest.mark.parametrize("hd", [64, 128])
def test_key_split_prefill_after_a_cached_prefix(hd):
    """A 1100-token prefill behind 10 cached positions: its query blocks
    straddle key blocks, so some key ranges hold no visible key for the first
    queries of a block (those ranges must weigh nothing in the merge); logits
    of the chunked prefill and the decode steps after it against the oracle."""
    s = synth.micro_shape(n_layer=1, n_embd=2 * hd, n_head=2, n_head_kv=1, head_dim=hd, n_ff=256,
                          n_vocab=500, max_seq_len=1200, name=f"prefix-split-{hd}")
    m = synth.random_model(s, hd + 3)
    prompt = synth.prompt_ids(s.n_vocab, 1110, 11)
    gm, om = gpu_model(m), oracle.OracleModel(m)
    gm.forward(prompt[:10], 0)
    om.forward(prompt[:10], 0)
    g, gid = gm.forward(prompt[10:], 10)
    st, ref, _ = om.forward(prompt[10:], 10)
    assert st == oracle.OK
    assert_logits_close(g, ref, f"hd {hd}: 1100 tokens after 10")
    tok = oracle.argmax(ref)
    for p in range(1110, 1113):
        g, _ = gm.forward([tok], p)
        _, ref, _ = om.forward([tok], p)
        assert_logits_close(g, ref, f"hd {hd}: decode at {p}")
        tok = oracle.argmax(ref)


@pytest.mark.parametrize("plen", [64, 97])
def test_big_gqa_shape_two_layers(plen):
    """hidden 4096, 32/8 heads, head_dim 128, FFN 14336, vocab 32000 untied (2
    layers). 64 tokens: the o and down projections on 32x64 tiles split over
    K; 97 tokens: on 64x128 tiles split over K (8 slices)."""
    s = synth.ModelShape("7b-width-2layer", n_layer=2, n_embd=4096, n_head=32, n_head_kv=8,
                         head_dim=128, n_ff=14336, n_vocab=32000, tied_output=False)
    m = synth.random_model(s, 6)
    prompt = synth.prompt_ids(s.n_vocab, plen, 7)
    gm = gpu_model(m)
    ids, err, ties = compare_generation(gm, oracle.OracleModel(m), prompt, 4, f"7b-width {plen}+4")
    log(f"7b-width {plen}: max abs err {err:.3g}")
    assert ties <= 1


@pytest.fixture(scope="module")
def big_full():
    """The full 7B-class shape (32 layers, 7.7 GB of Q8_0 weights)."""
    w, m, prompt = synth.workload_inputs("C5")
    log(f"7b full: {m.total_bytes / 1e9:.2f} GB generated")
    return m, prompt, gpu_model(m)


def test_big_gqa_full_depth_matches_oracle(big_full):
    """Short prompt at full depth against the oracle (its cost grows with T)."""
    m, prompt, gm = big_full
    ids, err, ties = compare_generation(gm, oracle.OracleModel(m), prompt[:4], 3, "7b full 4+3")
    log(f"7b full 4+3: max abs err {err:.3g}, near ties {ties}")
    assert ties <= 1


def test_big_gqa_full_depth_prefill_equals_decode_chain(big_full):
    """Prefill of 64 tokens (MFMA path) = the same tokens fed one at a time (GEMV path)."""
    m, prompt, gm = big_full
    toks = prompt[:64]
    full, _ = gm.forward(toks, 0)
    for i, t in enumerate(toks):
        step, _ = gm.forward([t], i)
    assert_logits_close(step, full, "7b full: prefill 64 vs 64 single-token steps")


def test_argmax_to_host_mapped_memory(tiny):
    """forward's argmax written by the last kernel into pinned host memory (by
    its device address) equals the argmax written to device memory, for the
    prefill and for decode steps through the captured graph."""
    from quantized_q8_gemv_amd.model import host_mapped_u32

    m, prompt, gm = tiny
    am_host, am_dev = host_mapped_u32()
    stream = torch.cuda.current_stream()
    nxt = None
    for k in range(6):
        toks, pos = (prompt, 0) if k == 0 else ([nxt], len(prompt) + k - 1)
        am_host[0] = -1
        assert gm.forward_async(toks, pos, argmax_out=am_dev) == 0
        stream.synchronize()
        host_id = int(am_host[0])
        ref = int(np.argmax(gm.logits.cpu().numpy()))
        log(f"host-mapped argmax step {k}: {host_id} (logits argmax {ref})")
        assert host_id == ref
        nxt = host_id


@pytest.mark.parametrize("plen", [6, 31, 64, 65, 300, 1024, 1025])
def test_prompt_lengths_around_split_k(tiny, plen):
    """Prompts on both sides of the split-K limits: short prompts split the
    o and down products' K steps over several workgroups whose partial sums
    the next norm kernel adds to the residual (the last layer's through the
    add-only form); at hidden size 576 prompts of up to 1024 tokens split,
    1025 take the plain accumulating GEMM. Logits of the prefill and of 3
    decode steps against the oracle."""
    m, _, gm = tiny
    prompt = synth.prompt_ids(m.shape.n_vocab, plen, 5)
    ids, err, ties = compare_generation(gm, oracle.OracleModel(m), prompt, 3, f"tiny {plen}+3")
    log(f"tiny {plen}+3: max abs err {err:.3g}, near ties {ties}")
    assert ties <= 1
