"""On-device greedy generation (q8l_generate) and long prompts at the 7B-class
widths against the CPU oracle.

q8l_generate runs the caller's loop of single-token forwards and argmax
readbacks ("生成一个 token", section 实验程序) with no host round trip: each
step's argmax becomes the next step's input on the device. Its ids are
compared with the oracle's greedy chain; where the two could legitimately
differ (a near tie in the oracle's logits) the oracle is run teacher-forced on
the GPU's ids and every GPU pick must be the oracle's argmax or within the
tolerance of it.
"""

import numpy as np
import pytest

import oracle
import synth
from helpers import ATOL, RTOL, assert_logits_close, compare_generation, gpu_model, log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


def device_generate(gm, prompt, steps):
    """Prefill (forward) then `steps` greedy steps in one q8l_generate call.
    Returns (id picked by the prefill, generated ids, last step's logits)."""
    from quantized_q8_gemv_amd import q8l as C

    _, first = gm.forward(prompt, 0)
    dev = torch.device("cuda:0")
    tok = torch.tensor([first], dtype=torch.int32, device=dev)
    ids = torch.zeros(steps, dtype=torch.int32, device=dev)
    st = gm.generate_async(tok, len(prompt), steps, ids)
    assert st == C.Q8L_OK, C.q8l_last_error(gm.handle)
    torch.cuda.synchronize()
    return first, ids.cpu().numpy().astype(np.int64).tolist(), gm.logits.cpu().numpy()


def check_against_oracle(om, prompt, first, ids, last_logits, what):
    """The oracle fed the prompt and then the GPU's own ids: every GPU pick
    must be the oracle's argmax at that step, except at a near tie (the
    oracle's top logit within twice the tolerance of the GPU's pick), and the
    last step's logits must be within tolerance. Returns the near-tie count."""
    st, lg, _ = om.forward(prompt, 0)
    assert st == oracle.OK
    chain = [first] + ids
    ties = 0
    pos = len(prompt)
    for k, pick in enumerate(chain):
        top = oracle.argmax(lg)
        if pick != top:
            bound = 2 * (ATOL + RTOL * abs(float(lg[top])))
            gap = float(lg[top]) - float(lg[pick])
            assert gap <= bound, f"{what} step {k}: GPU picked {pick}, oracle argmax {top} (gap {gap:.3g})"
            ties += 1
            log(f"{what} step {k}: near tie ({pick} vs {top}, gap {gap:.3g})")
        if k == len(chain) - 1:
            break
        st, lg, _ = om.forward([pick], pos + k)
        assert st == oracle.OK
        if k == len(chain) - 2:
            err = assert_logits_close(last_logits, lg, f"{what} last step logits")
            log(f"{what}: last-step max abs err {err:.3g}")
    return ties


def test_generate_135m_13_prompt_20_steps_matches_oracle():
    """The 135M-shaped workload (13-token prompt, 20 greedy steps) through the
    on-device loop: ids equal the oracle's greedy chain."""
    w, m, prompt = synth.workload_inputs("C2")
    gm = gpu_model(m)
    om = oracle.OracleModel(m)
    first, ids, last = device_generate(gm, prompt, 20)
    ref_ids, _ = om.generate(prompt, 20)
    ties = check_against_oracle(oracle.OracleModel(m), prompt, first, ids, last, "135m generate 13+20")
    if ties == 0:
        assert [first] + ids == ref_ids
    assert ties <= 1
    assert gm.cache_len == 13 + 20


def test_generate_crosses_attention_split_buckets():
    """One q8l_generate call whose steps cross 64 -> 65 and 128 -> 129 cached
    keys: the decode graph changes from one attention split (the attention
    kernel normalises) to two (merged in the o-projection's prologue) to
    three or four, inside the call."""
    w, m, _ = synth.workload_inputs("C1")
    prompt = synth.prompt_ids(m.shape.n_vocab, 60, 9)
    gm = gpu_model(m)
    first, ids, last = device_generate(gm, prompt, 80)
    ties = check_against_oracle(oracle.OracleModel(m), prompt, first, ids, last, "tiny generate 60+80")
    assert ties <= 1
    assert gm.cache_len == 140


def test_generate_head_dim_128_crosses_split_buckets():
    """Head size 128 (32-key attention splits), rows of 2048 weights (the
    register-activation decode kernels): one q8l_generate call from 20 cached
    keys to 80 crosses 32 -> 33 keys (one split, normalised by the attention
    kernel, to two, merged in the o-projection's prologue) and 64 -> 65 (to
    three and more, 33 KB of partials: merged by the combine kernel)."""
    s = synth.ModelShape("hd128-gen", n_layer=2, n_embd=2048, n_head=16, n_head_kv=4, head_dim=128,
                         n_ff=2048, n_vocab=500, tied_output=False, max_seq_len=256)
    m = synth.random_model(s, 12)
    prompt = synth.prompt_ids(s.n_vocab, 20, 10)
    gm = gpu_model(m)
    first, ids, last = device_generate(gm, prompt, 60)
    ties = check_against_oracle(oracle.OracleModel(m), prompt, first, ids, last, "hd128 generate 20+60")
    assert ties <= 1
    assert gm.cache_len == 80


def test_generate_135m_203_prompt_128_steps_crosses_257_keys():
    """The 203 + 128 workload as one q8l_generate call: the cache grows from
    204 to 331 keys, crossing the 4 -> 8 split bucket at 257."""
    w, m, prompt = synth.workload_inputs("C3")
    gm = gpu_model(m)
    first, ids, last = device_generate(gm, prompt, 128)
    ties = check_against_oracle(oracle.OracleModel(m), prompt, first, ids, last, "135m generate 203+128")
    assert ties <= 2


def test_big_gqa_two_layers_512_prompt_matches_oracle():
    """7B-class widths (hidden 4096, 32/8 heads, head_dim 128, FFN 14336,
    vocab 32000 untied), 2 layers, a 512-token prompt: the prefill GEMMs run
    on their large tiles at K = 4096 and K = 14336 with activations split
    into f16 pairs, and the MFMA attention covers 8 query blocks; then 4
    decode steps."""
    s = synth.ModelShape("7b-width-2layer", n_layer=2, n_embd=4096, n_head=32, n_head_kv=8,
                         head_dim=128, n_ff=14336, n_vocab=32000, tied_output=False)
    m = synth.random_model(s, 6)
    prompt = synth.prompt_ids(s.n_vocab, 512, 8)
    log("7b-width 2 layers: 512-token prefill")
    ids, err, ties = compare_generation(gpu_model(m), oracle.OracleModel(m), prompt, 4, "7b-width 512+4")
    log(f"7b-width 512+4: max abs err {err:.3g}, near ties {ties}")
    assert ties <= 1
