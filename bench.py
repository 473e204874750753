#!/usr/bin/env python3
"""Benchmark: batch-1 greedy generation with the Q8_0 Llama forward on one GPU.

One step = one generation of the workload as the pages time it ("生成一个
token", section 实验程序): a prompt prefill at position 0, then `decode_steps`
single-token forwards, each followed by the greedy argmax read back to the
host. Default workload: the SmolLM2-135M-shaped model (30 layers, hidden 576,
9/3 heads, vocab 49152 tied), 13-token prompt + 20 decode steps, random-init
Q8_0 weights and uniform random prompt ids (no trained weights are used).

Printed JSON line:
  value            decode tokens/s of the host loop (forward + argmax readback per token)
  prefill_tok_s    prompt tokens / prefill wall time (to the argmax readback)
  device_loop      decode on the device (q8l_generate: argmax feeds the next step
                   without host round trips), per-token time and HBM fraction
                   = algorithmic bytes per token (Q8_0 weights + norms + one
                   embedding row + KV cache read/written) / time / 8 TB/s
  device_loop_cache_flushed
                   the same per-token time with the 256 MB memory-side cache
                   flushed before each step (a 512 MiB copy outside the timed
                   region): the weights stream from HBM
  step_frac        the decode step's HBM-roofline fraction: algorithmic bytes per
                   token / device-loop time per token / 8 TB/s
  roofline         the decode kernel with the most time per step, its algorithmic
                   bytes per launch over its mean launch time (HIP events around
                   back-to-back launches, each on the next layer's weights), and
                   the same kernel's mean duration in the committed rocprofv3
                   summary of this workload (profile_us, profile_frac)
  cpu_baseline     the CPU oracle timed on a bounded sample of the same workload
                   (all threads, and one thread), with the host's CPU model
  host_loop_reps   min and median over the timed steps (per-token decode, prefill)
  configs          the other workloads, each measured the same way outside the
                   timed region: tiny (13 + 20), 203 + 128 (1 warm-up rep + 10
                   reps with a fresh cache, min and median), 4000 + 96 (decode
                   cost against cache length) and the 7B-class 512 + 128, each
                   with its own CPU-oracle sample

Other modes: --pmc-summary FETCH_DIR WRITE_DIR summarises two rocprofv3
counter runs (no GPU); --stats-summary CSV turns a rocprofv3 kernel_stats.csv
into the table kept in profiles/ (no GPU); --formats times one matmul per
block format; --kv-sweep prints one line per cache length (16 ... 4000 prompt
tokens on the 135M-shaped model): device-loop us/token and the attention
kernel's time at that length.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
FORMAT_BYTES = {"q8_0": (32, 34), "q5_0": (32, 22), "q4_k": (256, 144), "q6_k": (256, 210)}  # (weights, bytes)
# The pages' Metal figures for these workloads, on an Apple M2 Max -- another
# machine, quoted as context:
#   C2: 20 decode steps after a 13-token prompt, 2.6 ms mean per step incl. the
#       argmax readback ("生成一个 token", section "Metal：热缓存");
#   C3: 203-token prompt + 128 greedy steps, fresh cache per rep, best of 10
#       reps, Q8_0 on Metal 2.72 ms per token ("速度", sections
#       "两边量的是同一件事" and "小结").
PAGES_DECODE_MS = {"C2": 2.6, "C3": 2.72}
KIND_NAMES = ["embed", "qkv_rope_kv", "attn_decode", "oproj_residual", "gateup_silu",
              "down_residual", "lmhead", "argmax_finish"]
NKINDS = len(KIND_NAMES)
# source of each kind's kernel on the 135M shape, whose PMC summary is committed
KIND_SOURCES = {"embed": "quantized_q8_gemv_amd/csrc/k_misc.hip", "attn_decode": "quantized_q8_gemv_amd/csrc/k_attn.hip",
                "lmhead": "quantized_q8_gemv_amd/csrc/k_xgemv.hip", "argmax_finish": "quantized_q8_gemv_amd/csrc/k_gemv.hip"}
for _k in KIND_NAMES:
    KIND_SOURCES.setdefault(_k, "quantized_q8_gemv_amd/csrc/k_wgemv.hip")
# rocprofv3 PMC summaries of the decode kernels (FETCH_SIZE and WRITE_SIZE per
# dispatch, scaled by the same counters on a copy of known size); a summary
# counts only while the kernel source it was taken with is unchanged.
TRAFFIC_FILES = {"C2": "profiles/decode_kernels_135m_13+20_pmc_traffic.md"}


WAVE_GEMV_PAIRS = (1, 2, 4, 8, 9, 12, 16, 24)   # row lengths (64-weight pairs) of the wave-per-row GEMVs


def attn_chunk(hd):
    return 64 if hd <= 64 else 32


def decode_fused(s, kv_len, o_fmt="q8_0"):
    """Whether a decode step at this cache length runs the attention and the
    o-projection as one kernel (the runtime's rule: one attention split, the
    group's columns in whole 64-weight pairs, at most 16 KB of per-group
    partial rows, a Q8_0 or Q5_0 o-projection)."""
    G = s.n_head // s.n_head_kv
    return (kv_len <= attn_chunk(s.head_dim) and (G * s.head_dim) % 64 == 0 and G * s.head_dim // 64 <= 256
            and s.n_head_kv * s.n_embd * 4 <= 16 * 1024 and o_fmt in ("q8_0", "q5_0"))


def x_slices(pairs):
    """Slices of a row the register-activation GEMVs (k_x*) take it in: 1 for
    32..64 pairs, 2 up to 128, 4 up to 256; 0 when they do not take it."""
    if pairs < 32:
        return 0
    return 1 if pairs <= 64 else 2 if pairs <= 128 else 4 if pairs <= 256 else 0


def kernel_symbols(s, down_fmt="q8_0", kv_len=1):
    """Device symbol of each decode kernel kind at this shape (T = 1) and
    cache length. Rows of a few pairs run the wave-per-row kernels
    (k_w*<pairs>; their output layer several rows per wave,
    k_xlmhead_short); rows of 32 to 64 pairs the register-activation ones
    (k_x*; longer plain products in 2 or 4 slices, k_xmatmul1<slices>),
    q/k/v of such rows and other lengths the LDS-staged ones. A Q4_K / Q6_K
    down projection runs k_kq_gemv<format, rows per wave>. With the attention
    fused into the o-projection, the o-projection has no kernel of its own
    (None)."""
    multi = (s.n_embd // 64) * 272 > 40 * 1024  # rows longer than one LDS chunk
    o_multi = (s.q_dim // 64) * 272 > 40 * 1024
    down_multi = (s.n_ff // 64) * 272 > 40 * 1024
    ph, pq, pf = s.n_embd // 64, s.q_dim // 64, s.n_ff // 64
    wave_h = ph in WAVE_GEMV_PAIRS
    x_h = not wave_h and x_slices(ph) == 1

    def plain(pairs, lds_multi):
        if pairs in WAVE_GEMV_PAIRS:
            return f"k_wmatmul1<{pairs}>"
        if x_slices(pairs):
            return f"k_xmatmul1<{x_slices(pairs)}>"
        return "k_matmul1_chunked<false>" if lds_multi else "k_matmul1<false, false>"

    if down_fmt == "q8_0":
        down = plain(pf, down_multi)
    else:
        down = f"k_kq_gemv<{1 if down_fmt == 'q4_k' else 2}, {2 if s.n_embd >= 4096 else 1}>"
    fused = decode_fused(s, kv_len)
    oproj = None if fused else plain(pq, o_multi)
    return ["k_embed", f"k_wqkv1<{ph}>" if wave_h else f"k_qkv1<{str(multi).lower()}>",
            "k_attn_o1" if fused else "k_attn_decode", oproj,
            f"k_wgateup1<{ph}>" if wave_h else "k_xgateup1" if x_h else f"k_gateup1<{str(multi).lower()}>",
            down, "k_xlmhead1" if x_h else "k_xlmhead_short" if ph < 32 else f"k_lmhead1<{str(multi).lower()}>",
            "k_argmax_finish"]


def source_digest(path):
    import hashlib
    with open(os.path.join(ROOT, path), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(config, kind):
    """HBM bytes per launch of decode kernel `kind` from the committed PMC
    summary, or None if there is none or the kernel source changed since."""
    path = TRAFFIC_FILES.get(config)
    if not path or not os.path.exists(os.path.join(ROOT, path)):
        return None
    for line in open(os.path.join(ROOT, path)):
        if not line.startswith("traffic:"):
            continue
        f = dict(kv.split("=", 1) for kv in line.split()[1:])
        if f.get("kind") != kind:
            continue
        if source_digest(f["source"]) != f["sha256"]:
            return None
        return int(f["bytes_per_launch"])
    return None


# rocprofv3 --kernel-trace --stats summaries of the bench command per workload;
# a summary's figures count only while the sources it lists are unchanged.
STATS_FILES = {"C2": "profiles/decode_prefill_135m_13+20_kernel_stats.md",
               "C5": "profiles/decode_prefill_7b-gqa_512+128_kernel_stats.md"}
STATS_SOURCES = ["quantized_q8_gemv_amd/csrc/k_gemv.hip", "quantized_q8_gemv_amd/csrc/k_wgemv.hip",
                 "quantized_q8_gemv_amd/csrc/k_xgemv.hip", "quantized_q8_gemv_amd/csrc/k_attn.hip",
                 "quantized_q8_gemv_amd/csrc/runtime.cpp"]


def short_symbol(name):
    import re
    m = re.match(r"(?:void )?(?:q8l::\(anonymous namespace\)::|q8l::)?([^(]*)", name)
    return m.group(1).strip() if m and not name.startswith("_Z") else name


def stats_summary(csv_path):
    """The markdown table of a rocprofv3 kernel_stats.csv (one row per kernel
    symbol: calls, mean / min / max duration, share of GPU time) and the
    digests of the sources the profiled kernels were built from."""
    import csv
    rows = list(csv.DictReader(open(csv_path)))
    print("| kernel | calls | avg us | min us | max us | share % |")
    print("|---|---:|---:|---:|---:|---:|")
    for r in rows:
        print(f"| `{short_symbol(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
              f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    print()
    print("sources: " + " ".join(f"{p}={source_digest(p)}" for p in STATS_SOURCES))


def profiled_us(config, symbol):
    """Mean duration (us) of `symbol` in the committed kernel statistics of
    this workload, or None if there are none or a listed source changed."""
    path = STATS_FILES.get(config)
    if not path or not os.path.exists(os.path.join(ROOT, path)):
        return None
    us, fresh = None, False
    for line in open(os.path.join(ROOT, path)):
        if line.startswith("sources:"):
            pairs = dict(kv.split("=", 1) for kv in line.split()[1:])
            fresh = all(p in pairs and source_digest(p) == pairs[p] for p in STATS_SOURCES)
        elif line.startswith(f"| `{symbol}` |"):
            us = float(line.split("|")[3])
    return us if fresh else None


def pmc_summary(fetch_dir, write_dir, config="C2"):
    """Per-launch HBM traffic of each decode kernel kind from two rocprofv3
    counter runs of this script (--pmc FETCH_SIZE, then --pmc WRITE_SIZE; CSV
    output). Each counter is scaled by what it reads for the 1 GiB device copy
    of copy_bandwidth() (the largest __amd_rocclr_copyBuffer dispatches).
    Dispatches are assigned to kinds by symbol; the o-projection and the down
    projection share a symbol at some shapes and are told apart by what ran
    just before them (the attention kernels, or gate/up). Prints a markdown
    table and the `traffic:` lines read by measured_traffic()."""
    import csv
    import glob

    import synth
    _, model, prompt = synth.workload_inputs(config)
    s = model.shape
    syms = kernel_symbols(s, kv_len=len(prompt) + 1)
    alg_bytes = kernel_bytes(s, len(prompt) + 1)  # attention at the first decode step

    def load(d, counter):
        rows = []
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(path)):
                if r.get("Counter_Name") == counter:
                    rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
        per = {}
        for did, name, v in rows:  # a counter may come in several rows per dispatch
            n0, v0 = per.get(did, (name, 0.0))
            per[did] = (n0, v0 + v)
        return [(did, n, v) for did, (n, v) in sorted(per.items())]

    def kinds(disp):
        out, prev = [], ""
        for did, name, v in disp:
            short = name.replace("void ", "").replace("q8l::(anonymous namespace)::", "").replace("q8l::", "")
            short = short.split("(")[0].strip()
            kind = None
            for k, sym in enumerate(syms):
                if short == sym:
                    kind = KIND_NAMES[k]
            if short == syms[3] and short == syms[5]:
                kind = "oproj_residual" if prev.startswith("k_attn") else "down_residual"
            out.append((kind, short, v))
            prev = short
        return out

    res = {}
    scale = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        disp = load(d, counter)
        # the 1 GiB copies of copy_bandwidth() are the largest copy dispatches
        # (the 512 MiB cache-flush copies and the uploads are smaller)
        copies = sorted(v for _, n, v in disp if "copyBuffer" in n)
        big = [v for v in copies if v >= 0.9 * copies[-1]] if copies else []
        scale[counter] = (1 << 30) / (statistics.mean(big) * 1024) if big else float("nan")
        acc = {}
        for kind, short, v in kinds(disp):
            if kind:
                acc.setdefault(kind, (short, []))[1].append(v)
        for kind, (short, vals) in acc.items():
            res.setdefault(kind, {"symbol": short})[counter] = (len(vals), statistics.mean(vals))
    print(f"scale FETCH_SIZE {scale['FETCH_SIZE']:.4f}, WRITE_SIZE {scale['WRITE_SIZE']:.4f}")
    # the read-only check: the 1 GiB f32 sums of copy_bandwidth(), the largest
    # reduction dispatches of the FETCH_SIZE run
    sums = sorted(v for _, n, v in load(fetch_dir, "FETCH_SIZE") if "reduce" in n)
    if sums:
        big = [v for v in sums if v >= 0.9 * sums[-1]]
        read = statistics.mean(big) * 1024 * scale["FETCH_SIZE"]
        print(f"read-only check: a 1 GiB f32 sum reads {read:,.0f} bytes by the scaled FETCH_SIZE "
              f"({read / (1 << 30):.4f} of 1 GiB, {len(big)} dispatches)")
    print("| kind | symbol | dispatches | FETCH KiB | WRITE KiB | scaled bytes | algorithmic bytes | ratio |")
    print("|---|---|---:|---:|---:|---:|---:|---:|")
    lines = []
    for kind in KIND_NAMES:
        if kind == "embed":  # not a kernel of the decode step (its dispatches are the prefill's)
            continue
        if kind not in res or "FETCH_SIZE" not in res[kind] or "WRITE_SIZE" not in res[kind]:
            continue
        r = res[kind]
        n, f = r["FETCH_SIZE"]
        _, w = r["WRITE_SIZE"]
        b = int(round((f * scale["FETCH_SIZE"] + w * scale["WRITE_SIZE"]) * 1024))
        alg = alg_bytes[KIND_NAMES.index(kind)]
        print(f"| {kind} | `{r['symbol']}` | {n} | {f:.1f} | {w:.1f} | {b:,} | {alg:,} | "
              f"{b / alg if alg else float('nan'):.2f} |")
        src = KIND_SOURCES[kind]
        lines.append(f"traffic: kind={kind} bytes_per_launch={b} source={src} sha256={source_digest(src)}")
    print()
    print("\n".join(lines))


def copy_bandwidth(torch, nbytes=1 << 30, reps=5):
    """Device-to-device copy of `nbytes` (read + write) in GB/s; also the
    reference dispatch for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    # A read-only reference for the FETCH_SIZE scale: a sum over `nbytes` of
    # f32 (16-byte vector loads, nothing written but the result), checked
    # against the copy's scale by pmc_summary().
    c = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    for _ in range(2):
        c.sum()
    torch.cuda.synchronize()
    del c
    return 2 * nbytes / (ms * 1e-3) / 1e9


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


def q8_bytes(rows, cols):
    return rows * cols // 32 * 34


def fmt_bytes(fmt, rows, cols):
    per, size = FORMAT_BYTES[fmt]
    return rows * cols // per * size


def per_token_weight_bytes(model):
    """Every tensor's bytes once (projections in their block formats, norms,
    the output layer -- the embedding when tied) plus one embedding row."""
    s = model.shape
    embd = model["token_embd.weight"].nbytes
    total = sum(t.nbytes for t in model.tensors)
    if not s.tied_output:
        total -= embd
    return total + q8_bytes(1, s.n_embd)


def kv_bytes_per_position(s):
    return s.n_layer * 2 * s.n_head_kv * s.head_dim * 4


def kernel_bytes(s, kv_len, down_fmt="q8_0"):
    """Algorithmic bytes of one launch of each decode kernel kind (layer 0).
    Fused attention + o-projection (kind 2): the cache and q, the o weights
    and the per-group partial rows it writes; kind 3 is then 0."""
    H, QD, KVD, F, V = s.n_embd, s.q_dim, s.kv_dim, s.n_ff, s.n_vocab
    attn = kv_len * s.n_head_kv * s.head_dim * 4 * 2 + QD * 4
    oproj = q8_bytes(H, QD) + QD * 4 + 2 * H * 4
    fused = decode_fused(s, kv_len)
    return [
        q8_bytes(1, H) + H * 4,
        q8_bytes(QD + 2 * KVD, H) + 2 * H * 4 + (QD + 2 * KVD) * 4,
        attn + q8_bytes(H, QD) + s.n_head_kv * H * 4 if fused else attn,
        0 if fused else oproj,
        2 * q8_bytes(F, H) + 2 * H * 4 + F * 4,
        fmt_bytes(down_fmt, H, F) + F * 4 + 2 * H * 4,
        q8_bytes(V, H) + 2 * H * 4 + V * 4,
        0,
    ]


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def omp_threads(n=None):
    """Set (when n is given) and read the OpenMP thread count of the runtime
    the oracle's library uses (libgomp), or None without it."""
    try:
        g = ctypes.CDLL("libgomp.so.1")
    except OSError:
        return None
    if n is not None:
        g.omp_set_num_threads(int(n))
    g.omp_get_max_threads.restype = ctypes.c_int
    return int(g.omp_get_max_threads())


def cpu_baseline(model, prompt, steps, seconds, threads=None):
    """The oracle, as it stands, on the same workload: repeat the generation
    until `seconds` of CPU work; report decode tokens/s. For models whose
    oracle prefill alone would exceed the budget, the sample keeps the first
    four prompt tokens and as many decode steps as fit (at most 8): the
    decode rate is then an extrapolation from those steps."""
    import oracle

    oracle.build(force=False)
    prev = omp_threads()
    used = omp_threads(threads) if threads else prev
    om = oracle.OracleModel(model)
    params = sum(t.rows * t.cols for t in model.tensors)
    note = ""
    if params * len(prompt) > 2e10:          # oracle prefill alone would take long
        prompt = prompt[:4]
        steps = max(1, min(steps, 8, int(seconds * 2e9 / params)))
        note = "; prompt cut to its first 4 tokens and the decode to the first steps (per-token extrapolation)"
    t_dec, n_dec, reps, t_all0 = 0.0, 0, 0, time.perf_counter()
    while True:
        st, lg, _ = om.forward(prompt, 0)
        nxt = oracle.argmax(lg)
        t0 = time.perf_counter()
        for k in range(steps):
            st, lg, _ = om.forward([nxt], len(prompt) + k)
            nxt = oracle.argmax(lg)
        t_dec += time.perf_counter() - t0
        n_dec += steps
        reps += 1
        if time.perf_counter() - t_all0 >= seconds:
            break
    if threads and prev:
        omp_threads(prev)
    cores = used or int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or os.cpu_count()
    return {"value": n_dec / t_dec, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{reps} x (prefill {len(prompt)} + {steps} decode steps) of the same model; "
                      f"decode tokens/s over {t_dec:.1f} s of decode{note}"}


# The pages' CPU timings of one QMatMul on the down projection's shape, by
# block format ("速度", section "CPU GGUF"; minimum of 35 runs, Apple M2 Max,
# ms) -- another machine, quoted as context.
PAGES_MATMUL_MS = {("q8_0", 203): 0.8959, ("q4_k", 203): 0.6777, ("q6_k", 203): 1.1029, ("q8_0", 1): 0.0050}
PEAK_MFMA_F16_TFLOPS = 2500.0


def format_matmuls(reps):
    """Time Y = X W^T per block format through the single-op entries: the
    pages' down-projection shape [T, 1536] x [1536, 576] (T = 1 and 203) and a
    7B-sized one [T, 11008] x [11008, 4096]. One JSON line per case. T = 1 is
    HBM-bound (algorithmic bytes = the matrix + X + Y); T > 1 is compared with
    the dense f16 MFMA peak on its 2*N*K*T flops (the kernels issue twice that
    on the matrix cores: activations are an f16 pair hi + lo)."""
    import numpy as np
    import torch

    import synth
    from quantized_q8_gemv_amd import q8l as C

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    rng = np.random.default_rng(0)
    lines = []
    for (N, K, Ts, name) in ((576, 1536, (1, 203), "down 135M"), (4096, 11008, (1, 203, 512), "down 7B")):
        for fmt in ("q8_0", "q4_k", "q6_k"):
            if fmt == "q8_0":
                sc, q = synth.draw_q8_0(rng, N, K)
                raw = synth.pack_q8_0(sc, q)
            else:
                raw = synth.draw_k_quant(rng, N, K, fmt)
            Wd = torch.from_numpy(raw.reshape(-1)).to(dev)
            for T in Ts:
                X = torch.randn(T, K, device=dev)
                Y = torch.empty(T, N, device=dev)

                def call_on(st):
                    if fmt == "q8_0":
                        return C.q8l_op_matmul_q8_0(Wd, N, K, X, T, None, 0.0, 0, Y, st)
                    dt = C.Q8L_Q4_K if fmt == "q4_k" else C.Q8L_Q6_K
                    return C.q8l_op_matmul_kq(Wd, dt, N, K, X, T, 0, Y, st)

                def call():
                    return call_on(stream)

                for _ in range(3):
                    assert call() == C.Q8L_OK
                torch.cuda.synchronize()
                # the timed launches replay from a captured graph, so the events
                # see GPU time rather than the host's call rate
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    cs = torch.cuda.current_stream()
                    for _ in range(reps):
                        assert call_on(cs) == C.Q8L_OK
                g.replay()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                g.replay()
                e1.record(stream)
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) / reps * 1e3
                del g
                wbytes = raw.nbytes
                nbytes = wbytes + T * K * 4 + T * N * 4
                if T == 1:
                    ach = nbytes / (us * 1e-6) / 1e9
                    roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": round(ach / PEAK_HBM_GBS, 4)}
                else:
                    ach = 2.0 * N * K * T / (us * 1e-6) / 1e12
                    roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_MFMA_F16_TFLOPS,
                            "unit": "TFLOP/s", "frac": round(ach / PEAK_MFMA_F16_TFLOPS, 4)}
                pages = PAGES_MATMUL_MS.get((fmt, T)) if N == 576 else None
                line = {"metric": "single matmul time by block format", "format": fmt, "shape": name,
                        "N": N, "K": K, "T": T, "us": round(us, 2), "weight_bytes": int(wbytes),
                        "bytes_per_call": int(nbytes), "roofline": roof,
                        "pages_cpu_ms": pages, "reps": reps}
                print(json.dumps(line), flush=True)
                lines.append(line)
            del Wd
    return lines


class HostLoop:
    """The pages' generation loop on one model: prefill at position 0, then
    `steps` single-token forwards, each followed by the greedy id's readback.

    The greedy id goes to pinned host memory that the last kernel writes
    directly; the host polls that word (reset to -1, never a token id, before
    each forward) and reads the id as soon as it lands -- the 4-byte readback
    of each step, without a copy or a blocking stream sync (the next forward
    is ordered after the rest of the step by the stream)."""

    def __init__(self, gm, prompt, steps):
        import numpy as np
        import torch
        from quantized_q8_gemv_amd.model import host_mapped_u32

        self.gm, self.steps = gm, steps
        self.am_host, self.am_dev = host_mapped_u32()
        self.am_np = self.am_host.numpy()
        self.stream = torch.cuda.current_stream()
        self.tok = np.zeros(1, dtype=np.uint32)
        self.prompt = np.ascontiguousarray(np.asarray(prompt, dtype=np.uint32))

    def _read_id(self):
        deadline = time.perf_counter() + 10.0
        while self.am_np[0] == -1:
            if time.perf_counter() > deadline:
                self.stream.synchronize()
                if self.am_np[0] == -1:
                    raise RuntimeError("the forward did not write its argmax")
        return int(self.am_np[0])

    def generation(self):
        """One generation; returns (prefill seconds, decode seconds)."""
        from quantized_q8_gemv_amd import q8l as C

        t0 = time.perf_counter()
        self.am_np[0] = -1
        st = self.gm.forward_async(self.prompt, 0, argmax_out=self.am_dev)
        assert st == C.Q8L_OK, C.q8l_last_error(self.gm.handle)
        nxt = self._read_id()
        t1 = time.perf_counter()
        for k in range(self.steps):
            self.tok[0] = nxt
            self.am_np[0] = -1
            st = self.gm.forward_async(self.tok, len(self.prompt) + k, argmax_out=self.am_dev)
            assert st == C.Q8L_OK, C.q8l_last_error(self.gm.handle)
            nxt = self._read_id()
        t2 = time.perf_counter()
        self.stream.synchronize()
        return t1 - t0, t2 - t1


def device_loop(gm, prompt, steps, reps, segments=1):
    """Per-token time (ms) of q8l_generate after a prefill, HIP events around
    each of `segments` equal parts of the decode; returns a list per rep of
    the per-segment ms/token."""
    import torch
    from quantized_q8_gemv_amd import q8l as C

    per = steps // segments
    ids = torch.zeros(per, dtype=torch.int32, device="cuda:0")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(segments + 1)]
    out = []
    for r in range(reps):
        assert gm.forward_async(prompt, 0) == C.Q8L_OK
        tok = gm.argmax
        ev[0].record()
        for k in range(segments):
            assert gm.generate_async(tok, len(prompt) + k * per, per, ids) == C.Q8L_OK, C.q8l_last_error(gm.handle)
            tok = ids[per - 1:per]
            ev[k + 1].record()
        torch.cuda.synchronize()
        out.append([ev[k].elapsed_time(ev[k + 1]) / per for k in range(segments)])
    return out


def measure_config(key, cpu_seconds, with_cpu):
    """One workload measured the way the headline is, outside the timed
    region: host loop (decode ms/token and prefill ms, min and median over
    reps, each rep with a fresh cache: prefill at position 0 drops it), the
    device loop with its HBM-roofline fraction, and the oracle's rate. The
    long-context workload also reports the device loop per segment of 16
    steps against the cache length."""
    import torch

    import synth
    from quantized_q8_gemv_amd.model import Q8Model

    t0 = time.perf_counter()
    w, model, prompt = synth.workload_inputs(key)
    s = model.shape
    gm = Q8Model(synth.shape_fields(s), model.tensors, device="cuda:0")
    torch.cuda.synchronize()
    eprint(f"[bench] {key} {w.name}: model ready in {time.perf_counter() - t0:.1f} s")
    steps = w.decode_steps
    reps = w.reps if w.reps > 1 else 3
    loop = HostLoop(gm, prompt, steps)
    warm_pre, warm_dec = loop.generation()
    pre, dec = [], []
    for _ in range(reps):
        a, b = loop.generation()
        pre.append(a)
        dec.append(b)
    segments = 6 if key == "C4" else 1
    dl = device_loop(gm, prompt, steps, reps, segments)
    per_tok = [sum(r) / len(r) for r in dl]
    dev_ms = statistics.median(per_tok)
    W = per_token_weight_bytes(model)
    kvb = kv_bytes_per_position(s)
    b_tok = W + kvb * (len(prompt) + (steps + 1) / 2.0)
    out = {"workload": w.name, "model": s.name, "prompt_len": len(prompt), "decode_steps": steps, "reps": reps,
           "warmup_rep": {"prefill_ms": round(warm_pre * 1e3, 3),
                          "decode_ms_per_token": round(warm_dec / steps * 1e3, 4)},
           "decode_ms_per_token_host_loop": {"min": round(min(dec) / steps * 1e3, 4),
                                             "median": round(statistics.median(dec) / steps * 1e3, 4)},
           "decode_tok_s_host_loop": round(steps / statistics.median(dec), 1),
           "prefill_ms": {"min": round(min(pre) * 1e3, 3), "median": round(statistics.median(pre) * 1e3, 3)},
           "prefill_tok_s": round(len(prompt) / statistics.median(pre), 1),
           "device_loop_us_per_token": {"min": round(min(per_tok) * 1e3, 2), "median": round(dev_ms * 1e3, 2)},
           "bytes_per_token": int(b_tok),
           "step_frac": round(b_tok / (dev_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    if segments > 1:
        per = steps // segments
        seg = [statistics.median(r[k] for r in dl) for k in range(segments)]
        out["device_loop_by_kv_len"] = [
            {"kv_len": [len(prompt) + k * per + 1, len(prompt) + (k + 1) * per],
             "us_per_token": round(seg[k] * 1e3, 2),
             "step_frac": round((W + kvb * (len(prompt) + (k + 0.5) * per)) / (seg[k] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
            for k in range(segments)]
    if key in PAGES_DECODE_MS:
        out["pages_metal_ms_per_token"] = PAGES_DECODE_MS[key]
    del gm
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if with_cpu:
        out["cpu_baseline"] = cpu_baseline(model, prompt, steps, cpu_seconds)
    eprint(f"[bench] {key}: host loop {out['decode_ms_per_token_host_loop']['median']} ms/token, device loop "
           f"{out['device_loop_us_per_token']['median']} us/token (step_frac {out['step_frac']}), prefill "
           f"{out['prefill_tok_s']} tok/s")
    return out


def q5_0_as_q8_0(raw, rows, cols):
    """Q5_0 blocks rewritten as Q8_0 blocks with the same scale and the
    block's integers (nibble | fifth bit << 4) - 16: the same weights, the
    layout the library used before it streamed Q5_0 as it is."""
    import numpy as np

    import synth
    nb = cols // 32
    blk = raw.reshape(rows, nb, 22)
    d = blk[:, :, 0:2].copy().view("<f2").reshape(rows, nb)
    qh = blk[:, :, 2:6].copy().view("<u4").reshape(rows, nb)
    qs = blk[:, :, 6:22]
    bits = lambda first: (((qh[:, :, None] >> (np.arange(16, dtype=np.uint32) + first)) & 1) << 4).astype(np.uint8)
    q = np.concatenate([(qs & 15) | bits(0), (qs >> 4) | bits(16)], axis=2).astype(np.int16) - 16
    return synth.pack_q8_0(d, q.reshape(rows, cols).astype(np.int8))


# The pages' 4-bit file of the 135M model, per layer: q, k, o, gate and up in
# Q5_0, v in Q5_0 in every other layer (Q8_0 otherwise), down in Q4_K and Q6_K
# in alternate layers ("速度", section "CPU GGUF").
def q4_k_m_layer(l):
    return ["q5_0", "q5_0", "q5_0" if l % 2 else "q8_0", "q5_0", "q5_0", "q5_0", "q4_k" if l % 2 == 0 else "q6_k"]


def q5_compare(reps=5):
    """Decode with Q5_0 weights streamed as they are against the same
    weights expanded to Q8_0, at the 135M shape (13-token prompt, 20 steps)
    and the 7B-class one (128 + 32): every projection in Q5_0, and the pages'
    4-bit mix. One JSON line per (shape, mix, layout): weight and cache bytes
    per token, device-loop us/token (q8l_generate, HIP events; median of
    `reps` fresh-cache reps) and the HBM rate it implies."""
    import torch

    import synth
    from quantized_q8_gemv_amd.model import Q8Model

    for key in ("C2", "C5"):
        w = synth.WORKLOADS[key]
        s = w.model
        prompt = synth.prompt_ids(s.n_vocab, w.prompt_len, w.prompt_seed)
        steps = w.decode_steps
        for mix in ("all_q5_0", "q4_k_m"):
            fmts = [["q5_0"] * 7 if mix == "all_q5_0" else q4_k_m_layer(l) for l in range(s.n_layer)]
            t0 = time.perf_counter()
            native = synth.random_model_formats(s, w.seed, fmts)
            expanded = synth.Model(s, [synth.Tensor(t.name, "q8_0", t.rows, t.cols,
                                                    q5_0_as_q8_0(t.data, t.rows, t.cols))
                                       if t.dtype == "q5_0" else t for t in native.tensors])
            eprint(f"[bench] {key} {mix}: models drawn in {time.perf_counter() - t0:.1f} s")
            for layout, model in (("q5_0 native", native), ("q5_0 expanded to q8_0", expanded)):
                gm = Q8Model(synth.shape_fields(s), model.tensors, device="cuda:0")
                torch.cuda.synchronize()
                device_loop(gm, prompt, steps, 1)   # warm-up: builds the decode graphs
                per_tok = [r[0] for r in device_loop(gm, prompt, steps, reps)]
                ms = statistics.median(per_tok)
                W = per_token_weight_bytes(model)
                b_tok = W + kv_bytes_per_position(s) * (len(prompt) + (steps + 1) / 2.0)
                line = {"mode": "q5_compare", "model": s.name, "mix": mix, "layout": layout,
                        "prompt_len": len(prompt), "decode_steps": steps, "reps": reps,
                        "weight_bytes_per_token": int(W), "bytes_per_token": int(b_tok),
                        "us_per_token": round(ms * 1e3, 2), "us_per_token_min": round(min(per_tok) * 1e3, 2),
                        "hbm_gbs": round(b_tok / (ms * 1e-3) / 1e9, 1),
                        "step_frac": round(b_tok / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
                print(json.dumps(line), flush=True)
                del gm
                torch.cuda.synchronize()
                torch.cuda.empty_cache()
            del native, expanded


KV_SWEEP = [16, 64, 256, 1024, 2048, 4000]


def kv_sweep(kernel_reps, steps=16):
    """Decode cost against cache length on the 135M-shaped model: for each
    prompt length, prefill it, then `steps` greedy steps through q8l_generate
    (device loop, HIP events), and the attention kernel alone at that length
    (q8l_time_decode_kernels; with several splits, the merge kernel that
    follows it is not included)."""
    import torch

    import synth
    from quantized_q8_gemv_amd import q8l as C
    from quantized_q8_gemv_amd.model import Q8Model

    w, model, _ = synth.workload_inputs("C4")
    s = model.shape
    gm = Q8Model(synth.shape_fields(s), model.tensors, device="cuda:0")
    ids = torch.zeros(steps, dtype=torch.int32, device="cuda:0")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    W = per_token_weight_bytes(model)
    kvb = kv_bytes_per_position(s)
    chunk = 64 if s.head_dim <= 64 else 32
    for kv in KV_SWEEP:
        prompt = synth.prompt_ids(s.n_vocab, kv, 11)
        dl = []
        for r in range(5):
            assert gm.forward_async(prompt, 0) == C.Q8L_OK
            ev0.record()
            assert gm.generate_async(gm.argmax, kv, steps, ids) == C.Q8L_OK
            ev1.record()
            torch.cuda.synchronize()
            if r >= 1:
                dl.append(ev0.elapsed_time(ev1) / steps)
        assert gm.forward_async(prompt, 0) == C.Q8L_OK
        torch.cuda.synchronize()
        ms = (ctypes.c_float * (NKINDS + 1))()
        assert C.lib().q8l_time_decode_kernels(gm.handle, kernel_reps, ms,
                                               torch.cuda.current_stream().cuda_stream) == C.Q8L_OK
        dev_ms = statistics.median(dl)
        b_tok = W + kvb * (kv + (steps + 1) / 2.0)
        splits = -(-(kv + 1) // chunk)
        attn_bytes = (kv + 1) * s.n_head_kv * s.head_dim * 4 * 2 + s.q_dim * 4
        line = {"mode": "kv_sweep", "model": s.name, "kv_len": kv + 1, "decode_steps": steps,
                "us_per_token": round(dev_ms * 1e3, 2), "us_per_token_min": round(min(dl) * 1e3, 2),
                "hbm_gbs": round(b_tok / (dev_ms * 1e-3) / 1e9, 1),
                "attention_us": round(ms[2] * 1e3, 2), "attention_splits": splits,
                "attention_gbs": round(attn_bytes / (ms[2] * 1e-3) / 1e9, 1),
                "attention_us_per_token": round(ms[2] * 1e3 * s.n_layer, 1)}
        eprint(f"[bench] kv {kv + 1}: {line['us_per_token']} us/token, attention {line['attention_us']} us "
               f"({splits} splits)")
        print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="C2", help="workload key in synth.WORKLOADS")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-reps", type=int, default=50)
    ap.add_argument("--down-format", default="q8_0", choices=["q8_0", "q4_k", "q6_k", "q4_k_m"],
                    help="block format of the down projections (q4_k_m: Q4_K and Q6_K in alternate "
                         "layers, as the pages' 4-bit file holds them)")
    ap.add_argument("--formats", action="store_true",
                    help="time the single matmul per block format (Q8_0, Q4_K, Q6_K) instead")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this script; no GPU use")
    ap.add_argument("--no-configs", action="store_true",
                    help="measure only the --config workload (no per-workload block for the others)")
    ap.add_argument("--stats-summary", metavar="KERNEL_STATS_CSV",
                    help="print the profiles/ table of a rocprofv3 kernel_stats.csv; no GPU use")
    ap.add_argument("--q5-compare", action="store_true",
                    help="decode with Q5_0 weights as they are against the same weights expanded to Q8_0, "
                         "at the 135M and 7B-class shapes, instead (one JSON line per case)")
    ap.add_argument("--kv-sweep", action="store_true",
                    help="decode cost against cache length on the 135M-shaped model instead "
                         "(one JSON line per length)")
    args = ap.parse_args()
    if args.gpus != 1:
        eprint(f"bench.py runs on one GPU: this build has no multi-GPU path (--gpus {args.gpus}).")
        sys.exit(2)
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary, config=args.config)
        return
    if args.stats_summary:
        stats_summary(args.stats_summary)
        return
    if args.kv_sweep:
        kv_sweep(args.kernel_reps)
        return
    if args.q5_compare:
        q5_compare()
        return
    if args.formats:
        import torch
        format_matmuls(args.kernel_reps)
        # a copy of known size: the reference dispatch for scaling HBM counters
        eprint(f"[bench] device copy: {copy_bandwidth(torch):.0f} GB/s (1 GiB, read + write)")
        return

    import numpy as np
    import torch

    import synth
    from quantized_q8_gemv_amd import q8l as C
    from quantized_q8_gemv_amd.model import Q8Model, host_mapped_u32

    w, model, prompt = synth.workload_inputs(args.config)
    s = model.shape
    down_fmts = None
    if args.down_format != "q8_0":
        down_fmts = ([("q4_k", "q6_k")[l % 2] for l in range(s.n_layer)] if args.down_format == "q4_k_m"
                     else [args.down_format] * s.n_layer)
        model = synth.with_k_quants(model, ["q8_0"] * s.n_layer, down_fmts)
    down0 = down_fmts[0] if down_fmts else "q8_0"
    steps = w.decode_steps
    eprint(f"[bench] {w.name}: generating done, uploading {model.total_bytes / 1e6:.1f} MB")
    gm = Q8Model(synth.shape_fields(s), model.tensors, device="cuda:0")
    torch.cuda.synchronize()

    loop = HostLoop(gm, prompt, steps)
    generation = loop.generation

    for _ in range(args.warmup):
        generation()
    torch.cuda.synchronize()
    eprint(f"[bench] warmup {args.warmup} done; timing {args.steps} steps")
    t_start = time.perf_counter()
    pre, dec = [], []
    for _ in range(args.steps):
        a, b = generation()
        pre.append(a)
        dec.append(b)
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    ms_per_step = (t_end - t_start) / args.steps * 1e3
    value = args.steps * steps / sum(dec)
    prefill_tok_s = len(prompt) / statistics.median(pre)
    eprint(f"[bench] host loop: {value:.1f} decode tok/s, prefill {prefill_tok_s:.1f} tok/s")

    # Decode on the device: argmax feeds the next step, no host round trip.
    ids = torch.zeros(steps, dtype=torch.int32, device="cuda:0")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    dl = []
    for r in range(12):
        assert gm.forward_async(prompt, 0) == C.Q8L_OK
        ev0.record()
        assert gm.generate_async(gm.argmax, len(prompt), steps, ids) == C.Q8L_OK
        ev1.record()
        torch.cuda.synchronize()
        if r >= 2:
            dl.append(ev0.elapsed_time(ev1) / steps)
    dev_ms = statistics.median(dl)
    W = per_token_weight_bytes(model)
    kvb = kv_bytes_per_position(s)
    mean_kv = len(prompt) + (steps + 1) / 2.0
    b_tok = W + kvb * mean_kv
    dev_gbs = b_tok / (dev_ms * 1e-3) / 1e9

    # The same decode with the memory-side cache (256 MB) flushed before every
    # step: a 512 MiB device copy (1 GiB of traffic) runs between steps and
    # only the step itself (its state-setting kernel + the decode graph) is
    # timed, so the weights come from HBM as they would for a model that does
    # not fit that cache.
    flush_src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
    flush_dst = torch.empty_like(flush_src)
    cold = []
    for r in range(3):
        assert gm.forward_async(prompt, 0) == C.Q8L_OK
        for k in range(steps):
            flush_dst.copy_(flush_src)
            ev0.record()
            assert gm.generate_async(gm.argmax, len(prompt) + k, 1, ids) == C.Q8L_OK
            ev1.record()
            torch.cuda.synchronize()
            if r >= 1:
                cold.append(ev0.elapsed_time(ev1))
    del flush_src, flush_dst
    cold_ms = statistics.median(cold)
    cold_gbs = b_tok / (cold_ms * 1e-3) / 1e9
    eprint(f"[bench] device loop, cache flushed before each step: {cold_ms * 1e3:.1f} us/token, "
           f"{cold_gbs:.0f} GB/s algorithmic")
    eprint(f"[bench] device loop: {dev_ms * 1e3:.1f} us/token, {dev_gbs:.0f} GB/s algorithmic")

    # Per-kernel launch times (HIP events on the stream the kernels run on).
    assert gm.forward_async(prompt, 0) == C.Q8L_OK
    torch.cuda.synchronize()
    ms = (ctypes.c_float * (NKINDS + 1))()
    st = C.lib().q8l_time_decode_kernels(gm.handle, args.kernel_reps, ms,
                                         torch.cuda.current_stream().cuda_stream)
    assert st == C.Q8L_OK, C.q8l_last_error(gm.handle)
    # mean time per launch of back-to-back launches (the last entry: an empty
    # kernel, the dispatch gap alone)
    overhead = ms[NKINDS]
    raw = [ms[i] for i in range(NKINDS)]
    ms = raw
    kv_len = len(prompt) + 1
    kb = kernel_bytes(s, kv_len, down0)
    launches = [1, s.n_layer, s.n_layer, s.n_layer, s.n_layer, s.n_layer, 1, 1]
    launches = [n if raw[i] > 0 else 0 for i, n in enumerate(launches)]
    per_step = [ms[i] * launches[i] for i in range(NKINDS)]
    dom = max(range(NKINDS), key=lambda i: per_step[i])
    kernels = {KIND_NAMES[i]: {"us": round(ms[i] * 1e3, 2) if raw[i] > 0 else None, "bytes": kb[i],
                               "gbs": round(kb[i] / (ms[i] * 1e-3) / 1e9, 1) if raw[i] > 0 else 0.0,
                               "launches_per_token": launches[i]} for i in range(NKINDS)}
    achieved = kb[dom] / (ms[dom] * 1e-3) / 1e9
    traffic = measured_traffic(args.config, KIND_NAMES[dom]) if down_fmts is None else None
    symbol = kernel_symbols(s, down0, kv_len)[dom]
    prof_us = profiled_us(args.config, symbol) if down_fmts is None else None
    step_frac = round(dev_gbs / PEAK_HBM_GBS, 4)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                "kernel": KIND_NAMES[dom], "symbol": symbol,
                "bytes_per_launch": kb[dom], "us_per_launch": round(ms[dom] * 1e3, 2),
                "timing": "HIP events around back-to-back launches, launch r on layer r mod n_layer",
                "profile_us": prof_us,
                "profile_frac": (round(kb[dom] / (prof_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4) if prof_us else None),
                "profile": STATS_FILES.get(args.config) if prof_us else None,
                "empty_kernel_us": round(overhead * 1e3, 2),
                "step_frac": step_frac}
    copy_gbs = copy_bandwidth(torch)
    eprint(f"[bench] device copy: {copy_gbs:.0f} GB/s (1 GiB, read + write)")
    eprint(f"[bench] kernels: " + ", ".join(f"{k} {v['us']}us" for k, v in kernels.items() if v["us"] is not None))

    cpu = None
    if not args.no_cpu_baseline:
        eprint(f"[bench] cpu baseline (oracle) ~{args.cpu_seconds:.0f} s")
        cpu = cpu_baseline(model, prompt, steps, args.cpu_seconds)
        one = cpu_baseline(model, prompt, steps, max(2.0, args.cpu_seconds / 3), threads=1)
        cpu["value_1_thread"] = one["value"]
        cpu["sample_1_thread"] = one["sample"]

    configs = {}
    if not args.no_configs and args.config == "C2" and down_fmts is None:
        del gm
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        for key in ("C1", "C3", "C4", "C5"):
            configs[key] = measure_config(key, args.cpu_seconds / 2, not args.no_cpu_baseline)

    out = {
        "metric": "decode tokens/s (batch 1) + achieved HBM GB/s vs peak; prefill tokens/s",
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (round(value / (1e3 / PAGES_DECODE_MS[args.config]), 2)
                        if args.config in PAGES_DECODE_MS and down_fmts is None else None),
        "dtype": "f32 (Q8_0 int8 x f16-scale weights; decode f32 throughout; prefill MFMA on f16 hi+lo activation pairs, f32 accumulation)",
        "data": "synthetic: random-init Q8_0 weights, uniform random prompt ids",
        "config": {"workload": w.name + ("" if down_fmts is None else f" down={args.down_format}"),
                   "model": s.name, "layers": s.n_layer, "hidden": s.n_embd,
                   "heads": s.n_head, "kv_heads": s.n_head_kv, "vocab": s.n_vocab,
                   "prompt_len": len(prompt), "decode_steps": steps, "batch": 1,
                   "parallelism": "single GPU"},
        "prefill_tok_s": round(prefill_tok_s, 1),
        "decode_ms_per_token_host_loop": round(sum(dec) / (args.steps * steps) * 1e3, 4),
        # per timed step (one generation each): min and median over the steps
        "host_loop_reps": {"decode_ms_per_token_min": round(min(dec) / steps * 1e3, 4),
                           "decode_ms_per_token_median": round(statistics.median(dec) / steps * 1e3, 4),
                           "prefill_ms_min": round(min(pre) * 1e3, 3),
                           "prefill_ms_median": round(statistics.median(pre) * 1e3, 3)},
        "step_frac": step_frac,
        "device_loop": {"us_per_token": round(dev_ms * 1e3, 2),
                        "us_per_token_min": round(min(dl) * 1e3, 2),
                        "tok_s": round(1e3 / dev_ms, 1),
                        "bytes_per_token": int(b_tok),
                        "hbm_gbs": round(dev_gbs, 1),
                        "hbm_frac": round(dev_gbs / PEAK_HBM_GBS, 4)},
        "device_loop_cache_flushed": {"us_per_token": round(cold_ms * 1e3, 2),
                                      "hbm_gbs": round(cold_gbs, 1),
                                      "hbm_frac": round(cold_gbs / PEAK_HBM_GBS, 4),
                                      "flush": "512 MiB device copy before each step, outside the timed region"},
        "roofline": roofline,
        "copy_gbs": round(copy_gbs, 1),
        "kernels": kernels,
        "cpu_baseline": cpu,
        "configs": configs,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
