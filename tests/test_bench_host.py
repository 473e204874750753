"""Host-side logic of bench.py that needs no GPU: the counter summary that
turns two rocprofv3 --pmc runs into per-launch traffic of the decode kernels."""

import csv
import io
import os
import sys
from contextlib import redirect_stdout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402

FIELDS = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write(dirname, counter, rows):
    os.makedirs(dirname, exist_ok=True)
    with open(os.path.join(dirname, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Correlation_Id": i + 1, "Dispatch_Id": i + 1, "Kernel_Name": name,
                        "Counter_Name": counter, "Counter_Value": value})


def _dispatches(values, names):
    """One decode layer's dispatch sequence with the given counter values,
    between two 1 GiB copies (the reference dispatches)."""
    seq = [("__amd_rocclr_copyBuffer", values["copy"])]
    seq += [(names[k], values[k]) for k in ("embed", "qkv", "attn", "o", "gateup", "down", "lm") if k in names]
    seq += [("__amd_rocclr_copyBuffer", values["copy"]),
            ("__amd_rocclr_copyBuffer", values["copy"] / 2),  # a 512 MiB cache-flush copy: not a reference
            ("__amd_rocclr_copyBuffer", 3.0)]  # a small upload copy: not a reference dispatch
    if "sum" in values:  # the read-only reference: a 1 GiB f32 sum
        seq += [("void at::native::reduce_kernel<512, 1>(at::native::ReduceOp<float>)", values["sum"])]
    return seq


NS = "void q8l::(anonymous namespace)::"
FETCH = {"copy": 524288.0, "sum": 524800.0, "embed": 2.0, "qkv": 400.0, "attn": 30.0, "o": 280.0, "gateup": 1000.0,
         "down": 570.0, "lm": 15000.0}
WRITE = {"copy": 1048576.0, "embed": 1.0, "qkv": 8.0, "attn": 2.0, "o": 4.0, "gateup": 12.0,
         "down": 9.0, "lm": 270.0}


def _summary(tmp_path, names):
    _write(str(tmp_path / "f"), "FETCH_SIZE", _dispatches(FETCH, names))
    _write(str(tmp_path / "w"), "WRITE_SIZE", _dispatches(WRITE, names))
    buf = io.StringIO()
    with redirect_stdout(buf):
        bench.pmc_summary(str(tmp_path / "f"), str(tmp_path / "w"), config="C2")
    out = buf.getvalue()
    assert "scale FETCH_SIZE 2.0000, WRITE_SIZE 1.0000" in out
    # 524800 KiB * 2 = 1.00098 GiB
    assert "read-only check: a 1 GiB f32 sum reads 1,074,790,400 bytes by the scaled FETCH_SIZE (1.0010 of 1 GiB" in out
    return {l.split()[1].split("=")[1]: l for l in out.splitlines() if l.startswith("traffic:")}


def test_pmc_summary_scales_by_the_copy(tmp_path):
    """The 135M decode layer as it runs: wave-per-row q/k/v, gate/up and down,
    the attention fused with the o-projection, the output layer several rows
    per wave."""
    names = {"embed": NS + "k_embed(unsigned char const*, int)",
             "qkv": NS + "k_wqkv1<9>(q8l::(anonymous namespace)::WQkvArgs)",
             "attn": "q8l::(anonymous namespace)::k_attn_o1(q8l::AttnODecodeArgs)",
             "gateup": NS + "k_wgateup1<9>(q8l::(anonymous namespace)::WGateUpArgs)",
             "down": NS + "k_wmatmul1<24>(q8l::(anonymous namespace)::WMatmulArgs)",
             "lm": NS + "k_xlmhead_short(q8l::(anonymous namespace)::XLmHeadArgs)"}
    lines = _summary(tmp_path, names)
    # bytes = (FETCH KiB * 2 + WRITE KiB * 1) * 1024
    for kind, key in [("qkv_rope_kv", "qkv"), ("attn_decode", "attn"), ("gateup_silu", "gateup"),
                      ("down_residual", "down"), ("lmhead", "lm")]:
        want = int(round((FETCH[key] * 2 + WRITE[key]) * 1024))
        assert f"bytes_per_launch={want} " in lines[kind], (kind, lines[kind])
        src = bench.KIND_SOURCES[kind]
        assert f"sha256={bench.source_digest(src)}" in lines[kind]
    assert "oproj_residual" not in lines


def test_pmc_summary_tells_o_from_down(tmp_path, monkeypatch):
    """Where the o and down projections run the same kernel, a dispatch
    right after the attention is the o-projection."""
    mm = "k_matmul1<false, false>"
    monkeypatch.setattr(bench, "kernel_symbols", lambda s, down_fmt="q8_0", kv_len=1: [
        "k_embed", "k_qkv1<false>", "k_attn_decode", mm, "k_gateup1<false>", mm, "k_lmhead1<false>",
        "k_argmax_finish"])
    names = {"qkv": NS + "k_qkv1<false>(q8l::(anonymous namespace)::QkvArgs)",
             "attn": "q8l::(anonymous namespace)::k_attn_decode(q8l::AttnDecodeArgs)",
             "o": NS + mm + "(q8l::(anonymous namespace)::MatmulArgs)",
             "gateup": NS + "k_gateup1<false>(q8l::(anonymous namespace)::GateUpArgs)",
             "down": NS + mm + "(q8l::(anonymous namespace)::MatmulArgs)"}
    lines = _summary(tmp_path, names)
    for kind, key in [("oproj_residual", "o"), ("down_residual", "down")]:
        want = int(round((FETCH[key] * 2 + WRITE[key]) * 1024))
        assert f"bytes_per_launch={want} " in lines[kind], (kind, lines[kind])


def test_measured_traffic_follows_the_source_digest(tmp_path, monkeypatch):
    path = tmp_path / "t.md"
    src = bench.KIND_SOURCES["gateup_silu"]
    path.write_text(f"traffic: kind=gateup_silu bytes_per_launch=123 source={src} "
                    f"sha256={bench.source_digest(src)}\n"
                    f"traffic: kind=lmhead bytes_per_launch=456 source={src} sha256=0000000000000000\n")
    monkeypatch.setitem(bench.TRAFFIC_FILES, "C2", str(path))
    assert bench.measured_traffic("C2", "gateup_silu") == 123
    assert bench.measured_traffic("C2", "lmhead") is None     # digest of another source: stale
    assert bench.measured_traffic("C2", "embed") is None       # not measured
    assert synth.WORKLOADS["C2"].prompt_len == 13


def test_stats_summary_and_profiled_duration(tmp_path, monkeypatch):
    """--stats-summary turns a kernel_stats.csv into the profiles/ table with
    the sources' digests; profiled_us reads a symbol's mean back only while
    those digests match the sources."""
    stats = tmp_path / "k_kernel_stats.csv"
    with open(stats, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage",
                                          "MinNs", "MaxNs", "StdDev"])
        w.writeheader()
        w.writerow({"Name": "void q8l::(anonymous namespace)::k_gateup1<false>(q8l::(anonymous namespace)::GateUpArgs)",
                    "Calls": 30, "TotalDurationNs": 180000, "AverageNs": 6000.0, "Percentage": 55.0,
                    "MinNs": 5000, "MaxNs": 7000, "StdDev": 1.0})
        w.writerow({"Name": "k_attn_decode(q8l::AttnDecodeArgs)", "Calls": 30, "TotalDurationNs": 120000,
                    "AverageNs": 4000.0, "Percentage": 45.0, "MinNs": 3000, "MaxNs": 5000, "StdDev": 1.0})
    buf = io.StringIO()
    with redirect_stdout(buf):
        bench.stats_summary(str(stats))
    text = buf.getvalue()
    assert "| `k_gateup1<false>` | 30 | 6.00 | 5.00 | 7.00 | 55.00 |" in text
    assert "| `k_attn_decode` | 30 | 4.00 |" in text
    prof = tmp_path / "prof.md"
    prof.write_text(text)
    monkeypatch.setitem(bench.STATS_FILES, "CX", str(prof))
    assert bench.profiled_us("CX", "k_gateup1<false>") == 6.0
    assert bench.profiled_us("CX", "k_missing") is None
    # a changed source makes the table stale
    stale = text.replace(bench.source_digest(bench.STATS_SOURCES[0]), "0" * 16)
    prof.write_text(stale)
    assert bench.profiled_us("CX", "k_gateup1<false>") is None
