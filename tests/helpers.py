"""Shared helpers for the GPU parity tests."""

from __future__ import annotations

import sys
from typing import List, Sequence, Tuple

import numpy as np

import oracle
import synth

# Logits tolerance: element-wise |gpu - ref| <= ATOL + RTOL * |ref|.
ATOL = 2e-3
RTOL = 1e-3


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def assert_logits_close(gpu: np.ndarray, ref: np.ndarray, what: str = "") -> float:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape
    assert np.isfinite(gpu).all(), f"{what}: non-finite GPU logits"
    err = np.abs(gpu - ref)
    bound = ATOL + RTOL * np.abs(ref)
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} logits out of tolerance, max abs err "
                           f"{err.max():.3g} at {int(err.argmax())}")
    return float(err.max())


def top2_gap(lg: np.ndarray) -> float:
    s = np.sort(np.asarray(lg, dtype=np.float64))
    return float(s[-1] - s[-2])


def gpu_model(model: synth.Model, device: str = "cuda:0"):
    from quantized_q8_gemv_amd.model import Q8Model
    return Q8Model(synth.shape_fields(model.shape), model.tensors, device=device)


def compare_generation(gm, om: oracle.OracleModel, prompt: Sequence[int], steps: int,
                       what: str) -> Tuple[List[int], float, int]:
    """Prefill + greedy decode on both sides; logits checked every step.

    Greedy ids must match. If they diverge where the oracle's top-2 gap is
    within the observed error (a near tie), the divergence is reported and
    both sides continue with the oracle's id. Returns (ids, max abs error,
    number of near-tie divergences).
    """
    lg_g, id_g = gm.forward(prompt, 0)
    st, lg_o, _ = om.forward(prompt, 0)
    assert st == oracle.OK
    worst = assert_logits_close(lg_g, lg_o, f"{what} prefill")
    ids, ties = [], 0
    pos = len(prompt)
    for k in range(steps + 1):
        id_o = oracle.argmax(lg_o)
        if id_g != id_o:
            gap = top2_gap(lg_o)
            err = float(np.max(np.abs(lg_g.astype(np.float64) - lg_o)))
            assert gap <= err, f"{what} step {k}: greedy id {id_g} != oracle {id_o} (gap {gap:.3g})"
            ties += 1
            log(f"{what} step {k}: near-tie divergence (gap {gap:.3g} <= err {err:.3g})")
        ids.append(id_o)
        if k == steps:
            break
        lg_g, id_g = gm.forward([id_o], pos + k)
        st, lg_o, _ = om.forward([id_o], pos + k)
        assert st == oracle.OK
        worst = max(worst, assert_logits_close(lg_g, lg_o, f"{what} decode {k}"))
    return ids, worst, ties
