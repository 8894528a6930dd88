"""Shared helpers of the GPU parity tests: inputs from the seeded workloads,
the oracle's own quantisation of the same raw weights, and the per-row
tolerance check.  The oracle never receives anything the HIP path produced.
"""
from __future__ import annotations

import functools
import sys

import numpy as np
import torch

import oracle as O
import workloads as W

TOL = {"fp8": 2e-2, "mxfp4": 6e-2}


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def row_errors(out: np.ndarray, ref: np.ndarray):
    """max |out - ref| per row divided by the row RMS of ref (inf where the
    RMS is 0 and the row is not exactly 0)."""
    ref = ref.astype(np.float64)
    err = np.abs(out.astype(np.float64) - ref).max(axis=1)
    rms = np.sqrt(np.mean(ref ** 2, axis=1))
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(rms > 0, err / rms, np.where(err == 0, 0.0, np.inf))
    return rel


def assert_rows_close(out: np.ndarray, ref: np.ndarray, mode: str, what: str = ""):
    rel = row_errors(out, ref)
    worst = float(rel.max()) if rel.size else 0.0
    log(f"  {what} max row error / rms = {worst:.3e} (tol {TOL[mode]:.0e}) over {rel.size} rows")
    assert worst <= TOL[mode], f"{what}: max |out-ref|/rms = {worst} > {TOL[mode]}"


@functools.lru_cache(maxsize=4)
def oracle_weights_cpu(wl: W.Workload) -> O.QuantWeights:
    """Oracle-quantised weights of a small workload drawn on the host."""
    w13 = W.all_w13(wl).numpy()
    w2 = W.all_w2(wl).numpy()
    return O.quantize_weights(wl.mode, w13, w2)


def oracle_weights_subset(wl: W.Workload, experts, device) -> O.QuantWeights:
    """Oracle-quantised weights for the listed experts (others zero-filled),
    raw values drawn with the workload's generators on ``device``."""
    from oracle.from_workload import quantize_experts
    return quantize_experts(wl, experts, device)


def gpu_weights(M, cfg, wl: W.Workload, device="cuda", chunk: int = 16, source: str = "cuda"):
    """Quantised + preshuffled expert weights built by the library from the
    workload's raw weights (drawn on ``source``)."""
    ew = M.ExpertWeights(cfg, device)
    for e0 in range(0, wl.E, chunk):
        ex = range(e0, min(wl.E, e0 + chunk))
        w13 = W.all_w13(wl, ex, source).to(device)
        w2 = W.all_w2(wl, ex, source).to(device)
        ew.add_experts(e0, w13, w2)
        del w13, w2
    return ew.finalize()


def bf16_to_f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()
