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

TOL = {"fp8": 2e-2, "fp8_ue8m0": 2e-2, "mxfp4": 6e-2}


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


def assert_rows_close(out: np.ndarray, ref: np.ndarray, mode: str, what: str = "", allowance=None):
    """max_h (|out - ref| - allowance) per row <= TOL * row RMS of ref.
    ``allowance`` [rows, H] (default 0) is what re-quantisation ties may add
    (see requant_tie_allowance)."""
    if allowance is not None:
        dev = np.maximum(np.abs(out.astype(np.float64) - ref.astype(np.float64)) - allowance, 0.0)
        out = ref.astype(np.float64) + dev
    rel = row_errors(out, ref)
    worst = float(rel.max()) if rel.size else 0.0
    log(f"  {what} max row error / rms = {worst:.3e} (tol {TOL[mode]:.0e}) over {rel.size} rows")
    assert worst <= TOL[mode], f"{what}: max |out-ref|/rms = {worst} > {TOL[mode]}"


TIE_EPS = 1e-4  # relative distance to a rounding midpoint at which the code is a tie


def _tie_deltas(v: np.ndarray, grid: np.ndarray, eps: float):
    """For |v| against the positive code grid: the grid spacing where |v| lies
    within eps*|v| of a rounding midpoint (either neighbour is then a correct
    code), else 0."""
    mag = np.abs(v.astype(np.float64))
    mids = (grid[:-1] + grid[1:]) / 2
    gaps = grid[1:] - grid[:-1]
    i = np.clip(np.searchsorted(mids, mag), 1, len(mids) - 1)
    d_lo, d_hi = np.abs(mag - mids[i - 1]), np.abs(mids[i] - mag)
    near = np.where(d_lo < d_hi, i - 1, i)
    dist = np.minimum(d_lo, d_hi)
    return np.where((mag > 0) & (dist <= eps * mag), gaps[near], 0.0)


def requant_tie_allowance(stages, Q: O.QuantWeights, mode: str, hidden: int, eps: float = TIE_EPS):
    """Per output element, the largest change that intermediate codes at a
    rounding tie can make.  The oracle's GEMM1 sums in fp32 in one order, the
    kernel in another; where a SwiGLU value lies within ``eps`` (relative) of
    a rounding midpoint of its re-quantisation (an E4M3 code, or an E2M1 code
    and, when the group's amax is that close to a power of two, its E8M0
    exponent), either result is correct.  Its effect on token t is bounded by
    w[t,j] * |delta a_i| * |w2[e][:, i]| summed over the tied values.
    Returns float64 [tokens, hidden]."""
    ids, wts = stages["ids"], stages["weights"]
    n = ids.shape[0]
    bound = np.zeros((n, Q.w2.shape[1]), np.float64)
    w2abs = {}
    e4 = O.e4m3_value_table()
    g8 = np.unique(np.abs(e4[np.isfinite(e4)]))
    g4 = np.unique(np.abs(O.e2m1_value_table()))
    for (t, j), a in stages["a"].items():
        e = int(ids[t, j])
        if e not in w2abs:
            w2abs[e] = np.abs(O.dequant_expert(Q, e)[1].astype(np.float64))
        a = np.asarray(a, np.float32)
        delta = np.zeros(a.shape, np.float64)
        if mode == "fp8":
            for g0 in range(0, a.size, 128):
                grp = a[g0:g0 + 128]
                amax = float(np.max(np.abs(grp)))
                if amax == 0:
                    continue
                s = np.float32(amax / np.float32(448.0))
                delta[g0:g0 + 128] = _tie_deltas(grp / s, g8, eps) * float(s)
        elif mode == "fp8_ue8m0":
            for g0 in range(0, a.size, 128):
                grp = a[g0:g0 + 128].astype(np.float64)
                amax = float(np.max(np.abs(grp)))
                if amax == 0:
                    continue
                sc = 2.0 ** (int(O.ue8m0_scale_byte(amax)) - 127)
                d = _tie_deltas(grp / sc, g8, eps) * sc
                m = np.log2(amax / 448.0)
                if abs(m - np.round(m)) <= eps:
                    # amax sits at a power-of-two boundary of the scale: every
                    # code may move by one step of the larger scale
                    d = np.maximum(d, 2.0 * sc * 32.0 * (np.abs(grp) > 0))
                delta[g0:g0 + 128] = d
        else:
            for g0 in range(0, a.size, 32):
                grp = a[g0:g0 + 32].astype(np.float64)
                amax = float(np.max(np.abs(grp)))
                if amax == 0:
                    continue
                b = int(O.e8m0_scale_byte(amax))
                sc = 2.0 ** (b - 127)
                d = _tie_deltas(grp / sc, g4, eps) * sc
                m = np.log2(amax)
                if abs(m - np.round(m)) <= eps:
                    # the shared exponent itself is a tie: every code may move by up to one
                    # grid step of the larger of the two scales
                    d = np.maximum(d, 2.0 * sc * np.max(np.diff(g4)) * (np.abs(grp) > 0))
                delta[g0:g0 + 32] = d
        if np.any(delta):
            bound[t] += float(wts[t, j]) * (w2abs[e] @ delta)
    return bound[:, :hidden]


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


def check_gemm1_intermediate(wl: W.Workload, aq, as_, sid, npp, stages):
    """GEMM1's re-quantised intermediate (aq/as, rows by sorted position)
    against the oracle's stages: pad rows are all zero; a code may differ
    from the oracle's only by one step at a rounding boundary (the fp32
    summation order of GEMM1 differs), an FP8 scale by its own rounding, and a
    UE8M0 scale by one binade at a tie, rarely."""
    mode = wl.mode
    sid_h = sid.cpu().numpy()
    P = wl.T * wl.top_k
    rows = aq.numel() // (wl.Ip if mode != "mxfp4" else wl.Ip // 2)
    aq_h = aq.cpu().numpy().reshape(rows, -1)
    if mode == "fp8":
        as_h = as_.cpu().numpy().view(np.float32).reshape(rows, -1)
    elif mode == "fp8_ue8m0":
        as_h = as_.cpu().numpy().reshape(rows, -1)[:, :wl.Ip // 128]
    else:
        as_h = as_.cpu().numpy().reshape(rows, -1)
    total = mism = scale_moves = 0
    worst_scale = worst_val = 0.0
    for r in range(int(npp.item())):
        f = int(sid_h[r])
        if f >= P:
            assert np.all(aq_h[r] == 0) and np.all(as_h[r] == 0), "pad rows are zero"
            continue
        qo, so = stages["aq"][(f // wl.top_k, f % wl.top_k)]
        if mode == "fp8":
            # the scale is amax/448 of the fp32 intermediate: it inherits the
            # GEMM's accumulation-order difference
            rel = np.abs(as_h[r].astype(np.float64) - so) / np.maximum(so, 1e-30)
            worst_scale = max(worst_scale, float(rel.max()))
            dg = O.dequant_fp8_rows(aq_h[r][None], as_h[r][None])[0]
            do = O.dequant_fp8_rows(qo[None], so[None])[0]
            step = 32.0 / 448.0          # one code step at the top binade, relative to amax
        elif mode == "fp8_ue8m0":
            # a power-of-two scale: only an amax at a scale boundary (a tie) may
            # move it, by one binade
            dsc = np.abs(as_h[r].astype(np.int64) - so.astype(np.int64))
            assert dsc.max() <= 1
            scale_moves += int(np.count_nonzero(dsc))
            dg = O.dequant_fp8e8_rows(aq_h[r][None], as_h[r][None])[0]
            do = O.dequant_fp8e8_rows(qo[None], so[None])[0]
            # one top-binade step of the larger scale, relative to the
            # smallest amax a scale covers (224 * 2^e)
            step = 2 * 32.0 / 224.0 if dsc.max() else 32.0 / 224.0
        else:
            dg = O.dequant_mxfp4_rows(aq_h[r][None], as_h[r][None])[0]
            do = O.dequant_mxfp4_rows(qo[None], so[None])[0]
            step = 2.0 / 4.0             # E2M1 step 2 at the top, amax >= 4 units
        amax = np.abs(do).max()
        total += aq_h[r].size
        mism += int(np.count_nonzero(aq_h[r] != qo))
        if amax > 0:
            worst_val = max(worst_val, float(np.abs(dg - do).max() / amax) / step)
    log(f"  intermediate: {mism} of {total} code bytes differ; worst |deq diff|/(amax*step) {worst_val:.3e}; "
        f"worst FP8 scale rel diff {worst_scale:.2e}")
    # accumulation-order differences move a code by at most one step at a rounding boundary
    assert worst_val <= 1.01
    assert mism <= max(8, 0.01 * total)
    assert worst_scale <= 1e-3
    assert scale_moves <= 4
