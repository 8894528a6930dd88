"""Shared helpers of the GPU parity tests: inputs from the seeded workloads,
the oracle's own quantisation of the same raw weights, the check of GEMM1's
re-quantised intermediate, and the per-row tolerance check of the output.
The oracle never receives anything the HIP path produced.

The intermediate check.  GEMM1's fp32 sums run in another order on the GPU
than in the oracle, so a re-quantised code may legitimately differ from the
oracle's where the SwiGLU value sits at a rounding midpoint, and a group
scale may move where the group's largest value sits at a scale boundary.
``verify_intermediate`` accepts such a difference only when it is explained
by the two fp32 computations' error bound for that element:

  |h_gpu - h_oracle| <= C_ACC * u * sum_k |x_k w_k| + |h_oracle - h_exact|

with u = 2^-24, h_exact the fp64 sum of the same dequantised operands (the
oracle's own error is measured against it) and C_ACC covering the GPU's
summation structure: 32 K blocks of 128 added in fp32, each the sum of at
most 4 chained MFMAs whose internal sums stay within ~3u of sum |ab|, times
one scale product (first-order bound (31 + 12 + 2) u sum |ab| < 64 u sum |ab|,
plus the K split's piece sums).  The bound goes through the clamped SwiGLU
(silu is 1.1-Lipschitz; min and clamp are 1-Lipschitz), plus a few ulp for
each side's own silu evaluation, and into code units with the group scale.
Every code the kernel produced must then be the oracle's rounding of the
oracle's value under the kernel's scale, or one step away from it with that
value within the bound of the midpoint; every scale must be the oracle's, or
(fp32 scale) within its bound, or (power-of-two scale) one binade away with
the group's largest value within its bound of that binade's boundary.

The end-to-end allowance is then built from the intermediate differences
that actually occurred: per output element, sum_j w[t,j] * |w2_e| . |deq_gpu
- deq_oracle| of pair (t, j).  Nothing else widens the 2e-2 / 6e-2 bound.
"""
from __future__ import annotations

import functools
import os
import sys

import numpy as np
import torch

import oracle as O
import workloads as W

TOL = {"fp8": 2e-2, "fp8_ue8m0": 2e-2, "mxfp4": 6e-2}
U32 = 2.0 ** -24      # fp32 unit roundoff
C_ACC = 64            # GEMM1 sum: |h_gpu - h_exact| <= C_ACC * u * sum |x w| (see above)
EPI = 32 * U32        # relative error of either side's clamped SwiGLU evaluation
SILU_LIP = 1.1        # max |silu'(g)| = 1.0998...


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


# One line per checked output (test id, what was compared), printed by the
# terminal summary hook in conftest.py so that every run's log shows the
# intermediate flips and the share of the tolerance they took.
SUMMARY = []
_LAST_REPORT = {}


def _note(line: str):
    test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0].split("::")[-1]
    SUMMARY.append(f"{test}: {line}")


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
    ``allowance`` [rows, H] (default 0) is the effect of the intermediate
    codes the kernel verifiably rounded the other way (see
    verify_intermediate); the log gives the largest share of the
    tolerance it took."""
    ref64 = ref.astype(np.float64)
    out_in = out
    share = 0.0
    if allowance is not None:
        dev = np.maximum(np.abs(out.astype(np.float64) - ref64) - allowance, 0.0)
        rms = np.sqrt(np.mean(ref64 ** 2, axis=1))
        amax = allowance.max(axis=1) if allowance.size else np.zeros(len(ref64))
        with np.errstate(divide="ignore", invalid="ignore"):
            sh = np.where(rms > 0, amax / (TOL[mode] * rms), np.where(amax == 0, 0.0, np.inf))
        share = float(sh.max()) if sh.size else 0.0
        out = ref64 + dev
    raw = row_errors(np.asarray(out_in, np.float64), ref)
    rel = row_errors(out, ref)
    worst = float(rel.max()) if rel.size else 0.0
    worst_raw = float(raw.max()) if raw.size else 0.0
    log(f"  {what} max row error / rms = {worst:.3e} (tol {TOL[mode]:.0e}) over {rel.size} rows; "
        f"allowance took at most {share:.2%} of the tolerance (without it {worst_raw:.3e})")
    rep = _LAST_REPORT.get(os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0])
    flips = (f"{rep.code_flips} codes differ, {rep.tie_flips} verified ties (<= {rep.rel_to_mid:.1e} rel.), "
             f"{rep.scale_moves} scales" if rep is not None else "no intermediate check")
    _note(f"{what}: err {worst:.2e}/{TOL[mode]:.0e} of rms ({worst_raw:.2e} raw), {flips}, "
          f"allowance <= {share:.0%} of tol")
    assert worst <= TOL[mode], f"{what}: max |out-ref|/rms = {worst} > {TOL[mode]}"


# ----------------------------------------------------------------------------
# GEMM1 intermediate: what the kernel wrote, and its check
# ----------------------------------------------------------------------------

def _group(mode: str) -> int:
    return 32 if mode == "mxfp4" else 128


def _code_values(mode: str) -> np.ndarray:
    return O.e2m1_value_table() if mode == "mxfp4" else O.e4m3_value_table()


def _code_pos(mode: str, c: np.ndarray) -> np.ndarray:
    """Position of a code on the signed number line: magnitude code + 0.5,
    negated for a set sign bit (-0 and +0 are neighbours; adjacent codes are
    one apart)."""
    c = c.astype(np.int64)
    if mode == "mxfp4":
        mag, neg = c & 0x7, (c >> 3) & 1
    else:
        mag, neg = c & 0x7F, (c >> 7) & 1
    return np.where(neg == 1, -(mag + 0.5), mag + 0.5)


def _round_codes(mode: str, v: np.ndarray) -> np.ndarray:
    if mode == "mxfp4":
        return O.round_to_e2m1(np.clip(v, -O.E2M1_MAX, O.E2M1_MAX))
    return O.round_to_e4m3(np.clip(v, -O.E4M3_MAX, O.E4M3_MAX))


def gpu_intermediate_rows(mode: str, Ip: int, aq, as_, sid, npp, num_pairs: int, top_k: int, pairs):
    """The kernel's re-quantised intermediate for the listed pairs.

    ``aq``/``as_`` are GEMM1's outputs (rows by sorted position), ``sid`` the
    sorted pair ids and ``pairs`` a dict {(sample index, slot): flat pair f}.
    Pad rows (sorted ids >= P) below num_post_padded must be all zero.
    ``sid`` None: the rows are in pair order (the decode kernels' layout).
    Returns {(sample index, slot): (element codes uint8 [Ip], scale bytes
    [groups] as stored: float32 bits or E8M0)}."""
    row_bytes = Ip // 2 if mode == "mxfp4" else Ip
    aq_h = aq.cpu().numpy().reshape(-1)
    as_h = as_.cpu().numpy().reshape(-1)
    rows_total = aq_h.size // row_bytes
    aq_h = aq_h[:rows_total * row_bytes].reshape(rows_total, row_bytes)
    if mode == "fp8":
        as_h = as_h[:rows_total * (Ip // 128) * 4].view(np.float32).reshape(rows_total, Ip // 128)
    elif mode == "fp8_ue8m0":
        as_h = as_h[:rows_total * M_e8_ld(Ip)].reshape(rows_total, M_e8_ld(Ip))[:, :Ip // 128]
    else:
        as_h = as_h[:rows_total * (Ip // 32)].reshape(rows_total, Ip // 32)
    if sid is None:
        row_of = {f: f for f in range(num_pairs)}
    else:
        sid_h = sid.cpu().numpy()
        nrows = int(npp.item()) if torch.is_tensor(npp) else int(npp)
        live = sid_h[:nrows]
        pad = live >= num_pairs
        assert np.all(aq_h[:nrows][pad] == 0) and np.all(as_h[:nrows][pad] == 0), "pad rows are not zero"
        real = np.nonzero(~pad)[0]
        row_of = dict(zip(live[real].tolist(), real.tolist()))
    out = {}
    for key, f in pairs.items():
        r = row_of[f]
        codes = O.unpack_e2m1(aq_h[r][None])[0] if mode == "mxfp4" else aq_h[r].copy()
        out[key] = (codes, as_h[r].copy())
    return out


def M_e8_ld(cols_padded: int) -> int:
    """Row stride in bytes of UE8M0 activation-scale rows (whole dwords)."""
    return (cols_padded // 128 + 3) // 4 * 4


class IntermediateReport:
    def __init__(self):
        self.pairs = 0
        self.codes = 0
        self.code_flips = 0          # codes that differ from the oracle's (any reason)
        self.tie_flips = 0           # ... not explained by a moved scale: verified ties
        self.scale_moves = 0         # scales that differ from the oracle's
        self.window_used = 0.0       # largest |v - midpoint| / bound over the tie flips
        self.rel_to_mid = 0.0        # largest |v - midpoint| / |v| over the tie flips
        self.scale_window_used = 0.0

    def __str__(self):
        return (f"{self.pairs} pairs, {self.codes} codes: {self.code_flips} differ from the oracle "
                f"({self.tie_flips} verified rounding ties, at most {self.rel_to_mid:.1e} (relative) from the "
                f"midpoint, {self.window_used:.2f} of the element bound); {self.scale_moves} scales differ "
                f"(at most {self.scale_window_used:.2f} of the bound)")


def verify_pair(mode: str, limit: float, gpu_codes, gpu_scales, h_o, h_exact, habs, a_o, q_o, s_o,
                report: IntermediateReport):
    """Checks one pair's intermediate (see the module docstring); returns the
    elementwise |deq_gpu - deq_oracle| (float64 [Ip])."""
    G = _group(mode)
    Ip = a_o.size
    ng = Ip // G
    vmax = O.E2M1_MAX if mode == "mxfp4" else O.E4M3_MAX
    vals = _code_values(mode)
    magmask = 0x7 if mode == "mxfp4" else 0x7F
    codes_o = (O.unpack_e2m1(np.asarray(q_o)[None])[0] if mode == "mxfp4" else np.asarray(q_o)).reshape(ng, G)
    cg = np.asarray(gpu_codes).reshape(ng, G)
    h_o = np.asarray(h_o, np.float32).astype(np.float64)
    a = np.asarray(a_o, np.float32).astype(np.float64)
    # bound on |a_gpu - a_oracle| per element
    bh = C_ACC * U32 * habs + np.abs(h_o - h_exact)
    bg, bu = bh[:Ip], bh[Ip:]
    L = float(limit)
    gc = np.minimum(h_o[:Ip], L)
    uc = np.clip(h_o[Ip:], -L, L)
    with np.errstate(over="ignore"):
        sg = gc / (1.0 + np.exp(-gc))
    da = SILU_LIP * bg * (np.abs(uc) + bu) + np.abs(sg) * bu + (EPI + 2 * U32 * np.abs(gc)) * np.abs(a)
    a, da = a.reshape(ng, G), da.reshape(ng, G)
    amax = np.max(np.abs(a), axis=1)
    damax = np.max(da, axis=1)
    report.pairs += 1
    report.codes += Ip
    # the scales
    gs = np.asarray(gpu_scales)
    so = np.asarray(s_o)
    if mode == "fp8":
        sv_g = gs.astype(np.float32).astype(np.float64)
        sv_o = so.astype(np.float32).astype(np.float64)
        bound = damax / O.E4M3_MAX + 2 * U32 * sv_o
        d = np.abs(sv_g - sv_o)
        moved = d > 0
        assert np.all(d <= bound), f"fp32 scales {sv_g[d > bound]} vs {sv_o[d > bound]} beyond {bound[d > bound]}"
        if moved.any():
            report.scale_window_used = max(report.scale_window_used, float(np.max(d[moved] / bound[moved])))
    else:
        bgb, bob = gs.astype(np.int64), so.astype(np.int64)
        sv_g, sv_o = np.ldexp(1.0, bgb - 127), np.ldexp(1.0, bob - 127)
        moved = bgb != bob
        if moved.any():
            assert np.all(np.abs(bgb - bob)[moved] == 1) and np.all(np.minimum(bgb, bob)[moved] > 0), \
                f"scale bytes {bgb[moved]} vs {bob[moved]}"
            e_lo = np.minimum(bgb, bob)[moved] - 127
            edge = np.ldexp(O.E4M3_MAX, e_lo) if mode == "fp8_ue8m0" else np.ldexp(1.0, e_lo + 3)
            dist = np.abs(amax[moved] - edge)
            assert np.all(dist <= damax[moved]), (f"scale bytes {bgb[moved]} vs {bob[moved]}: amax "
                                                  f"{amax[moved]} is {dist} from the boundary {edge} "
                                                  f"(bound {damax[moved]})")
            report.scale_window_used = max(report.scale_window_used,
                                           float(np.max(dist / np.maximum(damax[moved], 1e-300))))
    report.scale_moves += int(np.count_nonzero(moved))
    # an all-zero group: zero scale and zero code magnitudes on both sides
    zero_o = amax == 0
    zero_g = (sv_g == 0) if mode == "fp8" else (gs.astype(np.int64) == 0)
    both0 = zero_o & zero_g
    assert np.all((cg[both0] & magmask) == 0), "an all-zero group has non-zero codes"
    if mode == "fp8":
        assert np.all(amax[zero_g] <= damax[zero_g]), "zero fp32 scale for a group that is not zero"
    # the codes, under the kernel's scale
    live = ~both0
    sig = np.where(sv_g > 0, sv_g, 1.0)[:, None]
    if mode == "fp8":   # the oracle's own arithmetic: an fp32 quotient (power-of-two scales divide exactly)
        v = (a.astype(np.float32) / sig.astype(np.float32)).astype(np.float64)
    else:
        v = a / sig
    v = np.clip(v, -vmax, vmax)
    ref = _round_codes(mode, v)
    bad = (cg != ref) & live[:, None]
    if bad.any():
        dv = da[bad] / sig.repeat(G, axis=1)[bad] + 4 * U32 * np.abs(v[bad])
        adj = np.abs(_code_pos(mode, cg[bad]) - _code_pos(mode, ref[bad])) == 1
        assert np.all(adj), f"codes {cg[bad][~adj]} more than one step from the oracle's rounding {ref[bad][~adj]}"
        mid = (vals[cg[bad]] + vals[ref[bad]]) / 2
        dist = np.abs(v[bad] - mid)
        ok = dist <= dv
        assert np.all(ok), (f"code(s) {cg[bad][~ok]} vs {ref[bad][~ok]} at value(s) {v[bad][~ok]} are "
                            f"{dist[~ok]} from the midpoint, beyond the element bound {dv[~ok]}")
        report.tie_flips += int(np.count_nonzero(bad))
        report.window_used = max(report.window_used, float(np.max(dist / dv)))
        report.rel_to_mid = max(report.rel_to_mid, float(np.max(dist / np.maximum(np.abs(v[bad]), 1e-300))))
    report.code_flips += int(np.count_nonzero(cg != codes_o))
    sv_g0 = np.where(both0, 0.0, sv_g)[:, None]
    sv_o0 = np.where(zero_o, 0.0, sv_o)[:, None]
    return np.abs(vals[cg] * sv_g0 - vals[codes_o] * sv_o0).reshape(-1)


def verify_intermediate(mode: str, limit: float, gpu_rows, stages, Q: O.QuantWeights, hidden: int):
    """Checks every pair of ``gpu_rows`` against the oracle's stages (see the
    module docstring) and returns (allowance float64 [sample tokens, hidden],
    report).  One pass per expert: its weights are dequantised once for the
    exact GEMM1 reference (fp64 sums of the dequantised operands) and for
    |w2| of the allowance."""
    ids, wts = stages["ids"], stages["weights"]
    xd = O.dequant_act(mode, stages["xq"], stages["xs"]).astype(np.float64)
    n = ids.shape[0]
    allowance = np.zeros((n, Q.w2.shape[1]), np.float64)
    report = IntermediateReport()
    by_expert = {}
    for (t, j) in gpu_rows:
        by_expert.setdefault(int(ids[t, j]), []).append((t, j))
    for e, keys in sorted(by_expert.items()):
        w13d, w2d = O.dequant_expert(Q, e)
        w64 = w13d.astype(np.float64)
        X = xd[[t for t, _ in keys]]
        hx = X @ w64.T
        habs = np.abs(X) @ np.abs(w64).T
        del w64
        w2abs = None
        for i, (t, j) in enumerate(keys):
            q_o, s_o = stages["aq"][(t, j)]
            cg, sg = gpu_rows[(t, j)]
            d = verify_pair(mode, limit, cg, sg, stages["h"][(t, j)], hx[i], habs[i], stages["a"][(t, j)], q_o,
                            s_o, report)
            if np.any(d):
                if w2abs is None:
                    w2abs = np.abs(w2d.astype(np.float64))
                allowance[t] += float(wts[t, j]) * (w2abs @ d)
    log(f"  intermediate: {report}")
    _LAST_REPORT[os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]] = report
    return allowance[:, :hidden], report


def pairs_of(tokens, top_k: int):
    """{(sample index, slot): flat pair index} of the sample tokens."""
    return {(i, j): int(t) * top_k + j for i, t in enumerate(tokens) for j in range(top_k)}


def check_intermediate_and_output(wl: W.Workload, out_rows: np.ndarray, aq, as_, sid, npp, ref, stages, Q,
                                  tokens=None, what: str = ""):
    """The kernel's intermediate (aq/as from GEMM1, rows by sorted position)
    against the oracle's stages, then the output rows of the sample
    (``out_rows`` [len(tokens), H], float32 of the bf16 output) against the
    oracle's within the mode's tolerance plus the effect of the intermediate
    differences that occurred.  ``tokens``: the sample (default all)."""
    toks = list(range(wl.T)) if tokens is None else list(tokens)
    rows = gpu_intermediate_rows(wl.mode, wl.Ip, aq, as_, sid, npp, wl.T * wl.top_k, wl.top_k,
                                 pairs_of(toks, wl.top_k))
    allowance, report = verify_intermediate(wl.mode, wl.swiglu_limit, rows, stages, Q, wl.H)
    assert_rows_close(out_rows, ref, wl.mode, what or wl.name, allowance=allowance)
    return report


def gpu_stage_chain(M, cfg, T: int, x_dev, lg_dev, ew, ksplit1=None):
    """The layer through the stage entry points, with the splits moe_forward
    plans: the front end (routing, permutation, quantisation of x), GEMM1 and
    GEMM2 + combine.  Returns a dict with the intermediate (aq, as_, sid,
    npp), the quantised x (xq, xs), routing (ids, w) and the output."""
    ids, w, sid, bexp, offs, npp, xq, xs = M.moe_route_permute_quant(cfg, x_dev, lg_dev)
    ks = M.plan_ksplit(cfg, T, 13) if ksplit1 is None else ksplit1
    aq, as_ = M.moe_grouped_gemm1_swiglu(cfg, T, xq, xs, sid, bexp, npp, ew.w13, ew.w13_scale, ksplit=ks)
    out = M.moe_grouped_gemm2_combine(cfg, T, aq, as_, sid, bexp, npp, ew.w2, ew.w2_scale, w)
    return dict(ids=ids, w=w, sid=sid, bexp=bexp, npp=npp, xq=xq, xs=xs, aq=aq, as_=as_, out=out)


def oracle_stages(wl: W.Workload, x: torch.Tensor, lg: torch.Tensor, Q: O.QuantWeights, tokens=None):
    """The oracle's output rows and stages on the (host copies of the) same
    inputs, for the sample tokens (default all)."""
    return O.moe_forward(x.float().cpu().numpy(), lg.cpu().numpy(), Q, wl.top_k, wl.swiglu_limit, wl.H, wl.I,
                         tokens=tokens, return_stages=True)


def decode_chain(M, cfg, x_dev, lg_dev, ew):
    """The decode entry points on the front end's routing and quantised x:
    moe_decode_gemm1_swiglu, then moe_decode_gemm2_combine.  Returns a dict
    with the routing (ids, w), the fp32 SwiGLU rows a32, the intermediate
    in pair order (aq, as_; sid None) and the output."""
    ids, w, sid, bexp, offs, npp, xq, xs = M.moe_route_permute_quant(cfg, x_dev, lg_dev)
    a32 = M.moe_decode_gemm1_swiglu(cfg, xq, xs, ids, ew.w13, ew.w13_scale)
    aq_b, as_b = M.decode_intermediate_bytes(cfg, x_dev.shape[0])
    aq = torch.zeros(aq_b, dtype=torch.uint8, device=a32.device)
    as_ = torch.zeros(as_b, dtype=torch.uint8, device=a32.device)
    out = M.moe_decode_gemm2_combine(cfg, a32, ids, w, ew.w2, ew.w2_scale, aq=aq, as_=as_)
    return dict(ids=ids, w=w, a32=a32, sid=None, npp=None, aq=aq, as_=as_, out=out, xq=xq, xs=xs)


def check_forward(M, wl: W.Workload, cfg, ew, x_dev, lg_dev, out, Q, tokens=None, what: str = ""):
    """moe_forward's output ``out`` equals the stage chain bit for bit; the
    chain's intermediate passes verify_intermediate; the sample rows of out
    match the oracle's within the tolerance plus the effect of the
    intermediate differences that occurred."""
    ch = gpu_stage_chain(M, cfg, wl.T, x_dev, lg_dev, ew)
    torch.cuda.synchronize()
    assert torch.equal(out.contiguous().view(torch.int16), ch["out"].view(torch.int16)), \
        "moe_forward differs from the stage entry points"
    ref, st = oracle_stages(wl, x_dev, lg_dev, Q, tokens)
    toks = list(range(wl.T)) if tokens is None else list(tokens)
    return check_intermediate_and_output(wl, bf16_to_f32(out)[toks], ch["aq"], ch["as_"], ch["sid"], ch["npp"], ref,
                                         st, Q, tokens=toks, what=what)


# ----------------------------------------------------------------------------
# Weights and inputs
# ----------------------------------------------------------------------------

@functools.lru_cache(maxsize=4)
def oracle_weights_cpu(wl: W.Workload) -> O.QuantWeights:
    """Oracle-quantised weights of a small workload drawn on the host."""
    w13 = W.all_w13(wl).numpy()
    w2 = W.all_w2(wl).numpy()
    return O.quantize_weights(wl.mode, w13, w2)


_QCACHE = {}


def _weight_key(wl: W.Workload, device: str):
    return (wl.H, wl.I, wl.Hp, wl.Ip, wl.E, wl.mode, wl.seed, str(device))


def oracle_weights_subset(wl: W.Workload, experts, device) -> O.QuantWeights:
    """Oracle-quantised weights for the listed experts (others zero-filled),
    raw values drawn with the workload's generators on ``device``.  Experts
    already quantised for a workload with the same weights are reused; new
    ones are quantised by the oracle on host threads (NumPy releases the GIL
    in its array operations), one expert per task."""
    key = _weight_key(wl, device)
    if key not in _QCACHE:
        _QCACHE.clear()
        E, Hp, Ip = wl.E, wl.Hp, wl.Ip
        if wl.mode == "mxfp4":
            arrs = (np.zeros((E, 2 * Ip, Hp // 2), np.uint8), np.zeros((E, 2 * Ip, Hp // 32), np.uint8),
                    np.zeros((E, Hp, Ip // 2), np.uint8), np.zeros((E, Hp, Ip // 32), np.uint8))
        else:
            sdt = np.float32 if wl.mode == "fp8" else np.uint8
            arrs = (np.zeros((E, 2 * Ip, Hp), np.uint8), np.zeros((E, 2 * Ip // 128, Hp // 128), sdt),
                    np.zeros((E, Hp, Ip), np.uint8), np.zeros((E, Hp // 128, Ip // 128), sdt))
        _QCACHE[key] = (O.QuantWeights(wl.mode, *arrs), set())
    Q, done = _QCACHE[key]
    todo = sorted(set(int(e) for e in experts) - done)
    if todo:
        from oracle.from_workload import quantize_experts
        part = quantize_experts(wl, todo, device)
        for e in todo:
            Q.w13[e], Q.s13[e], Q.w2[e], Q.s2[e] = part.w13[e], part.s13[e], part.w2[e], part.s2[e]
        del part
        done.update(todo)
    return Q


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
