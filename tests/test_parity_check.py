"""CPU pins of the GPU parity check itself (tests/parity_util.py): the
intermediate check accepts the oracle's own re-quantised intermediate with no
allowance, accepts a code rounded the other way only at a rounding midpoint
(and then allows exactly that code's effect on the output), and rejects a
code one step off away from a midpoint, a code two steps off, a scale off by
more than its bound, a power-of-two scale one binade off away from the
binade's boundary, and a pad row that is not zero.  The "kernel" rows here
are the oracle's own values, edited on the host."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from parity_util import (assert_rows_close, check_intermediate_and_output, gpu_intermediate_rows, pairs_of,
                         verify_intermediate, oracle_weights_cpu)

MODES = ["fp8", "fp8_ue8m0", "mxfp4"]


def _stages(wl):
    Q = oracle_weights_cpu(wl)
    x = W.activations(wl).float().numpy()
    lg = W.router_logits(wl).numpy()
    ref, st = O.moe_forward(x, lg, Q, wl.top_k, wl.swiglu_limit, wl.H, wl.I, return_stages=True)
    return Q, ref, st


def _oracle_rows(st, mode):
    """The oracle's own intermediate in the form gpu_intermediate_rows returns."""
    rows = {}
    for key, (q, s) in st["aq"].items():
        codes = O.unpack_e2m1(q[None])[0] if mode == "mxfp4" else q.copy()
        rows[key] = (codes, s.copy())
    return rows


def _bf16(v):
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.bfloat16).float().numpy()


@pytest.mark.parametrize("mode", MODES)
def test_oracle_intermediate_needs_no_allowance(mode):
    wl = W.WORKLOADS["tiny_fp8"].with_(mode=mode)
    Q, ref, st = _stages(wl)
    allow, rep = verify_intermediate(mode, wl.swiglu_limit, _oracle_rows(st, mode), st, Q, wl.H)
    assert rep.code_flips == 0 and rep.scale_moves == 0 and rep.tie_flips == 0
    assert not np.any(allow)
    assert_rows_close(_bf16(ref), ref, mode, "oracle vs itself", allowance=allow)


def _pick(st, mode):
    """A pair and an element of its largest-magnitude group whose code is
    not the group's largest (so changing it moves neither scale nor amax)."""
    key = sorted(st["aq"])[0]
    a = np.asarray(st["a"][key], np.float32)
    G = 32 if mode == "mxfp4" else 128
    g = int(np.argmax(np.abs(a).reshape(-1, G).max(axis=1)))
    grp = np.abs(a[g * G:(g + 1) * G])
    i = g * G + int(np.argsort(grp)[G // 2])
    return key, g, i


def _scale_value(mode, s):
    return float(np.float32(s)) if mode == "fp8" else float(np.ldexp(1.0, int(s) - 127))


def _neighbour_codes(mode, v):
    """(nearest code, the other code of the same rounding interval) of v."""
    vals = O.e2m1_value_table() if mode == "mxfp4" else O.e4m3_value_table()
    c = int((O.round_to_e2m1 if mode == "mxfp4" else O.round_to_e4m3)(np.array([v]))[0])
    fin = np.isfinite(vals)
    same_sign = np.signbit(vals) == np.signbit(v)
    cand = np.nonzero(fin & same_sign & (vals != vals[c]))[0]
    other = int(cand[np.argmin(np.abs(vals[cand] - v))])
    return c, other, vals


@pytest.mark.parametrize("mode", MODES)
def test_planted_tie_flip_is_accepted_with_its_exact_effect(mode):
    """One SwiGLU value put exactly on the midpoint of two codes (the oracle's
    stages re-quantised to match); the "kernel" takes the code that
    round-half-even does not.  Accepted as one tie, and the allowance is that
    code's exact effect on its token's output row."""
    wl = W.WORKLOADS["tiny_fp8"].with_(mode=mode)
    Q, ref, st = _stages(wl)
    key, g, i = _pick(st, mode)
    q, s = st["aq"][key]
    sig = _scale_value(mode, s[g])
    a = np.asarray(st["a"][key], np.float32).copy()
    c, other, vals = _neighbour_codes(mode, float(a[i]) / sig)
    mid = (vals[c] + vals[other]) / 2
    a_mid = np.float32(mid * sig)
    assert abs(float(a_mid) / sig - mid) <= 2.0 ** -23 * abs(mid)   # on the midpoint up to fp32 rounding
    a[i] = a_mid
    qq, ss = O.quant_act(mode, a[None])
    assert _scale_value(mode, ss[0][g]) == sig
    st2 = dict(st)
    st2["a"] = dict(st["a"])
    st2["a"][key] = a
    st2["aq"] = dict(st["aq"])
    st2["aq"][key] = (qq[0], ss[0])
    rows = _oracle_rows(st2, mode)
    codes = rows[key][0].copy()
    c_oracle = int(codes[i])
    assert c_oracle in (c, other)
    c_kernel = other if c_oracle == c else c
    codes[i] = c_kernel
    rows[key] = (codes, rows[key][1])
    allow, rep = verify_intermediate(mode, wl.swiglu_limit, rows, st2, Q, wl.H)
    assert rep.tie_flips == 1 and rep.code_flips == 1 and rep.scale_moves == 0
    t, j = key
    w2d = O.dequant_expert(Q, int(st["ids"][t, j]))[1].astype(np.float64)
    expect = float(st["weights"][t, j]) * abs(vals[c_kernel] - vals[c_oracle]) * sig * np.abs(w2d[:, i])[:wl.H]
    assert np.allclose(allow[t], expect, rtol=1e-12, atol=0)
    others = [r for r in range(allow.shape[0]) if r != t]
    assert not np.any(allow[others])


@pytest.mark.parametrize("mode", MODES)
def test_flip_away_from_a_midpoint_is_rejected(mode):
    wl = W.WORKLOADS["tiny_fp8"].with_(mode=mode)
    Q, ref, st = _stages(wl)
    key, g, i = _pick(st, mode)
    q, s = st["aq"][key]
    sig = _scale_value(mode, s[g])
    vals = O.e2m1_value_table() if mode == "mxfp4" else O.e4m3_value_table()
    rows = _oracle_rows(st, mode)
    codes = rows[key][0].copy()
    v = float(st["a"][key][i]) / sig
    c, other, _ = _neighbour_codes(mode, v)
    mid = (vals[c] + vals[other]) / 2
    assert abs(v - mid) > 1e-3 * abs(v)      # not a tie
    codes[i] = other
    rows[key] = (codes, rows[key][1])
    with pytest.raises(AssertionError):
        verify_intermediate(mode, wl.swiglu_limit, rows, st, Q, wl.H)


@pytest.mark.parametrize("mode", MODES)
def test_two_step_flip_is_rejected(mode):
    wl = W.WORKLOADS["tiny_fp8"].with_(mode=mode)
    Q, ref, st = _stages(wl)
    key, g, i = _pick(st, mode)
    rows = _oracle_rows(st, mode)
    codes = rows[key][0].copy()
    mag = 0x7 if mode == "mxfp4" else 0x7F
    c = int(codes[i])
    codes[i] = (c & ~mag) | ((c & mag) - 2 if (c & mag) >= 2 else (c & mag) + 2)
    rows[key] = (codes, rows[key][1])
    with pytest.raises(AssertionError):
        verify_intermediate(mode, wl.swiglu_limit, rows, st, Q, wl.H)


@pytest.mark.parametrize("mode", MODES)
def test_scale_off_is_rejected(mode):
    wl = W.WORKLOADS["tiny_fp8"].with_(mode=mode)
    Q, ref, st = _stages(wl)
    key, g, i = _pick(st, mode)
    rows = _oracle_rows(st, mode)
    sc = rows[key][1].copy()
    if mode == "fp8":
        sc[g] = np.float32(sc[g] * np.float32(1.001))
    else:
        sc[g] = sc[g] + 1     # one binade up, amax not at the boundary
    rows[key] = (rows[key][0], sc)
    with pytest.raises(AssertionError):
        verify_intermediate(mode, wl.swiglu_limit, rows, st, Q, wl.H)


def test_mx_scale_at_a_binade_boundary_is_accepted():
    """A group whose largest value is exactly a power of two may take either
    shared exponent; the codes must then be the rounding under the kernel's."""
    mode = "mxfp4"
    wl = W.WORKLOADS["tiny_fp8"].with_(mode=mode)
    Q, ref, st = _stages(wl)
    key, g, i = _pick(st, mode)
    a = np.asarray(st["a"][key], np.float32).copy()
    G = 32
    grp = a[g * G:(g + 1) * G]
    k = int(np.argmax(np.abs(grp)))
    e = int(np.floor(np.log2(abs(float(grp[k])))))
    # put the largest value a hair below 2^(e+1): the oracle keeps exponent
    # e - 2, a sum that lands just above takes e - 1
    grp[k] = np.float32(np.sign(grp[k]) * np.nextafter(np.float32(2.0 ** (e + 1)), np.float32(0)))
    a[g * G:(g + 1) * G] = grp
    st2 = dict(st)
    st2["a"] = dict(st["a"])
    st2["a"][key] = a
    qo, so = O.quant_mxfp4_rows(a[None])
    st2["aq"] = dict(st["aq"])
    st2["aq"][key] = (qo[0], so[0])
    b_o = int(so[0][g])
    b_g = b_o + 1
    codes = O.unpack_e2m1(qo)[0].copy()
    codes[g * G:(g + 1) * G] = O.round_to_e2m1(np.clip(grp.astype(np.float64) / np.ldexp(1.0, b_g - 127), -6, 6))
    sc = so[0].copy()
    sc[g] = b_g
    rows = _oracle_rows(st2, mode)
    rows[key] = (codes, sc)
    allow, rep = verify_intermediate(mode, wl.swiglu_limit, rows, st2, Q, wl.H)
    assert rep.scale_moves == 1
    t, _ = key
    assert np.any(allow[t])


def test_pad_rows_must_be_zero():
    mode, Ip, P, k = "fp8", 128, 4, 2
    sid = torch.tensor([0, 1, P, P, 2, 3, P, P], dtype=torch.int32)
    aq = torch.zeros(8, Ip, dtype=torch.uint8)
    as_ = torch.zeros(8, dtype=torch.float32).view(torch.uint8)
    rows = gpu_intermediate_rows(mode, Ip, aq, as_, sid, 8, P, k, pairs_of([0, 1], k))
    assert set(rows) == {(0, 0), (0, 1), (1, 0), (1, 1)}
    aq[3, 5] = 1
    with pytest.raises(AssertionError):
        gpu_intermediate_rows(mode, Ip, aq, as_, sid, 8, P, k, pairs_of([0, 1], k))


def test_end_to_end_check_on_oracle_rows():
    """check_intermediate_and_output with the oracle's own intermediate laid
    out by sorted position and its own output rounded to bf16."""
    wl = W.WORKLOADS["tiny_fp8"]
    Q, ref, st = _stages(wl)
    sid, bexp, offs, npp = O.permute_align(st["ids"], wl.E, 16)
    P = wl.T * wl.top_k
    aq = np.zeros((sid.size, wl.Ip), np.uint8)
    as_ = np.zeros((sid.size, wl.Ip // 128), np.float32)
    for r, f in enumerate(sid[:npp]):
        if f < P:
            aq[r], as_[r] = st["aq"][(int(f) // wl.top_k, int(f) % wl.top_k)]
    check_intermediate_and_output(wl, _bf16(ref), torch.from_numpy(aq), torch.from_numpy(as_.view(np.uint8)),
                                  torch.from_numpy(sid), npp, ref, st, Q)
