"""Pins of the oracle's GEMMs, clamped SwiGLU and whole layer (CPU only).

- dequantised GEMM: brute-force fp64 triple loop on 4 x 32 x 128 inputs
  (one FP8 128-block, four MX 32-groups) within the fp32 summation bound
  gamma_K * sum |a||b|;
- clamped SwiGLU (FreeToken PR #270, Summary): an infinite limit equals plain
  SwiGLU built from torch's silu; below the limit the clamp is inactive;
- layer: one expert with top-1 weight 1.0 equals a dense FFN; x = 0 gives 0;
  zero padding of H/I changes nothing; token permutation permutes the
  output; a brute-force pure-Python layer on a tiny input agrees.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W


def _gamma(K):
    u = 2.0 ** -24
    return K * u / (1 - K * u)


@pytest.mark.parametrize("mode", ["fp8", "fp8_ue8m0", "mxfp4"])
def test_dequant_gemm_brute_force_4x32x128(mode):
    rng = np.random.default_rng(20)
    a = rng.standard_normal((4, 128)).astype(np.float32)
    b = (rng.standard_normal((32, 128)) * 0.02).astype(np.float32)
    if mode == "fp8":
        qa, sa = O.quant_fp8_rows(a, 128)
        qb, sb = O.quant_fp8_weight(np.pad(b, ((0, 96), (0, 0))))
        ad = O.dequant_fp8_rows(qa, sa)
        bd = O.dequant_fp8_weight(qb, sb)[:32]
        tab = O.e4m3_value_table()
        # brute force: decode every code by table, scale, multiply in fp64
        A = [[float(np.float32(tab[qa[i, kk]] * sa[i, 0])) for kk in range(128)] for i in range(4)]
        B = [[float(np.float32(tab[qb[j, kk]] * sb[0, 0])) for kk in range(128)] for j in range(32)]
    elif mode == "fp8_ue8m0":
        qa, ba = O.quant_fp8e8_rows(a, 128)
        qb, bb = O.quant_fp8e8_weight(np.pad(b, ((0, 96), (0, 0))))
        ad = O.dequant_fp8e8_rows(qa, ba)
        bd = O.dequant_fp8e8_weight(qb, bb)[:32]
        tab = O.e4m3_value_table()
        A = [[tab[qa[i, kk]] * 2.0 ** (int(ba[i, 0]) - 127) for kk in range(128)] for i in range(4)]
        B = [[tab[qb[j, kk]] * 2.0 ** (int(bb[0, 0]) - 127) for kk in range(128)] for j in range(32)]
    else:
        pa, ba = O.quant_mxfp4_rows(a)
        pb, bb = O.quant_mxfp4_rows(b)
        ad = O.dequant_mxfp4_rows(pa, ba)
        bd = O.dequant_mxfp4_rows(pb, bb)
        vals = O.e2m1_value_table()

        def dec(p, bytes_, i, kk):
            byte = int(p[i, kk // 2])
            code = (byte & 0xF) if kk % 2 == 0 else (byte >> 4)
            return vals[code] * 2.0 ** (int(bytes_[i, kk // 32]) - 127)
        A = [[dec(pa, ba, i, kk) for kk in range(128)] for i in range(4)]
        B = [[dec(pb, bb, j, kk) for kk in range(128)] for j in range(32)]
    assert np.array_equal(ad, np.array(A, np.float32)) and np.array_equal(bd, np.array(B, np.float32))
    got = O.gemm_f32(ad, bd)
    for i in range(4):
        for j in range(32):
            exact = math.fsum(A[i][kk] * B[j][kk] for kk in range(128))
            bound = _gamma(128) * sum(abs(A[i][kk] * B[j][kk]) for kk in range(128))
            assert abs(float(got[i, j]) - exact) <= bound + 1e-30, (i, j)


def test_swiglu_infinite_limit_is_plain_swiglu():
    rng = np.random.default_rng(21)
    g = (rng.standard_normal(100000) * 8).astype(np.float32)
    u = (rng.standard_normal(100000) * 8).astype(np.float32)
    # silu against torch's implementation (x * sigmoid(x)): the two fp32
    # formulas may differ in the last bits, at most a few ulp
    s_ours = O.silu(g)
    s_ref = torch.nn.functional.silu(torch.from_numpy(g)).numpy()
    assert np.all(np.abs(s_ours - s_ref) <= 8 * np.spacing(np.abs(s_ref)))
    # with an infinite limit nothing is clamped: the result is silu(g) * up
    got = O.swiglu_clamped(g, u, float("inf"))
    ref = (torch.from_numpy(s_ref) * torch.from_numpy(u)).numpy()
    assert np.all(np.abs(got - ref) <= 16 * np.spacing(np.abs(ref)))
    assert np.array_equal(got, O.swiglu_clamped(g, u, np.float32(3.0e38)))


def test_swiglu_limit_inactive_below_limit_and_active_above():
    rng = np.random.default_rng(22)
    g = rng.uniform(-9.9, 9.9, 10000).astype(np.float32)
    u = rng.uniform(-9.9, 9.9, 10000).astype(np.float32)
    assert np.array_equal(O.swiglu_clamped(g, u, 10.0), O.swiglu_clamped(g, u, float("inf")))
    big = np.array([50.0, 10.0, 11.0, -50.0], np.float32)
    one = np.ones(4, np.float32)
    got = O.swiglu_clamped(big, one, 10.0)
    s10 = np.float32(10) / (np.float32(1) + np.exp(np.float32(-10)))
    assert got[0] == got[1] == got[2] == s10
    assert got[3] == O.swiglu_clamped(np.float32([-50.0]), one[:1], float("inf"))[0]   # gate only clamped from above
    up = np.array([50.0, -50.0, 3.0], np.float32)
    gg = np.full(3, 2.0, np.float32)
    got = O.swiglu_clamped(gg, up, 10.0)
    sg = O.silu(np.float32([2.0]))[0]
    assert got.tolist() == [sg * 10, sg * -10, sg * 3]


def _quantised(wl, device="cpu"):
    w13 = W.all_w13(wl).numpy()
    w2 = W.all_w2(wl).numpy()
    return O.quantize_weights(wl.mode, w13, w2)


TINY = W.WORKLOADS["tiny_fp8"]


def _close_rows(a, b, rel=1e-5):
    """max |a - b| per row within rel * row RMS of a: BLAS may sum in another
    order when the shapes differ, which moves fp32 results by a few ulp."""
    rms = np.sqrt(np.mean(a.astype(np.float64) ** 2, axis=1))
    return bool(np.all(np.abs(a - b).max(axis=1) <= rel * rms))


@pytest.mark.parametrize("mode", ["fp8", "fp8_ue8m0", "mxfp4"])
def test_single_expert_top1_equals_dense_ffn(mode):
    wl = TINY.with_(E=1, top_k=1, mode=mode, T=12)
    Q = _quantised(wl)
    x = W.activations(wl).float().numpy()
    lg = W.router_logits(wl).numpy()
    out = O.moe_forward(x, lg, Q, 1, wl.swiglu_limit, wl.H, wl.I)
    # dense FFN from the same quantisers, no routing
    xq, xs = O.quant_act(mode, O.pad_cols(x, wl.Hp))
    w13d, w2d = O.dequant_expert(Q, 0)
    h = O.gemm_f32(O.dequant_act(mode, xq, xs), w13d)
    a = O.swiglu_clamped(h[:, :wl.Ip], h[:, wl.Ip:], wl.swiglu_limit)
    aq, as_ = O.quant_act(mode, a)
    y = O.gemm_f32(O.dequant_act(mode, aq, as_), w2d)[:, :wl.H]
    assert np.array_equal(out, y)


@pytest.mark.parametrize("mode", ["fp8", "fp8_ue8m0", "mxfp4"])
def test_zero_input_gives_zero_output(mode):
    wl = TINY.with_(mode=mode)
    Q = _quantised(wl)
    out = O.moe_forward(np.zeros((wl.T, wl.H), np.float32), W.router_logits(wl).numpy(), Q,
                        wl.top_k, 10.0, wl.H, wl.I)
    assert np.all(out == 0)


@pytest.mark.parametrize("mode", ["fp8", "fp8_ue8m0", "mxfp4"])
def test_padding_is_invisible(mode):
    wl = TINY.with_(mode=mode)
    wlp = wl.with_(Hp=wl.H + 128, Ip=wl.I + 128)
    x = W.activations(wl).float().numpy()
    lg = W.router_logits(wl).numpy()
    out = O.moe_forward(x, lg, _quantised(wl), wl.top_k, 10.0, wl.H, wl.I)
    outp = O.moe_forward(x, lg, _quantised(wlp), wl.top_k, 10.0, wl.H, wl.I)
    # the GEMMs differ only by summation order over extra exact zeros
    assert _close_rows(out, outp)


def test_token_permutation_equivariance():
    wl = TINY.with_(T=24)
    Q = _quantised(wl)
    x = W.activations(wl).float().numpy()
    lg = W.router_logits(wl).numpy()
    out = O.moe_forward(x, lg, Q, wl.top_k, 10.0, wl.H, wl.I)
    perm = np.random.default_rng(23).permutation(wl.T)
    out2 = O.moe_forward(x[perm], lg[perm], Q, wl.top_k, 10.0, wl.H, wl.I)
    assert _close_rows(out[perm], out2)


def test_token_subset_equals_full_rows():
    wl = TINY
    Q = _quantised(wl)
    x = W.activations(wl).float().numpy()
    lg = W.router_logits(wl).numpy()
    full = O.moe_forward(x, lg, Q, wl.top_k, 10.0, wl.H, wl.I)
    sub = O.moe_forward(x, lg, Q, wl.top_k, 10.0, wl.H, wl.I, tokens=[3, 0, 11])
    assert _close_rows(full[[3, 0, 11]], sub)


@pytest.mark.parametrize("mode", ["fp8", "fp8_ue8m0", "mxfp4"])
def test_layer_brute_force_tiny(mode):
    """The whole layer written out with Python loops in fp64 from the stage
    definitions (own routing sort, own dot products, own SwiGLU); only the
    (separately pinned) quantisers are shared.  Catches swapped gate/up
    halves, a transposed w2, a wrong slot weight or combine order."""
    wl = TINY.with_(T=6, H=128, I=128, E=4, top_k=2, mode=mode)
    Q = _quantised(wl)
    x = W.activations(wl).float().numpy()
    lg = W.router_logits(wl).numpy()
    out = O.moe_forward(x, lg, Q, wl.top_k, wl.swiglu_limit, wl.H, wl.I)
    L = wl.swiglu_limit
    for t in range(wl.T):
        order = sorted(range(wl.E), key=lambda e: (-float(lg[t, e]), e))[:wl.top_k]
        m = max(float(lg[t, e]) for e in order)
        ex = [math.exp(float(lg[t, e]) - m) for e in order]
        wts = [v / sum(ex) for v in ex]
        xq, xs = O.quant_act(mode, x[t:t + 1])
        xd = O.dequant_act(mode, xq, xs)[0].astype(np.float64)
        acc = np.zeros(wl.H)
        for j, e in enumerate(order):
            w13d, w2d = O.dequant_expert(Q, e)
            a = np.zeros(wl.I)
            for i in range(wl.I):
                gate = math.fsum(xd * w13d[i].astype(np.float64))
                up = math.fsum(xd * w13d[wl.Ip + i].astype(np.float64))
                g = min(gate, L)
                a[i] = g / (1 + math.exp(-g)) * min(max(up, -L), L)
            aq, as_ = O.quant_act(mode, a.astype(np.float32)[None])
            ad = O.dequant_act(mode, aq, as_)[0].astype(np.float64)
            for h in range(wl.H):
                acc[h] += wts[j] * math.fsum(ad * w2d[h].astype(np.float64))
        rms = math.sqrt(float(np.mean(acc ** 2)))
        # fp32 vs fp64 arithmetic may move a requantised code by one step
        assert np.max(np.abs(out[t] - acc)) <= 2e-2 * rms, t
