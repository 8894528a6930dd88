"""GPU parity of the decode micro-batch kernels (T <= 16, block FP8): the
M-tiled GEMV entry points moe_decode_gemm1_swiglu and
moe_decode_gemm2_combine, against the oracle.

Every case: moe_decode_supported holds; on the routing and quantised x of
moe_route_permute_quant (bit-exact against the oracle elsewhere), the
intermediate that moe_decode_gemm2_combine stores (pair order) passes the
verified-tie check against the oracle's re-quantised SwiGLU; the fp32 SwiGLU
output a of moe_decode_gemm1_swiglu is within the fp32 accumulation bound of
the exact (fp64) GEMM1 of the same quantised operands through the clamped
SwiGLU; the output rows are within 2e-2 of the row RMS after the effect of
the intermediate codes that differed (parity_util); and two runs give the
same bytes.

Shapes: the 288-expert top-8 decode layer (H = 4096, I = 1024) at
T = 1 .. 16 in both scale formats (re-quantisation inside GEMM2 up to 4
tokens, a launch of its own above); smaller expert counts; H = 1024 / 2048
and I = 128 .. 512 (every K-block count the kernels take); ragged H and I;
the pair limit T*k = 128 with k = 16.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from parity_util import (bf16_to_f32, check_intermediate_and_output, decode_chain, gpu_weights, log,
                         oracle_stages, oracle_weights_cpu, oracle_weights_subset)

pytestmark = pytest.mark.gpu

M = None
_W = {}


@pytest.fixture(scope="module", autouse=True)
def lib():
    global M
    import mxfp4_quantized_weights_amd as mod
    M = mod
    yield mod
    _W.clear()
    torch.cuda.empty_cache()


def _small(wl) -> bool:
    """Weights drawn on the host (the oracle quantises all of them there);
    else drawn on the GPU, the oracle quantising only the routed experts from
    the same device draws."""
    return wl.E * wl.H * wl.I <= 64 * 1024 * 1024


def _weights(cfg, wl):
    key = (wl.H, wl.I, wl.Hp, wl.Ip, wl.E, wl.mode, wl.seed)
    if key not in _W:
        _W.clear()
        torch.cuda.empty_cache()
        _W[key] = gpu_weights(M, cfg, wl, source="cpu" if _small(wl) else "cuda")
    return _W[key]


DEC = W.WORKLOADS["decode_fp8"]
SMALL = W.Workload("dec_small", T=16, H=1024, I=256, E=48, top_k=8, mode="fp8", outlier_frac=0.01)

CASES = {
    "glm_T1": DEC.with_(T=1),
    "glm_T2": DEC.with_(T=2),
    "glm_T7": DEC.with_(T=7),
    "glm_T16": DEC.with_(T=16),
    "glm_ue8m0_T1": DEC.with_(T=1, mode="fp8_ue8m0"),
    "glm_ue8m0_T16": DEC.with_(T=16, mode="fp8_ue8m0"),
    "small_T1": SMALL.with_(T=1),
    "small_T16": SMALL,
    "small_ue8m0_T11": SMALL.with_(T=11, mode="fp8_ue8m0"),
    "h2048_i512_fused": W.Workload("dec_h2k", T=5, H=2048, I=512, E=96, top_k=6, mode="fp8"),
    "h1024_i128": W.Workload("dec_i128", T=9, H=1024, I=128, E=32, top_k=4, mode="fp8"),
    "ragged_h_i": W.Workload("dec_rag", T=9, H=1000, I=200, E=40, top_k=4, mode="fp8", Hp=1024, Ip=256),
    "k16_pairs128": W.Workload("dec_k16", T=8, H=1024, I=256, E=32, top_k=16, mode="fp8_ue8m0"),
    "no_limit_T3": SMALL.with_(T=3, swiglu_limit=float("inf")),
}


def _oracle_weights(wl, ids):
    if _small(wl):
        return oracle_weights_cpu(wl)
    return oracle_weights_subset(wl, np.unique(ids), "cuda")


@pytest.mark.parametrize("name", list(CASES))
def test_decode_matches_oracle(name):
    wl = CASES[name]
    cfg = M.make_cfg(wl.E, wl.top_k, wl.mode, wl.H, wl.I, wl.Hp, wl.Ip, block_m=16, swiglu_limit=wl.swiglu_limit)
    assert M.decode_supported(cfg, wl.T)
    log(f"decode {name}: {W.describe(wl)}")
    ew = _weights(cfg, wl)
    x = W.activations(wl, "cuda")
    lg = W.router_logits(wl, "cuda")
    ch = decode_chain(M, cfg, x, lg, ew)
    again = decode_chain(M, cfg, x, lg, ew)
    torch.cuda.synchronize()
    assert torch.equal(ch["out"].view(torch.int16), again["out"].view(torch.int16)), "decode runs differ"
    ids, _ = O.route_topk(lg.cpu().numpy(), wl.top_k)
    assert np.array_equal(ch["ids"].cpu().numpy(), ids)
    Q = _oracle_weights(wl, ids)
    ref, st = oracle_stages(wl, x, lg, Q)
    check_intermediate_and_output(wl, bf16_to_f32(ch["out"]), ch["aq"], ch["as_"], None, None, ref, st, Q,
                                  what=name)


def _exact_a(wl, Q, xq_o, xs_o, ids):
    """Exact (fp64) GEMM1 of the oracle's quantised x and weights for every
    pair, through the clamped SwiGLU in fp64, and the fp32 accumulation
    bound of each element (64 u * sum |x w| of gate and of up, through the
    clamped SwiGLU's slope)."""
    T, k, Hp, Ip = wl.T, wl.top_k, wl.Hp, wl.Ip
    xd = O.dequant_act(wl.mode, xq_o, xs_o).astype(np.float64)[:, :Hp]
    u = 2.0 ** -24
    h = np.zeros((T * k, Ip))
    bound = np.zeros((T * k, Ip))
    L = wl.swiglu_limit
    w13_of = {}
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            if e not in w13_of:
                w13_of[e] = O.dequant_expert(Q, e)[0].astype(np.float64)
            w13 = w13_of[e]
            acc = w13 @ xd[t]
            mag = np.abs(w13) @ np.abs(xd[t])
            g, up = acc[:Ip], acc[Ip:]
            gc = np.minimum(g, L)
            uc = np.clip(up, -L, L)
            sg = 1.0 / (1.0 + np.exp(-gc))
            h[t * k + j] = gc * sg * uc
            # |d/dg| <= 1.1 |uc|, |d/du| <= |silu(gc)|; the fp32 SwiGLU itself
            # (exp2 and reciprocal approximations): (32 + 2 |gc|) u |h|
            bound[t * k + j] = 64 * u * (1.1 * np.abs(uc) * mag[:Ip] + np.abs(gc * sg) * mag[Ip:]) + \
                (32 + 2 * np.abs(gc)) * u * np.abs(h[t * k + j]) + 1e-30
    return h, bound


@pytest.mark.parametrize("name", ["glm_T1", "glm_T16", "glm_ue8m0_T16", "ragged_h_i", "k16_pairs128"])
def test_decode_swiglu_within_accumulation_bound(name):
    """GEMM1's fp32 SwiGLU output a (before re-quantisation) of every pair against
    the exact product of the same quantised operands (the oracle's
    quantisation of x equals the kernels' bit for bit, checked elsewhere)."""
    wl = CASES[name]
    cfg = M.make_cfg(wl.E, wl.top_k, wl.mode, wl.H, wl.I, wl.Hp, wl.Ip, block_m=16, swiglu_limit=wl.swiglu_limit)
    ew = _weights(cfg, wl)
    x = W.activations(wl, "cuda")
    lg = W.router_logits(wl, "cuda")
    ch = decode_chain(M, cfg, x, lg, ew)
    torch.cuda.synchronize()
    ids, _ = O.route_topk(lg.cpu().numpy(), wl.top_k)
    assert np.array_equal(ch["ids"].cpu().numpy(), ids)
    Q = _oracle_weights(wl, ids)
    xq_o, xs_o = O.quant_act(wl.mode, O.pad_cols(x.float().cpu().numpy(), wl.Hp))
    a_ex, bound = _exact_a(wl, Q, xq_o, xs_o, ids)
    a_g = ch["a32"].cpu().numpy().astype(np.float64)
    err = np.abs(a_g - a_ex)
    worst = float(np.max(err / bound))
    log(f"decode a {name}: max |a - exact| / bound = {worst:.3f} over {a_g.size} values")
    assert worst <= 1.0
