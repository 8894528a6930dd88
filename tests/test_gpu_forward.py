"""GPU parity of the whole layer (moe_forward through the C ABI) against the
CPU oracle, on seeded inputs small enough for the oracle to finish in
seconds while still spanning several tiles, ragged tails and padding, plus
the method's degenerate cases.

Every check: moe_forward equals the stage entry points bit for bit; GEMM1's
re-quantised intermediate (from those entry points) equals the oracle's
except for codes verified to sit at a rounding midpoint within the element's
fp32 accumulation bound (parity_util.verify_intermediate); and max |out -
ref| <= tol * RMS of the oracle row, tol = 2e-2 (block FP8) or 6e-2 (MXFP4),
after adding only the effect of the intermediate codes that differed.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from parity_util import (assert_rows_close, bf16_to_f32, check_forward, check_intermediate_and_output,
                         gpu_weights, log, oracle_weights_cpu)

pytestmark = pytest.mark.gpu

M = None


@pytest.fixture(scope="module", autouse=True)
def lib():
    global M
    import mxfp4_quantized_weights_amd as mod
    M = mod
    yield mod


def _run(wl, block_m=None, ld_pad=0, stream=None):
    bm = block_m or M.pick_block_m(wl.T, wl.E, wl.top_k)
    cfg = M.make_cfg(wl.E, wl.top_k, wl.mode, wl.H, wl.I, wl.Hp, wl.Ip, block_m=bm,
                     swiglu_limit=wl.swiglu_limit)
    ew = gpu_weights(M, cfg, wl, source="cpu")
    x = W.activations(wl)
    lg = W.router_logits(wl)
    xd = torch.zeros(wl.T, wl.H + ld_pad, dtype=torch.bfloat16, device="cuda")
    xd[:, :wl.H] = x.cuda()
    out = torch.full((wl.T, wl.H + ld_pad), 7.0, dtype=torch.bfloat16, device="cuda")
    M.moe_forward(cfg, xd[:, :wl.H], lg.cuda(), *ew.tiled(), out=out[:, :wl.H])
    torch.cuda.synchronize()
    if ld_pad:
        assert torch.all(out[:, wl.H:] == 7.0), "columns past H must not be written"
    return cfg, ew, x, lg, out[:, :wl.H]


def _check(wl, cfg, ew, x, lg, out, tokens=None, what=""):
    """check_forward on the same inputs (x, lg host tensors; out the device output)."""
    return check_forward(M, wl, cfg, ew, x.cuda(), lg.cuda(), out, oracle_weights_cpu(wl), tokens=tokens,
                         what=what)


TINY = W.WORKLOADS["tiny_fp8"]
MID = W.Workload("mid", T=200, H=512, I=384, E=16, top_k=4, mode="fp8", outlier_frac=0.01)
STREAM = W.Workload("stream", T=2048, H=1536, I=1024, E=8, top_k=4, mode="fp8", outlier_frac=0.01)
SHORT_K = W.Workload("short_k", T=2048, H=2048, I=128, E=8, top_k=4, mode="fp8", outlier_frac=0.01)
# more per-pair GEMM2 rows than one y chunk holds (P * Hp * 2 bytes > 1 GiB):
# GEMM2 + combine run per column chunk (3840 columns, then a ragged
# 384-column tail of which 260 are real)
CHUNKED = W.Workload("chunked", T=16384, H=4100, I=256, E=8, top_k=8, mode="fp8", Hp=4224, outlier_frac=0.01)

CASES = {
    "tiny_fp8": (TINY, None),
    "tiny_mxfp4": (TINY.with_(mode="mxfp4"), None),
    "mid_fp8_bm16": (MID, 16),
    "mid_fp8_bm64": (MID, 64),
    "mid_fp8_bm128": (MID, 128),
    "mid_mxfp4_bm32": (MID.with_(mode="mxfp4"), 32),
    "mid_mxfp4_bm128": (MID.with_(mode="mxfp4"), 128),
    "padded_fp8": (W.Workload("pad", T=96, H=400, I=200, E=8, top_k=3, mode="fp8", Hp=512, Ip=256), 16),
    "padded_mxfp4": (W.Workload("pad", T=96, H=400, I=200, E=8, top_k=3, mode="mxfp4", Hp=512, Ip=384), 32),
    "skewed_fp8": (W.Workload("skew", T=160, H=256, I=256, E=32, top_k=8, mode="fp8", zipf_s=1.2), 64),
    "no_limit_fp8": (MID.with_(swiglu_limit=math.inf, T=64), 16),
    "tight_limit_mxfp4": (MID.with_(swiglu_limit=0.5, T=64, mode="mxfp4"), 16),
    "single_token_fp8": (MID.with_(T=1), 16),
    "single_expert_fp8": (MID.with_(E=1, top_k=1, T=40), 16),
    "all_experts_mxfp4": (W.Workload("kE", T=24, H=256, I=128, E=16, top_k=16, mode="mxfp4"), 16),
    "big_k_ragged_fp8": (W.Workload("rag", T=37, H=384, I=640, E=24, top_k=5, mode="fp8"), 32),
    # more (M block, N tile) items than workgroups: the persistent GEMMs walk
    # several items each and their load rings run across item boundaries
    "stream_fp8_bm64": (STREAM, 64),
    "stream_fp8_bm128": (STREAM, 128),
    "stream_mxfp4_bm64": (STREAM.with_(mode="mxfp4"), 64),
    "stream_mxfp4_bm128": (STREAM.with_(mode="mxfp4"), 128),
    # GEMM2 with a single K block (Ip = 128) and many items per workgroup: the
    # loads run several items ahead of the compute
    "short_k_fp8_bm128": (SHORT_K, 128),
    "short_k_fp8_bm16": (SHORT_K.with_(T=512), 16),
    "short_k_mxfp4_bm128": (SHORT_K.with_(mode="mxfp4"), 128),
    # items of exactly S-1 K blocks (S = ring depth: 3 for FP8 at block_m
    # 64/128, 4 at 16/32, 5 for MX) with many items per workgroup: the first
    # item ends inside the ring's prologue
    "ring_edge_fp8_bm128": (W.Workload("edge", T=2048, H=256, I=256, E=8, top_k=8, mode="fp8"), 128),
    "ring_edge_fp8_bm16": (W.Workload("edge", T=2048, H=384, I=384, E=8, top_k=8, mode="fp8"), 16),
    "ring_edge_mxfp4_bm64": (W.Workload("edge", T=2048, H=512, I=512, E=8, top_k=8, mode="mxfp4"), 64),
    "ring_edge_ue8m0_bm64": (W.Workload("edge", T=2048, H=256, I=256, E=8, top_k=8, mode="fp8_ue8m0"), 64),
    # block FP8 with UE8M0 (power-of-two) scales
    "tiny_ue8m0": (TINY.with_(mode="fp8_ue8m0"), None),
    "mid_ue8m0_bm16": (MID.with_(mode="fp8_ue8m0"), 16),
    "mid_ue8m0_bm128": (MID.with_(mode="fp8_ue8m0"), 128),
    "padded_ue8m0": (W.Workload("pad", T=96, H=400, I=200, E=8, top_k=3, mode="fp8_ue8m0", Hp=512, Ip=256), 32),
    "stream_ue8m0_bm128": (STREAM.with_(mode="fp8_ue8m0"), 128),
    "short_k_ue8m0_bm128": (SHORT_K.with_(mode="fp8_ue8m0"), 128),
    "short_k_ue8m0_bm16": (SHORT_K.with_(T=512, mode="fp8_ue8m0"), 16),
}


@pytest.mark.parametrize("name", list(CASES))
def test_forward_matches_oracle(name):
    wl, bm = CASES[name]
    log(f"forward {name}: {W.describe(wl)} block_m={bm}")
    cfg, ew, x, lg, out = _run(wl, bm)
    _check(wl, cfg, ew, x, lg, out, what=name)


def test_forward_with_row_strides():
    wl = MID.with_(T=50)
    log(f"forward strided: {W.describe(wl)}")
    cfg, ew, x, lg, out = _run(wl, 16, ld_pad=72)
    xd = torch.zeros(wl.T, wl.H + 72, dtype=torch.bfloat16, device="cuda")
    xd[:, :wl.H] = x.cuda()
    check_forward(M, wl, cfg, ew, xd[:, :wl.H], lg.cuda(), out, oracle_weights_cpu(wl), what="strided")


@pytest.mark.parametrize("mode,bm", [("fp8", 128), ("mxfp4", 64), ("fp8_ue8m0", 128)])
def test_chunked_gemm2_combine(mode, bm):
    """Column-chunked GEMM2 + combine (with an output row stride): moe_forward
    equals the stage entry points bit for bit, and sampled rows (first, last,
    and spread over the batch) match the oracle."""
    wl = CHUNKED.with_(mode=mode)
    log(f"chunked: {W.describe(wl)} block_m={bm}")
    cfg, ew, x, lg, out = _run(wl, bm, ld_pad=40)
    toks = sorted({0, wl.T - 1, *range(5, wl.T, 2711)})
    _check(wl, cfg, ew, x, lg, out, tokens=toks, what="chunked")


@pytest.mark.parametrize("mode", ["fp8", "fp8_ue8m0", "mxfp4"])
def test_forward_zero_input(mode):
    wl = MID.with_(T=33, mode=mode)
    cfg = M.make_cfg(wl.E, wl.top_k, mode, wl.H, wl.I, block_m=16)
    ew = gpu_weights(M, cfg, wl, source="cpu")
    out = M.moe_forward(cfg, torch.zeros(wl.T, wl.H, dtype=torch.bfloat16, device="cuda"),
                        W.router_logits(wl).cuda(), *ew.tiled())
    torch.cuda.synchronize()
    assert torch.all(out == 0)


def test_forward_zero_tokens():
    wl = MID
    cfg = M.make_cfg(wl.E, wl.top_k, "fp8", wl.H, wl.I, block_m=16)
    ew = gpu_weights(M, cfg, wl.with_(E=wl.E), source="cpu")
    out = M.moe_forward(cfg, torch.zeros(0, wl.H, dtype=torch.bfloat16, device="cuda"),
                        torch.zeros(0, wl.E, device="cuda"), *ew.tiled())
    torch.cuda.synchronize()
    assert out.shape == (0, wl.H)


@pytest.mark.parametrize("mode,T", [("fp8", 120), ("fp8_ue8m0", 120), ("mxfp4", 120), ("fp8", 3), ("mxfp4", 40)])
def test_forward_repeatable_and_equal_to_stages(mode, T):
    """Repeated runs give identical bits, and moe_forward equals the stage
    entry points called one by one (small batches take the two-launch front
    end inside moe_forward, the three stage kernels here)."""
    wl = MID.with_(mode=mode, T=T)
    log(f"repeatability {W.describe(wl)}")
    cfg, ew, x, lg, out1 = _run(wl, 32)
    xd, lgd = x.cuda(), lg.cuda()
    out2 = M.moe_forward(cfg, xd, lgd, *ew.tiled())
    # the three separate stage calls (small batches take the two-launch front
    # end inside moe_forward)
    ids, wts = M.moe_route_topk(lgd, wl.top_k)
    sid, bexp, offs, npp = M.moe_permute_align(ids, wl.E, 32)
    xq, xs = M.moe_quant_act(xd, wl.Hp, mode)
    aq, as_ = M.moe_grouped_gemm1_swiglu(cfg, wl.T, xq, xs, sid, bexp, npp, ew.w13, ew.w13_scale,
                                         ksplit=M.plan_ksplit(cfg, wl.T, 13))
    out3 = M.moe_grouped_gemm2_combine(cfg, wl.T, aq, as_, sid, bexp, npp, ew.w2, ew.w2_scale, wts)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(out1.view(torch.int16), out3.view(torch.int16))
    _check(wl, cfg, ew, x, lg, out1, what="forward")


def test_block_m_choices_agree():
    wl = MID.with_(T=150)
    for bm in (16, 32, 64, 128):
        cfg, ew, x, lg, out = _run(wl, bm)
        _check(wl, cfg, ew, x, lg, out, what=f"block_m {bm}")
