"""GPU parity of the K-split GEMMs used for small batches.

Each (block, N tile) work item is cut into ksplit pieces along K.  GEMM1
pieces store fp32 partial sums that a second kernel adds before the clamped
SwiGLU and the re-quantisation; GEMM2 pieces store y planes that the combine
adds.  Results differ from the unsplit launch by fp32 summation order (and,
for GEMM2, by each plane's own block-floating-point storage of the per-pair
rows), so the checks are those of the unsplit stages: the intermediate against the
oracle's stage values (a code moves by at most one step at a rounding
boundary), the layer output against the oracle rows within the mode's
tolerance, and moe_forward bit-identical to the stage entry points called with
the split the library plans.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from parity_util import (assert_rows_close, bf16_to_f32, check_gemm1_intermediate, gpu_weights, log,
                         oracle_weights_cpu, requant_tie_allowance)

pytestmark = pytest.mark.gpu

M = None


@pytest.fixture(scope="module", autouse=True)
def lib():
    global M
    import mxfp4_quantized_weights_amd as mod
    M = mod
    yield mod


# GEMM1 over K = 4096 (32 K blocks: splits 2, 4, 8 in every mode), few pairs
SPLIT1 = W.Workload("split1", T=5, H=4096, I=256, E=6, top_k=2, mode="fp8", outlier_frac=0.02)
# GEMM2 over K = Ip = 1024 (8 K blocks: split 2), ragged hidden size
SPLIT2 = W.Workload("split2", T=5, H=1000, I=1000, E=6, top_k=2, mode="fp8", Hp=1024, Ip=1024, outlier_frac=0.02)
MODES = ["fp8", "fp8_ue8m0", "mxfp4"]


def _setup(wl, bm):
    cfg = M.make_cfg(wl.E, wl.top_k, wl.mode, wl.H, wl.I, wl.Hp, wl.Ip, block_m=bm, swiglu_limit=wl.swiglu_limit)
    ew = gpu_weights(M, cfg, wl, source="cpu")
    x = W.activations(wl)
    lg = W.router_logits(wl)
    xd, lgd = x.cuda(), lg.cuda()
    ids, wts = M.moe_route_topk(lgd, wl.top_k)
    sid, bexp, offs, npp = M.moe_permute_align(ids, wl.E, bm)
    xq, xs = M.moe_quant_act(xd, wl.Hp, wl.mode)
    return cfg, ew, x, lg, (ids, wts, sid, bexp, npp, xq, xs)


def _oracle_stages(wl, x, lg):
    Q = oracle_weights_cpu(wl)
    ref, st = O.moe_forward(x.float().numpy(), lg.numpy(), Q, wl.top_k, wl.swiglu_limit, wl.H, wl.I,
                            return_stages=True)
    return ref, st, requant_tie_allowance(st, Q, wl.mode, wl.H)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("bm", [16, 128])
def test_gemm1_splitk_stage(mode, bm):
    wl = SPLIT1.with_(mode=mode)
    log(f"gemm1 split {W.describe(wl)} BM={bm}")
    cfg, ew, x, lg, (ids, wts, sid, bexp, npp, xq, xs) = _setup(wl, bm)
    _, st, _ = _oracle_stages(wl, x, lg)
    for ks in (1, 2, 4, 8):
        P = wl.T * wl.top_k
        need = ks * P * 2 * wl.Ip * 4 + P * 4   # partial sums, then each pair's sorted row
        assert M.splitk_bytes(cfg, wl.T, 13, ks) == (0 if ks == 1 else -(-need // 256) * 256)
        aq, as_ = M.moe_grouped_gemm1_swiglu(cfg, wl.T, xq, xs, sid, bexp, npp, ew.w13, ew.w13_scale, ksplit=ks)
        torch.cuda.synchronize()
        log(f"  ksplit {ks}")
        check_gemm1_intermediate(wl, aq, as_, sid, npp, st)


@pytest.mark.parametrize("mode", MODES)
def test_gemm2_splitk_combine(mode):
    wl = SPLIT2.with_(mode=mode)
    log(f"gemm2 split {W.describe(wl)}")
    cfg, ew, x, lg, (ids, wts, sid, bexp, npp, xq, xs) = _setup(wl, 16)
    ref, _, tie = _oracle_stages(wl, x, lg)
    aq, as_ = M.moe_grouped_gemm1_swiglu(cfg, wl.T, xq, xs, sid, bexp, npp, ew.w13, ew.w13_scale)
    outs = {}
    for ks in (1, 2):
        out = torch.full((wl.T, wl.H + 24), 7.0, dtype=torch.bfloat16, device="cuda")
        M.moe_grouped_gemm2_combine(cfg, wl.T, aq, as_, sid, bexp, npp, ew.w2, ew.w2_scale, wts,
                                    out=out[:, :wl.H], ksplit=ks)
        torch.cuda.synchronize()
        assert torch.all(out[:, wl.H:] == 7.0), "columns past H must not be written"
        outs[ks] = bf16_to_f32(out[:, :wl.H])
        assert_rows_close(outs[ks], ref, mode, f"gemm2 ksplit {ks}", allowance=tie)
    # the two differ by fp32 summation order (at most one bf16 rounding step)
    # and by the block-floating-point storage of the per-pair rows, which each
    # piece encodes on its own: every stored term is within 2^-14 of its
    # 64-column group's largest |w y|, so the 2k terms of an element stay well
    # under 2^-7 of the row RMS
    d = np.abs(outs[1] - outs[2])
    rms = np.sqrt(np.mean(np.square(outs[1]), axis=1, keepdims=True))
    assert np.all(d <= 2.0 ** -7 * (np.maximum(np.abs(outs[1]), np.abs(outs[2])) + rms) + 1e-30)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("wl0,bm", [(SPLIT1, 16), (SPLIT2, 16), (SPLIT2, 128)])
def test_forward_planned_split_equals_stages(mode, wl0, bm):
    """moe_forward with its planned splits is repeatable, equals the stage
    entry points called with the same splits, and matches the oracle."""
    wl = wl0.with_(mode=mode)
    cfg, ew, x, lg, (ids, wts, sid, bexp, npp, xq, xs) = _setup(wl, bm)
    k1, k2 = M.plan_ksplit(cfg, wl.T, 13), M.plan_ksplit(cfg, wl.T, 2)
    log(f"forward split {W.describe(wl)} BM={bm}: planned ksplit GEMM1 {k1}, GEMM2 {k2}")
    assert k1 > 1
    xd, lgd = x.cuda(), lg.cuda()
    out1 = M.moe_forward(cfg, xd, lgd, *ew.tiled())
    out2 = M.moe_forward(cfg, xd, lgd, *ew.tiled())
    aq, as_ = M.moe_grouped_gemm1_swiglu(cfg, wl.T, xq, xs, sid, bexp, npp, ew.w13, ew.w13_scale, ksplit=k1)
    out3 = M.moe_grouped_gemm2_combine(cfg, wl.T, aq, as_, sid, bexp, npp, ew.w2, ew.w2_scale, wts)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(out1.view(torch.int16), out3.view(torch.int16))
    ref, _, tie = _oracle_stages(wl, x, lg)
    assert_rows_close(bf16_to_f32(out1), ref, mode, "forward", allowance=tie)


def test_splitk_single_token_all_experts_zero():
    """A token whose x is all zero gives all-zero intermediates and output
    through the split path (zero scales, zero codes)."""
    wl = SPLIT1.with_(T=1)
    cfg, ew, x, lg, _ = _setup(wl, 16)
    out = M.moe_forward(cfg, torch.zeros(1, wl.H, dtype=torch.bfloat16, device="cuda"), lg.cuda(), *ew.tiled())
    torch.cuda.synchronize()
    assert M.plan_ksplit(cfg, 1, 13) == 8
    assert torch.all(out.float() == 0)
