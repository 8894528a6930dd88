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
the split the library plans.  The intermediate check is
parity_util.verify_intermediate: every code that differs from the oracle's
must sit at a rounding midpoint within the element's fp32 accumulation
bound, and only those codes' effect is added to the output tolerance.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from parity_util import (assert_rows_close, bf16_to_f32, gpu_intermediate_rows, gpu_weights, log,
                         oracle_stages, oracle_weights_cpu, oracle_weights_subset, pairs_of, verify_intermediate)

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
    return ref, st, Q


def _verify(wl, aq, as_, sid, npp, st, Q):
    """The intermediate against the oracle's stages; -> output allowance."""
    rows = gpu_intermediate_rows(wl.mode, wl.Ip, aq, as_, sid, npp, wl.T * wl.top_k, wl.top_k,
                                 pairs_of(range(wl.T), wl.top_k))
    return verify_intermediate(wl.mode, wl.swiglu_limit, rows, st, Q, wl.H)[0]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("bm", [16, 128])
def test_gemm1_splitk_stage(mode, bm):
    wl = SPLIT1.with_(mode=mode)
    log(f"gemm1 split {W.describe(wl)} BM={bm}")
    cfg, ew, x, lg, (ids, wts, sid, bexp, npp, xq, xs) = _setup(wl, bm)
    _, st, Q = _oracle_stages(wl, x, lg)
    for ks in (1, 2, 4, 8):
        P = wl.T * wl.top_k
        need = ks * P * 2 * wl.Ip * 4 + P * 4   # partial sums, then each pair's sorted row
        assert M.splitk_bytes(cfg, wl.T, 13, ks) == (0 if ks == 1 else -(-need // 256) * 256)
        aq, as_ = M.moe_grouped_gemm1_swiglu(cfg, wl.T, xq, xs, sid, bexp, npp, ew.w13, ew.w13_scale, ksplit=ks)
        torch.cuda.synchronize()
        log(f"  ksplit {ks}")
        _verify(wl, aq, as_, sid, npp, st, Q)


@pytest.mark.parametrize("mode", MODES)
def test_gemm2_splitk_combine(mode):
    wl = SPLIT2.with_(mode=mode)
    log(f"gemm2 split {W.describe(wl)}")
    cfg, ew, x, lg, (ids, wts, sid, bexp, npp, xq, xs) = _setup(wl, 16)
    ref, st, Q = _oracle_stages(wl, x, lg)
    aq, as_ = M.moe_grouped_gemm1_swiglu(cfg, wl.T, xq, xs, sid, bexp, npp, ew.w13, ew.w13_scale)
    torch.cuda.synchronize()
    tie = _verify(wl, aq, as_, sid, npp, st, Q)
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
    ref, st, Q = _oracle_stages(wl, x, lg)
    tie = _verify(wl, aq, as_, sid, npp, st, Q)
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


# Tail split: more (block, N tile) items than workgroups (one per compute
# unit, 256 on the MI355X) and not a multiple of them: 40 experts x 8 N tiles
# at block_m 16 (some experts take two blocks) give ~360 GEMM1 items, one
# whole round and a leftover round that the tail split cuts into K pieces;
# at block_m 64 and 128 (one block per expert) 320 items.
# K = 1024 (8 K blocks): pieces of 4 K blocks (ksplit -2) in every mode.
TAIL1 = W.Workload("tail1", T=48, H=1024, I=1024, E=40, top_k=8, mode="fp8", outlier_frac=0.02)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("bm", [16, 32, 64, 128])
def test_gemm1_tail_split_stage(mode, bm):
    """GEMM1 with the tail split (whole rounds unsplit, the leftover items in
    K pieces finished by the second kernel) against the oracle's stages, and
    moe_forward (which plans it) equal to the stage entry points."""
    wl = TAIL1.with_(mode=mode)
    log(f"gemm1 tail split {W.describe(wl)} BM={bm}")
    cfg, ew, x, lg, (ids, wts, sid, bexp, npp, xq, xs) = _setup(wl, bm)
    items = int(npp.item()) // bm * (wl.Ip // 128)
    log(f"  {items} GEMM1 items")
    assert items > 256 or bm == 32
    ref, st, Q = _oracle_stages(wl, x, lg)
    # planned at every block_m for block FP8, at block_m 16 / 32 for MXFP4
    # (which still takes it when asked)
    planned = -2 if bm <= 32 or mode != "mxfp4" else 1
    assert M.plan_ksplit(cfg, wl.T, 13) == planned
    assert M.splitk_bytes(cfg, wl.T, 13, -2) > 0
    res = {}
    for ks in (1, -2):
        aq, as_ = M.moe_grouped_gemm1_swiglu(cfg, wl.T, xq, xs, sid, bexp, npp, ew.w13, ew.w13_scale, ksplit=ks)
        torch.cuda.synchronize()
        log(f"  ksplit {ks}")
        res[ks] = (aq, as_, _verify(wl, aq, as_, sid, npp, st, Q))
    aq, as_, tie = res[planned]
    xd, lgd = x.cuda(), lg.cuda()
    out1 = M.moe_forward(cfg, xd, lgd, *ew.tiled())
    out3 = M.moe_grouped_gemm2_combine(cfg, wl.T, aq, as_, sid, bexp, npp, ew.w2, ew.w2_scale, wts)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out3.view(torch.int16))
    assert_rows_close(bf16_to_f32(out1), ref, mode, "tail forward", allowance=tie)


@pytest.mark.parametrize("mode", MODES)
def test_gemm1_tail_split_few_items(mode):
    """A tail launch with fewer items than half a round (ksplit -2 asked of
    the stage entry point): no whole round, every item is cut into pieces,
    and the intermediate matches the oracle's as the unsplit launch does."""
    wl = TAIL1.with_(mode=mode, T=6, E=8, top_k=2)
    log(f"gemm1 tail split, few items {W.describe(wl)}")
    cfg, ew, x, lg, (ids, wts, sid, bexp, npp, xq, xs) = _setup(wl, 16)
    items = int(npp.item()) // 16 * (wl.Ip // 128)
    log(f"  {items} GEMM1 items")
    assert items <= 128
    ref, st, Q = _oracle_stages(wl, x, lg)
    for ks in (1, -2):
        aq, as_ = M.moe_grouped_gemm1_swiglu(cfg, wl.T, xq, xs, sid, bexp, npp, ew.w13, ew.w13_scale, ksplit=ks)
        torch.cuda.synchronize()
        log(f"  ksplit {ks}")
        _verify(wl, aq, as_, sid, npp, st, Q)


@pytest.mark.parametrize("mode,T", [("fp8", 64), ("fp8_ue8m0", 64), ("mxfp4", 64), ("fp8", 8)])
def test_gemm1_tail_split_full_size(mode, T):
    """At the decode shape (T = 64, H = 4096, I = 1024, 288 experts; ~1860
    GEMM1 items: 7 whole rounds and 72 items left, under half a round), the
    unsplit launch and every tail split give an intermediate that passes the
    oracle check on a token sample that includes tokens of the last blocks
    (whose items are the leftover ones the tail split cuts).  At T = 8 (~460
    items: 208 left, over half a round) a tail launch runs every item whole:
    bit-identical to the unsplit launch."""
    wl = W.WORKLOADS["decode_fp8"].with_(mode=mode, T=T)
    cfg = M.make_cfg(wl.E, wl.top_k, wl.mode, wl.H, wl.I, wl.Hp, wl.Ip, block_m=16, swiglu_limit=wl.swiglu_limit)
    log(f"gemm1 tail split, full size: {W.describe(wl)}")
    ew = gpu_weights(M, cfg, wl)
    x, lg = W.activations(wl, "cuda"), W.router_logits(wl, "cuda")
    ids, wts, sid, bexp, offs, npp, xq, xs = M.moe_route_permute_quant(cfg, x, lg)
    torch.cuda.synchronize()
    rows = int(npp.item())
    rows_total = M.max_blocks(wl.T * wl.top_k, wl.E, 16) * 16
    items = rows // 16 * 8
    log(f"  {items} GEMM1 items")
    # sample: tokens spread over the batch plus tokens of the last 9 blocks
    P = wl.T * wl.top_k
    tail_pairs = [int(f) for f in sid.cpu().numpy()[max(0, rows - 9 * 16):rows] if f < P]
    toks = sorted(set(np.linspace(0, wl.T - 1, 4).round().astype(int).tolist()) |
                  set(f // wl.top_k for f in tail_pairs[::max(1, len(tail_pairs) // 4)][:4]))
    ido, _ = O.route_topk(lg.cpu().numpy()[toks], wl.top_k)
    Q = oracle_weights_subset(wl, np.unique(ido), "cuda")
    ref, st = oracle_stages(wl, x, lg, Q, tokens=toks)
    log(f"  oracle on tokens {toks}")
    outs = {}
    for ks in (1, -2, -4, -8):
        aq, as_ = M.moe_grouped_gemm1_swiglu(cfg, wl.T, xq, xs, sid, bexp, npp, ew.w13, ew.w13_scale, ksplit=ks)
        torch.cuda.synchronize()
        log(f"  ksplit {ks}")
        g = gpu_intermediate_rows(wl.mode, wl.Ip, aq, as_, sid, npp, P, wl.top_k, pairs_of(toks, wl.top_k))
        verify_intermediate(wl.mode, wl.swiglu_limit, g, st, Q, wl.H)
        outs[ks] = (aq.cpu().numpy().reshape(rows_total, -1)[:rows], as_.cpu().numpy().reshape(rows_total, -1)[:rows])
    if 2 * (items % 256) > 256:
        for ks in (-2, -4, -8):
            assert np.array_equal(outs[ks][0], outs[1][0]) and np.array_equal(outs[ks][1], outs[1][1])
