"""Full-size workloads on the GPU, in the launch configuration the benchmark
uses (block_m from pick_block_m, all experts resident), checked against the
oracle on sampled tokens (the layer is row-independent, so the oracle
computes only those rows, with only the experts they route to).

Bit-exact over the whole workload: routing ids and the permutation.  Bit-exact
on the sampled experts: the quantised weight bytes and scales.  Tolerance on
the sampled output rows: 2e-2 (block FP8) / 6e-2 (MXFP4) times the row RMS,
after the re-quantisation tie allowance (see parity_util).
"""
import gc

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from parity_util import (assert_rows_close, bf16_to_f32, gpu_weights, log, oracle_weights_subset,
                         requant_tie_allowance)

pytestmark = pytest.mark.gpu

M = None
_CACHE = {}


@pytest.fixture(scope="module", autouse=True)
def lib():
    global M
    import mxfp4_quantized_weights_amd as mod
    M = mod
    yield mod
    _CACHE.clear()
    gc.collect()
    torch.cuda.empty_cache()


def _weights(cfg, wl):
    key = (wl.H, wl.I, wl.Hp, wl.Ip, wl.E, wl.mode, wl.seed)
    if key not in _CACHE:
        _CACHE.clear()
        gc.collect()
        torch.cuda.empty_cache()
        _CACHE[key] = gpu_weights(M, cfg, wl, source="cuda")
    return _CACHE[key]


@pytest.mark.parametrize("name", ["decode_fp8", "prefill_fp8", "prefill_fp8_16k", "skewed_padded_fp8", "prefill_mxfp4", "tp4_decode_fp8",
                                  "tp8_prefill_fp8", "tp4_prefill_mxfp4", "shared_expert_fp8", "shared_expert_mxfp4",
                                  "decode_fp8_ue8m0", "prefill_fp8_ue8m0"])
def test_fullsize_sampled(name):
    wl = W.WORKLOADS[name]
    bm = M.pick_block_m(wl.T, wl.E, wl.top_k)
    log(f"full size {W.describe(wl)} block_m={bm}")
    cfg = M.make_cfg(wl.E, wl.top_k, wl.mode, wl.H, wl.I, wl.Hp, wl.Ip, block_m=bm, swiglu_limit=wl.swiglu_limit)
    ew = _weights(cfg, wl)
    x = W.activations(wl, "cuda")
    lg = W.router_logits(wl, "cuda")
    out = M.moe_forward(cfg, x, lg, *ew.tiled())
    ids, wts = M.moe_route_topk(lg, wl.top_k)
    sid, bexp, offs, npp = M.moe_permute_align(ids, wl.E, bm)
    torch.cuda.synchronize()
    lg_h = lg.cpu().numpy()
    ido, wo = O.route_topk(lg_h, wl.top_k)
    assert np.array_equal(ids.cpu().numpy(), ido)
    assert np.allclose(wts.cpu().numpy(), wo, rtol=2e-6, atol=0)
    so, bo, oo, no = O.permute_align(ido, wl.E, bm)
    assert np.array_equal(sid.cpu().numpy(), so) and np.array_equal(bexp.cpu().numpy(), bo)
    active = int(np.count_nonzero(np.bincount(ido.reshape(-1), minlength=wl.E)))
    log(f"  routing/permutation bit-exact; active experts {active}; num_post_padded {no}")

    rng = np.random.default_rng(5)
    toks = sorted({0, wl.T - 1, int(rng.integers(1, wl.T - 1))})
    experts = np.unique(ido[toks])
    log(f"  oracle on tokens {toks} ({len(experts)} experts)")
    Q = oracle_weights_subset(wl, experts, "cuda")
    for e in experts[:3]:
        assert np.array_equal(ew.q13[e].cpu().numpy(), Q.w13[e])
        assert np.array_equal(ew.q2[e].cpu().numpy(), Q.w2[e])
        assert np.array_equal(ew.s13[e].cpu().numpy().view(np.uint8), Q.s13[e].view(np.uint8))
        assert np.array_equal(ew.s2[e].cpu().numpy().view(np.uint8), Q.s2[e].view(np.uint8))
    ref, st = O.moe_forward(x.float().cpu().numpy(), lg_h, Q, wl.top_k, wl.swiglu_limit, wl.H, wl.I, tokens=toks,
                            return_stages=True)
    tie = requant_tie_allowance(st, Q, wl.mode, wl.H)
    assert_rows_close(bf16_to_f32(out)[toks], ref, wl.mode, name, allowance=tie)
