"""Full-size workloads on the GPU, in the launch configuration the benchmark
uses (block_m from pick_block_m, all experts resident, the splits moe_forward
plans), checked against the oracle.

Bit-exact over the whole batch: routing ids, the permutation, and the
quantised activations (codes and scales) that the front end of moe_forward
writes.  Bit-exact on the sampled experts: the quantised weight bytes and
scales.  moe_forward equals the stage entry points bit for bit.  On a sample
of tokens spread over the batch (first, last, evenly strided; 64 for the
decode, prefill, MXFP4 and skewed workloads): GEMM1's re-quantised
intermediate passes the verified-tie check, and the output rows are within
2e-2 (block FP8) / 6e-2 (MXFP4) of the row RMS after adding only the effect
of the intermediate codes that differed (see parity_util).  The layer is
row-independent, so the oracle computes only the sampled rows, with only the
experts they route to.
"""
import gc

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from parity_util import (bf16_to_f32, check_intermediate_and_output, gpu_stage_chain, gpu_weights, log,
                         oracle_stages, oracle_weights_subset)

pytestmark = pytest.mark.gpu

M = None
_CACHE = {}

# tokens sampled per workload (the rest: 16)
SAMPLE = {"decode_fp8": 64, "prefill_fp8": 64, "prefill_mxfp4": 64, "skewed_padded_fp8": 64}


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


def sample_tokens(T: int, n: int):
    """n tokens spread over [0, T): the first, the last and evenly strided."""
    return sorted(set(np.linspace(0, T - 1, min(n, T)).round().astype(int).tolist()))


@pytest.mark.parametrize("name", ["decode_fp8", "prefill_fp8", "prefill_fp8_16k", "skewed_padded_fp8", "prefill_mxfp4",
                                  "tp4_decode_fp8", "tp8_prefill_fp8", "tp4_prefill_mxfp4", "shared_expert_fp8",
                                  "shared_expert_mxfp4", "decode_fp8_ue8m0", "prefill_fp8_ue8m0"])
def test_fullsize_sampled(name):
    wl = W.WORKLOADS[name]
    bm = M.pick_block_m(wl.T, wl.E, wl.top_k)
    log(f"full size {W.describe(wl)} block_m={bm}")
    cfg = M.make_cfg(wl.E, wl.top_k, wl.mode, wl.H, wl.I, wl.Hp, wl.Ip, block_m=bm, swiglu_limit=wl.swiglu_limit)
    ew = _weights(cfg, wl)
    x = W.activations(wl, "cuda")
    lg = W.router_logits(wl, "cuda")
    out = M.moe_forward(cfg, x, lg, *ew.tiled())
    ch = gpu_stage_chain(M, cfg, wl.T, x, lg, ew)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ch["out"].view(torch.int16)), "moe_forward differs from the stages"

    # whole batch, bit-exact: routing, permutation, quantised x
    lg_h = lg.cpu().numpy()
    ido, wo = O.route_topk(lg_h, wl.top_k)
    assert np.array_equal(ch["ids"].cpu().numpy(), ido)
    assert np.allclose(ch["w"].cpu().numpy(), wo, rtol=2e-6, atol=0)
    so, bo, oo, no = O.permute_align(ido, wl.E, bm)
    assert np.array_equal(ch["sid"].cpu().numpy(), so) and np.array_equal(ch["bexp"].cpu().numpy(), bo)
    assert int(ch["npp"].item()) == no
    xq_o, xs_o = O.quant_act(wl.mode, O.pad_cols(x.float().cpu().numpy(), wl.Hp))
    assert np.array_equal(ch["xq"].cpu().numpy(), xq_o), "quantised x codes differ"
    xs_g = ch["xs"].cpu().numpy()
    if wl.mode == "fp8_ue8m0":
        xs_g = xs_g[:, :wl.Hp // 128]
    assert np.array_equal(xs_g.view(np.uint8), np.ascontiguousarray(xs_o).view(np.uint8)), "quantised x scales differ"
    active = int(np.count_nonzero(np.bincount(ido.reshape(-1), minlength=wl.E)))
    log(f"  routing, permutation and the {wl.T}x{wl.Hp} quantised x bit-exact; active experts {active}; "
        f"num_post_padded {no}")

    toks = sample_tokens(wl.T, SAMPLE.get(name, 16))
    experts = np.unique(ido[toks])
    log(f"  oracle on {len(toks)} tokens ({len(experts)} experts)")
    Q = oracle_weights_subset(wl, experts, "cuda")
    for e in experts[:: max(1, len(experts) // 4)]:
        assert np.array_equal(ew.q13[e].cpu().numpy(), Q.w13[e])
        assert np.array_equal(ew.q2[e].cpu().numpy(), Q.w2[e])
        assert np.array_equal(ew.s13[e].cpu().numpy().view(np.uint8), Q.s13[e].view(np.uint8))
        assert np.array_equal(ew.s2[e].cpu().numpy().view(np.uint8), Q.s2[e].view(np.uint8))
    ref, st = oracle_stages(wl, x, lg, Q, tokens=toks)
    check_intermediate_and_output(wl, bf16_to_f32(out)[toks], ch["aq"], ch["as_"], ch["sid"], ch["npp"], ref, st, Q,
                                  tokens=toks, what=name)
