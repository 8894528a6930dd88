"""moe_forward captured in a HIP graph (torch.cuda.CUDAGraph on one stream)
and replayed: every replay, with new inputs written into the captured input
buffers and the program's own eager work and synchronisations in between,
gives bit for bit the output of an eager moe_forward on the same inputs.

Serving runs the decode layer this way (sglang PR #38546 "[AMD]
[GLM-5.3-Flash Day 0] Enable FP8 and Quark MXFP4 MoE on gfx950", Test plan:
decode graph capture).  The layer enqueues kernels only: no host sync, no
allocation, no memset, and every launch reads its batch size from arguments
fixed at capture and its per-batch counts (the padded row count) from device
memory, so a replay with new values in the same buffers is a new forward.
Shapes: the decode layer at T = 1 and 64 (one-launch and two-launch front
ends, K split and tail split) and the prefill layer at T = 4096 (288 experts,
top-8, H = 4096, I = 1024, block FP8); plus an MXFP4 decode batch.
"""
import pytest
import torch

import workloads as W
from parity_util import gpu_weights, log

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


def _weights(cfg, wl):
    key = (wl.H, wl.I, wl.E, wl.mode, wl.seed)
    if key not in _W:
        _W.clear()
        torch.cuda.empty_cache()
        _W[key] = gpu_weights(M, cfg, wl, source="cuda")
    return _W[key]


CASES = {
    "decode_T1": W.WORKLOADS["decode_fp8"].with_(T=1),
    "decode_T64": W.WORKLOADS["decode_fp8"],
    "prefill_T4096": W.WORKLOADS["prefill_fp8"],
    "mxfp4_T16": W.WORKLOADS["prefill_mxfp4"].with_(T=16),
}


@pytest.mark.parametrize("name", list(CASES))
def test_forward_graph_replay_equals_eager(name):
    wl = CASES[name]
    bm = M.pick_block_m(wl.T, wl.E, wl.top_k)
    cfg = M.make_cfg(wl.E, wl.top_k, wl.mode, wl.H, wl.I, wl.Hp, wl.Ip, block_m=bm, swiglu_limit=wl.swiglu_limit)
    log(f"graph capture {W.describe(wl)} block_m={bm} ksplit {M.plan_ksplit(cfg, wl.T, 13)}/"
        f"{M.plan_ksplit(cfg, wl.T, 2)}")
    ew = _weights(cfg, wl)
    tiled = ew.tiled()
    x = W.activations(wl, "cuda")
    lg = W.router_logits(wl, "cuda")
    out_g = torch.empty(wl.T, wl.H, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(M.workspace_bytes(cfg, wl.T), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):      # warm-up on the capture stream
        M.moe_forward(cfg, x, lg, *tiled, out=out_g, ws=ws)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        M.moe_forward(cfg, x, lg, *tiled, out=out_g, ws=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        # new inputs in the captured buffers (drawn with other seeds)
        wl_r = wl.with_(seed=wl.seed + 101 + rep)
        x.copy_(W.activations(wl_r, "cuda"))
        lg.copy_(W.router_logits(wl_r, "cuda"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        # eager work of the program between replays, then the reference
        ref = M.moe_forward(cfg, x.clone(), lg.clone(), *tiled)
        torch.cuda.synchronize()
        same = torch.equal(out_g.view(torch.int16), ref.view(torch.int16))
        log(f"  replay {rep}: bit-identical to eager: {same}")
        assert same
