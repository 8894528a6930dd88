"""moe_forward_noalloc (the entry point for callers that cannot allocate:
its scratch is the library's static device array) against moe_forward (the
same kernels with a caller workspace), through the C ABI: bit-identical
outputs on two calls in a row, the second with a smaller batch (so stale
contents of the shared array from the first call must not matter), in each
weight contract; a batch whose scratch exceeds the array is refused before
anything is launched."""
import pytest
import torch

import workloads as W
from parity_util import gpu_weights, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    import mxfp4_quantized_weights_amd as mod
    return mod


@pytest.mark.parametrize("mode", ["fp8", "mxfp4", "fp8_ue8m0"])
def test_noalloc_equals_forward_twice(M, mode):
    wl0 = W.WORKLOADS["decode_fp8"].with_(mode=mode, E=64)
    for T in (64, 9):
        wl = wl0.with_(T=T)
        bm = M.pick_block_m(wl.T, wl.E, wl.top_k)
        cfg = M.make_cfg(wl.E, wl.top_k, mode, wl.H, wl.I, block_m=bm, swiglu_limit=wl.swiglu_limit)
        if T == 64:
            ew = gpu_weights(M, cfg, wl, source="cuda")
        log(f"no-alloc {W.describe(wl)} block_m={bm} scratch {M.workspace_bytes(cfg, T)} of "
            f"{M.MOE_NOALLOC_SCRATCH_BYTES} bytes")
        assert M.workspace_bytes(cfg, T) <= M.MOE_NOALLOC_SCRATCH_BYTES
        x = W.activations(wl, "cuda")
        lg = W.router_logits(wl, "cuda")
        ref = M.moe_forward(cfg, x, lg, *ew.tiled())
        out = torch.full((wl.T, wl.H), 3.0, dtype=torch.bfloat16, device="cuda")
        M.moe_forward_noalloc(cfg, x, lg, *ew.tiled(), out=out)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"T={T}: outputs differ"


def test_noalloc_refuses_oversized_batch(M):
    wl = W.WORKLOADS["prefill_fp8"].with_(E=8, T=4096)
    cfg = M.make_cfg(wl.E, wl.top_k, wl.mode, wl.H, wl.I, block_m=128)
    assert M.workspace_bytes(cfg, wl.T) > M.MOE_NOALLOC_SCRATCH_BYTES
    x = torch.zeros(wl.T, wl.H, dtype=torch.bfloat16, device="cuda")
    lg = torch.zeros(wl.T, wl.E, dtype=torch.float32, device="cuda")
    w = torch.zeros(16, dtype=torch.uint8, device="cuda")   # never read: the call is refused first
    out = torch.full((wl.T, wl.H), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(M.MoeError) as ei:
        M.moe_forward_noalloc(cfg, x, lg, w, w, w, w, out=out)
    assert ei.value.status == 6   # MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
