"""Seeded synthetic workloads for the routed-expert MoE layer.

This module only draws random inputs (router logits, activations, raw fp32
weights) and describes the workload shapes.  It holds none of the layer's
arithmetic: no quantisation, routing or GEMM.  Both the CPU oracle and the
HIP path take their inputs from here.

Every tensor has its own torch generator, seeded from (workload seed, tensor
name, expert), so any single expert's weights can be regenerated on its own,
on the host or on the GPU, without drawing the others.  Values drawn on the
CPU and on the GPU differ (different generators); a test always feeds both
sides from the same draw.

Shapes and distributions follow the MoE layer of the GLM-5.3-Flash-style
model the pages describe (288 routed experts, top-8), with synthetic hidden
and intermediate sizes:
  x ~ N(0, 1) in bf16 (optionally 1% of entries scaled by 30 so that the
  SwiGLU clamp at 10 fires); router logits ~ N(0, 1) (optionally plus
  3 * ln p_e for a Zipf(s = 1.2) expert popularity, popularity rank = expert
  id); weights ~ N(0, 0.02) (standard deviation 0.02), zero-padded.
"""
from __future__ import annotations

import dataclasses
import hashlib

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    I: int
    E: int
    top_k: int
    mode: str  # "fp8", "fp8_ue8m0" or "mxfp4"
    Hp: int = 0
    Ip: int = 0
    swiglu_limit: float = 10.0
    outlier_frac: float = 0.0   # fraction of x entries scaled by outlier_scale
    outlier_scale: float = 30.0
    zipf_s: float = 0.0         # > 0: skewed router logits
    zipf_weight: float = 3.0
    seed: int = 0

    def __post_init__(self):
        if not self.Hp:
            object.__setattr__(self, "Hp", -(-self.H // 128) * 128)
        if not self.Ip:
            object.__setattr__(self, "Ip", -(-self.I // 128) * 128)

    def with_(self, **kw) -> "Workload":
        """Copy with fields replaced; padded sizes follow a changed H / I unless
        given explicitly."""
        if "H" in kw and "Hp" not in kw:
            kw["Hp"] = 0
        if "I" in kw and "Ip" not in kw:
            kw["Ip"] = 0
        return dataclasses.replace(self, **kw)

    @property
    def pairs(self) -> int:
        return self.T * self.top_k

    def flops(self) -> float:
        """Algorithmic FLOPs of the two GEMMs on real (unpadded) sizes:
        2*T*k*H*(2I) + 2*T*k*I*H = 6*T*k*H*I."""
        return 6.0 * self.T * self.top_k * self.H * self.I


WORKLOADS = {
    # tiny block-FP8 layer: a few tiles, parity only
    "tiny_fp8": Workload("tiny_fp8", T=16, H=256, I=128, E=8, top_k=2, mode="fp8"),
    # decode-shaped block-FP8 layer (all 288 experts resident, ~240 active)
    "decode_fp8": Workload("decode_fp8", T=64, H=4096, I=1024, E=288, top_k=8, mode="fp8"),
    # prefill-shaped block-FP8 layer with activation outliers
    "prefill_fp8": Workload("prefill_fp8", T=4096, H=4096, I=1024, E=288, top_k=8, mode="fp8",
                            outlier_frac=0.01),
    # the same layer at a long prefill (16384 tokens, ~455 per expert): enough
    # tokens per expert weight byte that the MFMA, not HBM, is the bound
    "prefill_fp8_16k": Workload("prefill_fp8_16k", T=16384, H=4096, I=1024, E=288, top_k=8, mode="fp8",
                                outlier_frac=0.01),
    # MXFP4 w4a4 layer
    "prefill_mxfp4": Workload("prefill_mxfp4", T=4096, H=4096, I=1024, E=288, top_k=8,
                              mode="mxfp4"),
    # skewed routing, padded hidden/intermediate sizes
    "skewed_padded_fp8": Workload("skewed_padded_fp8", T=2048, H=4000, I=1000, E=288, top_k=8,
                                  mode="fp8", Hp=4096, Ip=1024, zipf_s=1.2),
    # one GPU's share of the layer under tensor parallelism over I (each GPU
    # holds Ip/n of the gate and up halves and the matching w2 columns)
    "tp4_decode_fp8": Workload("tp4_decode_fp8", T=64, H=4096, I=256, E=288, top_k=8, mode="fp8"),
    "tp8_prefill_fp8": Workload("tp8_prefill_fp8", T=4096, H=4096, I=128, E=288, top_k=8, mode="fp8",
                                outlier_frac=0.01),
    "tp4_prefill_mxfp4": Workload("tp4_prefill_mxfp4", T=4096, H=4096, I=256, E=288, top_k=8,
                                  mode="mxfp4"),
    # a shared expert: one dense FFN under the same contracts (E = 1, top-1,
    # routing weight 1)
    "shared_expert_fp8": Workload("shared_expert_fp8", T=4096, H=4096, I=1024, E=1, top_k=1, mode="fp8",
                                  outlier_frac=0.01),
    "shared_expert_mxfp4": Workload("shared_expert_mxfp4", T=64, H=4096, I=1024, E=1, top_k=1,
                                    mode="mxfp4"),
    # block FP8 with UE8M0 (power-of-two) weight and activation scales
    "decode_fp8_ue8m0": Workload("decode_fp8_ue8m0", T=64, H=4096, I=1024, E=288, top_k=8, mode="fp8_ue8m0"),
    "prefill_fp8_ue8m0": Workload("prefill_fp8_ue8m0", T=4096, H=4096, I=1024, E=288, top_k=8,
                                  mode="fp8_ue8m0", outlier_frac=0.01),
}



def _seed(wl: Workload, tag: str, index: int = 0) -> int:
    h = hashlib.sha256(f"{wl.seed}/{tag}/{index}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(wl: Workload, tag: str, index: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(wl, tag, index))
    return g


def router_logits(wl: Workload, device="cpu") -> torch.Tensor:
    """float32 [T, E]."""
    g = _gen(wl, "logits", 0, device)
    lg = torch.randn(wl.T, wl.E, generator=g, device=device, dtype=torch.float32)
    if wl.zipf_s > 0:
        ranks = torch.arange(1, wl.E + 1, dtype=torch.float64)
        p = ranks ** (-wl.zipf_s)
        p = p / p.sum()
        lg = lg + (wl.zipf_weight * torch.log(p)).to(torch.float32).to(device)
    return lg.contiguous()


def activations(wl: Workload, device="cpu") -> torch.Tensor:
    """bfloat16 [T, H]."""
    g = _gen(wl, "x", 0, device)
    x = torch.randn(wl.T, wl.H, generator=g, device=device, dtype=torch.float32)
    if wl.outlier_frac > 0:
        g2 = _gen(wl, "outlier", 0, device)
        mask = torch.rand(wl.T, wl.H, generator=g2, device=device) < wl.outlier_frac
        x = torch.where(mask, x * wl.outlier_scale, x)
    return x.to(torch.bfloat16).contiguous()


def expert_w13(wl: Workload, e: int, device="cpu") -> torch.Tensor:
    """float32 [2*Ip, Hp]: gate rows [0, I), up rows [Ip, Ip + I), real columns
    [0, H); everything else zero."""
    g = _gen(wl, "w13", e, device)
    raw = torch.randn(2 * wl.I, wl.H, generator=g, device=device, dtype=torch.float32) * 0.02
    out = torch.zeros(2 * wl.Ip, wl.Hp, device=device, dtype=torch.float32)
    out[:wl.I, :wl.H] = raw[:wl.I]
    out[wl.Ip:wl.Ip + wl.I, :wl.H] = raw[wl.I:]
    return out


def expert_w2(wl: Workload, e: int, device="cpu") -> torch.Tensor:
    """float32 [Hp, Ip]: real block [0, H) x [0, I); everything else zero."""
    g = _gen(wl, "w2", e, device)
    raw = torch.randn(wl.H, wl.I, generator=g, device=device, dtype=torch.float32) * 0.02
    out = torch.zeros(wl.Hp, wl.Ip, device=device, dtype=torch.float32)
    out[:wl.H, :wl.I] = raw
    return out


def all_w13(wl: Workload, experts=None, device="cpu") -> torch.Tensor:
    ex = range(wl.E) if experts is None else experts
    return torch.stack([expert_w13(wl, e, device) for e in ex])


def all_w2(wl: Workload, experts=None, device="cpu") -> torch.Tensor:
    ex = range(wl.E) if experts is None else experts
    return torch.stack([expert_w2(wl, e, device) for e in ex])


def pick_block_m(wl_or_T, E: int = 0, top_k: int = 0) -> int:
    """Rows per expert block: 16 / 32 when experts see few tokens (decode),
    else 128.  A host-side launch choice, not part of the method."""
    if isinstance(wl_or_T, Workload):
        T, E, top_k = wl_or_T.T, wl_or_T.E, wl_or_T.top_k
    else:
        T = wl_or_T
    per_expert = T * top_k / max(E, 1)
    if per_expert <= 16:
        return 16
    if per_expert <= 32:
        return 32
    return 128


def describe(wl: Workload) -> str:
    return (f"{wl.name}: T={wl.T} H={wl.H}(Hp={wl.Hp}) I={wl.I}(Ip={wl.Ip}) E={wl.E} "
            f"top_k={wl.top_k} mode={wl.mode} limit={wl.swiglu_limit} seed={wl.seed}")


__all__ = ["Workload", "WORKLOADS", "router_logits", "activations", "expert_w13", "expert_w2",
           "all_w13", "all_w2", "pick_block_m", "describe"]
