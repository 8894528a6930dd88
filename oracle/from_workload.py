"""Oracle-side preparation of a seeded workload: draws the raw fp32 weights of
the requested experts with the workload's generators and quantises them with
the oracle's own quantisers.  Test infrastructure only (tests, smoke check,
the benchmark's cpu_baseline leg)."""
from __future__ import annotations

import numpy as np

import workloads as W

from . import moe_oracle as O


def quantize_experts(wl: W.Workload, experts, device="cpu") -> O.QuantWeights:
    """QuantWeights with the listed experts filled in (the others stay zero),
    raw values drawn on ``device`` with the workload's per-expert generators."""
    experts = sorted(set(int(e) for e in experts))
    E, Hp, Ip = wl.E, wl.Hp, wl.Ip
    if wl.mode == "mxfp4":
        q13 = np.zeros((E, 2 * Ip, Hp // 2), np.uint8)
        s13 = np.zeros((E, 2 * Ip, Hp // 32), np.uint8)
        q2 = np.zeros((E, Hp, Ip // 2), np.uint8)
        s2 = np.zeros((E, Hp, Ip // 32), np.uint8)
        quant13 = quant2 = O.quant_mxfp4_rows
    else:
        sdt = np.float32 if wl.mode == "fp8" else np.uint8
        q13 = np.zeros((E, 2 * Ip, Hp), np.uint8)
        s13 = np.zeros((E, 2 * Ip // 128, Hp // 128), sdt)
        q2 = np.zeros((E, Hp, Ip), np.uint8)
        s2 = np.zeros((E, Hp // 128, Ip // 128), sdt)
        quant13 = quant2 = O.quant_fp8_weight if wl.mode == "fp8" else O.quant_fp8e8_weight
    for e in experts:
        w13 = W.expert_w13(wl, e, device).cpu().numpy()
        w2 = W.expert_w2(wl, e, device).cpu().numpy()
        q13[e], s13[e] = quant13(w13)
        q2[e], s2[e] = quant2(w2)
    return O.QuantWeights(wl.mode, q13, s13, q2, s2)
