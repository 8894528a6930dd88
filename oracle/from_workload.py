"""Oracle-side preparation of a seeded workload: draws the raw fp32 weights of
the requested experts with the workload's generators and quantises them with
the oracle's own quantisers.  Test infrastructure only (tests, smoke check,
the benchmark's cpu_baseline leg)."""
from __future__ import annotations

import concurrent.futures
import os

import numpy as np

import workloads as W

from . import moe_oracle as O


def quantize_experts(wl: W.Workload, experts, device="cpu", threads: int = 0) -> O.QuantWeights:
    """QuantWeights with the listed experts filled in (the others stay zero),
    raw values drawn on ``device`` with the workload's per-expert generators.
    Experts are quantised one per task on ``threads`` host threads (default:
    the CPUs this process may use, at most 16; NumPy releases the GIL in its
    array operations); each expert's result is the same as a serial run's."""
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
    def one(e, w13, w2):
        q13[e], s13[e] = quant13(w13)
        q2[e], s2[e] = quant2(w2)

    n = threads or min(16, len(os.sched_getaffinity(0)))
    with concurrent.futures.ThreadPoolExecutor(n) as ex:
        futs = []
        for e in experts:   # raw weights are drawn on the calling thread
            futs.append(ex.submit(one, e, W.expert_w13(wl, e, device).cpu().numpy(),
                                  W.expert_w2(wl, e, device).cpu().numpy()))
            if len(futs) >= 2 * n:
                futs.pop(0).result()
        for f in futs:
            f.result()
    return O.QuantWeights(wl.mode, q13, s13, q2, s2)
