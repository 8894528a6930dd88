"""Benchmark of the routed-expert MoE layer on one MI355X.

One step = one moe_forward over one batch of synthetic tokens: top-k routing,
permutation, activation quantisation, GEMM1 + clamped SwiGLU +
re-quantisation, GEMM2 + weighted combine.  Inputs (router logits, bf16
activations, quantised + preshuffled weights of all experts) are resident in
HBM before the timed region starts.

The default workload is the prefill layer: T = 4096 tokens, H = 4096,
I = 1024, 288 experts, top-8, block FP8 (e4m3 weights with 128x128 scales,
dynamic 1x128 activations), 1% of x scaled by 30 -- the largest
configuration of the benchmark that fits one GPU.

Prints one JSON line with tokens/s (whole job), effective TFLOP/s
(6*T*k*H*I per step on the real sizes), the roofline of the dominant kernel
(its average duration from HIP events recorded on the launch stream around
the same kernels, called through the stage entry points) with the attainable
ceiling min(peak, intensity x HBM bandwidth), the CPU oracle's throughput on
a bounded sample of the same workload, and (unless --no-extras) the decode
(T = 64) and MXFP4 (T = 4096) layers measured the same way, plus the decode
layer at T = 1 .. 64 replayed from a HIP graph, as extra keys, and what the
part itself delivers beside the published peaks (a read stream's and a device
copy's GB/s, each MFMA instruction's TFLOP/s: `box_measured`).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = {"fp8": 5000.0, "fp8_ue8m0": 5000.0, "mxfp4": 10100.0}   # dense, TFLOP/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="prefill_fp8")
    ap.add_argument("--T", type=int, default=0, help="override the token count")
    ap.add_argument("--block-m", type=int, default=0)
    ap.add_argument("--cpu-sample", type=int, default=-1,
                    help="tokens in the oracle's timed sample (0 = skip; default -1: the whole batch)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the extra decode and MXFP4 measurements")
    ap.add_argument("--no-breakdown", action="store_true")
    ap.add_argument("--decode-sweep", action="store_true",
                    help="only the graph-replayed decode sweep (T = 1 .. 64) of the decode layer")
    ap.add_argument("--decode-path", default="forward", choices=["forward", "gemv"],
                    help="decode sweep through moe_forward or through the decode (GEMV) entry points (T <= 16)")
    ap.add_argument("--weight-copies", type=int, default=1,
                    help="rotate over this many copies of the weights, one per step, so that no "
                         "step finds the previous step's weights in the memory-side cache")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 3 device-to-device copies of MIB MiB (calibrates HBM byte counters) and exit")
    return ap.parse_args()


def copy_calibration(mib: int):
    """Plain device copy of known size: FETCH_SIZE / WRITE_SIZE of these
    dispatches give the counters' scale against true bytes."""
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_dispatch": n * 4}), flush=True)


def box_measured(M):
    """What this part delivers beside the published peaks: a 2 GiB read with the
    GEMMs' kind of load (the library's stream diagnostic), a 1 GiB device copy
    (read + write bytes over its time; medians of 5) and each matrix-core
    instruction the GEMMs use, from the library's rate diagnostic (8
    independent accumulator chains per wave, 4 waves per SIMD, no memory
    traffic; median of 3 launches of ~3 ms)."""
    import torch
    n = (1 << 30) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)

    def med_ms(fn, reps):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        return sorted(ts)[len(ts) // 2]

    copy_gbs = 2 * n * 4 / (med_ms(lambda: b.copy_(a), 5) * 1e-3) / 1e9
    del b
    big = torch.ones(2 * n, dtype=torch.float32, device="cuda")   # 2 GiB, read once per launch
    read_gbs = big.numel() * 4 / (med_ms(lambda: M.moe_diag_stream_read(big), 5) * 1e-3) / 1e9
    del a, big
    sink = torch.empty(M.DIAG_MFMA_RATE_WORKGROUPS * 256, dtype=torch.float32, device="cuda")
    tflops = {}
    for kind, name, iters in ((0, "f16_16x16x32", 12000), (1, "fp8_16x16x128", 6000), (2, "fp4_16x16x128", 12000)):
        flop = M.DIAG_MFMA_RATE_WORKGROUPS * 4 * iters * 8 * M.DIAG_MFMA_RATE_FLOP[kind]
        ms = med_ms(lambda: M.moe_diag_mfma_rate(kind, iters, sink), 3)
        tflops[name] = round(flop / (ms * 1e-3) / 1e12, 1)
    return {"read_gbs": round(read_gbs, 1), "copy_gbs": round(copy_gbs, 1), "mfma_tflops": tflops,
            "spec": {"hbm_gbs": HBM_PEAK_GBS, "f16_tflops": 2500.0, "fp8_tflops": 5000.0, "fp4_tflops": 10100.0}}


def algorithmic_bytes(wl, ids, M):
    """Bytes the layer must move at least once: the weights and scales of
    every expert with at least one pair, x, the logits and the output; plus,
    per kernel, what it must read/write (documented next to the roofline)."""
    import numpy as np
    counts = np.bincount(ids.reshape(-1), minlength=wl.E)
    active = int(np.count_nonzero(counts))
    Hp, Ip = wl.Hp, wl.Ip
    P = wl.T * wl.top_k
    if wl.mode in ("fp8", "fp8_ue8m0"):
        sb = 4 if wl.mode == "fp8" else 1   # bytes per block scale (UE8M0: one byte in HBM)
        w13 = 2 * Ip * Hp + (2 * Ip // 128) * (Hp // 128) * sb
        w2 = Hp * Ip + (Hp // 128) * (Ip // 128) * sb
        xq = wl.T * (Hp + Hp // 128 * sb)
        aq = P * (Ip + Ip // 128 * sb)
    else:
        w13 = 2 * Ip * Hp // 2 + 2 * Ip * Hp // 32
        w2 = Hp * Ip // 2 + Hp * Ip // 32
        xq = wl.T * (Hp // 2 + Hp // 32)
        aq = P * (Ip // 2 + Ip // 32)
    layer = active * (w13 + w2) + wl.T * wl.H * 2 + wl.T * wl.E * 4 + wl.T * wl.H * 2
    gemm1 = active * w13 + xq + aq
    gemm2 = active * w2 + aq + wl.T * wl.H * 2 + P * 4   # + the output and the routing weights
    return dict(active_experts=active, layer=layer, gemm1=gemm1, gemm2=gemm2,
                w13_per_expert=w13, w2_per_expert=w2)


def recorded_traffic(workload: str, T: int, block_m: int):
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary (calibrated against a plain
    copy), or None when there is none, it was taken at another token count
    or block size, or the GEMM source changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{workload}_hbm_counters.md")
    if not os.path.exists(path):
        return None
    src = os.path.join(ROOT, "mxfp4_quantized_weights_amd", "csrc", "gemm.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    for line in open(path):
        if line.startswith("TRAFFIC "):
            kv = dict(t.split("=", 1) for t in line.split()[1:])
            if kv.get("gemm_src_sha256") != sha or kv.get("T") != str(T) or kv.get("block_m") != str(block_m):
                return None
            return int(kv["read_bytes"]) + int(kv["write_bytes"])
    return None


def cpu_baseline(wl, x, lg, sample_tokens: int):
    """The oracle, as it stands, on the first `sample_tokens` tokens of the
    same workload (all of them when `sample_tokens` < 0): timed from bf16
    activations + quantised weights to the fp32 output (routing, activation
    quantisation, dequantisation, GEMMs, SwiGLU, re-quantisation, combine).
    Weight quantisation is done beforehand and not timed."""
    import numpy as np
    import oracle as O
    from threadpoolctl import threadpool_info
    from oracle.from_workload import quantize_experts
    n = wl.T if sample_tokens < 0 else min(sample_tokens, wl.T)
    toks = list(range(n))
    lg_h = lg.cpu().numpy()
    x_h = x.float().cpu().numpy()
    ids, _ = O.route_topk(lg_h[toks], wl.top_k)
    Q = quantize_experts(wl, np.unique(ids), "cuda")
    # the sample is timed until about 10 s of oracle work have run (at most 5
    # passes); the median pass gives the rate
    passes = []
    while len(passes) < 5 and sum(passes) < 10.0:
        t0 = time.perf_counter()
        O.moe_forward(x_h, lg_h, Q, wl.top_k, wl.swiglu_limit, wl.H, wl.I, tokens=toks)
        passes.append(time.perf_counter() - t0)
    dt = float(np.median(passes))
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    return {"value": len(toks) / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{'all' if len(toks) == wl.T else 'first'} {len(toks)} of {wl.T} tokens of {wl.name} "
                      f"({len(np.unique(ids))} experts); {len(passes)} timed passes, {sum(passes):.1f} s, "
                      f"median {dt:.2f} s; weight quantisation excluded; "
                      f"host affinity {len(os.sched_getaffinity(0))} cpus"}


def build_weights(M, cfg, wl, dev, copies: int):
    """Quantised + preshuffled weights of every expert (drawn on the GPU,
    quantised and preshuffled by the library); only the tiled copies stay."""
    import torch
    import workloads as W
    ew = M.ExpertWeights(cfg, dev)
    for e0 in range(0, wl.E, 16):
        ex = range(e0, min(wl.E, e0 + 16))
        ew.add_experts(e0, W.all_w13(wl, ex, "cuda"), W.all_w2(wl, ex, "cuda"))
    ew.finalize()
    ew.q13 = ew.s13 = ew.q2 = ew.s2 = None
    torch.cuda.empty_cache()
    out = [tuple(ew.tiled())]
    for _ in range(1, max(1, copies)):
        out.append(tuple(t.clone() for t in out[0]))
    return out


def measure(M, wl, args, copies=None, steps=None, warmup=None, breakdown=True, block_m=None):
    """Times `steps` moe_forward steps of workload `wl` (after `warmup`
    untimed ones), then the same kernels through the stage entry points with
    HIP events on the launch stream.  Returns (result dict, weight copies,
    x, logits)."""
    import numpy as np
    import torch
    import workloads as W
    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
    bm = (args.block_m if block_m is None else block_m) or M.pick_block_m(wl.T, wl.E, wl.top_k)
    cfg = M.make_cfg(wl.E, wl.top_k, wl.mode, wl.H, wl.I, wl.Hp, wl.Ip, block_m=bm,
                     swiglu_limit=wl.swiglu_limit)
    dev = torch.device("cuda", 0)
    if copies is None:
        copies = build_weights(M, cfg, wl, dev, args.weight_copies)
    x = W.activations(wl, "cuda")
    lg = W.router_logits(wl, "cuda")
    out = torch.empty(wl.T, wl.H, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(M.workspace_bytes(cfg, wl.T), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        w13, s13, w2, s2 = copies[i % len(copies)]
        M.moe_forward(cfg, x, lg, w13, s13, w2, s2, out=out, ws=ws, stream=stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = wall * 1e3 / steps

    ids, wts = M.moe_route_topk(lg, wl.top_k)
    nbytes = algorithmic_bytes(wl, ids.cpu().numpy(), M)
    kern, spread = {}, None
    ks1 = M.plan_ksplit(cfg, wl.T, 13)
    if breakdown:
        # the stages moe_forward runs: the front end (routing, permutation,
        # quantisation of x; one launch for small batches), GEMM1, GEMM2 +
        # combine, with HIP events recorded on the launch stream between them
        names = ["front_end", "gemm1_swiglu", "gemm2_combine"]
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(steps)]
        aq_b, as_b = M.intermediate_bytes(cfg, wl.T)
        nb = M.max_blocks(wl.T * wl.top_k, wl.E, bm)
        sid = torch.empty(nb * bm, dtype=torch.int32, device=dev)
        bexp = torch.empty(nb, dtype=torch.int32, device=dev)
        offs = torch.empty(wl.E + 1, dtype=torch.int32, device=dev)
        npp = torch.empty(1, dtype=torch.int32, device=dev)
        import ctypes
        lib = M.lib()
        cfgp = ctypes.byref(cfg)
        sp = stream.cuda_stream
        xq, xs = M._act_buffers(cfg.quant_mode, wl.T, wl.Hp, dev)
        aq = torch.empty(aq_b, dtype=torch.uint8, device=dev)
        as_ = torch.empty(as_b, dtype=torch.uint8, device=dev)
        # GEMM1 with the K split moe_forward plans (small batches: GEMM1 pieces
        # plus the SwiGLU/re-quantisation kernel)
        part_b = M.splitk_bytes(cfg, wl.T, 13, ks1)
        part = torch.empty(max(part_b, 1), dtype=torch.uint8, device=dev)

        def staged(evs, i):
            w13, s13, w2, s2 = copies[i % len(copies)]
            evs[0].record(stream)
            lib.moe_route_permute_quant(cfgp, wl.T, lg.data_ptr(), x.data_ptr(), wl.H, ids.data_ptr(),
                                        wts.data_ptr(), sid.data_ptr(), bexp.data_ptr(), offs.data_ptr(),
                                        npp.data_ptr(), xq.data_ptr(), xs.data_ptr(), sp)
            evs[1].record(stream)
            lib.moe_grouped_gemm1_swiglu_splitk(cfgp, wl.T, xq.data_ptr(), xs.data_ptr(), sid.data_ptr(),
                                                bexp.data_ptr(), npp.data_ptr(), w13.data_ptr(), s13.data_ptr(),
                                                aq.data_ptr(), as_.data_ptr(), ks1, part.data_ptr(), part_b, sp)
            evs[2].record(stream)
            lib.moe_grouped_gemm2_combine(cfgp, wl.T, aq.data_ptr(), as_.data_ptr(), sid.data_ptr(),
                                          bexp.data_ptr(), npp.data_ptr(), w2.data_ptr(), s2.data_ptr(),
                                          wts.data_ptr(), out.data_ptr(), wl.H, ws.data_ptr(), ws.numel(), sp)
            evs[3].record(stream)

        for i in range(min(warmup, steps)):
            staged(ev[i], i)
        torch.cuda.synchronize()
        for i in range(steps):
            staged(ev[i], i)
        torch.cuda.synchronize()
        for j, n in enumerate(names):
            kern[n] = float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(steps)])) * 1e3  # us
        tot = np.array([ev[i][0].elapsed_time(ev[i][len(names)]) for i in range(steps)]) * 1e3
        g1 = np.array([ev[i][1].elapsed_time(ev[i][2]) for i in range(steps)]) * 1e3
        spread = {n: {"p10": round(float(np.percentile(a, 10)), 2), "median": round(float(np.median(a)), 2),
                      "p90": round(float(np.percentile(a, 90)), 2)}
                  for n, a in (("step", tot), ("gemm1_swiglu", g1))}

    peak_f = MFMA_PEAK_TFLOPS[wl.mode]
    flops = wl.flops()
    tflops = flops / (ms * 1e-3) / 1e12
    bw = HBM_PEAK_GBS * 1e9
    # the layer's attainable step time: the larger of its MFMA time at the
    # format's dense peak and its algorithmic bytes at the HBM peak
    layer_floor = max(flops / (peak_f * 1e12), nbytes["layer"] / bw)
    roof = None
    if kern:
        # GEMM1 is bound by HBM or by the MFMA peak of the layer's format,
        # whichever its arithmetic intensity (real sizes) puts it under
        dur = kern["gemm1_swiglu"] * 1e-6
        flops1 = 4.0 * wl.T * wl.top_k * wl.I * wl.H
        floor1 = max(flops1 / (peak_f * 1e12), nbytes["gemm1"] / bw)
        mfma_bound = flops1 / (peak_f * 1e12) > nbytes["gemm1"] / bw
        common = {"traffic": recorded_traffic(wl.name, wl.T, bm),
                  "kernel": ("moe_gemm_stream (GEMM1 + clamped SwiGLU + re-quantisation)" if ks1 == 1 else
                             f"moe_gemm_stream (GEMM1, leftover items in {-ks1} K pieces) + gemm1_tail_finish"
                             if ks1 < 0 else f"moe_gemm_stream (GEMM1, K split {ks1}) + swiglu_requant"),
                  "kernel_us": round(kern["gemm1_swiglu"], 2), "algorithmic_bytes": nbytes["gemm1"],
                  "algorithmic_flops": flops1,
                  # attainable = min(peak, intensity x HBM bandwidth), and the
                  # kernel's fraction of it
                  "intensity_flop_per_byte": round(flops1 / nbytes["gemm1"], 2),
                  "attainable_tflops": round(min(peak_f, flops1 / nbytes["gemm1"] * bw / 1e12), 1),
                  "achieved_tflops": round(flops1 / dur / 1e12, 1),
                  "attainable_frac": round(floor1 / dur, 4),
                  "hbm_frac": round(nbytes["gemm1"] / dur / bw, 4),
                  "mfma_frac": round(flops1 / dur / 1e12 / peak_f, 4)}
        if mfma_bound:
            tf = flops1 / dur / 1e12
            roof = {"bound": "mfma", "achieved": round(tf, 1), "peak": peak_f, "unit": "TFLOP/s",
                    "frac": round(tf / peak_f, 4), **common}
        else:
            gbs = nbytes["gemm1"] / dur / 1e9
            roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(gbs / HBM_PEAK_GBS, 4), **common}
    res = {
        "ms_per_step": round(ms, 4),
        "tokens_per_s": round(wl.T / (ms * 1e-3), 1),
        "config": {"workload": wl.name, "T": wl.T, "H": wl.H, "I": wl.I, "Hp": wl.Hp, "Ip": wl.Ip, "E": wl.E,
                   "top_k": wl.top_k, "quant": wl.mode, "block_m": bm, "swiglu_limit": wl.swiglu_limit,
                   "ksplit": [ks1, M.plan_ksplit(cfg, wl.T, 2)]},
        "effective_tflops": round(tflops, 3),
        "mfma_frac": round(tflops / peak_f, 5),
        "layer_hbm_frac": round(nbytes["layer"] / (ms * 1e-3) / bw, 4),
        "layer_attainable_us": round(layer_floor * 1e6, 1),
        "layer_attainable_frac": round(layer_floor / (ms * 1e-3), 4),
        "active_experts": nbytes["active_experts"],
        "layer_algorithmic_bytes": nbytes["layer"],
        "kernels_us": {k: round(v, 2) for k, v in kern.items()},
        "events_us": spread,
        "roofline": roof,
    }
    return res, copies, x, lg


def graph_replay(M, wl, copies, sets: int = 8, reps: int = 40, block_m: int = 0, path: str = "forward"):
    """Device-side step time of the layer with the host out of the loop: one
    HIP graph (torch.cuda.CUDAGraph) holds `sets` moe_forward calls, each on
    its own seeded input batch (so consecutive steps route to different
    experts and read their weights from HBM, not from the memory-side cache),
    and is replayed `reps` times.  This is how a serving loop runs the decode
    layer.  Returns the mean step time and the layer's fraction of HBM
    bandwidth over the mean algorithmic bytes of the sets.  path "gemv": the
    same layer through the decode entry points (front end, then
    moe_decode_gemm1_swiglu and moe_decode_gemm2_combine) instead of
    moe_forward."""
    import numpy as np
    import torch
    import workloads as W
    bm = block_m or M.pick_block_m(wl.T, wl.E, wl.top_k)
    cfg = M.make_cfg(wl.E, wl.top_k, wl.mode, wl.H, wl.I, wl.Hp, wl.Ip, block_m=bm,
                     swiglu_limit=wl.swiglu_limit)
    ins = []
    for j in range(sets):
        wj = wl.with_(seed=wl.seed + 1000 + j)
        ins.append((W.activations(wj, "cuda"), W.router_logits(wj, "cuda")))
    outs = [torch.empty(wl.T, wl.H, dtype=torch.bfloat16, device="cuda") for _ in range(sets)]
    ws = torch.empty(M.workspace_bytes(cfg, wl.T), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())

    if path == "gemv":
        P = wl.T * wl.top_k
        a32 = torch.empty(P, wl.Ip, dtype=torch.float32, device="cuda")
        aq_b, as_b = M.decode_intermediate_bytes(cfg, wl.T)
        aq = torch.empty(aq_b, dtype=torch.uint8, device="cuda")
        as_ = torch.empty(as_b, dtype=torch.uint8, device="cuda")

    def calls():
        for j, (x, lg) in enumerate(ins):
            w13, s13, w2, s2 = copies[j % len(copies)]
            if path == "gemv":
                ids, w, _, _, _, _, xq, xs = M.moe_route_permute_quant(cfg, x, lg)
                M.moe_decode_gemm1_swiglu(cfg, xq, xs, ids, w13, s13, a=a32)
                M.moe_decode_gemm2_combine(cfg, a32, ids, w, w2, s2, out=outs[j], aq=aq, as_=as_)
            else:
                M.moe_forward(cfg, x, lg, w13, s13, w2, s2, out=outs[j], ws=ws)

    with torch.cuda.stream(stream):
        calls()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        calls()
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) * 1e6 / (reps * sets)
    layer, active = [], []
    for _, lg in ins:
        ids, _ = M.moe_route_topk(lg, wl.top_k)
        nb = algorithmic_bytes(wl, ids.cpu().numpy(), M)
        layer.append(nb["layer"])
        active.append(nb["active_experts"])
    del g
    torch.cuda.synchronize()
    return {"T": wl.T, "path": path, "block_m": bm, "us_per_step": round(us, 2),
            "tokens_per_s": round(wl.T / (us * 1e-6), 1),
            "active_experts_mean": round(float(np.mean(active)), 1),
            "layer_hbm_frac": round(float(np.mean(layer)) / (us * 1e-6) / (HBM_PEAK_GBS * 1e9), 4),
            "ksplit": [M.plan_ksplit(cfg, wl.T, 13), M.plan_ksplit(cfg, wl.T, 2)]}


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer's multi-GPU "
              "sharding is described, not built", file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads as W
    import mxfp4_quantized_weights_amd as M

    torch.cuda.set_device(0)
    if args.decode_sweep:
        wl = W.WORKLOADS["decode_fp8"]
        bm = M.pick_block_m(wl.T, wl.E, wl.top_k)
        cfg = M.make_cfg(wl.E, wl.top_k, wl.mode, wl.H, wl.I, wl.Hp, wl.Ip, block_m=bm,
                         swiglu_limit=wl.swiglu_limit)
        copies = build_weights(M, cfg, wl, torch.device("cuda", 0), args.weight_copies)
        ts = (1, 2, 4, 8, 16) if args.decode_path == "gemv" else (1, 2, 4, 8, 16, 32, 64)
        for t in ts:
            print(json.dumps({"decode_sweep_graph": graph_replay(M, wl.with_(T=t), copies, path=args.decode_path)}),
                  flush=True)
        return
    wl = W.WORKLOADS[args.workload]
    if args.T:
        wl = wl.with_(T=args.T)
    r, copies, x, lg = measure(M, wl, args, breakdown=not args.no_breakdown)
    res = {
        "metric": "MoE layer tokens/s + effective TFLOP/s (% of MFMA/HBM roofline), 1 MI355X",
        "value": r["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4e2m1" if wl.mode == "mxfp4" else "fp8e4m3",
        "data": "synthetic (seeded N(0,1) activations/logits, N(0,0.02) weights, quantised by the library)",
        **{k: v for k, v in r.items() if k not in ("ms_per_step", "tokens_per_s")},
        "weight_copies": len(copies),
        "cpu_baseline": None,
    }
    if args.cpu_sample != 0:
        res["cpu_baseline"] = cpu_baseline(wl, x, lg, args.cpu_sample)
    if not args.no_extras and not args.T and args.workload == "prefill_fp8":
        # the decode layer shares the prefill layer's weights; the MXFP4 layer
        # has its own
        extras = {}
        d, _, _, _ = measure(M, W.WORKLOADS["decode_fp8"], args, copies=copies, breakdown=not args.no_breakdown,
                             block_m=0)
        extras["decode_fp8"] = d
        # decode micro-batches, replayed from a HIP graph as a serving loop
        # runs them (same weights)
        extras["decode_sweep_graph"] = [graph_replay(M, W.WORKLOADS["decode_fp8"].with_(T=t), copies)
                                        for t in (1, 2, 4, 8, 16, 32, 64)]
        del copies
        torch.cuda.empty_cache()
        m, _, _, _ = measure(M, W.WORKLOADS["prefill_mxfp4"], args, breakdown=not args.no_breakdown, block_m=0)
        extras["prefill_mxfp4"] = m
        res["extra"] = extras
        box = res["box_measured"] = box_measured(M)
        # each roofline's fraction of what this part measurably reaches: the
        # read stream for HBM-bound kernels, the rate of the MFMA instruction
        # the kernel runs (f16 for block FP8, FP4 for MXFP4) for MFMA-bound ones
        for r in (res, extras["decode_fp8"], extras["prefill_mxfp4"]):
            roof = r["roofline"]
            if roof["bound"] == "hbm":
                roof["frac_of_box_read"] = round(roof["achieved"] / box["read_gbs"], 4)
            else:
                inst = "fp4_16x16x128" if r["config"]["quant"] == "mxfp4" else "f16_16x16x32"
                roof["frac_of_box_mfma"] = round(roof["achieved_tflops"] / box["mfma_tflops"][inst], 4)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
