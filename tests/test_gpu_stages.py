"""GPU parity of each stage of the layer against the CPU oracle (through the C ABI).

Bit-exact: routing ids, permutation arrays, activation and weight quantiser
bytes and scales, the preshuffled layout.  Tolerance: routing weights
(float, rtol 2e-6); the GEMM1 intermediate codes may differ from the oracle's
only at a rounding midpoint within the element's fp32 accumulation bound
(parity_util.verify_intermediate).
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from parity_util import log

pytestmark = pytest.mark.gpu

M = None


@pytest.fixture(scope="module", autouse=True)
def lib():
    global M
    import mxfp4_quantized_weights_amd as mod
    M = mod
    yield mod


def _spread_values(rng, rows, cols):
    """Rows of very different magnitudes, including fp32 subnormal rows, an
    all-zero group, negative zeros and exact ties."""
    v = rng.standard_normal((rows, cols)).astype(np.float32)
    v *= np.exp2(rng.integers(-40, 40, (rows, 1))).astype(np.float32)
    v[0] *= np.float32(1e-38)          # subnormal row
    v[1, :] = 0.0
    v[2, :64] = -0.0
    v[3, 5] = -0.0
    v[4, :] = rng.integers(-8, 9, cols).astype(np.float32)  # integers: exact halfway cases
    return v


def _fp8_decision_rows():
    """Groups of 128 values whose quotients v / s lie on, or one or two fp32
    steps beside, every positive E4M3 value and every midpoint between
    neighbouring values (both signs), for several group scales s = amax / 448
    (amax = the group's first value: 448, so that s = 1, and scales that are
    not powers of two).  These are the quotients whose E4M3 code is decided
    closest, so a quantiser that does not form the IEEE quotient, or rounds
    it otherwise, shows here."""
    tab = O.e4m3_value_table()[:0x7F].astype(np.float64)  # codes 0x00 .. 0x7E
    targets = np.concatenate([tab, (tab[:-1] + tab[1:]) / 2])
    groups = []
    for amax in (448.0, 3.7, 1.37e-3, 77.7, 2.9e5):
        a32 = np.float32(amax)
        sc = a32 / np.float32(448.0)
        vals = []
        for t in targets:
            v0 = np.float32(t) * sc
            for v in (np.nextafter(np.nextafter(v0, np.float32(-np.inf)), np.float32(-np.inf)),
                      np.nextafter(v0, np.float32(-np.inf)), v0, np.nextafter(v0, np.float32(np.inf)),
                      np.nextafter(np.nextafter(v0, np.float32(np.inf)), np.float32(np.inf))):
                if 0 < v <= a32:
                    vals += [v, -v]
        vals = np.array(vals, np.float32)
        for i in range(0, len(vals), 127):
            g = np.zeros(128, np.float32)
            g[0] = a32 if (i // 127) % 2 == 0 else -a32
            chunk = vals[i:i + 127]
            g[1:1 + len(chunk)] = chunk
            groups.append(g)
    while len(groups) % 8:
        groups.append(np.zeros(128, np.float32))
    return np.stack(groups).reshape(-1, 8 * 128)


def test_quant_act_fp8_every_code_and_midpoint():
    """Block-FP8 activation codes at every decision point (_fp8_decision_rows),
    bit-exact against the oracle: the code is the RNE E4M3 code of the IEEE
    quotient fl32(v / s) (reading r4)."""
    v = _fp8_decision_rows()
    rows, cols = v.shape
    log(f"quant_act fp8 decision rows: {rows} x {cols}")
    q, s = M.moe_quant_act(torch.from_numpy(v).cuda(), cols, "fp8")
    torch.cuda.synchronize()
    qo, so = O.quant_act("fp8", v)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))
    qg = q.cpu().numpy()
    bad = np.argwhere(qg != qo)
    assert len(bad) == 0, f"{len(bad)} codes differ, e.g. v={v[tuple(bad[0])]!r}: {qg[tuple(bad[0])]:#x} vs {qo[tuple(bad[0])]:#x}"


def test_quant_act_mxfp4_every_code_and_midpoint():
    """MXFP4 activation codes at every decision point: groups of 32 whose
    largest value fixes the E8M0 scale (6 * 2^k: scale 2^k) and whose other
    values, scaled by 2^-k, lie on or one or two fp32 steps beside every E2M1
    value and every midpoint between neighbours, both signs.  Bit-exact
    against the oracle (RNE on the code grid, reading r7/r8)."""
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    targets = np.concatenate([grid, (grid[:-1] + grid[1:]) / 2]).astype(np.float32)
    groups = []
    for k in (0, -3, 5, -20):
        sc = np.float32(2.0 ** k)
        vals = []
        for t in targets:
            v0 = t * sc
            lo1 = np.nextafter(v0, np.float32(-np.inf))
            hi1 = np.nextafter(v0, np.float32(np.inf))
            for v in (np.nextafter(lo1, np.float32(-np.inf)), lo1, v0, hi1, np.nextafter(hi1, np.float32(np.inf))):
                if 0 < v <= 6 * sc:
                    vals += [v, -v]
        vals = np.array(vals, np.float32)
        for i in range(0, len(vals), 31):
            g = np.zeros(32, np.float32)
            g[0] = 6 * sc
            chunk = vals[i:i + 31]
            g[1:1 + len(chunk)] = chunk
            groups.append(g)
    while len(groups) % 32:
        groups.append(np.zeros(32, np.float32))
    v = np.stack(groups).reshape(-1, 1024)
    log(f"quant_act mxfp4 decision rows: {v.shape[0]} x {v.shape[1]}")
    q, s = M.moe_quant_act(torch.from_numpy(v).cuda(), v.shape[1], "mxfp4")
    torch.cuda.synchronize()
    qo, so = O.quant_act("mxfp4", v)
    assert np.array_equal(s.cpu().numpy(), so)
    assert np.array_equal(q.cpu().numpy(), qo)


@pytest.mark.parametrize("mode", ["fp8", "fp8_ue8m0", "mxfp4"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quant_act_bitexact(mode, dtype):
    log(f"quant_act mode={mode} dtype={dtype}")
    rng = np.random.default_rng(100)
    rows, cols, cols_p, ld = 37, 300, 384, 320
    v = _spread_values(rng, rows, ld)
    t = torch.from_numpy(v)
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    vals = t.float().numpy()[:, :cols]
    x = t.cuda()[:, :cols]
    q, s = M.moe_quant_act(x, cols_p, mode)
    torch.cuda.synchronize()
    qo, so = O.quant_act(mode, O.pad_cols(vals, cols_p))
    assert np.array_equal(q.cpu().numpy(), qo)
    if mode == "fp8":
        assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))
    elif mode == "fp8_ue8m0":
        sh = s.cpu().numpy()
        G = cols_p // 128
        assert sh.shape == (rows, M.e8_scale_ld(cols_p))
        assert np.array_equal(sh[:, :G], so)
        assert np.all(sh[:, G:] == 0)
    else:
        assert np.array_equal(s.cpu().numpy(), so)


def test_quant_act_ue8m0_scale_edges():
    """UE8M0 exponent boundaries: group maxima at exactly 448 * 2^k, one fp32
    step above and below it, and at 1.75 * 2^k boundaries, plus subnormal
    maxima; every group of a row has its own maximum."""
    log("quant_act ue8m0 edges")
    rows, G = 24, 16
    v = np.zeros((rows, G * 128), np.float32)
    rng = np.random.default_rng(103)
    k = 0
    for r in range(rows):
        for g in range(G):
            base = np.float32(np.ldexp(448.0, int(rng.integers(-140, 100))))
            amax = [base, np.nextafter(base, np.float32(np.inf)), np.nextafter(base, np.float32(0)),
                    np.float32(np.ldexp(1.75, int(rng.integers(-100, 100)))), np.float32(3e-41)][k % 5]
            k += 1
            grp = (rng.uniform(-1, 1, 128) * amax).astype(np.float32)
            grp[int(rng.integers(0, 128))] = -amax if k % 2 else amax
            v[r, g * 128:(g + 1) * 128] = grp
    q, s = M.moe_quant_act(torch.from_numpy(v).cuda(), G * 128, "fp8_ue8m0")
    torch.cuda.synchronize()
    qo, so = O.quant_act("fp8_ue8m0", v)
    assert np.array_equal(q.cpu().numpy(), qo)
    assert np.array_equal(s.cpu().numpy()[:, :G], so)


@pytest.mark.parametrize("mode", ["fp8", "fp8_ue8m0", "mxfp4"])
def test_quant_weights_bitexact(mode):
    log(f"quant_weights mode={mode}")
    rng = np.random.default_rng(101)
    E, N, K = 3, 256, 384
    w = (rng.standard_normal((E, N, K)) * 0.02).astype(np.float32)
    w[1, :128, :128] = 0.0
    w[2, 128:, 256:] *= 1e4
    w[0, 5, 7] = -0.0
    q, s = M.moe_quant_weights(torch.from_numpy(w).cuda(), mode)
    torch.cuda.synchronize()
    for e in range(E):
        if mode == "fp8":
            qo, so = O.quant_fp8_weight(w[e])
            assert np.array_equal(s[e].cpu().numpy().view(np.uint32), so.view(np.uint32))
        elif mode == "fp8_ue8m0":
            qo, so = O.quant_fp8e8_weight(w[e])
            assert np.array_equal(s[e].cpu().numpy(), so)
        else:
            qo, so = O.quant_mxfp4_rows(w[e])
            assert np.array_equal(s[e].cpu().numpy(), so)
        assert np.array_equal(q[e].cpu().numpy(), qo)


@pytest.mark.parametrize("T,E,k", [(64, 288, 8), (4096, 288, 8), (33, 8, 2), (7, 1, 1), (5, 16, 16),
                                   (3, 1024, 16), (129, 65, 3)])
def test_route_topk(T, E, k):
    log(f"route_topk T={T} E={E} k={k}")
    rng = np.random.default_rng(T * 1000 + E)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    if T > 10:
        lg[:T // 3] = rng.integers(-2, 3, (T // 3, E)).astype(np.float32)  # heavy ties
        lg[T // 3, :] = -0.0
        lg[T // 3, ::2] = 0.0
    ids, w = M.moe_route_topk(torch.from_numpy(lg).cuda(), k)
    torch.cuda.synchronize()
    ido, wo = O.route_topk(lg, k)
    assert np.array_equal(ids.cpu().numpy(), ido)
    assert np.allclose(w.cpu().numpy(), wo, rtol=2e-6, atol=0)


@pytest.mark.parametrize("T,E,k,BM,skew", [(1, 288, 8, 16, False), (64, 288, 8, 16, False),
                                           (4096, 288, 8, 128, False), (2048, 288, 8, 64, True),
                                           (300, 8, 2, 32, False), (0, 8, 2, 16, False),
                                           (1000, 1024, 16, 16, False), (17, 1, 1, 128, False),
                                           (513, 16, 4, 16, True), (200, 8, 4, 16, "dup"),
                                           (3000, 64, 8, 32, "dup"), (100, 16, 3, 64, "bad"),
                                           (2000, 288, 8, 128, "dup1"), (70000, 288, 8, 128, False),
                                           (70001, 64, 2, 16, True)])
def test_permute_align_bitexact(T, E, k, BM, skew):
    """Includes tokens that list an expert twice ("dup": the pairs keep f
    order; "dup1": only a few tokens in one token chunk do), ids outside
    [0, E) ("bad": skipped by both sides), and token counts that split into
    the maximum number of chunks with several 64-token rounds per wave."""
    log(f"permute_align T={T} E={E} k={k} BM={BM} skew={skew}")
    rng = np.random.default_rng(T + 7 * E + BM)
    if skew == "dup":
        ids = rng.integers(0, E, (T, k)).astype(np.int32)
        ids[::3, 1] = ids[::3, 0]
    elif skew == "dup1":
        ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
        ids[600:605, 3] = ids[600:605, 5]
    elif skew == "bad":
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        ids[::5, 0] = -1
        ids[1::7, 1] = E + 3
    elif skew:
        p = (np.arange(1, E + 1) ** -1.5)
        p /= p.sum()
        ids = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32) \
            if T else np.zeros((0, k), np.int32)
    else:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32) \
            if T else np.zeros((0, k), np.int32)
    sid, bexp, offs, npp = M.moe_permute_align(torch.from_numpy(ids).cuda(), E, BM)
    torch.cuda.synchronize()
    so, bo, oo, no = O.permute_align(ids, E, BM)
    assert int(npp.item()) == no
    assert np.array_equal(offs.cpu().numpy(), oo)
    assert np.array_equal(sid.cpu().numpy(), so)
    assert np.array_equal(bexp.cpu().numpy(), bo)


def _row_tile(which, Ip, N, g, i):
    """Row tile at position i of N tile g (TILED_V2): w13 = 8 gate tiles then
    the matching 8 up tiles; w2 = 16 consecutive tiles, None past N/16."""
    if which == 13:
        return 8 * g + i if i < 8 else Ip // 16 + 8 * g + (i - 8)
    t = 16 * g + i
    return t if t < N // 16 else None


def _tile_run(mode, which):
    """Documented tile run R of each matrix: w2 4; w13 16, MXFP4 w13 1."""
    if which == 2:
        return 4
    return 1 if mode == "mxfp4" else 16


def _runs(a, R):
    """[E, NG, KB', 16, ...] (position-major per K block) -> storage order
    [E, NG, 16/R, KB', R, ...], flattened."""
    E, NG, KB = a.shape[:3]
    rest = a.shape[4:]
    b = a.reshape(E, NG, KB, 16 // R, R, *rest)
    return np.moveaxis(b, 3, 2).reshape(-1)


def _tiled_fp8_reference(q, E, N, K, which, Ip, R):
    """The documented TILED_V2 FP8 layout, rebuilt on the host: tile
    [h][lane = 16*(K quarter) + row][16 bytes] at position i of N tile g and
    K block kb, stored [e][g][i / R][kb][i % R]."""
    KB, NG = K // 128, -(-N // 256)
    out = np.zeros((E, NG, KB, 16, 2, 64, 16), np.uint8)
    for g in range(NG):
        for i in range(16):
            rt = _row_tile(which, Ip, N, g, i)
            if rt is None:
                continue
            t = q[:, rt * 16:(rt + 1) * 16, :].reshape(E, 16, KB, 4, 2, 16)  # e, row, kb, quarter, h, byte
            out[:, g, :, i] = t.transpose(0, 2, 4, 3, 1, 5).reshape(E, KB, 2, 64, 16)
    return _runs(out, R)


def _tiled_mx_reference(q, s, E, N, K, which, Ip, R):
    """TILED_V2 MX: tiles [lane][16 bytes], stored as the FP8 tiles; scale
    word rows [lane][byte j = K block 4q + j] stored [e][g][i / R][q][i % R]."""
    KB, NG = K // 128, -(-N // 256)
    KB4 = (KB + 3) // 4
    w = np.zeros((E, NG, KB, 16, 64, 16), np.uint8)
    sc = np.zeros((E, NG, KB4, 16, 64, 4), np.uint8)
    for g in range(NG):
        for i in range(16):
            rt = _row_tile(which, Ip, N, g, i)
            if rt is None:
                continue
            t = q[:, rt * 16:(rt + 1) * 16, :].reshape(E, 16, KB, 4, 16)  # e, row, kb, quarter, byte
            w[:, g, :, i] = t.transpose(0, 2, 3, 1, 4).reshape(E, KB, 64, 16)
            s5 = s[:, rt * 16:(rt + 1) * 16, :].reshape(E, 16, KB, 4)  # e, row, kb, 32-group in block
            for kb in range(KB):
                for quarter in range(4):
                    sc[:, g, kb // 4, i, quarter * 16:(quarter + 1) * 16, kb % 4] = s5[:, :, kb, quarter]
    return _runs(w, R), _runs(sc, R)


@pytest.mark.parametrize("mode", ["fp8", "fp8_ue8m0", "mxfp4"])
def test_preshuffle_layout(mode):
    log(f"preshuffle mode={mode}")
    rng = np.random.default_rng(102)
    E, Hp, Ip = 3, 384, 640
    cfg = M.make_cfg(E, 2, mode, Hp, Ip)
    for which, N, K in ((13, 2 * Ip, Hp), (2, Hp, Ip)):
        if mode == "fp8":
            q = rng.integers(0, 256, (E, N, K), dtype=np.uint8)
            s = rng.standard_normal((E, N // 128, K // 128)).astype(np.float32)
        elif mode == "fp8_ue8m0":
            q = rng.integers(0, 256, (E, N, K), dtype=np.uint8)
            s = rng.integers(0, 255, (E, N // 128, K // 128), dtype=np.uint8)
            s.reshape(-1)[:3] = [0, 1, 254]
        else:
            q = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
            s = rng.integers(0, 255, (E, N, K // 32), dtype=np.uint8)
        qo, so = M.moe_preshuffle_weights(cfg, which, torch.from_numpy(q).cuda(), torch.from_numpy(s).cuda())
        torch.cuda.synchronize()
        if mode == "fp8":
            assert np.array_equal(qo.cpu().numpy(), _tiled_fp8_reference(q, E, N, K, which, Ip, _tile_run(mode, which)))
            assert np.array_equal(so.cpu().numpy().view(np.float32), s.reshape(-1))
        elif mode == "fp8_ue8m0":
            # same tiles; the scale bytes as their exact fp32 values
            assert np.array_equal(qo.cpu().numpy(), _tiled_fp8_reference(q, E, N, K, which, Ip, _tile_run(mode, which)))
            assert np.array_equal(so.cpu().numpy().view(np.float32), O.e8m0_to_f32(s).reshape(-1))
        else:
            w_ref, s_ref = _tiled_mx_reference(q, s, E, N, K, which, Ip, _tile_run(mode, which))
            assert np.array_equal(qo.cpu().numpy(), w_ref)
            assert np.array_equal(so.cpu().numpy(), s_ref)


@pytest.mark.parametrize("mode,BM", [("fp8", 16), ("fp8", 64), ("mxfp4", 32), ("mxfp4", 128), ("fp8_ue8m0", 16),
                                     ("fp8_ue8m0", 128)])
def test_gemm1_swiglu_stage(mode, BM):
    """GEMM1 + clamped SwiGLU + re-quantisation, fed by the (bit-exact) GPU
    routing/permutation/quantisation stages; the oracle recomputes everything
    from the raw inputs."""
    wl = W.Workload("gemm1", T=48, H=512, I=384, E=8, top_k=2, mode=mode, outlier_frac=0.02)
    log(f"gemm1 stage {W.describe(wl)} BM={BM}")
    cfg = M.make_cfg(wl.E, wl.top_k, mode, wl.H, wl.I, block_m=BM)
    x = W.activations(wl)
    lg = W.router_logits(wl)
    from parity_util import gpu_intermediate_rows, gpu_weights, oracle_weights_cpu, pairs_of, verify_intermediate
    ew = gpu_weights(M, cfg, wl, source="cpu")
    xd, lgd = x.cuda(), lg.cuda()
    ids, wts = M.moe_route_topk(lgd, wl.top_k)
    sid, bexp, offs, npp = M.moe_permute_align(ids, wl.E, BM)
    xq, xs = M.moe_quant_act(xd, wl.Hp, mode)
    aq, as_ = M.moe_grouped_gemm1_swiglu(cfg, wl.T, xq, xs, sid, bexp, npp, ew.w13, ew.w13_scale)
    torch.cuda.synchronize()
    Q = oracle_weights_cpu(wl)
    _, st = O.moe_forward(x.float().numpy(), lg.numpy(), Q, wl.top_k, wl.swiglu_limit, wl.H, wl.I,
                          return_stages=True)
    rows = gpu_intermediate_rows(mode, wl.Ip, aq, as_, sid, npp, wl.T * wl.top_k, wl.top_k,
                                 pairs_of(range(wl.T), wl.top_k))
    verify_intermediate(mode, wl.swiglu_limit, rows, st, Q, wl.H)


@pytest.mark.parametrize("T,E,k,BM,mode,ldpad", [(1, 288, 8, 16, "fp8", 0), (7, 288, 8, 16, "mxfp4", 24),
                                                 (64, 288, 8, 16, "fp8_ue8m0", 0), (64, 1024, 16, 32, "fp8", 8),
                                                 (33, 8, 2, 64, "mxfp4", 0), (64, 1, 1, 128, "fp8", 0),
                                                 (65, 288, 8, 16, "fp8", 0), (300, 64, 4, 32, "mxfp4", 0),
                                                 (16, 1024, 16, 16, "fp8", 0), (17, 288, 8, 16, "fp8_ue8m0", 8)])
def test_route_permute_quant_equals_stages(T, E, k, BM, mode, ldpad):
    """moe_route_permute_quant (one launch up to 16 tokens, else two) gives exactly the
    results of moe_route_topk + moe_permute_align + moe_quant_act, and those
    match the oracle."""
    log(f"route_permute_quant T={T} E={E} k={k} BM={BM} mode={mode} ldpad={ldpad}")
    H = 400
    cfg = M.make_cfg(E, k, mode, H, 256, block_m=BM)
    rng = np.random.default_rng(T + E + BM)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    if T > 4:
        lg[: T // 3] = rng.integers(-2, 3, (T // 3, E)).astype(np.float32)  # ties
    xf = rng.standard_normal((T, H + ldpad)).astype(np.float32)
    xf[:, 7] *= 40
    xb = torch.from_numpy(xf).to(torch.bfloat16).cuda()
    x = xb[:, :H]
    lgd = torch.from_numpy(lg).cuda()
    ids, w, sid, bexp, offs, npp, xq, xs = M.moe_route_permute_quant(cfg, x, lgd)
    ids2, w2 = M.moe_route_topk(lgd, k)
    sid2, bexp2, offs2, npp2 = M.moe_permute_align(ids2, E, BM)
    xq2, xs2 = M.moe_quant_act(x, cfg.pad.hidden_padded, mode)
    torch.cuda.synchronize()
    for a, b in ((ids, ids2), (sid, sid2), (bexp, bexp2), (offs, offs2), (npp, npp2), (xq, xq2)):
        assert torch.equal(a, b)
    assert torch.equal(w.view(torch.int32), w2.view(torch.int32))
    assert torch.equal(xs.view(torch.uint8), xs2.view(torch.uint8))
    ido, _ = O.route_topk(lg, k)
    assert np.array_equal(ids.cpu().numpy(), ido)
    so, bo, oo, no = O.permute_align(ido, E, BM)
    assert np.array_equal(sid.cpu().numpy(), so) and int(npp.item()) == no
    qo, _ = O.quant_act(mode, O.pad_cols(x.float().cpu().numpy(), cfg.pad.hidden_padded))
    assert np.array_equal(xq.cpu().numpy(), qo)
