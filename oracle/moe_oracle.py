"""Plain, slow CPU oracle for the routed-expert MoE layer (block FP8 and OCP MXFP4).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this module:
only the test suite, the smoke check of the package entry point and the
``cpu_baseline`` leg of the benchmark call it.  It shares no code, table or
constant generator with the HIP library; it is NumPy on the host, written
from the method's definition step by step.

Sources (page title and section):
  [P1] sglang PR #38546 "[AMD] [GLM-5.3-Flash Day 0] Enable FP8 and Quark MXFP4
       MoE on gfx950" -- Summary (block FP8 [128,128] weights with dynamic FP8
       activations; OCP MXFP4 1x32; separate contiguous gate/up halves; clamped
       SwiGLU with swiglu_limit=10.0) and the contract table (padding metadata
       recorded and forwarded).
  [P4] "[AMD] [GLM5] Opt-in prefill-only FP8 dense projection GEMM for MLA
       q_b/o_proj (gfx950)" -- Modifications (e4m3 weights with a 128x128
       UE8M0, i.e. power-of-two, block scale).
  [P3] FreeToken PR #270 "glm5_next: support GLM-5.3-Flash (hybrid KDA + DSA,
       mHC, NVFP4 expert offload)" -- Summary (288-expert top-8 routing; the
       clamped SwiGLU silu(min(gate, lim)) * clamp(up, -lim, lim), where an
       infinite limit leaves plain SwiGLU unchanged).
  Where the pages are silent, each function states the reading it takes
  (top-k ties, renormalised softmax weights, scale arithmetic, amax == 0,
  E8M0 exponent rule, E2M1 rounding and saturation).

Precision: the pages fix fp32 for the quantiser scales and the dequantised
GEMMs; every such step here is done in float32 with NumPy's IEEE operations
(division is correctly rounded).  Routing weights are computed in float64 and
rounded once to float32.

Parity status per function (what pins it is in the tests):
  route_topk, permute_align, e4m3/e2m1 code tables, quant_fp8_*, quant_fp8e8_*
  (UE8M0 scales), quant_mxfp4_*,
  gemm (dequantised fp32), swiglu_clamped, moe_forward: pinned by brute force,
  library casts, closed forms and invariants.  No function is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

F32 = np.float32

_CHUNK_ELEMS = 1 << 19  # rows are processed in pieces of about this many elements


def _row_chunks(rows: int, cols: int):
    """Row ranges covering [0, rows) with about _CHUNK_ELEMS elements each.
    Only bounds temporary memory; every row is computed the same way."""
    step = max(1, _CHUNK_ELEMS // max(cols, 1))
    for r0 in range(0, rows, step):
        yield r0, min(rows, r0 + step)

# ----------------------------------------------------------------------------
# Code tables, written from the format definitions.
# ----------------------------------------------------------------------------

E4M3_MAX = 448.0  # largest finite OCP E4M3FN magnitude: exponent field 15, mantissa 6


def e4m3_value_table() -> np.ndarray:
    """All 256 OCP E4M3FN codes decoded to float64 (NaN for 0x7F/0xFF).

    Definition: sign bit 7, exponent bits 6..3 with bias 7, mantissa bits 2..0.
    Exponent field 0 encodes subnormals m/8 * 2**-6.  E4M3FN has no infinities;
    only S.1111.111 is NaN, so exponent field 15 still holds finite values up
    to 1.75 * 2**8 = 448.
    """
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        ef = (code >> 3) & 0xF
        m = code & 0x7
        if ef == 0xF and m == 0x7:
            vals[code] = np.nan
        elif ef == 0:
            vals[code] = sign * (m / 8.0) * 2.0 ** (1 - 7)
        else:
            vals[code] = sign * (1.0 + m / 8.0) * 2.0 ** (ef - 7)
    return vals


E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])  # codes 0..7, bit 3 = sign
E2M1_MAX = 6.0


def e2m1_value_table() -> np.ndarray:
    """All 16 OCP E2M1 codes decoded to float64: bit 3 sign, bits 2..1 exponent
    (bias 1), bit 0 mantissa; exponent field 0 is the subnormal 0 / 0.5."""
    vals = np.empty(16, dtype=np.float64)
    for code in range(16):
        sign = -1.0 if code & 0x8 else 1.0
        ef = (code >> 1) & 0x3
        m = code & 0x1
        mag = (m * 0.5) if ef == 0 else (1.0 + 0.5 * m) * 2.0 ** (ef - 1)
        vals[code] = sign * mag
    return vals


def _round_to_grid(mag: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Index of the nearest grid value for non-negative ``mag`` (float64),
    ties going to the even index.  ``grid`` is increasing and its index is the
    magnitude code, so "even index" is "even code" (round-half-to-even)."""
    idx = np.searchsorted(grid, mag, side="left")  # grid[idx-1] < mag <= grid[idx]
    idx = np.clip(idx, 1, len(grid) - 1)
    lo = grid[idx - 1]
    hi = grid[idx]
    dlo = mag - lo
    dhi = hi - mag
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (idx % 2 == 0))
    out = np.where(pick_hi, idx, idx - 1)
    out = np.where(mag <= grid[0], 0, out)
    return out.astype(np.int64)


_E4M3_POS = e4m3_value_table()[0:0x7F]  # codes 0x00..0x7E, increasing


def round_to_e4m3(v: np.ndarray) -> np.ndarray:
    """Round values with |v| <= 448 to the nearest E4M3FN code, ties to even.
    The sign bit is kept, also for zero (-0.0 and negative values that round to
    zero give 0x80)."""
    v = np.asarray(v, dtype=np.float64)
    if np.any(np.abs(v) > E4M3_MAX) or np.any(np.isnan(v)):
        raise ValueError("round_to_e4m3 expects finite |v| <= 448 (saturate first)")
    mag_code = _round_to_grid(np.abs(v), _E4M3_POS)
    sign = np.signbit(v).astype(np.int64) << 7
    return (mag_code | sign).astype(np.uint8)


def round_to_e2m1(v: np.ndarray) -> np.ndarray:
    """Round values with |v| <= 6 to the nearest E2M1 code, ties to even code;
    the sign bit (bit 3) is kept, also for zero."""
    v = np.asarray(v, dtype=np.float64)
    if np.any(np.abs(v) > E2M1_MAX) or np.any(np.isnan(v)):
        raise ValueError("round_to_e2m1 expects finite |v| <= 6 (saturate first)")
    mag_code = _round_to_grid(np.abs(v), E2M1_VALUES)
    sign = np.signbit(v).astype(np.int64) << 3
    return (mag_code | sign).astype(np.uint8)


# ----------------------------------------------------------------------------
# Block FP8: e4m3 codes with one fp32 dequant scale per group  [P1 Summary]
# ----------------------------------------------------------------------------

def _fp8_groups(g: np.ndarray):
    """Quantise groups of float32 values laid out along the last axis of ``g``
    ([..., G]); returns (codes uint8 [..., G], scales float32 [...]).

    Reading of the scale arithmetic: s = fl32(amax / 448), then
    q = RNE_e4m3(clamp(fl32(v / s), -448, 448)); both divisions are IEEE fp32.
    Reading for amax == 0: s = 0 and every code of the group is 0x00 (no
    division).
    """
    g = np.asarray(g, dtype=F32)
    amax = np.max(np.abs(g), axis=-1)
    s = (amax / F32(E4M3_MAX)).astype(F32)
    nz = amax > 0
    safe = np.where(nz, s, F32(1))[..., None]
    r = (g / safe).astype(F32)
    r = np.clip(r, F32(-E4M3_MAX), F32(E4M3_MAX))
    q = round_to_e4m3(r)
    q = np.where(nz[..., None], q, np.uint8(0)).astype(np.uint8)
    return q, np.where(nz, s, F32(0)).astype(F32)


def quant_fp8_rows(v: np.ndarray, group: int = 128):
    """Dynamic per-row activation quantisation: one e4m3 code per element and
    one fp32 scale per 1 x ``group`` run along the last axis.

    ``v`` is float32 [rows, K] with K a multiple of ``group`` (callers zero-pad).
    Returns (q uint8 [rows, K], s float32 [rows, K/group]).
    """
    v = np.asarray(v, dtype=F32)
    rows, K = v.shape
    assert K % group == 0
    q = np.zeros((rows, K), np.uint8)
    s = np.zeros((rows, K // group), F32)
    for r0, r1 in _row_chunks(rows, K):
        qq, ss = _fp8_groups(v[r0:r1].reshape(r1 - r0, K // group, group))
        q[r0:r1] = qq.reshape(r1 - r0, K)
        s[r0:r1] = ss
    return q, s


def quant_fp8_weight(w: np.ndarray, block: int = 128):
    """Block FP8 weight quantisation with one fp32 scale per [128, 128] block
    [P1 Summary].  ``w`` is float32 [N, K], both multiples of ``block``.
    Returns (q uint8 [N, K], s float32 [N/block, K/block]).  The scale is the
    dequant multiplier (the runtime ``weight_scale_inv`` of [P1 Scope])."""
    w = np.asarray(w, dtype=F32)
    N, K = w.shape
    assert N % block == 0 and K % block == 0
    q = np.zeros((N, K), np.uint8)
    s = np.zeros((N // block, K // block), F32)
    for i in range(N // block):  # one 128-row band of blocks at a time
        band = w[i * block:(i + 1) * block].reshape(block, K // block, block).transpose(1, 0, 2)
        qq, s[i] = _fp8_groups(band.reshape(K // block, block * block))
        q[i * block:(i + 1) * block] = qq.reshape(K // block, block, block).transpose(1, 0, 2).reshape(block, K)
    return q, s


def dequant_fp8_rows(q: np.ndarray, s: np.ndarray, group: int = 128) -> np.ndarray:
    """fp32 value of each element: fl32(code value * group scale)."""
    tab = e4m3_value_table().astype(F32)
    rows, K = q.shape
    out = np.zeros((rows, K), F32)
    for r0, r1 in _row_chunks(rows, K):
        out[r0:r1] = tab[q[r0:r1]] * np.repeat(s[r0:r1].astype(F32), group, axis=1)
    return out


def dequant_fp8_weight(q: np.ndarray, s: np.ndarray, block: int = 128) -> np.ndarray:
    """fp32 value of each weight: fl32(code value * scale of its 128x128 block)."""
    return dequant_fp8_rows(q, np.repeat(np.asarray(s, F32), block, axis=0), block)


# ----------------------------------------------------------------------------
# Block FP8 with UE8M0 scales: e4m3 codes, one power-of-two scale per group,
# stored as an unsigned E8M0 exponent byte.  [P4] "[AMD] [GLM5] Opt-in
# prefill-only FP8 dense projection GEMM for MLA q_b/o_proj (gfx950)",
# Modifications: e4m3 weights with a 128x128 UE8M0 scale.
# ----------------------------------------------------------------------------

def ue8m0_exponent(amax):
    """Smallest integer e with 448 * 2**e >= amax, for finite amax > 0.

    Reading: the block scale amax/448 is rounded UP to a power of two, so
    that no value of the group needs saturation (|v| / 2**e <= 448).  Exact:
    start one below floor(log2 amax) - 8 and step up while 448 * 2**e is still
    below amax (both sides are exact in float64).  Works elementwise."""
    amax = np.asarray(amax, dtype=np.float64)
    e = floor_log2(amax) - 9
    for _ in range(3):  # 448 * 2**(E - 9) < 2**E <= amax, and 448 * 2**(E - 7) > 2**(E + 1) > amax
        e = np.where(np.ldexp(E4M3_MAX, e) < amax, e + 1, e)
    return e


def ue8m0_scale_byte(amax):
    """E8M0 byte of a UE8M0 block: ue8m0_exponent(amax) + 127 clamped to
    [0, 254].  Reading for amax == 0 (zero rows, all-pad blocks): byte 0 with
    all-zero codes, as for the MX scales."""
    amax = np.asarray(amax, dtype=np.float64)
    b = np.clip(ue8m0_exponent(np.where(amax > 0, amax, 1.0)) + 127, 0, 254)
    return np.where(amax > 0, b, 0).astype(np.uint8)


def _fp8_ue8m0_groups(g: np.ndarray):
    """Groups along the last axis of float32 ``g`` -> (codes uint8 [..., G],
    scale bytes uint8 [...]).  q = RNE_e4m3(v / 2**(b - 127)); the division by
    a power of two is exact (done in float64), and |v| / 2**(b-127) <= 448 by
    the choice of b, so no value saturates."""
    g = np.asarray(g, dtype=F32).astype(np.float64)
    amax = np.max(np.abs(g), axis=-1)
    b = ue8m0_scale_byte(amax)
    r = g / np.ldexp(1.0, b.astype(np.int64) - 127)[..., None]
    q = round_to_e4m3(np.clip(r, -E4M3_MAX, E4M3_MAX))
    q = np.where((amax > 0)[..., None], q, np.uint8(0)).astype(np.uint8)
    return q, b


def quant_fp8e8_rows(v: np.ndarray, group: int = 128):
    """Per-row activation quantisation with UE8M0 scales: one e4m3 code per
    element and one E8M0 byte per 1 x ``group`` run along the last axis.
    Returns (q uint8 [rows, K], b uint8 [rows, K/group])."""
    v = np.asarray(v, dtype=F32)
    rows, K = v.shape
    assert K % group == 0
    q = np.zeros((rows, K), np.uint8)
    b = np.zeros((rows, K // group), np.uint8)
    for r0, r1 in _row_chunks(rows, K):
        qq, bb = _fp8_ue8m0_groups(v[r0:r1].reshape(r1 - r0, K // group, group))
        q[r0:r1] = qq.reshape(r1 - r0, K)
        b[r0:r1] = bb
    return q, b


def quant_fp8e8_weight(w: np.ndarray, block: int = 128):
    """Weights [N, K] -> (q uint8 [N, K], b uint8 [N/block, K/block]): one
    UE8M0 scale per [128, 128] block."""
    w = np.asarray(w, dtype=F32)
    N, K = w.shape
    assert N % block == 0 and K % block == 0
    q = np.zeros((N, K), np.uint8)
    b = np.zeros((N // block, K // block), np.uint8)
    for i in range(N // block):
        band = w[i * block:(i + 1) * block].reshape(block, K // block, block).transpose(1, 0, 2)
        qq, b[i] = _fp8_ue8m0_groups(band.reshape(K // block, block * block))
        q[i * block:(i + 1) * block] = qq.reshape(K // block, block, block).transpose(1, 0, 2).reshape(block, K)
    return q, b


def e8m0_to_f32(b: np.ndarray) -> np.ndarray:
    """2**(b - 127) as float32 (exact: 2**-127 is an fp32 subnormal)."""
    return np.ldexp(1.0, np.asarray(b, np.int64) - 127).astype(F32)


def dequant_fp8e8_rows(q: np.ndarray, b: np.ndarray, group: int = 128) -> np.ndarray:
    """fp32 value of each element: code value * 2**(b - 127) (exact)."""
    return dequant_fp8_rows(q, e8m0_to_f32(b), group)


def dequant_fp8e8_weight(q: np.ndarray, b: np.ndarray, block: int = 128) -> np.ndarray:
    return dequant_fp8_weight(q, e8m0_to_f32(b), block)


# ----------------------------------------------------------------------------
# OCP MXFP4: E2M1 codes, two per byte, one E8M0 scale per 1 x 32 along K  [P1]
# ----------------------------------------------------------------------------

MX_GROUP = 32


def floor_log2(a):
    """floor(log2 a) for finite a > 0, exact (from the binary exponent,
    subnormals included): frexp gives a = m * 2**e with m in [0.5, 1)."""
    _, e = np.frexp(np.asarray(a, dtype=np.float64))
    return e.astype(np.int64) - 1


def e8m0_scale_byte(amax):
    """Shared exponent of an MX block: 2**(floor(log2 amax) - 2), where 2 is
    the exponent of E2M1's largest power of two (4.0), stored biased by 127 and
    clamped to the byte range [0, 254] (0xFF is the E8M0 NaN).  Reading for
    amax == 0: byte 0.  Works elementwise on arrays."""
    amax = np.asarray(amax, dtype=np.float64)
    b = np.clip(floor_log2(np.where(amax > 0, amax, 1.0)) - 2 + 127, 0, 254)
    return np.where(amax > 0, b, 0).astype(np.uint8)


def quant_mxfp4_rows(v: np.ndarray):
    """MXFP4 quantisation of float32 [rows, K] (K a multiple of 32).

    Per 1 x 32 group: byte b from ``e8m0_scale_byte``; each element is divided
    by 2**(b - 127) (exact, done in float64), saturated to [-6, 6] and rounded
    to the nearest E2M1 code, ties to even.  Element 2i goes in the low nibble
    of byte i and element 2i+1 in the high nibble.
    Returns (packed uint8 [rows, K/2], scale bytes uint8 [rows, K/32]).
    """
    v = np.asarray(v, dtype=F32)
    rows, K = v.shape
    assert K % MX_GROUP == 0
    packed = np.zeros((rows, K // 2), np.uint8)
    sb = np.zeros((rows, K // MX_GROUP), np.uint8)
    for r0, r1 in _row_chunks(rows, K):
        grp = v[r0:r1].reshape(r1 - r0, K // MX_GROUP, MX_GROUP).astype(np.float64)
        b = e8m0_scale_byte(np.max(np.abs(grp), axis=-1))
        scaled = grp / np.ldexp(1.0, b.astype(np.int64) - 127)[..., None]
        scaled = np.clip(scaled, -E2M1_MAX, E2M1_MAX)
        codes = round_to_e2m1(scaled).reshape(r1 - r0, K)
        packed[r0:r1] = codes[:, 0::2] | (codes[:, 1::2] << 4)
        sb[r0:r1] = b
    return packed, sb


def unpack_e2m1(packed: np.ndarray) -> np.ndarray:
    """uint8 [rows, K/2] -> uint8 codes [rows, K] (low nibble = even element)."""
    rows, half = packed.shape
    codes = np.zeros((rows, half * 2), np.uint8)
    codes[:, 0::2] = packed & 0xF
    codes[:, 1::2] = packed >> 4
    return codes


def dequant_mxfp4_rows(packed: np.ndarray, sb: np.ndarray) -> np.ndarray:
    """fp32 value of each element: E2M1 value * 2**(b - 127) (exact)."""
    tab = e2m1_value_table()
    rows, half = packed.shape
    out = np.zeros((rows, half * 2), F32)
    for r0, r1 in _row_chunks(rows, half * 2):
        vals = tab[unpack_e2m1(packed[r0:r1])]
        scale = np.ldexp(1.0, sb[r0:r1].astype(np.int64) - 127)
        out[r0:r1] = vals * np.repeat(scale, MX_GROUP, axis=1)
    return out


# ----------------------------------------------------------------------------
# Routing  [P3 Summary: 288-expert top-8 routing]
# ----------------------------------------------------------------------------

def route_topk(logits: np.ndarray, top_k: int):
    """Top-k experts per token from fp32 router logits.

    Reading: selection on the raw logits, ordered by descending value with ties
    going to the lower expert id (-0.0 ties +0.0); slot j holds the j-th best.
    Weights are the softmax over the selected logits, i.e. softmax over all E
    followed by renormalisation over the chosen k: w_j = exp(l_j - l_max) /
    sum_i exp(l_i - l_max), computed in float64 and rounded to float32.
    Returns (ids int32 [T, k], weights float32 [T, k]).
    """
    logits = np.asarray(logits, dtype=F32)
    T, E = logits.shape
    ids = np.zeros((T, top_k), np.int32)
    w = np.zeros((T, top_k), F32)
    expert = np.arange(E)
    for t in range(T):
        order = np.lexsort((expert, -logits[t].astype(np.float64)))  # last key is primary
        sel = order[:top_k]
        ids[t] = sel
        l = logits[t, sel].astype(np.float64)
        ex = np.exp(l - l.max())
        w[t] = (ex / ex.sum()).astype(F32)
    return ids, w


def max_blocks(num_pairs: int, num_experts: int, block_m: int) -> int:
    """Upper bound on the number of BM-row blocks after padding every expert's
    segment to a multiple of BM: sum_e ceil(c_e/BM) <= (P + E*(BM-1))/BM, and
    every non-empty block holds at least one pair, so it is also <= P."""
    return min(num_pairs, (num_pairs + num_experts * (block_m - 1)) // block_m)


def permute_align(ids: np.ndarray, num_experts: int, block_m: int):
    """Counting sort of the T*k (token, slot) pairs by expert.

    Pair f = t*k + j.  Expert e's segment starts at offsets[e], holds the pairs
    routed to e in increasing f, and is padded with the sentinel P = T*k to a
    multiple of BM; experts with no pairs get no block.  Every block of BM rows
    belongs to one expert (block_expert).  Arrays are sized for the worst case
    (max_blocks blocks); entries past num_post_padded hold P / -1.
    Reading for ids outside [0, E) (not produced by routing): such pairs are
    not routed to any expert and appear nowhere in sorted_ids.
    Returns (sorted_ids int32 [max_blocks*BM], block_expert int32 [max_blocks],
             offsets int32 [E+1], num_post_padded int).
    """
    ids = np.asarray(ids, dtype=np.int64)
    P = ids.size
    flat = ids.reshape(-1)
    nb = max_blocks(P, num_experts, block_m)
    counts = np.zeros(num_experts, np.int64)
    for e in flat:
        if 0 <= e < num_experts:
            counts[e] += 1
    padded = ((counts + block_m - 1) // block_m) * block_m
    offsets = np.zeros(num_experts + 1, np.int64)
    offsets[1:] = np.cumsum(padded)
    sorted_ids = np.full(nb * block_m, P, np.int32)
    block_expert = np.full(nb, -1, np.int32)
    cursor = offsets[:-1].copy()
    for f in range(P):
        e = flat[f]
        if not 0 <= e < num_experts:
            continue
        sorted_ids[cursor[e]] = f
        cursor[e] += 1
    for e in range(num_experts):
        for b in range(offsets[e] // block_m, offsets[e + 1] // block_m):
            block_expert[b] = e
    return sorted_ids, block_expert, offsets.astype(np.int32), int(offsets[-1])


# ----------------------------------------------------------------------------
# Clamped SwiGLU  [P3 Summary; P1 Summary: swiglu_limit=10.0]
# ----------------------------------------------------------------------------

def silu(g: np.ndarray) -> np.ndarray:
    g = np.asarray(g, dtype=F32)
    return (g / (F32(1) + np.exp(-g))).astype(F32)


def swiglu_clamped(gate: np.ndarray, up: np.ndarray, limit: float) -> np.ndarray:
    """silu(min(gate, limit)) * clamp(up, -limit, limit), float32.  With an
    infinite limit this is plain silu(gate) * up."""
    lim = F32(limit)
    g = np.minimum(np.asarray(gate, F32), lim)
    u = np.clip(np.asarray(up, F32), -lim, lim)
    return (silu(g) * u).astype(F32)


# ----------------------------------------------------------------------------
# The layer
# ----------------------------------------------------------------------------

def gemm_f32(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """a [M, K] @ b[N, K]^T in float32 (dequantised operands, fp32 GEMM)."""
    return np.matmul(np.asarray(a, F32), np.asarray(b, F32).T).astype(F32)


class QuantWeights:
    """Quantised expert weights in the canonical (oracle) layout.

    mode "fp8":  w13 uint8 [E, 2Ip, Hp], s13 float32 [E, 2Ip/128, Hp/128];
                 w2  uint8 [E, Hp, Ip],  s2  float32 [E, Hp/128, Ip/128].
    mode "fp8_ue8m0": as "fp8" with uint8 E8M0 scale bytes in place of the
                 float32 scales.
    mode "mxfp4": w13 uint8 [E, 2Ip, Hp/2], s13 uint8 [E, 2Ip, Hp/32];
                  w2  uint8 [E, Hp, Ip/2],  s2  uint8 [E, Hp, Ip/32].
    Gate rows are [0, Ip) and up rows [Ip, 2Ip) of w13 (separate contiguous
    halves, [P1 Summary]); each half is zero-padded from I to Ip rows and every
    matrix from H to Hp / I to Ip columns.
    """

    def __init__(self, mode, w13, s13, w2, s2):
        self.mode, self.w13, self.s13, self.w2, self.s2 = mode, w13, s13, w2, s2


def quantize_weights(mode: str, w13: np.ndarray, w2: np.ndarray) -> QuantWeights:
    """Quantise padded float32 weights w13 [E, 2Ip, Hp] and w2 [E, Hp, Ip]."""
    E = w13.shape[0]
    if mode == "fp8":
        q13, s13, q2, s2 = [], [], [], []
        for e in range(E):
            a, b = quant_fp8_weight(w13[e]); q13.append(a); s13.append(b)
            a, b = quant_fp8_weight(w2[e]); q2.append(a); s2.append(b)
        return QuantWeights(mode, np.stack(q13), np.stack(s13), np.stack(q2), np.stack(s2))
    if mode == "fp8_ue8m0":
        q13, s13, q2, s2 = [], [], [], []
        for e in range(E):
            a, b = quant_fp8e8_weight(w13[e]); q13.append(a); s13.append(b)
            a, b = quant_fp8e8_weight(w2[e]); q2.append(a); s2.append(b)
        return QuantWeights(mode, np.stack(q13), np.stack(s13), np.stack(q2), np.stack(s2))
    if mode == "mxfp4":
        q13, s13, q2, s2 = [], [], [], []
        for e in range(E):
            a, b = quant_mxfp4_rows(w13[e]); q13.append(a); s13.append(b)
            a, b = quant_mxfp4_rows(w2[e]); q2.append(a); s2.append(b)
        return QuantWeights(mode, np.stack(q13), np.stack(s13), np.stack(q2), np.stack(s2))
    raise ValueError(mode)


def dequant_expert(W: QuantWeights, e: int):
    """fp32 w13[e] [2Ip, Hp] and w2[e] [Hp, Ip]."""
    if W.mode == "fp8":
        return dequant_fp8_weight(W.w13[e], W.s13[e]), dequant_fp8_weight(W.w2[e], W.s2[e])
    if W.mode == "fp8_ue8m0":
        return dequant_fp8e8_weight(W.w13[e], W.s13[e]), dequant_fp8e8_weight(W.w2[e], W.s2[e])
    return dequant_mxfp4_rows(W.w13[e], W.s13[e]), dequant_mxfp4_rows(W.w2[e], W.s2[e])


def quant_act(mode: str, v: np.ndarray):
    """Dynamic activation quantisation of float32 rows: FP8 1x128 (fp32 or
    UE8M0 scales) or MXFP4 1x32."""
    if mode == "fp8":
        return quant_fp8_rows(v, 128)
    if mode == "fp8_ue8m0":
        return quant_fp8e8_rows(v, 128)
    if mode == "mxfp4":
        return quant_mxfp4_rows(v)
    raise ValueError(mode)


def dequant_act(mode: str, q: np.ndarray, s: np.ndarray) -> np.ndarray:
    if mode == "fp8":
        return dequant_fp8_rows(q, s, 128)
    if mode == "fp8_ue8m0":
        return dequant_fp8e8_rows(q, s, 128)
    if mode == "mxfp4":
        return dequant_mxfp4_rows(q, s)
    raise ValueError(mode)


def pad_cols(v: np.ndarray, cols: int) -> np.ndarray:
    out = np.zeros((v.shape[0], cols), F32)
    out[:, :v.shape[1]] = v
    return out


def moe_forward(x: np.ndarray, logits: np.ndarray, W: QuantWeights, top_k: int,
                swiglu_limit: float, hidden: int, inter: int, tokens=None,
                return_stages: bool = False):
    """The routed-expert MoE layer, stage by stage.

    x: float32 (bf16 values) [T, H]; logits float32 [T, E]; W: QuantWeights.
    ``tokens`` optionally restricts the output to a subset of token indices
    (the layer is row-independent, so a sample is computed exactly as in the
    full run).  Returns float32 [len(tokens) or T, H].

    1. route: top-k ids and renormalised weights.
    2. quantise x per token (once per token, not per slot), zero-padded to Hp.
    3. per (token, slot) pair with expert e: h = deq(xq[t]) . deq(w13[e])^T,
       fp32.
    4. a = silu(min(h[:Ip], L)) * clamp(h[Ip:], -L, L).
    5. re-quantise a from fp32 per pair row (FP8 1x128 or MXFP4 1x32 over Ip).
    6. y = deq(aq) . deq(w2[e])^T, fp32.
    7. out[t] = sum over slots j = 0..k-1, in slot order, of fl32(w[t,j] * y),
       accumulated in fp32; first H columns.

    With ``return_stages`` it also returns the routing, the quantised input,
    per (sample token, slot) pair the GEMM1 output ``h`` (fp32, gate columns
    then up columns), the SwiGLU output ``a`` (fp32, before re-quantisation)
    and its codes/scales ``aq``, and the per-pair ``y``.
    """
    mode = W.mode
    x = np.asarray(x, F32)
    T = x.shape[0]
    Ip = W.w2.shape[2] * (2 if mode == "mxfp4" else 1)
    Hp = W.w2.shape[1]
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    ids, wts = route_topk(np.asarray(logits, F32)[tok], top_k)
    xq, xs = quant_act(mode, pad_cols(x[tok], Hp))
    xd = dequant_act(mode, xq, xs)
    n = len(tok)
    y = np.zeros((n, top_k, Hp), F32)
    aq_all = {}
    a_all = {}
    h_all = {}
    for e in np.unique(ids):
        w13d, w2d = dequant_expert(W, int(e))
        rows = np.argwhere(ids == e)  # (token index in sample, slot) pairs, increasing f
        h = gemm_f32(xd[rows[:, 0]], w13d)
        a = swiglu_clamped(h[:, :Ip], h[:, Ip:], swiglu_limit)
        aq, as_ = quant_act(mode, a)
        ad = dequant_act(mode, aq, as_)
        yy = gemm_f32(ad, w2d)
        for i, (t, j) in enumerate(rows):
            y[t, j] = yy[i]
            if return_stages:
                aq_all[(int(t), int(j))] = (aq[i], as_[i])
                a_all[(int(t), int(j))] = a[i]
                h_all[(int(t), int(j))] = h[i]
    out = np.zeros((n, Hp), F32)
    for j in range(top_k):
        out = (out + (wts[:, j:j + 1] * y[:, j]).astype(F32)).astype(F32)
    out = out[:, :hidden]
    if return_stages:
        return out, dict(ids=ids, weights=wts, xq=xq, xs=xs, y=y, aq=aq_all, a=a_all, h=h_all)
    return out

