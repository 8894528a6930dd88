"""Pins of the oracle's number formats and quantisers (CPU only).

Each check compares the oracle with something other than itself: the
published format definitions (tests/golden/ocp_formats.json), torch's
float8_e4m3fn conversion (a library cast), brute-force nearest-value search,
bit-level exponent extraction, and invariants that follow from the
quantiser's definition.
"""
import json
import os
import struct

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "ocp_formats.json")))


# ---------------------------------------------------------------- E4M3 -----

def test_e4m3_table_matches_torch_decode():
    ours = O.e4m3_value_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_e4m3_table_matches_spec_examples():
    g = GOLDEN["e4m3"]
    tab = O.e4m3_value_table()
    for code, val in g["examples"]:
        assert tab[code] == val and np.signbit(tab[code]) == np.signbit(val), code
    assert sorted(np.flatnonzero(np.isnan(tab)).tolist()) == g["nan_codes"]
    assert np.nanmax(tab) == g["max_normal"] == O.E4M3_MAX
    pos = tab[(tab > 0) & ~np.isnan(tab)]
    assert pos.min() == g["min_subnormal"]


def _e4m3_boundary_values():
    """Every code value, every midpoint between neighbours, and the fp32
    neighbours of every midpoint, over the whole finite range, both signs."""
    tab = O.e4m3_value_table()[:0x7F]
    mids = (tab[:-1] + tab[1:]) / 2
    mids32 = mids.astype(np.float32)
    assert np.array_equal(mids32.astype(np.float64), mids)  # midpoints are exact in fp32
    up = np.nextafter(mids32, np.float32(np.inf))
    dn = np.nextafter(mids32, np.float32(-np.inf))
    v = np.concatenate([tab.astype(np.float32), mids32, up, dn])
    v = v[np.abs(v) <= 448]
    return np.concatenate([v, -v]).astype(np.float32)


def _torch_e4m3(v32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(v32.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_round_to_e4m3_matches_torch_cast_on_boundaries():
    v = _e4m3_boundary_values()
    assert np.array_equal(O.round_to_e4m3(v), _torch_e4m3(v))


def test_round_to_e4m3_matches_torch_cast_random():
    rng = np.random.default_rng(1)
    mags = np.exp2(rng.uniform(-14, 8.8, size=400_000))
    v = (mags * rng.choice([-1, 1], size=mags.size)).astype(np.float32)
    v = np.clip(v, -448, 448).astype(np.float32)
    assert np.array_equal(O.round_to_e4m3(v), _torch_e4m3(v))


def test_round_to_e4m3_ties_to_even_and_sign_of_zero():
    # 1.0625 lies halfway between 1.0 (0x38) and 1.125 (0x39): even code wins
    assert O.round_to_e4m3(np.array([1.0625]))[0] == 0x38
    # 1.1875 lies halfway between 1.125 (0x39) and 1.25 (0x3A)
    assert O.round_to_e4m3(np.array([1.1875]))[0] == 0x3A
    # half the smallest subnormal rounds to zero (even), keeping the sign
    assert O.round_to_e4m3(np.array([2.0 ** -10]))[0] == 0x00
    assert O.round_to_e4m3(np.array([-2.0 ** -10]))[0] == 0x80
    assert O.round_to_e4m3(np.array([-0.0]))[0] == 0x80
    with pytest.raises(ValueError):
        O.round_to_e4m3(np.array([449.0]))


def test_fp8_group_quantiser_invariants():
    rng = np.random.default_rng(2)
    v = (rng.standard_normal((64, 512)) * np.exp2(rng.integers(-20, 20, (64, 1)))).astype(np.float32)
    v[3, 128:256] = 0.0           # an all-zero group
    v[5, :128] = -0.0             # an all-negative-zero group
    v[7, 0] = -0.0                # a negative zero inside a non-zero group
    q, s = O.quant_fp8_rows(v, 128)
    assert q.shape == (64, 512) and s.shape == (64, 4) and s.dtype == np.float32
    # amax == 0 reading: scale 0, codes 0x00
    assert s[3, 1] == 0 and np.all(q[3, 128:256] == 0)
    assert s[5, 0] == 0 and np.all(q[5, :128] == 0)
    assert q[7, 0] == 0x80
    # s = fl32(amax / 448)
    amax = np.abs(v.reshape(64, 4, 128)).max(-1)
    assert np.array_equal(s, (amax / np.float32(448)).astype(np.float32))
    # the group's largest element maps to the largest code 0x7E
    qg = (q.reshape(64, 4, 128) & 0x7F).max(-1)
    assert np.all(qg[amax > 0] == 0x7E)
    # each code is the torch RNE cast of the saturated fp32 quotient
    r = np.clip(v.reshape(64, 4, 128) / np.where(s > 0, s, 1)[..., None], -448, 448).astype(np.float32)
    ref = _torch_e4m3(r.reshape(64, 512))
    nz = np.repeat(amax > 0, 128, axis=1)
    assert np.array_equal(q[nz], ref[nz])


def test_fp8_saturation_when_quotient_exceeds_448():
    # amax / fl32(amax/448) can land just above 448 in fp32; it must saturate
    found = False
    for a in np.linspace(1.0, 2.0, 20001, dtype=np.float32):
        s = np.float32(a / np.float32(448))
        if np.float32(a / s) > 448:
            found = True
            v = np.zeros((1, 128), np.float32)
            v[0, 0] = a
            q, _ = O.quant_fp8_rows(v)
            assert q[0, 0] == 0x7E
            break
    assert found


def test_fp8_weight_blocks_are_independent_groups():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((256, 384)) * 0.02).astype(np.float32)
    w[128:, 256:] *= 1000
    q, s = O.quant_fp8_weight(w)
    assert s.shape == (2, 3)
    for i in range(2):
        for j in range(3):
            blk = w[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            qb, sb = O.quant_fp8_rows(blk.reshape(1, -1), 128 * 128)
            assert sb[0, 0] == s[i, j]
            assert np.array_equal(qb.reshape(128, 128), q[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128])


def test_fp8_dequant_is_code_value_times_scale():
    rng = np.random.default_rng(4)
    q = rng.integers(0, 256, (8, 256)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0
    s = rng.uniform(1e-4, 1.0, (8, 2)).astype(np.float32)
    d = O.dequant_fp8_rows(q, s, 128)
    tv = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float32)
    ref = (tv * torch.from_numpy(np.repeat(s, 128, axis=1))).numpy()
    assert np.array_equal(d, ref)


# ---------------------------------------------------------------- E2M1 -----

def test_e2m1_table_matches_spec():
    tab = O.e2m1_value_table()
    ref = np.array(GOLDEN["e2m1"]["values_by_code"])
    assert np.array_equal(tab, ref) and np.array_equal(np.signbit(tab), np.signbit(ref))


def test_e2m1_rounding_spec_examples():
    for v, code in GOLDEN["e2m1"]["round_half_even"]:
        assert O.round_to_e2m1(np.array([np.float32(v)]))[0] == code, v


def test_e2m1_rounding_matches_brute_force():
    rng = np.random.default_rng(5)
    grid = O.E2M1_VALUES
    v = rng.uniform(-6, 6, 20000)
    mids = (grid[:-1] + grid[1:]) / 2
    v = np.concatenate([v, mids, -mids, grid, -grid, np.nextafter(mids, 0), np.nextafter(mids, 7)])
    got = O.round_to_e2m1(v)
    for x, c in zip(v, got):
        d = [abs(abs(x) - g) for g in grid]
        best = min(d)
        cands = [i for i, di in enumerate(d) if di == best]
        want = cands[0] if len(cands) == 1 else [i for i in cands if i % 2 == 0][0]
        want |= 8 if np.signbit(x) else 0
        assert c == want, (x, c, want)


# ---------------------------------------------------------------- E8M0 -----

def _floor_log2_bits(a: float) -> int:
    """floor(log2 a) of a positive fp32 value from its bit pattern."""
    u = struct.unpack("<I", struct.pack("<f", a))[0]
    ef = (u >> 23) & 0xFF
    if ef:
        return ef - 127
    m = u & 0x7FFFFF
    return (m.bit_length() - 1) - 149


def test_e8m0_examples_from_spec_rule():
    for amax, b in GOLDEN["e8m0"]["examples_amax_to_byte"]:
        assert int(O.e8m0_scale_byte(np.float32(amax))) == b, amax


def test_e8m0_matches_bit_extraction_over_all_binades():
    rng = np.random.default_rng(6)
    vals = []
    for e in range(-149, 128):
        for m in (1.0, 1.5, 1.9999999, 1.0000001):
            x = np.float32(np.ldexp(m, e))
            if x > 0 and np.isfinite(x):
                vals.append(x)
    vals += list(rng.uniform(0, 1, 1000).astype(np.float32) * np.float32(1e-38))
    for a in vals:
        want = min(max(_floor_log2_bits(float(a)) - 2 + 127, 0), 254)
        assert int(O.e8m0_scale_byte(a)) == want, a
    assert int(O.e8m0_scale_byte(0.0)) == 0


def test_mxfp4_quantiser_invariants_and_round_trip():
    rng = np.random.default_rng(7)
    v = (rng.standard_normal((32, 256)) * np.exp2(rng.integers(-30, 30, (32, 1)))).astype(np.float32)
    v[1, 32:64] = 0
    v[2, 0] = -0.0
    p, b = O.quant_mxfp4_rows(v)
    assert p.shape == (32, 128) and b.shape == (32, 8)
    codes = O.unpack_e2m1(p)
    # packing: even element in the low nibble
    assert np.array_equal(codes[:, 0::2], p & 0xF) and np.array_equal(codes[:, 1::2], p >> 4)
    assert b[1, 1] == 0 and np.all(codes[1, 32:64] == 0)
    assert codes[2, 0] == 8
    g = codes.reshape(32, 8, 32) & 7
    amax = np.abs(v.reshape(32, 8, 32)).max(-1)
    # every non-zero group holds a code of magnitude 4.0 (code 6) or 6.0 (code 7)
    assert np.all(np.isin(g.max(-1)[amax > 0], [6, 7]))
    # round trip: quantising the dequantised values gives back the same bits
    d = O.dequant_mxfp4_rows(p, b)
    p2, b2 = O.quant_mxfp4_rows(d)
    assert np.array_equal(p2, p) and np.array_equal(b2, b)
    # dequant = code value * 2^(b-127)
    ref = O.E2M1_VALUES[g] * np.where(codes.reshape(32, 8, 32) & 8, -1, 1) * np.exp2(b.astype(np.float64) - 127)[..., None]
    assert np.array_equal(d.reshape(32, 8, 32).astype(np.float64), ref)


def test_mxfp4_error_bound():
    # |v - deq(q)| <= half the code spacing at the top binade: 2^(b-127) for |v|/2^(b-127) in [4, 6],
    # and saturation error < 2 * 2^(b-127) above 6
    rng = np.random.default_rng(8)
    v = rng.standard_normal((16, 512)).astype(np.float32)
    p, b = O.quant_mxfp4_rows(v)
    d = O.dequant_mxfp4_rows(p, b)
    unit = np.repeat(np.exp2(b.astype(np.float64) - 127), 32, axis=1)
    assert np.all(np.abs(d - v) <= 2 * unit)


# ------------------------------------------------------ FP8 with UE8M0 -----
# "[AMD] [GLM5] Opt-in prefill-only FP8 dense projection GEMM for MLA
# q_b/o_proj (gfx950)", Modifications: e4m3 with a 128x128 UE8M0 scale.  The
# reading pinned here: the scale is 2^e with e the smallest integer such
# that 448 * 2^e >= amax, stored as the E8M0 byte e + 127.

def _ue8m0_exponent_exact(amax: float) -> int:
    """Smallest e with 448 * 2^e >= amax, by exact rational comparison."""
    from fractions import Fraction
    a = Fraction(float(amax))
    e = 0
    while Fraction(448) * Fraction(2) ** e < a:
        e += 1
    while Fraction(448) * Fraction(2) ** (e - 1) >= a:
        e -= 1
    return e


def _ue8m0_amax_cases():
    rng = np.random.default_rng(30)
    vals = []
    for e in range(-149, 128):
        for m in (1.0, 1.5, 1.75, 1.7500001, 1.7499999, 1.9999999, 1.0000001):
            x = np.float32(np.ldexp(m, e))
            if x > 0 and np.isfinite(x):
                vals.append(x)
    for k in range(-140, 119):  # exactly 448 * 2^k and its fp32 neighbours
        x = np.float32(np.ldexp(448.0, k))
        if x > 0 and np.isfinite(x):
            vals += [x, np.nextafter(x, np.float32(np.inf)), np.nextafter(x, np.float32(0))]
    vals += list(np.exp2(rng.uniform(-140, 127, 2000)).astype(np.float32))
    return [v for v in vals if v > 0 and np.isfinite(v)]


def test_ue8m0_exponent_is_minimal_by_exact_comparison():
    cases = _ue8m0_amax_cases()
    got = O.ue8m0_exponent(np.array(cases, np.float32))
    for a, e in zip(cases, got):
        assert int(e) == _ue8m0_exponent_exact(a), a


def test_ue8m0_byte_examples_and_clamp():
    # amax 448 -> 2^0 (byte 127); just above 448 -> 2^1; 224 -> 2^-1; 1.0 -> 2^-8
    assert int(O.ue8m0_scale_byte(448.0)) == 127
    assert int(O.ue8m0_scale_byte(np.nextafter(np.float32(448), np.float32(1e9)))) == 128
    assert int(O.ue8m0_scale_byte(224.0)) == 126
    assert int(O.ue8m0_scale_byte(1.0)) == 127 - 8
    assert int(O.ue8m0_scale_byte(1.75)) == 127 - 8     # 448 * 2^-8 = 1.75 exactly
    assert int(O.ue8m0_scale_byte(1.76)) == 127 - 7
    # tiny amax: the exponent is below -127 and the byte clamps to 0 (2^-127)
    assert int(O.ue8m0_scale_byte(np.float32(1e-40))) == 0
    assert int(O.ue8m0_scale_byte(0.0)) == 0


def test_fp8e8_group_quantiser_invariants():
    rng = np.random.default_rng(31)
    v = (rng.standard_normal((64, 512)) * np.exp2(rng.integers(-30, 30, (64, 1)))).astype(np.float32)
    v[3, 128:256] = 0.0
    v[5, :128] = -0.0
    v[7, 0] = -0.0
    v[9] *= np.float32(1e-38)   # subnormal amax
    q, b = O.quant_fp8e8_rows(v, 128)
    assert q.shape == (64, 512) and b.shape == (64, 4) and b.dtype == np.uint8
    assert b[3, 1] == 0 and np.all(q[3, 128:256] == 0)
    assert b[5, 0] == 0 and np.all(q[5, :128] == 0)
    assert q[7, 0] == 0x80
    amax = np.abs(v.reshape(64, 4, 128)).max(-1).astype(np.float64)
    e = b.astype(np.int64) - 127
    nz = amax > 0
    # power-of-two scale just large enough: amax in (224 * 2^e, 448 * 2^e]
    # (unless the byte clamped at 0)
    hi = np.ldexp(448.0, e)
    assert np.all(amax[nz] <= hi[nz])
    unclamped = nz & (b > 0)
    assert np.all(amax[unclamped] > hi[unclamped] / 2)
    # the group's largest magnitude code lies in [0x76 (224), 0x7E (448)]
    qg = (q.reshape(64, 4, 128) & 0x7F).max(-1)
    assert np.all((qg[unclamped] >= 0x76) & (qg[unclamped] <= 0x7E))
    # each code is torch's RNE cast of v / 2^e, which is exact in fp32 here
    r = (v.reshape(64, 4, 128).astype(np.float64) / np.ldexp(1.0, e)[..., None])
    assert np.all(np.abs(r) <= 448)
    ref = _torch_e4m3(r.astype(np.float32).reshape(64, 512))
    mask = np.repeat(nz, 128, axis=1)
    assert np.array_equal(q[mask], ref[mask])


def test_fp8e8_dequant_exact_and_round_trip():
    rng = np.random.default_rng(32)
    v = (rng.standard_normal((16, 384)) * np.exp2(rng.integers(-20, 20, (16, 1)))).astype(np.float32)
    q, b = O.quant_fp8e8_rows(v, 128)
    d = O.dequant_fp8e8_rows(q, b, 128)
    tv = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ref = tv * np.repeat(np.exp2(b.astype(np.float64) - 127), 128, axis=1)
    assert np.array_equal(d.astype(np.float64), ref)
    # re-quantising the dequantised values gives back the same bits wherever
    # the group's largest code is above 224 (a largest code of exactly 224
    # halves the next scale)
    q2, b2 = O.quant_fp8e8_rows(d, 128)
    keep = (q.reshape(16, 3, 128) & 0x7F).max(-1) > 0x76
    assert np.array_equal(b2[keep], b[keep])
    assert np.array_equal(q2.reshape(16, 3, 128)[keep], q.reshape(16, 3, 128)[keep])
    # error bound: half a code step at the top binade, 16 * 2^e
    assert np.all(np.abs(d - v) <= np.repeat(np.exp2(b.astype(np.float64) - 127), 128, axis=1) * 16)


def test_fp8e8_weight_blocks_are_independent_groups():
    rng = np.random.default_rng(33)
    w = (rng.standard_normal((256, 384)) * 0.02).astype(np.float32)
    w[128:, 256:] *= 1000
    w[:128, 128:256] = 0
    q, b = O.quant_fp8e8_weight(w)
    assert b.shape == (2, 3) and b[0, 1] == 0
    for i in range(2):
        for j in range(3):
            blk = w[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            qb, bb = O.quant_fp8e8_rows(blk.reshape(1, -1), 128 * 128)
            assert bb[0, 0] == b[i, j]
            assert np.array_equal(qb.reshape(128, 128), q[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128])
