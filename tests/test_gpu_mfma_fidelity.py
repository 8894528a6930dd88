"""Why GEMM1 widens FP8 to f16 instead of using the FP8 matrix-core
instruction: measured sums of one K block (16 x 16 outputs over K = 128 of
e4m3 codes) from each instruction against the exact fp64 sum.

GEMM1's output is re-quantised, and the parity check accepts a differing
intermediate code only within the fp32 accumulation bound of GEMM1's sum
(64 u sum |ab|, u = 2^-24, parity_util.C_ACC).  The f16 path stays within a
few u of sum |ab| per K block; the FP8 instruction drops low-order bits of
small products when a large one is present (a K block with one product of 1
and 127 products of 2^-18 comes back short), far beyond that bound.  GEMM2's
output is not re-quantised and keeps the FP8 instruction.
"""
import numpy as np
import pytest
import torch

import oracle as O
from parity_util import C_ACC, U32, log

pytestmark = pytest.mark.gpu

M = None


@pytest.fixture(scope="module", autouse=True)
def lib():
    global M
    import mxfp4_quantized_weights_amd as mod
    M = mod
    yield mod


TAB = O.e4m3_value_table()


def _exact(a, b):
    A, B = TAB[a.astype(np.int64)], TAB[b.astype(np.int64)]
    return A @ B.T, np.abs(A) @ np.abs(B).T


def _run(kind, a, b):
    out = M.moe_diag_mfma_tile(kind, torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda())
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _rel(kind, a, b):
    ex, ab = _exact(a, b)
    return np.abs(_run(kind, a, b) - ex) / np.maximum(ab, 1e-300)


def test_f16_path_sum_is_fp32_faithful_and_fp8_is_not_on_small_terms():
    rng = np.random.default_rng(11)
    a = O.round_to_e4m3(np.clip(rng.standard_normal((16, 128)) * 16, -448, 448))
    b = O.round_to_e4m3(np.clip(rng.standard_normal((16, 128)) * 16, -448, 448))
    # row 0 of A and of B: one product 1 * 1, then 127 products 2^-9 * 2^-9
    one, tiny = O.round_to_e4m3(np.array([1.0]))[0], O.round_to_e4m3(np.array([2.0 ** -9]))[0]
    a[0, :] = tiny
    b[0, :] = tiny
    a[0, 0] = b[0, 0] = one
    ex, ab = _exact(a, b)
    assert ex[0, 0] == 1.0 + 127 * 2.0 ** -18
    got16, got8 = _run(1, a, b), _run(0, a, b)
    e16 = abs(got16[0, 0] - ex[0, 0]) / ab[0, 0]
    e8 = abs(got8[0, 0] - ex[0, 0]) / ab[0, 0]
    log(f"  C[0,0] exact 1 + 127*2^-18; f16 path 1 + {(got16[0, 0] - 1) / 2 ** -18:.2f}*2^-18 "
        f"({e16 / U32:.1f} u of sum|ab|); FP8 MFMA 1 + {(got8[0, 0] - 1) / 2 ** -18:.2f}*2^-18 ({e8 / U32:.1f} u)")
    assert e16 <= 4 * U32
    assert e8 > C_ACC * U32, "the FP8 instruction kept the small products"


def test_random_tiles_error_statistics():
    """Codes of N(0,1) values under a 1x128 scale (amax -> 448): the f16
    path's error stays within a few u of sum |ab| on every output; the FP8
    instruction's is logged (its largest over the tiles is reported)."""
    rng = np.random.default_rng(12)
    worst16 = worst8 = 0.0
    med8 = []
    for _ in range(24):
        va, vb = rng.standard_normal((16, 128)), rng.standard_normal((16, 128))
        a = O.round_to_e4m3(np.clip(va / np.abs(va).max(axis=1, keepdims=True) * 448, -448, 448))
        b = O.round_to_e4m3(np.clip(vb / np.abs(vb).max(axis=1, keepdims=True) * 448, -448, 448))
        r16, r8 = _rel(1, a, b), _rel(0, a, b)
        worst16, worst8 = max(worst16, float(r16.max())), max(worst8, float(r8.max()))
        med8.append(float(np.median(r8)))
    log(f"  over 24 tiles: f16 path max {worst16 / U32:.2f} u of sum|ab|; FP8 MFMA max {worst8 / U32:.1f} u, "
        f"median {np.median(med8) / U32:.1f} u")
    assert worst16 <= 4 * U32


@pytest.mark.parametrize("kind", [0, 1, 2])
def test_mfma_rate_diagnostic_runs(kind):
    # the rate loop of each instruction runs to completion and leaves finite
    # sums in its sink (its timing is bench.py's business)
    sink = M.moe_diag_mfma_rate(kind, 16)
    torch.cuda.synchronize()
    s = sink.cpu().numpy()
    assert s.shape == (M.DIAG_MFMA_RATE_WORKGROUPS * 256,)
    assert np.isfinite(s).all()
    log(f"mfma rate kind {kind}: sink sum {float(s.sum()):.4g}")


@pytest.mark.parametrize("words", [4, 4 * 1001, 4 * (256 * 4 * 512 * 3 + 12345)])
def test_stream_diagnostic_reads_every_word_once(words):
    # the XOR of the per-thread checksums is the XOR of every 32-bit word of
    # the buffer exactly when each 16-byte word is read once (one word; fewer
    # words than workgroups; several unrolled rounds per workgroup with a
    # ragged tail)
    rng = np.random.default_rng(words)
    host = rng.integers(-2**31, 2**31, size=words, dtype=np.int64).astype(np.int32)
    src = torch.from_numpy(host).cuda()
    sink = M.moe_diag_stream_read(src)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy())
    assert got == np.bitwise_xor.reduce(host)
