"""CPU pins of the re-quantisation tie allowance used by the GPU parity
tests: it is zero away from rounding midpoints, and a code planted at a tie
and rounded the other way moves the oracle's output by no more than the
allowance (and by exactly the bound when a single weight column is
involved)."""
import numpy as np

import oracle as O
import workloads as W
from parity_util import oracle_weights_cpu, requant_tie_allowance, _tie_deltas


def test_tie_deltas_grid():
    e4 = O.e4m3_value_table()
    g8 = np.unique(np.abs(e4[np.isfinite(e4)]))
    # 1.0625 is the midpoint of 1.0 and 1.125; 1.0 is a code
    d = _tie_deltas(np.array([1.0625, -1.0625, 1.0, 0.0, 300.0]), g8, 1e-4)
    assert d[0] == d[1] == 0.125 and d[2] == 0 and d[3] == 0 and d[4] == 0


def _stages(wl):
    Q = oracle_weights_cpu(wl)
    x = W.activations(wl).float().numpy()
    lg = W.router_logits(wl).numpy()
    return Q, O.moe_forward(x, lg, Q, wl.top_k, wl.swiglu_limit, wl.H, wl.I, return_stages=True)


def test_allowance_covers_a_planted_flip():
    wl = W.WORKLOADS["tiny_fp8"]
    Q, (ref, st) = _stages(wl)
    assert requant_tie_allowance(st, Q, "fp8", wl.H).shape == ref.shape
    # plant: an intermediate row whose values all sit on E4M3 codes of its
    # scale (no ties), except value i, put exactly on the midpoint of 1.0 and
    # 1.125; the allowance is then exactly the effect of that one code
    t, j = 0, 0
    s = np.float32(0.01)
    e4 = O.e4m3_value_table()
    g8 = np.unique(np.abs(e4[np.isfinite(e4)]))
    rng = np.random.default_rng(3)
    a = (g8[rng.integers(0, len(g8), 128)] * rng.choice([-1.0, 1.0], 128)).astype(np.float32) * s
    a[0] = np.float32(448.0) * s  # amax -> scale s
    i = 7
    a[i] = np.float32(1.0625) * s
    assert np.float32(np.max(np.abs(a)) / np.float32(448.0)) == s
    st2 = dict(st)
    st2["a"] = {(t, j): a}
    bound = requant_tie_allowance(st2, Q, "fp8", wl.H)[t]
    e = int(st["ids"][t, j])
    w2d = O.dequant_expert(Q, e)[1].astype(np.float64)
    change = float(st["weights"][t, j]) * 0.125 * float(s) * np.abs(w2d[:, i])[:wl.H]
    assert np.allclose(bound, change, rtol=1e-9, atol=0)
    # and the two roundings of the planted value really differ by that much
    q_lo, q_hi = O.round_to_e4m3(np.array([1.0])), O.round_to_e4m3(np.array([1.125]))
    assert e4[q_hi[0]] - e4[q_lo[0]] == 0.125


def test_allowance_zero_when_no_ties():
    wl = W.WORKLOADS["tiny_fp8"]
    Q, (ref, st) = _stages(wl)
    bound = requant_tie_allowance(st, Q, "fp8", wl.H, eps=0.0)
    assert not np.any(bound)
