"""Pins of the oracle's routing and permutation (CPU only).

Routing ids are checked against brute force (pure-Python sort of
(-value, id) pairs) on 200 random batches plus tie-heavy integer batches,
following the id-identity test of FreeToken PR #270 "glm5_next: support
GLM-5.3-Flash (hybrid KDA + DSA, mHC, NVFP4 expert offload)", Summary (router
ids identical to a reference top-k on 200 random batches), with the tie order
fixed to the lower expert id.  Weights are checked against scipy's softmax on
the selected logits; the permutation against a brute-force segment build and
its invariants.
"""
import numpy as np
import pytest
import scipy.special

import oracle as O


def _brute_topk(row, k):
    pairs = sorted((-float(v), e) for e, v in enumerate(row))
    return [e for _, e in pairs[:k]]


@pytest.mark.parametrize("batch", range(200))
def test_route_ids_random_batches(batch):
    rng = np.random.default_rng(1000 + batch)
    T = int(rng.integers(1, 9))
    E = int(rng.choice([8, 33, 64, 288]))
    k = int(rng.integers(1, min(E, 16) + 1))
    lg = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = O.route_topk(lg, k)
    for t in range(T):
        assert ids[t].tolist() == _brute_topk(lg[t], k)
        # stable argsort of the negated logits gives the same prefix
        assert ids[t].tolist() == np.argsort(-lg[t].astype(np.float64), kind="stable")[:k].tolist()


def test_route_ids_tie_heavy():
    rng = np.random.default_rng(7)
    for _ in range(50):
        T, E, k = 4, 288, 8
        lg = rng.integers(-3, 4, (T, E)).astype(np.float32)
        ids, _ = O.route_topk(lg, k)
        for t in range(T):
            assert ids[t].tolist() == _brute_topk(lg[t], k)


def test_route_signed_zero_ties_go_to_lower_id():
    lg = np.full((1, 6), -1.0, np.float32)
    lg[0, 4] = 0.0
    lg[0, 1] = -0.0
    ids, w = O.route_topk(lg, 2)
    assert ids[0].tolist() == [1, 4]
    assert w[0, 0] == w[0, 1] == np.float32(0.5)


def test_route_ids_invariant_under_power_of_two_scaling():
    rng = np.random.default_rng(8)
    lg = rng.standard_normal((32, 288)).astype(np.float32)
    ids, _ = O.route_topk(lg, 8)
    for s in (0.5, 2.0, 1024.0):
        ids2, _ = O.route_topk(lg * np.float32(s), 8)
        assert np.array_equal(ids, ids2)


def test_route_weights_closed_form():
    rng = np.random.default_rng(9)
    lg = (rng.standard_normal((64, 288)) * 3).astype(np.float32)
    ids, w = O.route_topk(lg, 8)
    sel = np.take_along_axis(lg, ids.astype(np.int64), axis=1).astype(np.float64)
    ref = scipy.special.softmax(sel, axis=1)
    assert np.allclose(w, ref, rtol=1e-6, atol=0)
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1) <= 8 * 2.0 ** -24)
    # weights follow slot order (descending logits)
    assert np.all(np.diff(w, axis=1) <= 0)
    # softmax over all E then renormalised over the chosen k is the same thing
    full = scipy.special.softmax(lg.astype(np.float64), axis=1)
    fsel = np.take_along_axis(full, ids.astype(np.int64), axis=1)
    assert np.allclose(w, fsel / fsel.sum(1, keepdims=True), rtol=1e-6)


def test_route_single_expert_weight_is_one():
    lg = np.random.default_rng(10).standard_normal((5, 1)).astype(np.float32)
    ids, w = O.route_topk(lg, 1)
    assert np.all(ids == 0) and np.all(w == np.float32(1.0))


# ------------------------------------------------------- permute-align -----

def _brute_permute(ids, E, BM):
    flat = ids.reshape(-1).tolist()
    P = len(flat)
    seg = []
    blocks = []
    offsets = [0]
    for e in range(E):
        fs = [f for f in range(P) if flat[f] == e]
        padded = -(-len(fs) // BM) * BM
        seg += fs + [P] * (padded - len(fs))
        blocks += [e] * (padded // BM)
        offsets.append(offsets[-1] + padded)
    return seg, blocks, offsets


@pytest.mark.parametrize("case", range(30))
def test_permute_align_brute_force(case):
    rng = np.random.default_rng(2000 + case)
    E = int(rng.choice([1, 3, 8, 17]))
    k = int(rng.integers(1, min(E, 4) + 1))
    T = int(rng.integers(0, 40))
    BM = int(rng.choice([16, 32, 64, 128]))
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32) if T else np.zeros((0, k), np.int32)
    sorted_ids, block_expert, offsets, npp = O.permute_align(ids, E, BM)
    seg, blocks, offs = _brute_permute(ids, E, BM)
    P = T * k
    nb = O.max_blocks(P, E, BM)
    assert len(sorted_ids) == nb * BM and len(block_expert) == nb
    assert npp == offs[-1] == len(seg) and npp <= nb * BM
    assert sorted_ids[:npp].tolist() == seg
    assert np.all(sorted_ids[npp:] == P)
    assert block_expert[:npp // BM].tolist() == blocks
    assert np.all(block_expert[npp // BM:] == -1)
    assert offsets.tolist() == offs


def test_permute_align_invariants_large():
    rng = np.random.default_rng(11)
    T, E, k, BM = 512, 288, 8, 16
    lg = rng.standard_normal((T, E)).astype(np.float32)
    ids, _ = O.route_topk(lg, k)
    sorted_ids, block_expert, offsets, npp = O.permute_align(ids, E, BM)
    P = T * k
    real = sorted_ids[sorted_ids < P]
    assert np.array_equal(np.sort(real), np.arange(P))          # each pair exactly once
    counts = np.bincount(ids.reshape(-1), minlength=E)
    padded = -(-counts // BM) * BM
    assert np.array_equal(np.diff(offsets), padded)
    flat = ids.reshape(-1)
    for e in range(E):
        s = sorted_ids[offsets[e]:offsets[e + 1]]
        r = s[s < P]
        assert np.all(np.diff(r) > 0) and np.all(flat[r] == e)   # ascending, right expert
        assert np.all(block_expert[offsets[e] // BM:offsets[e + 1] // BM] == e)


def test_max_blocks_bound_is_tight_enough():
    # worst case: every expert gets one pair -> E blocks when P >= E
    assert O.max_blocks(288, 288, 128) == 288
    assert O.max_blocks(8, 288, 16) == 8
    assert O.max_blocks(512, 288, 16) == (512 + 288 * 15) // 16


def test_permute_align_skips_out_of_range_ids():
    ids = np.array([[0, 5], [-1, 1], [1, 0]], np.int32)
    sorted_ids, block_expert, offsets, npp = O.permute_align(ids, 2, 16)
    assert npp == 32 and offsets.tolist() == [0, 16, 32]
    assert sorted_ids[:3].tolist() == [0, 5, 6] and np.all(sorted_ids[3:16] == 6)
    assert sorted_ids[16:18].tolist() == [3, 4] and np.all(sorted_ids[18:] == 6)


def test_permute_align_duplicate_experts_keep_f_order():
    ids = np.array([[1, 1], [0, 1]], np.int32)
    sorted_ids, _, offsets, _ = O.permute_align(ids, 2, 16)
    assert sorted_ids[offsets[1]:offsets[1] + 3].tolist() == [0, 1, 3]
