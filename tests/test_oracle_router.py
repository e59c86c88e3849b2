"""Pins for the oracle's routing and permutation.

The int8 card's model table (row "Weights") describes routed experts picked
by a router; the readings (top-k by logit, ties to the lower expert, softmax
over the k chosen, stable expert-sorted permutation) are pinned here against
a Python brute force, a library softmax and the permutation invariants.
"""

import numpy as np
import torch

from oracle import router


def _brute(logits, k):
    t_count, e_count = logits.shape
    ids = []
    for t in range(t_count):
        order = sorted(range(e_count), key=lambda e: (-float(logits[t, e]), e))
        ids.append(order[:k])
    return np.array(ids)


def _check_permutation(ids, e_count, off, sp, pos):
    flat = ids.reshape(-1)
    p_count = flat.size
    assert off[0] == 0 and off[-1] == p_count and np.all(np.diff(off) >= 0)
    assert np.array_equal(np.sort(sp), np.arange(p_count))
    assert np.array_equal(sp[pos], np.arange(p_count))
    for e in range(e_count):
        seg = sp[off[e]:off[e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg) > 0)                   # stable: increasing pair index
        assert seg.size == np.count_nonzero(flat == e)


def test_topk_matches_sorted_brute_force_with_ties():
    rng = np.random.default_rng(21)
    lg = np.round(rng.standard_normal((50, 16)), 1).astype(np.float32)  # many exact ties
    lg[3] = 0.5                                                          # all equal
    ids, w = router.topk(lg, 5)
    assert np.array_equal(ids, _brute(lg, 5))
    assert np.array_equal(ids[3], np.arange(5))


def test_nan_logits_rank_last_by_index():
    # NaN after every number, -inf included; NaNs among themselves by index
    rng = np.random.default_rng(23)
    lg = rng.standard_normal((6, 12)).astype(np.float32)
    lg[0, [2, 5, 7]] = np.nan
    lg[1] = np.nan
    lg[2, :6] = -np.inf
    lg[2, 6:] = np.nan
    lg[3, [0, 11]] = np.nan
    lg[3, 4] = np.inf
    lg[4, ::2] = np.nan
    lg[4, 1::2] = -np.inf
    for k in (1, 4, 12):
        ids, w = router.topk(lg, k)
        want = []
        for t in range(lg.shape[0]):
            key = lambda e: (1 if np.isnan(lg[t, e]) else 0, 0.0 if np.isnan(lg[t, e]) else -float(lg[t, e]), e)
            want.append(sorted(range(lg.shape[1]), key=key)[:k])
        assert np.array_equal(ids, np.array(want))
        assert np.all((ids >= 0) & (ids < lg.shape[1]))
        sel = np.take_along_axis(lg, ids, 1)
        has_nan = np.isnan(sel).any(axis=1)
        assert np.all(np.isnan(w[has_nan])) and np.all(np.isfinite(w[~has_nan & np.isfinite(sel).all(axis=1)]))
    assert list(router.topk(lg, 3)[0][1]) == [0, 1, 2]          # all NaN: the lowest indices
    assert list(router.topk(lg, 8)[0][2]) == [0, 1, 2, 3, 4, 5, 6, 7]  # -inf before NaN


def test_negative_zero_ties_positive_zero():
    lg = np.zeros((1, 4), dtype=np.float32)
    lg[0, 0] = -0.0
    ids, _ = router.topk(lg, 2)
    assert list(ids[0]) == [0, 1]


def test_softmax_weights_against_torch():
    rng = np.random.default_rng(22)
    lg = rng.standard_normal((40, 128)).astype(np.float32) * 3
    ids, w = router.topk(lg, 8)
    sel = np.take_along_axis(lg, ids, 1).astype(np.float64)
    want = torch.softmax(torch.from_numpy(sel), dim=1).numpy()
    np.testing.assert_allclose(w, want, rtol=1e-14, atol=0)
    assert np.all(np.diff(w, axis=1) <= 0)                 # slots in descending logit order
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-15)


def test_k_equals_e_selects_everything_in_order():
    lg = np.array([[0.1, 0.3, -1.0, 0.3]], dtype=np.float32)
    ids, w = router.topk(lg, 4)
    assert list(ids[0]) == [1, 3, 0, 2]


def test_permutation_invariants_and_hand_case():
    ids = np.array([[2, 0], [0, 1], [2, 1]])
    r = router.permute(ids, 4)
    off, sp, pos = r
    # pairs: p0->e2, p1->e0, p2->e0, p3->e1, p4->e2, p5->e1
    assert list(off) == [0, 2, 4, 6, 6]
    assert list(sp) == [1, 2, 3, 5, 0, 4]
    assert list(pos) == [4, 0, 1, 2, 5, 3]
    _check_permutation(ids, 4, off, sp, pos)


def test_permutation_random_skewed():
    rng = np.random.default_rng(23)
    lg = rng.standard_normal((300, 64)).astype(np.float32) + rng.standard_normal(64).astype(np.float32) * 2
    res = router.route(lg, 6)
    _check_permutation(res["ids"], 64, res["expert_off"], res["sorted_pairs"], res["pair_pos"])
    # distinct experts per token
    assert all(len(set(r)) == 6 for r in res["ids"])
