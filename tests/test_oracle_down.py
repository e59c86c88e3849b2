"""Pins for the oracle's bf16 grouped down projection and weighted combine.

Source: int8 card, model table row "Weights" (the routed experts' down
projections stay bf16). The readings (bf16 act operand, slot-order combine
with the router weights) are pinned by a pure-Python brute force that walks
tokens and slots directly (no sorted order, no inverse permutation), by a
library matrix product on the single-expert special case, by linearity and
one-hot invariants, and by exact rounding cases of the act operand.
"""

import numpy as np
import torch

from oracle import down, numfmt, router


def _case(seed=5, t_count=3, e_count=4, k=2, h=6, i_dim=10):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((t_count, e_count)).astype(np.float32)
    r = router.route(lg, k)
    w = numfmt.bf16_round(rng.standard_normal((e_count, h, i_dim)) * 0.02)
    act_pair = rng.standard_normal((t_count * k, i_dim)).astype(np.float32)   # one row per pair p = t k + j
    act_sorted = act_pair[r["sorted_pairs"]]                                   # the layout the step consumes
    return r, w, act_pair, act_sorted, k


def test_brute_force_by_token_and_slot():
    r, w, act_pair, act_sorted, k = _case()
    out = down.down_combine(act_sorted, w, r["expert_off"], r["pair_pos"], r["weights"], k)
    t_count, h = out.shape[0], w.shape[1]
    for t in range(t_count):
        for hh in range(h):
            total = 0.0
            for j in range(k):
                e = int(r["ids"][t, j])
                p = t * k + j
                dot = 0.0
                for i in range(w.shape[2]):
                    a = float(np.float32(act_pair[p, i]))
                    a16 = float(torch.tensor(a, dtype=torch.float32).to(torch.bfloat16).to(torch.float64))
                    dot += float(w[e, hh, i]) * a16
                total += float(r["weights"][t, j]) * dot
            assert abs(out[t, hh] - total) <= 1e-12 * (1 + abs(total))


def test_single_expert_is_a_library_matmul():
    # E = 1, k = 1: every pair is its own token, weight 1, and the step is
    # bf16(act) @ W^T, a plain matrix product.
    rng = np.random.default_rng(11)
    t_count, h, i_dim = 7, 5, 12
    lg = rng.standard_normal((t_count, 1)).astype(np.float32)
    r = router.route(lg, 1)
    w = numfmt.bf16_round(rng.standard_normal((1, h, i_dim)))
    act = rng.standard_normal((t_count, i_dim)).astype(np.float32)
    out = down.down_combine(act, w, r["expert_off"], r["pair_pos"], r["weights"], 1)
    a16 = torch.from_numpy(act).to(torch.bfloat16).to(torch.float64)
    ref = torch.nn.functional.linear(a16, torch.from_numpy(w[0])).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-15)


def test_combine_is_linear_in_the_weights_and_one_hot_selects_a_row():
    r, w, _, act_sorted, k = _case(seed=8, t_count=5, e_count=6, k=3)
    y = down.down_grouped(act_sorted, w, r["expert_off"])
    base = down.combine(y, r["pair_pos"], r["weights"], k)
    np.testing.assert_allclose(down.combine(y, r["pair_pos"], 2.5 * r["weights"], k), 2.5 * base, rtol=1e-14)
    for j in range(k):
        onehot = np.zeros_like(r["weights"])
        onehot[:, j] = 1.0
        got = down.combine(y, r["pair_pos"], onehot, k)
        for t in range(got.shape[0]):
            # the row of pair t k + j in sorted order holds that pair
            row = int(np.nonzero(r["sorted_pairs"] == t * k + j)[0][0])
            np.testing.assert_array_equal(got[t], y[row])


def test_rows_are_taken_by_their_expert():
    # distinct constant weights per expert make y reveal which expert a row used
    r, w, _, act_sorted, k = _case(seed=3, t_count=4, e_count=5, k=2, h=3, i_dim=4)
    e_count = w.shape[0]
    w_const = np.stack([np.full(w.shape[1:], float(e + 1)) for e in range(e_count)])
    ones = np.ones_like(act_sorted)
    y = down.down_grouped(ones, w_const, r["expert_off"])
    off = r["expert_off"]
    for e in range(e_count):
        np.testing.assert_array_equal(y[off[e]:off[e + 1]], (e + 1) * ones.shape[1])


def test_act_operand_is_rounded_to_bf16_nearest_even():
    # one expert, one output, weight 1 on input 0: y equals bf16(act[0])
    lg = np.zeros((4, 1), dtype=np.float32)
    r = router.route(lg, 1)
    w = np.zeros((1, 1, 2))
    w[0, 0, 0] = 1.0
    vals = np.array([1 + 2.0 ** -9, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8 + 2.0 ** -20)], dtype=np.float32)
    act = np.stack([vals, np.zeros(4, dtype=np.float32)], axis=1)
    y = down.down_grouped(act, w, r["expert_off"])[:, 0]
    # below half an ulp -> down; a tie -> the even neighbour (1.0, then 1 + 2^-6);
    # above the tie -> away
    np.testing.assert_array_equal(y, [1.0, 1.0, 1 + 2.0 ** -6, -(1 + 2.0 ** -7)])


def test_rows_subset_matches_full():
    r, w, _, act_sorted, k = _case(seed=9, t_count=6, e_count=3, k=2)
    full = down.down_grouped(act_sorted, w, r["expert_off"])
    rows = np.array([0, 5, 2, 11, 7])
    np.testing.assert_array_equal(down.down_grouped(act_sorted, w, r["expert_off"], rows=rows), full[rows])
