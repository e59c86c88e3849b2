"""bf16 grouped down projection and the weighted combine (fp64).

Test infrastructure: only the tests, the package smoke check and the bench's
CPU baseline use this module; the GPU path never does.

The int8 card's model table (row "Weights") keeps the routed experts' down
projections in bf16 as the checkpoint ships them; the cards show neither
that product nor how the k expert outputs of a token are merged. Readings:
  * an expert's down weight is W_down[e] of shape [H, I] (H = the hidden
    size K of the gate_up input, I = N / 2), row-major, bf16;
  * the product takes bf16 operands: the act rows (float32 out of the
    gate_up epilogue) are rounded to bf16, nearest-even, first;
  * for the pair in expert-sorted row r of expert e,
        y[r, h] = sum_i W_down[e, h, i] * bf16(act[r, i]);
  * the k outputs of token t are merged with its router weights, slot by
    slot:  out[t, h] = sum_j w[t, j] * y[pos[t k + j], h],
    where pos is the routing's inverse permutation.
Products of two bf16 values are exact in fp64; the sums round at fp64.
"""

import numpy as np

from .numfmt import bf16_round


def _expert_of_rows(expert_off, rows):
    off = np.asarray(expert_off, dtype=np.int64)
    return np.searchsorted(off, rows, side="right") - 1


def down_grouped(act, w_down, expert_off, rows=None):
    """y [R, H] for the requested sorted rows (all P by default).

    act [P, I] float32 values (rounded to bf16 here), w_down [E, H, I] fp64
    holding bf16 values, expert_off [E + 1].
    """
    a = bf16_round(np.asarray(act, dtype=np.float64))
    w = np.asarray(w_down, dtype=np.float64)
    p_count = int(np.asarray(expert_off)[-1])
    r = np.arange(p_count) if rows is None else np.asarray(rows, dtype=np.int64)
    e = _expert_of_rows(expert_off, r)
    y = np.zeros((r.size, w.shape[1]), dtype=np.float64)
    for ex in np.unique(e):
        sel = np.nonzero(e == ex)[0]
        y[sel] = a[r[sel]] @ w[ex].T          # one expert's rows, one matrix product
    return y


def combine(y, pair_pos, weights, topk):
    """out [T, H] = sum_j weights[t, j] * y[pair_pos[t k + j]], slot order j."""
    y = np.asarray(y, dtype=np.float64)
    w = np.asarray(weights, dtype=np.float64)
    pos = np.asarray(pair_pos, dtype=np.int64).reshape(-1, topk)
    out = np.zeros((pos.shape[0], y.shape[1]), dtype=np.float64)
    for j in range(topk):
        out += w[:, j:j + 1] * y[pos[:, j]]
    return out


def down_combine(act, w_down, expert_off, pair_pos, weights, topk):
    """The whole step: out [T, H]."""
    return combine(down_grouped(act, w_down, expert_off), pair_pos, weights, topk)
