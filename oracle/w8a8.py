"""The W8A8 int8 g128 format ("i8g") on the grouped gate_up (fp64).

Test infrastructure: only the tests, the package smoke check and the bench's
CPU baseline use this module; the GPU path never does.

Source: "Gemma 4 12B-it · int8 · for radiance", header table row "Format"
(int8 weights with one bf16 scale per 128 weights; int8 activations with one
scale per token and 128 values) and "How it was made", step 2 (round to
nearest, no calibration data). The int5 card's header table, row "Format",
uses the same activation form for calls above 64 rows, so this is the
many-rows (prefill-shaped) form. Readings:
  * weights, per row n and group g of 128 along K: s = bf16(amax / 127)
    (the stored scale is the one the codes are formed with); q = round half
    to even of w / s, clamped to [-127, 127]; an all-zero group stores s = 0
    and q = 0. No rotation: the card names none.
  * activations, per token t and group g: sx = float32(amax / 127), one
    rounding of the exact quotient (the card gives no scale type; float32 as
    for the FP8 activation scales); qx = round half to even of
    float32(x / sx), clamped to [-127, 127] (two roundings, as a float32
    device computes them); amax == 0 gives sx = 0 and qx = 0.
  * the product on the grouped layout of the int8 path:
        gu[r, n] = sum_g sw[e, n, g] * sx[t, g] * sum_{kk in g} qw[e, n, kk] * qx[t, kk]
    with the same GELU-tanh(gate) * up epilogue (gateup.epilogue). The
    integer group sums are exact; the rest rounds at fp64.
"""

import numpy as np

from .gateup import _rows_of
from .numfmt import bf16_round

GROUP = 128
QMAX = 127


def quantize_i8g_weights(w):
    """w [..., N, K] -> (codes int8 [..., N, K], scales fp64 [..., N, K/128] holding bf16 values)."""
    w = np.asarray(w, dtype=np.float64)
    lead, k_dim = w.shape[:-1], w.shape[-1]
    g = w.reshape(*lead, k_dim // GROUP, GROUP)
    s = bf16_round(np.abs(g).max(axis=-1) / QMAX)
    safe = np.where(s > 0, s, 1.0)
    q = np.clip(np.rint(g / safe[..., None]), -QMAX, QMAX)
    q = np.where(s[..., None] > 0, q, 0.0)
    return q.reshape(*lead, k_dim).astype(np.int8), s


def quantize_i8_activations(x):
    """Activations [T, K] (fp64 values, e.g. bf16) -> (codes int8 [T, K], float32 scales [T, K/128])."""
    x = np.asarray(x, dtype=np.float64)
    t, k = x.shape
    g = x.reshape(t, k // GROUP, GROUP)
    amax = np.max(np.abs(g), axis=-1, keepdims=True)
    sx = (amax / QMAX).astype(np.float32)              # exact quotient, rounded once
    sx64 = sx.astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio32 = np.where(sx64 == 0, 0.0, g / sx64).astype(np.float32)   # float32 division
    q = np.clip(np.rint(ratio32.astype(np.float64)), -QMAX, QMAX)
    q = np.where(sx64 == 0, 0.0, q)
    return q.reshape(t, k).astype(np.int8), sx[..., 0]


def gateup_i8g(qx, sx, codes, scales, expert_off, sorted_pairs, topk, rows=None):
    """Grouped W8A8 gate_up.

    qx int8 [T, K] and sx float32 [T, K/128] from quantize_i8_activations,
    codes int8 [E, N, K], scales fp64 [E, N, K/128] (bf16 values).
    Returns gu [R, N] for the requested sorted rows (all P rows by default).
    """
    # integer-valued fp64 operands: every partial sum of int8 x int8 products
    # over a group is an integer below 2^21, so the fp64 matmul is exact in
    # any summation order
    qx = np.asarray(qx, dtype=np.float64)
    sx = np.asarray(sx, dtype=np.float64)
    n_rows, k_dim = codes.shape[1], codes.shape[2]
    n_groups = k_dim // GROUP
    r, e = _rows_of(expert_off, rows)
    t = np.asarray(sorted_pairs, dtype=np.int64)[r] // topk
    gu = np.zeros((r.size, n_rows))
    for ex in np.unique(e):
        sel = np.nonzero(e == ex)[0]
        xs = qx[t[sel]].reshape(sel.size, n_groups, GROUP)
        w = np.asarray(codes[ex], dtype=np.float64).reshape(n_rows, n_groups, GROUP)
        sw = np.asarray(scales[ex], dtype=np.float64)                     # [N, G]
        acc = np.zeros((sel.size, n_rows))
        for g in range(n_groups):
            isum = xs[:, g, :] @ w[:, g, :].T                             # exact integers
            acc += isum * sw[:, g][None, :] * sx[t[sel], g][:, None]
        gu[sel] = acc
    return gu
