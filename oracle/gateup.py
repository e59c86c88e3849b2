"""Grouped gate_up products and the GELU-tanh(gate) * up epilogue (fp64).

int8 Hadamard-domain product (int8 card, model table row "Weights"): for the
pair in expert-sorted row r, owned by expert e and token t = sorted[r] // k,
    gu[r, n] = sum_g s[e, n, g] * sum_{kk in group g} q[e, n, kk] * x_rot[t, kk]
with x_rot the bf16 rotated activations. Since H128/sqrt(128) is orthonormal
this approximates the unrotated W x (the tests bound the gap).

FP8 block product (FP8 card, model table row "Weights"):
    gu[r, n] = sum_g sw[e, n // 128, g] * sx[t, g]
                     * sum_{kk in g} dec(qw[e, n, kk]) * dec(qx[t, kk]).

Readings (the cards are silent): the N = 2I rows of an expert's gate_up are
[gate rows 0..I-1 ; up rows I..2I-1]; the activation is GELU with the tanh
approximation, act[r, i] = gelu_tanh(gu[r, i]) * gu[r, I + i]; outputs stay
in expert-sorted row order; the router weights are not applied here.

Inner sums are exact in fp64 (integer or 4-bit-mantissa codes times bf16 or
E4M3 values, 128 terms); the outer sums round at fp64.
"""

import numpy as np

from .numfmt import e4m3_decode

GROUP = 128


def gelu_tanh(g):
    """0.5 g (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3))), fp64."""
    g = np.asarray(g, dtype=np.float64)
    return 0.5 * g * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (g + 0.044715 * g ** 3)))


def epilogue(gu):
    """gu [P, 2I] -> act [P, I] = gelu_tanh(gate) * up."""
    gu = np.asarray(gu, dtype=np.float64)
    i = gu.shape[1] // 2
    return gelu_tanh(gu[:, :i]) * gu[:, i:]


def _rows_of(expert_off, rows):
    """(row r, expert e) for the requested sorted rows (all if rows is None)."""
    off = np.asarray(expert_off, dtype=np.int64)
    p_count = int(off[-1])
    r = np.arange(p_count) if rows is None else np.asarray(rows, dtype=np.int64)
    e = np.searchsorted(off, r, side="right") - 1
    return r, e


def gateup_i8h(x_rot, codes, scales, expert_off, sorted_pairs, topk, rows=None):
    """Grouped int8 Hadamard-domain gate_up.

    x_rot [T, K] fp64 (bf16 values), codes int8 [E, N, K], scales fp64
    [E, N, K/128] (bf16 values), expert_off [E+1], sorted_pairs [P].
    Returns gu [R, N] for the requested sorted rows (all P rows by default).
    """
    x_rot = np.asarray(x_rot, dtype=np.float64)
    n_rows, k_dim = codes.shape[1], codes.shape[2]
    n_groups = k_dim // GROUP
    r, e = _rows_of(expert_off, rows)
    t = np.asarray(sorted_pairs, dtype=np.int64)[r] // topk
    gu = np.zeros((r.size, n_rows))
    for ex in np.unique(e):
        sel = np.nonzero(e == ex)[0]
        xs = x_rot[t[sel]].reshape(sel.size, n_groups, GROUP)
        q = codes[ex].astype(np.float64).reshape(n_rows, n_groups, GROUP)
        s = np.asarray(scales[ex], dtype=np.float64)          # [N, G]
        acc = np.zeros((sel.size, n_rows))
        for g in range(n_groups):
            partial = xs[:, g, :] @ q[:, g, :].T               # exact inner sums
            acc += partial * s[:, g][None, :]
        gu[sel] = acc
    return gu


def gateup_fp8blk(qx, sx, codes, scales, expert_off, sorted_pairs, topk, rows=None):
    """Grouped FP8 E4M3 128x128-block gate_up.

    qx uint8 [T, K] and sx float32 [T, K/128] from the activation quantizer,
    codes uint8 [E, N, K], scales fp64 [E, N/128, K/128] (bf16 values).
    Returns gu [R, N] for the requested sorted rows (all P rows by default).
    """
    xq = e4m3_decode(qx)
    sx = np.asarray(sx, dtype=np.float64)
    n_rows, k_dim = codes.shape[1], codes.shape[2]
    n_groups = k_dim // GROUP
    r, e = _rows_of(expert_off, rows)
    t = np.asarray(sorted_pairs, dtype=np.int64)[r] // topk
    gu = np.zeros((r.size, n_rows))
    for ex in np.unique(e):
        sel = np.nonzero(e == ex)[0]
        xs = xq[t[sel]].reshape(sel.size, n_groups, GROUP)
        w = e4m3_decode(codes[ex]).reshape(n_rows, n_groups, GROUP)
        sw = np.repeat(np.asarray(scales[ex], dtype=np.float64), GROUP, axis=0)  # [N, G]
        acc = np.zeros((sel.size, n_rows))
        for g in range(n_groups):
            partial = xs[:, g, :] @ w[:, g, :].T
            acc += partial * sw[:, g][None, :] * sx[t[sel], g][:, None]
        gu[sel] = acc
    return gu
