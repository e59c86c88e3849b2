"""Dense int8 linears with an f16 scale per row and 128 of K (fp64).

Test infrastructure: only the tests, the package smoke check and the bench's
CPU baseline use this module; the GPU path never does.

The int8 card, model table row "Speculator": the DFlash drafter's linears
and head are int8 with an f16 scale per row and 128 of K; its recipe lines
(section "How this file was made") give them `rtn codes=i8 group=128
scale=f16 clamp=sym` with no transform and no search rule. Readings:
  * per row n and group g of 128 along K: s = f16(amax / 127), rounded
    before the codes are formed (the stored scale is the one used);
  * q = round half to even of w / s, clamped to [-127, 127]; an all-zero
    group stores s = 0 and q = 0;
  * the linear takes bf16 activations x [T, K] unrotated:
        y[t, n] = sum_g s[n, g] * sum_{k in g} q[n, k] * x[t, k].
Inner sums are exact in fp64; the outer sum rounds at fp64.
"""

import numpy as np

from .numfmt import f16_round

GROUP = 128
QMAX = 127


def quantize_i8_f16(w):
    """w [N, K] -> (codes int8 [N, K], scales fp64 [N, K/128] holding f16 values)."""
    w = np.asarray(w, dtype=np.float64)
    n_rows, k_dim = w.shape
    g = w.reshape(n_rows, k_dim // GROUP, GROUP)
    s = f16_round(np.abs(g).max(axis=-1) / QMAX)
    safe = np.where(s > 0, s, 1.0)
    q = np.clip(np.rint(g / safe[..., None]), -QMAX, QMAX)
    q = np.where(s[..., None] > 0, q, 0.0)
    return q.reshape(n_rows, k_dim).astype(np.int8), s


def linear_i8_f16(x, codes, scales):
    """y [T, N] = per-group scaled int8 products with x [T, K] (fp64 values)."""
    x = np.asarray(x, dtype=np.float64)
    q = np.asarray(codes, dtype=np.float64)
    n_rows, k_dim = q.shape
    g = k_dim // GROUP
    # per group: [T, N] partial products, then weighted by that group's scales
    xg = x.reshape(x.shape[0], g, GROUP)
    qg = q.reshape(n_rows, g, GROUP)
    part = np.einsum("tgk,ngk->tng", xg, qg)
    return (part * np.asarray(scales, dtype=np.float64)[None, :, :]).sum(axis=-1)
