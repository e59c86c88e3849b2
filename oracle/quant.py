"""Offline weight quantizers and the FP8 activation quantizer (fp64).

int8 Hadamard-domain codes. The int8 card, model table row "Weights": the
routed experts' gate_up weights are int8 codes in -127..127, in the 128-wide
Hadamard domain, one bf16 scale per row and per 128 of K, rounded to nearest
with a scale search; its recipe (section "How this file was made") adds a
symmetric clamp. The cards do not print the search, so these readings hold:
  * candidates: the group's absolute maximum shrunk by f in 1.00, 0.98, ...,
    0.80 (eleven steps of 0.02), divided by 127;
  * each candidate scale is rounded to bf16 BEFORE the codes are formed and
    scored, so the score is that of what is stored;
  * codes: round half to even of w / s, clamped to [-127, 127];
  * objective: sum of squared errors in the rotated domain; ties keep the
    earlier candidate (the larger f);
  * an all-zero group stores s = 0 and q = 0.

FP8 block codes. The FP8 card, model table row "Weights" and its recipe:
E4M3 per 128x128 block with a bf16 scale per block. Reading: s = bf16 of
blockmax / 448, codes = E4M3 of w / s with saturation; an all-zero block
stores s = 0 and q = 0.

FP8 activations. The FP8 card gives bf16 activations; a native FP8 product
needs FP8 activations too. Reading (precedent: the int8 12B card and the
int5 31B card, header table row "Format", one activation scale per token and
128 values): per token and per 128 of K, sx = amax / 448 as a float32
(IEEE single division: the fp64 quotient of two float32 values rounded once
to float32 is that quotient), qx = E4M3 (nearest even, saturating) of the
float32 quotient x / sx; a group with sx == 0 stores qx = 0.
"""

import numpy as np

from .numfmt import bf16_round, e4m3_encode_sat, e4m3_decode

GROUP = 128
QMAX = 127
SHRINK = tuple((100 - 2 * i) / 100.0 for i in range(11))  # 1.00 .. 0.80


def quantize_i8h_group(w, factors=SHRINK):
    """One group of rotated weights (fp64, any length) -> (scale, codes, i*).

    Plain loop over the candidate factors, as the search is described.
    """
    w = np.asarray(w, dtype=np.float64)
    a = np.max(np.abs(w))
    if a == 0:
        return 0.0, np.zeros(w.shape, dtype=np.int8), 0
    best = None
    for i, f in enumerate(factors):
        s = float(bf16_round(f * a / QMAX))
        if s == 0.0:
            q = np.zeros(w.shape)
        else:
            q = np.clip(np.rint(w / s), -QMAX, QMAX)
        sse = float(np.sum((w - s * q) ** 2))
        if best is None or sse < best[0]:
            best = (sse, s, q, i)
    _, s, q, i = best
    return s, q.astype(np.int8), i


def quantize_i8h(w_rot, factors=SHRINK):
    """Rotated weights [..., N, K] -> (codes int8 [..., N, K], scales fp64
    [..., N, K/128] holding bf16 values, chosen factor index [..., N, K/128]).

    Vectorised over groups; the per-group arithmetic is that of
    quantize_i8h_group (the tests check the two agree).
    """
    w_rot = np.asarray(w_rot, dtype=np.float64)
    k = w_rot.shape[-1]
    assert k % GROUP == 0
    g = w_rot.reshape(w_rot.shape[:-1] + (k // GROUP, GROUP))
    a = np.max(np.abs(g), axis=-1, keepdims=True)
    best_sse = np.full(a.shape, np.inf)
    best_s = np.zeros(a.shape)
    best_q = np.zeros(g.shape)
    best_i = np.zeros(a.shape, dtype=np.int64)
    for i, f in enumerate(factors):
        s = bf16_round(f * a / QMAX)
        with np.errstate(divide="ignore", invalid="ignore"):
            q = np.where(s == 0, 0.0, np.clip(np.rint(g / s), -QMAX, QMAX))
        sse = np.sum((g - s * q) ** 2, axis=-1, keepdims=True)
        better = sse < best_sse          # strict: ties keep the earlier f
        best_sse = np.where(better, sse, best_sse)
        best_s = np.where(better, s, best_s)
        best_i = np.where(better, i, best_i)
        best_q = np.where(better, q, best_q)
    zero = a == 0
    best_s = np.where(zero, 0.0, best_s)
    best_q = np.where(zero, 0.0, best_q)
    codes = best_q.reshape(w_rot.shape).astype(np.int8)
    return codes, best_s[..., 0], best_i[..., 0]


def dequantize_i8h(codes, scales):
    """W_hat[..., n, k] = s[..., n, k // 128] * q[..., n, k] (fp64)."""
    codes = np.asarray(codes, dtype=np.float64)
    s = np.repeat(np.asarray(scales, dtype=np.float64), GROUP, axis=-1)
    return s * codes


def quantize_fp8_blocks(w):
    """Weights [..., N, K] (N, K multiples of 128) -> (E4M3 codes uint8
    [..., N, K], scales fp64 [..., N/128, K/128] holding bf16 values)."""
    w = np.asarray(w, dtype=np.float64)
    n, k = w.shape[-2:]
    assert n % GROUP == 0 and k % GROUP == 0
    lead = w.shape[:-2]
    b = w.reshape(lead + (n // GROUP, GROUP, k // GROUP, GROUP))
    amax = np.max(np.abs(b), axis=(-3, -1), keepdims=True)
    s = bf16_round(amax / 448.0)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(s == 0, 0.0, b / s)
    codes = e4m3_encode_sat(ratio).reshape(w.shape)
    return codes, s[..., :, 0, :, 0]


def dequantize_fp8_blocks(codes, scales):
    """W_hat = s[block] * decode(q) (fp64)."""
    v = e4m3_decode(codes)
    s = np.asarray(scales, dtype=np.float64)
    s = np.repeat(np.repeat(s, GROUP, axis=-2), GROUP, axis=-1)
    return s * v


def quantize_fp8_activations(x):
    """bf16 activations [T, K] (fp64 values) -> (E4M3 codes uint8 [T, K],
    float32 scales [T, K/128])."""
    x = np.asarray(x, dtype=np.float64)
    t, k = x.shape
    g = x.reshape(t, k // GROUP, GROUP)
    amax = np.max(np.abs(g), axis=-1, keepdims=True)
    sx = (amax / 448.0).astype(np.float32)            # one rounding to float32
    sx64 = sx.astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio32 = np.where(sx64 == 0, 0.0, g / sx64).astype(np.float32)
    codes = e4m3_encode_sat(ratio32.astype(np.float64))
    codes = np.where(sx64 == 0, np.uint8(0), codes)
    return codes.reshape(t, k).astype(np.uint8), sx[..., 0]
