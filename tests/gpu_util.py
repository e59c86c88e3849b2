"""Helpers shared by the GPU parity tests: tolerance checks, bf16 near-tie
analysis for the rotation, and device upload of generator data.

Tolerance for float32 outputs (gate_up and act) against the fp64 oracle:
elementwise |gpu - oracle| <= 1e-4 |oracle| + 1e-5.
"""

import numpy as np
import torch

from oracle import gateup, hadamard, numfmt, quant

RTOL, ATOL = 1e-4, 1e-5


def assert_close(gpu, ref, what, rtol=RTOL, atol=ATOL):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU values"
    err = np.abs(gpu - ref)
    lim = rtol * np.abs(ref) + atol
    bad = err > lim
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside |d| <= {rtol}|ref| + {atol}; "
                             f"worst ratio {np.max(err / lim):.3g}; first {idx.tolist()} "
                             f"gpu={gpu[tuple(idx[0])]!r} ref={ref[tuple(idx[0])]!r}")


def assert_close_nan(gpu, ref, what, rtol=RTOL, atol=ATOL):
    """assert_close where NaN is expected: NaN exactly where the oracle has
    NaN, the other values within the tolerance."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(gpu), nan), f"{what}: NaN positions differ"
    if (~nan).any():
        assert_close(gpu[~nan], ref[~nan], what, rtol, atol)


def cuda(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype) if t.dtype.itemsize == dtype.itemsize and t.dtype != dtype else t.to(dtype)
    return t.cuda()


def bf16_cuda(bits):
    """uint16 bf16 bit patterns (numpy) -> bf16 tensor on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def bf16_bits_of(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def fwht_tie_window(x):
    """Per-output bound on how far the float32 rotation (7 butterfly stages,
    one multiply by a rounded 1/sqrt(128)) can sit from the exact value:
    (7 + 2) * 2^-24 * sum_j |x_j| / sqrt(128), per 128-block, with margin."""
    xb = np.abs(np.asarray(x, dtype=np.float64)).reshape(x.shape[0], -1, 128)
    s = xb.sum(-1, keepdims=True) / np.sqrt(128.0)
    return np.broadcast_to(12 * 2.0 ** -24 * s, xb.shape).reshape(x.shape)


def near_tie_mask(exact, window):
    """True where the exact value lies within `window` of the midpoint
    between its two neighbouring bf16 values (where a float32 evaluation
    may round either way)."""
    ae = np.abs(np.asarray(exact, dtype=np.float64))
    ar = numfmt.bf16_round(ae)
    bits = numfmt.bf16_to_bits(ar).astype(np.int64)
    other_bits = np.where(ae >= ar, bits + 1, np.maximum(bits - 1, 0))
    other = numfmt.bf16_from_bits(other_bits.astype(np.uint16))
    mid = (ar + other) / 2
    return np.abs(ae - mid) <= window


def check_rotation(x_bits, y_bits):
    """GPU rotation y (bf16 bits) of x (bf16 bits) against the oracle: equal
    everywhere except where the float32 evaluation may legitimately round
    differently. The GPU value is the bf16 rounding of a float32 result within
    `fwht_tie_window` of the exact value, so any difference must satisfy
    |gpu - exact| <= window + half a bf16 step, and the exact value must lie
    within the window of a rounding midpoint. Returns the number of
    differences."""
    x = numfmt.bf16_from_bits(x_bits)
    exact = hadamard.rotate_blocks(x)
    want = numfmt.bf16_round(exact)
    got = numfmt.bf16_from_bits(y_bits)
    diff = got != want
    if not diff.any():
        return 0
    win = fwht_tie_window(x)
    tie = near_tie_mask(exact, win)
    assert np.all(tie[diff]), f"{(diff & ~tie).sum()} differences away from any rounding tie"
    mag = np.maximum(np.abs(got), np.abs(exact))[diff]
    half = np.ldexp(1.0, np.frexp(mag + 1e-300)[1] - 9)
    err = np.abs(got - exact)[diff]
    assert np.all(err <= win[diff] + half), "a difference beyond the float32 error bound"
    return int(diff.sum())


def check_with_rotation_slack(x, codes, sbits, r, topk, gu, act):
    """gate_up / act computed on the GPU from UNROTATED activations x (fp64
    values of bf16) against the oracle chain (rotate, round to bf16, grouped
    product, epilogue). The tolerance is the usual 1e-4 |ref| + 1e-5, widened
    only where the float32 rotation may round x_rot either way (one bf16 step
    there, carried through |W| to each output, and through gelu with
    |gelu'| < 1.13 to act)."""
    exact = hadamard.rotate_blocks(x)
    x_rot = numfmt.bf16_round(exact)
    scales = numfmt.bf16_from_bits(sbits)
    ref = gateup.gateup_i8h(x_rot, codes, scales, r["expert_off"], r["sorted_pairs"], topk)
    tie = near_tie_mask(exact, fwht_tie_window(x))
    ulp = np.ldexp(1.0, np.frexp(np.abs(x_rot) + 1e-300)[1] - 8)
    slack_x = np.where(tie, ulp, 0.0)
    off, sp = r["expert_off"], r["sorted_pairs"]
    what = quant.dequantize_i8h(codes, scales)
    slack = np.zeros_like(ref)
    for row in range(ref.shape[0]):
        e = np.searchsorted(off, row, side="right") - 1
        slack[row] = np.abs(what[e]) @ slack_x[sp[row] // topk]
    I = codes.shape[1] // 2
    if gu is not None:
        g = gu.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(g))
        assert np.all(np.abs(g - ref) <= 1e-4 * np.abs(ref) + 1e-5 + slack)
    if act is not None:
        ref_act = gateup.epilogue(ref)
        dg, du = slack[:, :I], slack[:, I:]
        act_slack = 1.13 * dg * (np.abs(ref[:, I:]) + du) + np.abs(gateup.gelu_tanh(ref[:, :I])) * du
        a = act.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(a))
        assert np.all(np.abs(a - ref_act) <= 1e-4 * np.abs(ref_act) + 1e-5 + act_slack)
