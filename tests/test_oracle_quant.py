"""Pins for the oracle's quantizers.

int8: the int8 card's model table (row "Weights": int8 codes -127..127, one
bf16 scale per row and 128 of K, round to nearest with a scale search) and
recipe (symmetric clamp, search rule). FP8: the FP8 card (E4M3 per 128x128
block, bf16 scale). FP8 activations: one float32 scale per token and 128
values (the int8 12B card, header table row "Format").
"""

import json
import os

import numpy as np
import torch

from oracle import numfmt, quant

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _bf16_torch(x):
    """bf16 rounding by torch (float32 intermediate: exact for these inputs)."""
    return float(torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).double())


def _brute_force_group(w, factors):
    # pure-Python loops, independent of the vectorised oracle
    a = max(abs(v) for v in w)
    best = None
    for i, f in enumerate(factors):
        s = _bf16_torch(f * a / 127.0)
        q = [max(-127, min(127, round(v / s))) for v in w]   # round(): ties to even
        sse = sum((v - s * c) ** 2 for v, c in zip(w, q))
        if best is None or sse < best[0]:
            best = (sse, s, q, i)
    return best


def test_vectorised_matches_group_loop():
    rng = np.random.default_rng(11)
    w = rng.standard_normal((5, 6, 256)) * 0.02
    codes, scales, idx = quant.quantize_i8h(w)
    for a in range(5):
        for n in range(6):
            for g in range(2):
                s, q, i = quant.quantize_i8h_group(w[a, n, 128 * g:128 * (g + 1)])
                assert s == scales[a, n, g] and i == idx[a, n, g]
                assert np.array_equal(q, codes[a, n, 128 * g:128 * (g + 1)])


def test_brute_force_tiny_groups():
    rng = np.random.default_rng(12)
    for trial in range(12):
        w = rng.standard_normal(128) * 0.02
        if trial % 3 == 0:
            w[rng.integers(128)] *= 8.0       # an outlier makes shrinking pay
        codes, scales, idx = quant.quantize_i8h(w[None, :])
        sse, s, q, i = _brute_force_group(list(w), quant.SHRINK)
        assert scales[0, 0] == s and idx[0, 0] == i
        assert list(codes[0]) == q


def test_hand_computed_case():
    case = json.load(open(os.path.join(GOLD, "quant_i8h_case.json")))
    w = np.array([float.fromhex(v) for v in case["weights"]], dtype=np.float64)
    codes, scales, idx = quant.quantize_i8h(w[None, :])
    assert int(idx[0, 0]) == case["chosen_index"]
    assert scales[0, 0] == float.fromhex(case["scale"])
    assert list(codes[0]) == case["codes"]


def test_exact_group_keeps_full_scale():
    # all entries +-a with a/127 a power of two: f = 1 is exact, SSE 0, chosen first
    w = np.where(np.arange(128) % 3 == 0, -1.0, 1.0) * 127 * 2.0 ** -8
    codes, scales, idx = quant.quantize_i8h(w[None, :])
    assert idx[0, 0] == 0 and scales[0, 0] == 2.0 ** -8
    assert np.array_equal(codes[0], np.where(np.arange(128) % 3 == 0, -127, 127))


def test_invariants_on_random_layer():
    rng = np.random.default_rng(13)
    w = rng.standard_normal((4, 32, 512)) * 0.02
    w[0, 0, :128] = 0.0                                       # an all-zero group
    codes, scales, idx = quant.quantize_i8h(w)
    assert codes.dtype == np.int8 and codes.min() >= -127 and codes.max() <= 127
    assert np.array_equal(numfmt.bf16_round(scales), scales)  # stored scales are bf16
    assert scales[0, 0, 0] == 0 and np.all(codes[0, 0, :128] == 0)
    # the chosen candidate is never worse than the plain absmax scale (f = 1)
    g = w.reshape(4, 32, 4, 128)
    s_full = numfmt.bf16_round(np.max(np.abs(g), -1, keepdims=True) / 127)
    with np.errstate(divide="ignore", invalid="ignore"):
        q_full = np.where(s_full == 0, 0, np.clip(np.rint(g / s_full), -127, 127))
    sse_full = np.sum((g - s_full * q_full) ** 2, -1)
    what = quant.dequantize_i8h(codes, scales).reshape(4, 32, 4, 128)
    sse = np.sum((g - what) ** 2, -1)
    assert np.all(sse <= sse_full * (1 + 1e-12))
    # unclipped entries are within half a step of their code
    s = np.repeat(scales, 128, -1)
    inside = np.abs(codes) < 127
    err = np.abs(w - s * codes)
    assert np.all(err[inside] <= s[inside] / 2 * (1 + 1e-12))


def test_fp8_blocks_against_torch_cast():
    rng = np.random.default_rng(14)
    w = rng.standard_normal((2, 256, 256)).astype(np.float32) * np.float32(0.02)
    codes, scales = quant.quantize_fp8_blocks(w)
    assert scales.shape == (2, 2, 2)
    for e in range(2):
        for nb in range(2):
            for kb in range(2):
                blk = w[e, 128 * nb:128 * (nb + 1), 128 * kb:128 * (kb + 1)].astype(np.float64)
                s = _bf16_torch(np.max(np.abs(blk)) / 448.0)
                assert scales[e, nb, kb] == s
                ratio = blk / s
                # torch's cast rounds from float32; compare where float32 holds the ratio exactly
                r32 = ratio.astype(np.float32)
                exact = r32.astype(np.float64) == ratio
                sat = np.abs(ratio) > 448
                want = torch.from_numpy(np.clip(r32, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
                got = codes[e, 128 * nb:128 * (nb + 1), 128 * kb:128 * (kb + 1)]
                assert np.array_equal(got[exact | sat], want[exact | sat])
                # and everywhere the decoded value is the nearest E4M3 value of the ratio
                dec = numfmt.e4m3_decode(got)
                grid = numfmt.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
                near = np.min(np.abs(np.abs(ratio)[..., None] - grid[None, None, :]), -1)
                assert np.all(np.abs(np.abs(dec) - np.minimum(np.abs(ratio), 448)) <= near + 1e-12)


def test_fp8_block_dequantize_brute_force_and_bound():
    # W_hat[e, n, k] = s[e, n // 128, k // 128] * value of code[e, n, k]: each
    # element computed one by one, the code's value from torch's own E4M3FN
    # decoder (independent of the oracle's codec)
    rng = np.random.default_rng(16)
    w = rng.standard_normal((2, 256, 384)) * 0.02
    w[1, :128, 128:256] = 0.0                                # a zero block
    w[0, 5, 7] = 3.0                                         # a block with one large value
    codes, scales = quant.quantize_fp8_blocks(w)
    what = quant.dequantize_fp8_blocks(codes, scales)
    assert what.shape == w.shape
    tv = torch.from_numpy(codes.reshape(-1)).view(torch.float8_e4m3fn).to(torch.float64).numpy().reshape(codes.shape)
    rows = rng.integers(0, 256, 40)
    cols = rng.integers(0, 384, 40)
    for e in range(2):
        for n, k in zip(rows.tolist(), cols.tolist()):
            assert what[e, n, k] == scales[e, n // 128, k // 128] * float(tv[e, n, k])
    assert np.array_equal(what, np.repeat(np.repeat(scales, 128, -2), 128, -1) * tv)
    assert np.all(what[1, :128, 128:256] == 0)
    # round trip: within half an E4M3 step of w / s (steps: 2^(e - 3) for
    # normals, 2^-9 below 2^-6), times s; the block maximum itself is exact to
    # the scale's bf16 rounding (|w / s| lands within one E4M3 step of 448)
    sb = np.repeat(np.repeat(scales, 128, -2), 128, -1)
    nz = sb > 0
    r = np.abs(w[nz] / sb[nz])
    step = np.where(r >= 2.0 ** -6, np.ldexp(1.0, np.floor(np.log2(np.maximum(r, 2.0 ** -6))).astype(int) - 3),
                    2.0 ** -9)
    sat = r > 448
    err = np.abs(w[nz] - what[nz]) / sb[nz]
    assert np.all(err[~sat] <= step[~sat] / 2 * (1 + 1e-12))
    assert np.all(err[sat] <= r[sat] - 448 + 1e-12)


def test_fp8_zero_block():
    w = np.zeros((128, 128))
    codes, scales = quant.quantize_fp8_blocks(w)
    assert scales[0, 0] == 0 and np.all(codes == 0)


def test_fp8_activation_quantizer_against_float32_division():
    rng = np.random.default_rng(15)
    x = torch.from_numpy(rng.standard_normal((9, 512)).astype(np.float32)).to(torch.bfloat16)
    x[3, 128:256] = 0.0                                      # an all-zero group
    x[4, :128] *= 1e-30                                      # tiny values
    xd = x.double().numpy()
    codes, sx = quant.quantize_fp8_activations(xd)
    # float32 division by torch (IEEE single, correctly rounded)
    xf = x.float().reshape(9, 4, 128)
    amax = xf.abs().amax(-1, keepdim=True)
    sx_t = amax / torch.tensor(448.0, dtype=torch.float32)
    assert np.array_equal(sx, sx_t[..., 0].numpy())
    ratio = torch.where(sx_t == 0, torch.zeros_like(xf), xf / sx_t)
    want = ratio.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).reshape(9, 512).numpy()
    want = np.where(np.repeat(sx_t[..., 0].numpy(), 128, -1) == 0, 0, want)
    assert np.array_equal(codes, want)
