"""Pins for the W8A8 int8 g128 form (oracle/w8a8.py).

Source: "Gemma 4 12B-it · int8 · for radiance", header table row "Format"
and "How it was made", step 2. The activation quantizer is pinned by numpy's
IEEE float32 division for the scale, hand-derived round-half-to-even ties,
the half-step error bound, exact power-of-two scaling and zero groups; the
weight quantizer by torch's bf16 cast and the same properties; the product
by pure-Python brute force, by the identity with one dense matmul of the
dequantized operands, and by the quantization error bound against the
unquantized product.
"""

import math

import numpy as np
import torch

from oracle import numfmt, router, w8a8


def test_activation_scale_is_ieee_float32_division():
    rng = np.random.default_rng(0)
    x = numfmt.bf16_round(rng.standard_normal((16, 1024)) * 10.0 ** rng.uniform(-6, 4, (16, 1)))
    _, sx = w8a8.quantize_i8_activations(x)
    amax = np.abs(x.reshape(16, 8, 128)).max(axis=-1).astype(np.float32)   # exact: bf16 values
    np.testing.assert_array_equal(sx, amax / np.float32(127))               # numpy float32 division


def test_activation_ties_round_to_even():
    # amax = 127 gives sx = 1 exactly, so x / sx = x and the ties are the inputs'
    row = np.zeros(128)
    row[:8] = [127.0, 2.5, 3.5, -2.5, 0.5, -0.5, 126.5, -1.5]
    q, sx = w8a8.quantize_i8_activations(row[None, :])
    assert sx[0, 0] == 1.0
    assert q[0, :8].tolist() == [127, 2, 4, -2, 0, 0, 126, -2]


def test_activation_codes_properties():
    rng = np.random.default_rng(1)
    x = numfmt.bf16_round(rng.standard_normal((8, 512)) * 3.0)
    x[2, 128:256] = 0.0                                     # an all-zero group
    q, sx = w8a8.quantize_i8_activations(x)
    assert q.dtype == np.int8 and np.abs(q.astype(int)).max() <= 127
    g = x.reshape(8, 4, 128)
    qg = q.astype(np.float64).reshape(8, 4, 128)
    s = sx.astype(np.float64)
    assert s[2, 1] == 0 and not qg[2, 1].any()
    live = s > 0
    err = np.abs(g - s[..., None] * qg)
    # round-to-nearest of the float32 quotient: half a step, plus the quotient's own
    # rounding (at most half an ulp of 127 in float32, i.e. 127 * 2^-24 steps)
    assert np.all(err[live] <= (s[live] * (0.5 + 127 * 2.0 ** -24) * (1 + 1e-12))[:, None])
    idx = np.abs(g).argmax(axis=-1)
    top = np.take_along_axis(qg, idx[..., None], axis=-1)[..., 0]
    np.testing.assert_array_equal(np.abs(top[live]), 127)


def test_activation_power_of_two_scaling():
    rng = np.random.default_rng(2)
    x = numfmt.bf16_round(rng.standard_normal((4, 256)))
    q1, s1 = w8a8.quantize_i8_activations(x)
    q2, s2 = w8a8.quantize_i8_activations(x * 2.0 ** -7)
    np.testing.assert_array_equal(q1, q2)
    np.testing.assert_array_equal(s2, s1 * np.float32(2.0 ** -7))


def test_weight_quantizer_against_torch_bf16_cast():
    rng = np.random.default_rng(3)
    w = rng.standard_normal((2, 16, 384)) * 0.02
    w[1, 5, :128] = 0.0
    q, s = w8a8.quantize_i8g_weights(w)
    amax = np.abs(w.reshape(2, 16, 3, 128)).max(axis=-1)
    ref = torch.from_numpy(amax / 127).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(s, ref)
    assert s[1, 5, 0] == 0 and not q[1, 5, :128].any()
    qg = q.astype(np.float64).reshape(2, 16, 3, 128)
    g = w.reshape(2, 16, 3, 128)
    live = s > 0
    ratio = np.where(live[..., None], np.abs(g) / np.where(live, s, 1.0)[..., None], 0.0)
    err = np.abs(g - s[..., None] * qg)
    unclamped = ratio < 127.5
    bound = np.broadcast_to((s / 2)[..., None], g.shape)
    assert np.all(err[unclamped] <= bound[unclamped] * (1 + 1e-12))
    assert np.abs(q.astype(int)).max() <= 127


def _tiny_case(seed=41, t_count=3, e_count=4, k=2, n_rows=6, k_dim=256):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((t_count, e_count)).astype(np.float32)
    x = numfmt.bf16_round(rng.standard_normal((t_count, k_dim)))
    qx, sx = w8a8.quantize_i8_activations(x)
    codes = rng.integers(-127, 128, size=(e_count, n_rows, k_dim)).astype(np.int8)
    scales = numfmt.bf16_round(rng.uniform(1e-3, 1e-2, size=(e_count, n_rows, k_dim // 128)))
    r = router.route(lg, k)
    return qx, sx, codes, scales, r, k


def test_product_brute_force_python_loops():
    qx, sx, codes, scales, r, k = _tiny_case()
    gu = w8a8.gateup_i8g(qx, sx, codes, scales, r["expert_off"], r["sorted_pairs"], k)
    off, sp = r["expert_off"], r["sorted_pairs"]
    e_count, n_rows, k_dim = codes.shape
    for e in range(e_count):
        for row in range(off[e], off[e + 1]):
            t = sp[row] // k
            for n in range(n_rows):
                total = 0.0
                for kk in range(k_dim):        # both operands dequantized, one term at a time
                    total += (float(scales[e, n, kk // 128]) * int(codes[e, n, kk])) * \
                             (float(sx[t, kk // 128]) * int(qx[t, kk]))
                assert math.isclose(gu[row, n], total, rel_tol=1e-12, abs_tol=1e-15)


def test_product_equals_one_dense_matmul_of_dequantized_operands():
    qx, sx, codes, scales, r, k = _tiny_case(seed=42, t_count=9, e_count=5, k=3, n_rows=16, k_dim=512)
    gu = w8a8.gateup_i8g(qx, sx, codes, scales, r["expert_off"], r["sorted_pairs"], k)
    xd = torch.from_numpy(np.repeat(sx.astype(np.float64), 128, axis=1) * qx)          # [T, K]
    off, sp = r["expert_off"], r["sorted_pairs"]
    for e in range(codes.shape[0]):
        wd = torch.from_numpy(np.repeat(scales[e], 128, axis=1) * codes[e])            # [N, K]
        rows = np.arange(off[e], off[e + 1])
        if rows.size == 0:
            continue
        ref = (xd[torch.from_numpy(sp[rows] // k)] @ wd.T).numpy()
        np.testing.assert_allclose(gu[rows], ref, rtol=1e-12, atol=1e-15)


def test_rows_subset_matches_full():
    qx, sx, codes, scales, r, k = _tiny_case(seed=43, t_count=7)
    full = w8a8.gateup_i8g(qx, sx, codes, scales, r["expert_off"], r["sorted_pairs"], k)
    rows = np.array([0, 3, 5, full.shape[0] - 1])
    part = w8a8.gateup_i8g(qx, sx, codes, scales, r["expert_off"], r["sorted_pairs"], k, rows=rows)
    np.testing.assert_array_equal(part, full[rows])


def test_quantized_product_within_error_bound_of_the_dense_one():
    rng = np.random.default_rng(44)
    t_count, e_count, k, n_rows, k_dim = 6, 3, 2, 32, 1024
    x = numfmt.bf16_round(rng.standard_normal((t_count, k_dim)))
    w = rng.standard_normal((e_count, n_rows, k_dim)) * 0.02
    qx, sx = w8a8.quantize_i8_activations(x)
    codes, scales = w8a8.quantize_i8g_weights(w)
    r = router.route(rng.standard_normal((t_count, e_count)).astype(np.float32), k)
    gu = w8a8.gateup_i8g(qx, sx, codes, scales, r["expert_off"], r["sorted_pairs"], k)
    off, sp = r["expert_off"], r["sorted_pairs"]
    ex = np.repeat(sx.astype(np.float64) * (0.5 + 127 * 2.0 ** -24), 128, axis=1)  # per-element bounds
    worst = 0.0
    for e in range(e_count):
        ew = np.repeat(scales[e] / 2, 128, axis=1)
        ew = np.maximum(ew, np.abs(w[e] - np.repeat(scales[e], 128, axis=1) * codes[e]))   # clamped elements
        for row in range(off[e], off[e + 1]):
            t = sp[row] // k
            exact = w[e] @ x[t]
            bound = (np.abs(x[t])[None, :] * ew + np.abs(w[e]) * ex[t][None, :] + ew * ex[t][None, :]).sum(axis=1)
            assert np.all(np.abs(gu[row] - exact) <= bound * (1 + 1e-9))
            worst = max(worst, np.abs(gu[row] - exact).max())
    assert worst > 0                                       # the codes do round
