"""Pins for the drafter's dense int8 linears with f16 scales (oracle/dense.py)
and the binary16 codec (oracle/numfmt.py).

Source: int8 card, model table row "Speculator" and the recipe lines
`rtn codes=i8 group=128 scale=f16 clamp=sym` (section "How this file was
made"). The codec is pinned against numpy's float16 cast and bit views; the
quantizer by the properties round-to-nearest must have (error within half a
step, the group maximum at +-127, zero groups, f16-representable scales equal
to numpy's cast of amax / 127); the product by pure-Python brute force, a
one-hot read-out of the dequantized weights, and the RTN error bound against
the dense product.
"""

import numpy as np

from oracle import dense, numfmt


def test_f16_round_matches_numpy_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.uniform(-9, 5, 20000),
        [0.0, -0.0, 65504.0, 65519.99, 65520.0, -70000.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26,
         1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 2.0 ** -14 - 2.0 ** -25],
    ])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).astype(np.float64)
    np.testing.assert_array_equal(numfmt.f16_round(x), ref)


def test_f16_bits_round_trip_against_numpy_views():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 16, 50000).astype(np.uint16)
    bits = bits[(bits & 0x7C00) != 0x7C00]                 # finite values only
    vals = bits.view(np.float16).astype(np.float64)
    np.testing.assert_array_equal(numfmt.f16_from_bits(bits), vals)
    nz = vals != 0                                        # the sign of zero is kept; compare where nonzero
    np.testing.assert_array_equal(numfmt.f16_to_bits(vals[nz]), bits[nz])
    assert numfmt.f16_to_bits(np.array([np.inf]))[0] == 0x7C00


def test_quantizer_properties():
    rng = np.random.default_rng(2)
    w = rng.standard_normal((16, 512)) * 0.02
    w[3, 128:256] = 0.0                                  # an all-zero group
    q, s = dense.quantize_i8_f16(w)
    assert q.dtype == np.int8 and np.abs(q.astype(int)).max() <= 127
    g = w.reshape(16, 4, 128)
    qg = q.astype(np.float64).reshape(16, 4, 128)
    assert s[3, 1] == 0 and not qg[3, 1].any()
    amax = np.abs(g).max(axis=-1)
    ref_s = (amax / 127).astype(np.float16).astype(np.float64)        # numpy's cast
    np.testing.assert_array_equal(s, ref_s)
    np.testing.assert_array_equal(numfmt.f16_round(s), s)
    live = s > 0
    err = np.abs(g - s[..., None] * qg)
    assert np.all(err[live] <= s[live][:, None] / 2 * (1 + 1e-12) + 1e-300)
    # the largest element of each group lands on +-127
    idx = np.abs(g).argmax(axis=-1)
    top = np.take_along_axis(qg, idx[..., None], axis=-1)[..., 0]
    np.testing.assert_array_equal(np.abs(top[live]), 127)


def test_linear_brute_force_python_loops():
    rng = np.random.default_rng(3)
    t_count, n_rows, k_dim = 2, 3, 256
    codes = rng.integers(-127, 128, size=(n_rows, k_dim)).astype(np.int8)
    scales = numfmt.f16_round(rng.uniform(1e-4, 1e-2, size=(n_rows, k_dim // 128)))
    x = numfmt.bf16_round(rng.standard_normal((t_count, k_dim)))
    y = dense.linear_i8_f16(x, codes, scales)
    for t in range(t_count):
        for n in range(n_rows):
            total = 0.0
            for kk in range(k_dim):
                total += float(scales[n, kk // 128]) * int(codes[n, kk]) * float(x[t, kk])
            assert abs(y[t, n] - total) <= 1e-12 * (1 + abs(total))


def test_one_hot_reads_out_the_dequantized_weights():
    rng = np.random.default_rng(4)
    w = rng.standard_normal((8, 384)) * 0.05
    q, s = dense.quantize_i8_f16(w)
    x = np.eye(384)[[0, 127, 128, 200, 383]]
    y = dense.linear_i8_f16(x, q, s)
    for row, kk in enumerate([0, 127, 128, 200, 383]):
        np.testing.assert_array_equal(y[row], s[:, kk // 128] * q[:, kk])


def test_rtn_error_bound_against_the_dense_product():
    rng = np.random.default_rng(5)
    w = rng.standard_normal((32, 1024)) * 0.02
    x = numfmt.bf16_round(rng.standard_normal((4, 1024)))
    q, s = dense.quantize_i8_f16(w)
    y = dense.linear_i8_f16(x, q, s)
    exact = x @ w.T
    bound = (np.abs(x).reshape(4, 1, 8, 128).sum(-1) * (s[None] / 2)).sum(-1)
    assert np.all(np.abs(y - exact) <= bound * (1 + 1e-9))
    assert np.abs(y - exact).max() > 0                   # the bound is not vacuous: codes do round
