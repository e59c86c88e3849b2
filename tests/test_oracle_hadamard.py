"""Pins for the oracle's 128-wide Hadamard rotation.

The int8 card puts the experts' gate_up codes in the 128-wide Hadamard
domain (model table, row "Weights"; recipe transform fwht128). Pinned by the
defining identities of a Sylvester-Hadamard matrix, an independent Kronecker
construction, the dense product, and orthogonality.
"""

import numpy as np

from oracle import hadamard, numfmt


def _kron_build(n):
    # H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]]
    h = np.array([[1]], dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def test_h_times_ht_is_128_identity():
    h = hadamard.sylvester()
    assert h.dtype == np.int64
    assert np.array_equal(h @ h.T, 128 * np.eye(128, dtype=np.int64))


def test_matches_kronecker_recursion():
    assert np.array_equal(hadamard.sylvester(), _kron_build(128))


def test_known_rows():
    h = hadamard.sylvester()
    assert np.all(h[0] == 1) and np.all(h[:, 0] == 1)
    assert np.array_equal(h[1], np.tile([1, -1], 64))
    assert np.array_equal(h[2], np.tile([1, 1, -1, -1], 32))
    assert np.array_equal(h[64], np.concatenate([np.ones(64), -np.ones(64)]))
    parity = np.array([bin(j).count("1") % 2 for j in range(128)])
    assert np.array_equal(h[127], np.where(parity == 0, 1, -1))


def test_fwht_of_unit_vectors_is_columns():
    h = hadamard.sylvester()
    eye = np.eye(128)
    assert np.array_equal(hadamard.fwht(eye), h.T.astype(np.float64))  # row j of result = column j


def test_fwht_equals_dense_product():
    rng = np.random.default_rng(1)
    v = rng.integers(-1000, 1000, size=(37, 128)).astype(np.float64)  # integers: exact
    assert np.array_equal(hadamard.fwht(v), v @ hadamard.sylvester().T)


def test_fwht_of_ones():
    y = hadamard.fwht(np.ones(128))
    assert y[0] == 128 and np.all(y[1:] == 0)


def test_normalised_rotation_is_involution_and_orthogonal():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((16, 512))
    y = hadamard.rotate_blocks(x)
    np.testing.assert_allclose(hadamard.rotate_blocks(y), x, rtol=0, atol=1e-13)
    # block norms and dot products are preserved
    xb = x.reshape(16, 4, 128)
    yb = y.reshape(16, 4, 128)
    np.testing.assert_allclose(np.linalg.norm(yb, axis=-1), np.linalg.norm(xb, axis=-1), rtol=1e-13)
    a, b = xb[0], xb[1]
    ra, rb = yb[0], yb[1]
    np.testing.assert_allclose(np.sum(ra * rb, -1), np.sum(a * b, -1), rtol=1e-12, atol=1e-12)


def test_blocks_are_independent():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((3, 384))
    y = hadamard.rotate_blocks(x)
    for b in range(3):
        np.testing.assert_allclose(y[:, 128 * b:128 * (b + 1)],
                                   hadamard.rotate_blocks(x[:, 128 * b:128 * (b + 1)]), atol=0)


def test_weight_and_activation_rotation_preserve_products():
    # W x == (W H) (H x) with H orthonormal and symmetric
    rng = np.random.default_rng(4)
    w = rng.standard_normal((64, 256))
    x = rng.standard_normal(256)
    lhs = w @ x
    rhs = hadamard.rotate_blocks(w) @ hadamard.rotate_blocks(x)
    np.testing.assert_allclose(rhs, lhs, rtol=1e-12, atol=1e-12)


def test_activation_rotation_rounds_exact_value_once():
    rng = np.random.default_rng(5)
    x = numfmt.bf16_round(rng.standard_normal((8, 256)))
    got = hadamard.rotate_activations_bf16(x)
    h = hadamard.sylvester().astype(np.float64) / np.sqrt(128.0)
    exact = (x.reshape(8, 2, 128) @ h.T).reshape(8, 256)
    # result is bf16 and within half a bf16 ulp of the exact value
    assert np.array_equal(numfmt.bf16_round(got), got)
    ulp = np.ldexp(1.0, np.frexp(np.abs(exact))[1] - 8)
    assert np.all(np.abs(got - exact) <= ulp / 2 * (1 + 1e-12))
