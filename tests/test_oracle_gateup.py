"""Pins for the oracle's grouped gate_up products and epilogue.

int8 Hadamard-domain product: int8 card, model table row "Weights"; FP8 block
product: FP8 card, model table row "Weights". Pinned by pure-Python brute
force on tiny cases, a special case that reads out code columns, the
Cauchy-Schwarz bound against the dense unrotated product, and a library
GELU for the epilogue.
"""

import math

import numpy as np
import torch

import synth
from oracle import gateup, hadamard, numfmt, quant, router


def _tiny_case(seed=31, t_count=3, e_count=4, k=2, n_rows=6, k_dim=256):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((t_count, e_count)).astype(np.float32)
    x = numfmt.bf16_round(rng.standard_normal((t_count, k_dim)))
    codes = rng.integers(-127, 128, size=(e_count, n_rows, k_dim)).astype(np.int8)
    scales = numfmt.bf16_round(rng.uniform(1e-3, 1e-2, size=(e_count, n_rows, k_dim // 128)))
    r = router.route(lg, k)
    return x, codes, scales, r, k


def test_i8h_brute_force_python_loops():
    x, codes, scales, r, k = _tiny_case()
    gu = gateup.gateup_i8h(x, codes, scales, r["expert_off"], r["sorted_pairs"], k)
    off, sp = r["expert_off"], r["sorted_pairs"]
    e_count, n_rows, k_dim = codes.shape
    for e in range(e_count):
        for row in range(off[e], off[e + 1]):
            t = sp[row] // k
            for n in range(n_rows):
                total = 0.0
                for kk in range(k_dim):        # dense dequantized weight, one term at a time
                    total += float(scales[e, n, kk // 128]) * int(codes[e, n, kk]) * float(x[t, kk])
                assert math.isclose(gu[row, n], total, rel_tol=1e-12, abs_tol=1e-12)


def test_i8h_unit_vector_reads_code_columns():
    x, codes, scales, r, k = _tiny_case(seed=32)
    ones = np.ones_like(scales)
    j = 200
    xe = np.zeros_like(x)
    xe[:, j] = 1.0
    gu = gateup.gateup_i8h(xe, codes, ones, r["expert_off"], r["sorted_pairs"], k)
    e_of_row = np.searchsorted(r["expert_off"], np.arange(gu.shape[0]), side="right") - 1
    for row in range(gu.shape[0]):
        assert np.array_equal(gu[row], codes[e_of_row[row], :, j].astype(np.float64))


def test_i8h_rows_subset_matches_full():
    x, codes, scales, r, k = _tiny_case(seed=33)
    full = gateup.gateup_i8h(x, codes, scales, r["expert_off"], r["sorted_pairs"], k)
    rows = [4, 0, 5]
    part = gateup.gateup_i8h(x, codes, scales, r["expert_off"], r["sorted_pairs"], k, rows=rows)
    assert np.array_equal(part, full[rows])


def test_quantized_rotated_product_within_error_bound():
    # the tiny layer, end to end through the oracle: dense W x vs the Hadamard-domain product
    L = synth.layer("tiny")
    lg = synth.router_logits(L)
    x = synth.bf16_bits_to_f64(synth.activations_bf16(L))
    w = np.stack([synth.dense_weights(L, e) for e in range(L.E)]).astype(np.float64)
    w_rot = hadamard.rotate_blocks(w)
    codes, scales, _ = quant.quantize_i8h(w_rot)
    x_rot = hadamard.rotate_activations_bf16(x)
    r = router.route(lg, L.topk)
    gu = gateup.gateup_i8h(x_rot, codes, scales, r["expert_off"], r["sorted_pairs"], L.topk)
    w_hat = quant.dequantize_i8h(codes, scales)
    x_rot_exact = hadamard.rotate_blocks(x)
    off, sp = r["expert_off"], r["sorted_pairs"]
    for e in range(L.E):
        for row in range(off[e], off[e + 1]):
            t = sp[row] // L.topk
            y = w[e] @ x[t]                                          # unrotated dense product
            bound = (np.linalg.norm(w_rot[e] - w_hat[e], axis=1) * np.linalg.norm(x[t])
                     + np.linalg.norm(w_hat[e], axis=1) * np.linalg.norm(x_rot_exact[t] - x_rot[t]))
            assert np.all(np.abs(y - gu[row]) <= bound * (1 + 1e-9) + 1e-12)
    # and the quantized product is a close approximation overall
    rel = np.linalg.norm(gu - np.stack([w[np.searchsorted(off, i, 'right') - 1] @ x[sp[i] // L.topk]
                                          for i in range(gu.shape[0])])) / np.linalg.norm(gu)
    assert rel < 0.02


def test_gelu_closed_forms_and_library():
    g = np.linspace(-12, 12, 4001)
    assert gateup.gelu_tanh(np.array([0.0]))[0] == 0.0
    # 0.5 g (1 + tanh(z)) - 0.5 (-g)(1 + tanh(-z)) = g, since tanh is odd
    np.testing.assert_allclose(gateup.gelu_tanh(g) - gateup.gelu_tanh(-g), g, rtol=0, atol=1e-14)
    want = torch.nn.functional.gelu(torch.from_numpy(g), approximate="tanh").numpy()
    np.testing.assert_allclose(gateup.gelu_tanh(g), want, rtol=1e-14, atol=1e-15)


def test_epilogue_pairs_gate_with_up():
    gu = np.array([[1.0, -2.0, 3.0, 5.0]])
    act = gateup.epilogue(gu)
    want = torch.nn.functional.gelu(torch.tensor([1.0, -2.0], dtype=torch.float64), approximate="tanh").numpy() * [3.0, 5.0]
    np.testing.assert_allclose(act[0], want, rtol=1e-15)


def test_fp8_brute_force_python_loops():
    rng = np.random.default_rng(34)
    t_count, e_count, k, n_rows, k_dim = 3, 3, 2, 256, 256
    lg = rng.standard_normal((t_count, e_count)).astype(np.float32)
    x = numfmt.bf16_round(rng.standard_normal((t_count, k_dim)))
    w = rng.standard_normal((e_count, n_rows, k_dim)) * 0.02
    codes, scales = quant.quantize_fp8_blocks(w)
    qx, sx = quant.quantize_fp8_activations(x)
    r = router.route(lg, k)
    gu = gateup.gateup_fp8blk(qx, sx, codes, scales, r["expert_off"], r["sorted_pairs"], k)
    dq = numfmt.e4m3_decode(qx)
    dw = numfmt.e4m3_decode(codes)
    off, sp = r["expert_off"], r["sorted_pairs"]
    for e in range(e_count):
        for row in range(off[e], off[e + 1]):
            t = sp[row] // k
            for n in (0, 1, 127, 128, 200, 255):
                total = 0.0
                for kk in range(k_dim):
                    total += (float(scales[e, n // 128, kk // 128]) * float(sx[t, kk // 128])
                              * float(dw[e, n, kk]) * float(dq[t, kk]))
                assert math.isclose(gu[row, n], total, rel_tol=1e-12, abs_tol=1e-12)
    # the quantized product approximates the dense product
    for row in range(gu.shape[0]):
        e = np.searchsorted(off, row, "right") - 1
        y = w[e] @ x[sp[row] // k]
        assert np.linalg.norm(gu[row] - y) / np.linalg.norm(y) < 0.1
