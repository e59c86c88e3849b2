"""GPU parity: linear_i8f16 (the drafter's dense int8 linears with f16 group
scales) against the oracle.

Elementwise |gpu - oracle| <= 1e-4 |oracle| + 1e-5 on y [T, N]. Small cases
quantize dense N(0, 0.02^2) weights with the oracle's RTN quantizer; the
full-size stand-in (16 tokens, K = 2048, N = 4096) uses generator codes and is
compared in full. Cases cover one group (three idle waves), more groups than
one batch per wave, token counts below, at and above the 16-token tile
(ragged), zero-scale groups with nonzero codes, f16 subnormal and large
scales, and T = 0.
"""

import numpy as np
import pytest
import torch

import int8_hadamard_domain_amd as i8h
import synth
from oracle import dense, numfmt
from tests.gpu_util import assert_close, bf16_cuda

pytestmark = pytest.mark.gpu


def f16_cuda(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.float16).cuda()


def run(xbits, codes, sbits):
    y = i8h.linear_i8f16(bf16_cuda(xbits), torch.from_numpy(np.ascontiguousarray(codes)).cuda(), f16_cuda(sbits))
    torch.cuda.synchronize()
    return y.cpu().numpy()


def quantized(n_rows, k_dim, seed):
    w = np.random.default_rng(seed).standard_normal((n_rows, k_dim)) * 0.02
    q, s = dense.quantize_i8_f16(w)
    return q, numfmt.f16_to_bits(s)


@pytest.mark.parametrize("T,K,N,seed", [(1, 128, 16, 0), (5, 256, 48, 1), (16, 512, 64, 2), (17, 384, 32, 3),
                                        (33, 1024, 64, 4), (16, 4096, 256, 5), (3, 2048, 112, 6),
                                        (20, 2560, 48, 8)])
def test_linear_small(T, K, N, seed):
    q, sbits = quantized(N, K, seed)
    xbits = synth.drafter_activations_bf16(T, K, seed)
    ref = dense.linear_i8_f16(synth.bf16_bits_to_f64(xbits), q, numfmt.f16_from_bits(sbits))
    assert_close(run(xbits, q, sbits), ref, f"linear T{T} K{K} N{N}")


def test_zero_scale_groups_and_extreme_scales():
    T, K, N = 9, 512, 32
    rng = np.random.default_rng(7)
    q = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    s = rng.uniform(1e-4, 1e-2, size=(N, K // 128))
    s[0, 1] = 0.0                         # nonzero codes, zero scale: the group adds nothing
    s[1, :] = 2.0 ** -20                  # f16 subnormals
    s[2, :] = 3.0e3                       # large scales
    sbits = numfmt.f16_to_bits(numfmt.f16_round(s))
    xbits = synth.drafter_activations_bf16(T, K, 7)
    ref = dense.linear_i8_f16(synth.bf16_bits_to_f64(xbits), q, numfmt.f16_from_bits(sbits))
    assert_close(run(xbits, q, sbits), ref, "linear extreme scales")


def test_full_size_stand_in_and_repeatability():
    d = synth.DRAFTER
    q, sbits = synth.synthetic_i8f16(d["N"], d["K"], d["seed"])
    xbits = synth.drafter_activations_bf16(d["T"], d["K"], d["seed"])
    y1 = run(xbits, q, sbits)
    y2 = run(xbits, q, sbits)
    np.testing.assert_array_equal(y1, y2)
    ref = dense.linear_i8_f16(synth.bf16_bits_to_f64(xbits), q, numfmt.f16_from_bits(sbits))
    assert_close(y1, ref, "linear drafter stand-in")


def test_zero_tokens_is_a_no_op():
    y = i8h.linear_i8f16(torch.empty((0, 256), dtype=torch.bfloat16, device="cuda"),
                         torch.zeros((32, 256), dtype=torch.int8, device="cuda"),
                         torch.zeros((32, 2), dtype=torch.float16, device="cuda"))
    assert y.shape == (0, 32)
