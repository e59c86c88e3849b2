"""GPU parity: hadamard128_rotate against the oracle rotation.

The oracle rounds the exact rotated value once to bf16; the GPU runs the
butterflies in float32 and rounds at the end. The two must agree everywhere
except where the exact value lies within the float32 error bound of a bf16
rounding midpoint; there the results must be adjacent bf16 values.
"""

import numpy as np
import pytest
import torch

import int8_hadamard_domain_amd as i8h
import synth
from tests.gpu_util import bf16_bits_of, bf16_cuda, check_rotation

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny", "decode", "verify", "prefill"])
def test_workload_activations(gpu_available, name):
    L = synth.layer(name)
    x = synth.activations_bf16(L)
    print(f"fwht {name} T={L.T} K={L.K}", flush=True)
    y = i8h.hadamard128_rotate(bf16_cuda(x))
    torch.cuda.synchronize()
    n = check_rotation(x, bf16_bits_of(y))
    assert n <= max(4, x.size // 2000)


@pytest.mark.parametrize("T,K", [(1, 128), (3, 384), (17, 4096), (129, 256), (2, 8192)])
def test_shapes(gpu_available, T, K):
    rng = np.random.default_rng(T * 10 + K)
    x = synth.to_bf16_bits((rng.standard_normal((T, K)) * np.exp(rng.uniform(-8, 8, (T, K)))).astype(np.float32))
    y = i8h.hadamard128_rotate(bf16_cuda(x))
    torch.cuda.synchronize()
    check_rotation(x, bf16_bits_of(y))


def test_in_place_and_strided(gpu_available):
    rng = np.random.default_rng(3)
    T, K, ld = 9, 512, 520
    full = synth.to_bf16_bits(rng.standard_normal((T, ld)).astype(np.float32))
    xt = bf16_cuda(full)
    ref_in = full[:, :K].copy()
    # strided input into a contiguous output
    y = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
    lib = i8h.lib()
    import ctypes
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = lib.hadamard128_rotate(ctypes.c_void_p(xt.data_ptr()), ld, ctypes.c_void_p(y.data_ptr()), K, T, K, st)
    assert rc == 0
    torch.cuda.synchronize()
    check_rotation(ref_in, bf16_bits_of(y))
    # padding columns of the strided source are untouched; in place over the strided rows
    rc = lib.hadamard128_rotate(ctypes.c_void_p(xt.data_ptr()), ld, ctypes.c_void_p(xt.data_ptr()), ld, T, K, st)
    assert rc == 0
    torch.cuda.synchronize()
    after = bf16_bits_of(xt)
    assert np.array_equal(after[:, K:], full[:, K:])
    check_rotation(ref_in, after[:, :K])


def test_special_values(gpu_available):
    x = np.zeros((4, 256), dtype=np.float32)
    x[1, :128] = 1.0                        # -> sqrt(128) e_0
    x[2, 5] = -3.0                          # -> a signed Hadamard column
    x[3] = np.linspace(-100, 100, 256)
    xb = synth.to_bf16_bits(x)
    y = i8h.hadamard128_rotate(bf16_cuda(xb))
    torch.cuda.synchronize()
    yb = bf16_bits_of(y)
    assert np.all(yb[0] == 0)
    check_rotation(xb, yb)
