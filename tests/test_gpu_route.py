"""GPU parity: moe_route_permute against the oracle's routing.

ids, expert_off, sorted_pairs and pair_pos must match bit for bit; the
softmax weights within 1e-4 relative + 1e-5 absolute. Covers the single-block
path (T <= 4) and the three-kernel path, ties, skewed loads, the largest
expert count and top-k the ABI accepts, and expert counts that are not a
multiple of the wavefront.
"""

import numpy as np
import pytest
import torch

import int8_hadamard_domain_amd as i8h
import synth
from oracle import router
from tests.gpu_util import assert_close, assert_close_nan

pytestmark = pytest.mark.gpu


def _run_and_compare(lg, k, nan_weights=False):
    print(f"route T={lg.shape[0]} E={lg.shape[1]} k={k}", flush=True)
    ref = router.route(lg, k)
    out = i8h.moe_route_permute(torch.from_numpy(lg).cuda(), k)
    torch.cuda.synchronize()
    for key in ("topk_ids", "expert_off", "sorted_pairs", "pair_pos"):
        got = out[key].cpu().numpy()
        want = ref["ids" if key == "topk_ids" else key]
        assert np.array_equal(got, want.reshape(got.shape)), key
    if nan_weights:
        assert_close_nan(out["topk_w"].cpu().numpy(), ref["weights"], "topk_w")
    else:
        assert_close(out["topk_w"].cpu().numpy(), ref["weights"], "topk_w")


@pytest.mark.parametrize("name", ["tiny", "decode", "verify", "prefill", "fp8"])
def test_workloads(gpu_available, name):
    L = synth.layer(name)
    _run_and_compare(synth.router_logits(L), L.topk)


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (3, 64, 32), (4, 1024, 32), (5, 100, 7),
                                   (37, 300, 5), (300, 2, 1), (1000, 1024, 32), (257, 128, 8)])
def test_shapes(gpu_available, T, E, k):
    rng = np.random.default_rng(T * 7919 + E * 31 + k)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    _run_and_compare(lg, k)


def test_ties_and_equal_rows(gpu_available):
    rng = np.random.default_rng(5)
    lg = np.round(rng.standard_normal((200, 128)), 1).astype(np.float32)  # heavy ties
    lg[7] = 0.25                                                           # a fully tied row
    lg[8] = -0.0
    lg[8, ::3] = 0.0                                                       # +0 and -0 tie
    _run_and_compare(lg, 8)
    _run_and_compare(lg[:3], 8)                                            # small path


def test_skew_all_to_one_expert(gpu_available):
    lg = np.zeros((600, 64), dtype=np.float32)
    lg[:, 5] = 10.0
    lg[:, 9] = 5.0
    _run_and_compare(lg, 2)


@pytest.mark.parametrize("T", [3, 40])
def test_nan_logits(gpu_available, T):
    # NaN ranks after every number (-inf included), NaNs by index: ids stay
    # valid experts, so nothing downstream indexes out of range. T = 3 takes
    # the single-block path, T = 40 the three-kernel path.
    rng = np.random.default_rng(31 + T)
    E, k = 128, 8
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[0] = np.nan                                  # a row of NaNs only
    lg[1, rng.choice(E, 20, replace=False)] = np.nan
    lg[1, [3, 50]] = 9.0                            # large values beside NaNs
    lg[2, :64] = -np.inf
    lg[2, 64:] = np.nan                             # -inf before NaN
    if T > 3:
        lg[3:, ::5] = np.nan                        # NaNs in every row
        lg[5, :] = np.nan
    _run_and_compare(lg, k, nan_weights=True)


@pytest.mark.parametrize("T,E,k,K", [(128, 128, 8, 2048), (2048, 128, 8, 2048), (3, 64, 4, 256),
                                     (100, 96, 3, 384), (257, 300, 5, 128), (40, 1024, 32, 512),
                                     (300, 16, 1, 256)])
def test_route_permute_rotate(gpu_available, T, E, k, K):
    # routing and the rotation of the routed rows in one call: the routing
    # outputs equal the oracle's (and moe_route_permute's) bit for bit, x_rot
    # equals hadamard128_rotate's bit for bit and the oracle's up to the proven
    # rounding-tie window
    from tests.gpu_util import bf16_bits_of, bf16_cuda, check_rotation
    rng = np.random.default_rng(T * 31 + E + k + K)
    lg = (rng.standard_normal((T, E)) + 0.5 * rng.standard_normal((1, E))).astype(np.float32)
    xb = synth.to_bf16_bits((rng.standard_normal((T, K)) * np.where(rng.random(K) < 0.01, 20.0, 1.0))
                            .astype(np.float32))
    print(f"route+rotate T={T} E={E} k={k} K={K}", flush=True)
    ref = router.route(lg, k)
    d_lg, d_x = torch.from_numpy(lg).cuda(), bf16_cuda(xb)
    out = i8h.moe_route_permute_rotate(d_lg, d_x, k)
    plain = i8h.moe_route_permute(d_lg, k)
    xr = i8h.hadamard128_rotate(d_x)
    torch.cuda.synchronize()
    for key in ("topk_ids", "expert_off", "sorted_pairs", "pair_pos"):
        got = out[key].cpu().numpy()
        assert np.array_equal(got, ref["ids" if key == "topk_ids" else key].reshape(got.shape)), key
        assert torch.equal(out[key], plain[key]), key
    assert torch.equal(out["topk_w"], plain["topk_w"])
    assert_close(out["topk_w"].cpu().numpy(), ref["weights"], "topk_w")
    assert torch.equal(out["x_rot"].view(torch.int16), xr.view(torch.int16))
    check_rotation(xb, bf16_bits_of(out["x_rot"]))


def test_route_permute_rotate_in_place(gpu_available):
    from tests.gpu_util import bf16_cuda
    rng = np.random.default_rng(77)
    T, E, k, K = 96, 128, 8, 1024
    lg = rng.standard_normal((T, E)).astype(np.float32)
    xb = synth.to_bf16_bits(rng.standard_normal((T, K)).astype(np.float32))
    d_x = bf16_cuda(xb)
    want = i8h.hadamard128_rotate(d_x)
    out = i8h.moe_route_permute_rotate(torch.from_numpy(lg).cuda(), d_x, k, x_rot=d_x)
    torch.cuda.synchronize()
    assert out["x_rot"].data_ptr() == d_x.data_ptr()
    assert torch.equal(d_x.view(torch.int16), want.view(torch.int16))
