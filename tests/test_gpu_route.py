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
from tests.gpu_util import assert_close

pytestmark = pytest.mark.gpu


def _run_and_compare(lg, k):
    print(f"route T={lg.shape[0]} E={lg.shape[1]} k={k}", flush=True)
    ref = router.route(lg, k)
    out = i8h.moe_route_permute(torch.from_numpy(lg).cuda(), k)
    torch.cuda.synchronize()
    for key in ("topk_ids", "expert_off", "sorted_pairs", "pair_pos"):
        got = out[key].cpu().numpy()
        want = ref["ids" if key == "topk_ids" else key]
        assert np.array_equal(got, want.reshape(got.shape)), key
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
