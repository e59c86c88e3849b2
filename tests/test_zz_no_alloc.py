"""The allocation-free routing call (moe_route_permute_noalloc) against the
workspace form (moe_route_permute), both through the C ABI: identical
outputs bit for bit, on two calls in a row (the second with fewer pairs, so
it runs over what the first left in the library's scratch), on the
three-kernel path and the single-block path, and for the largest size the
scratch admits. Sizes beyond it are refused before any launch."""

import ctypes

import numpy as np
import pytest
import torch

import int8_hadamard_domain_amd as i8h

pytestmark = pytest.mark.gpu

KEYS = ("topk_ids", "topk_w", "expert_off", "sorted_pairs", "pair_pos")


def _outputs(T, E, k):
    dev = torch.device("cuda")
    return {"topk_ids": torch.full((T, k), -7, dtype=torch.int32, device=dev),
            "topk_w": torch.full((T, k), -7.0, dtype=torch.float32, device=dev),
            "expert_off": torch.full((E + 1,), -7, dtype=torch.int32, device=dev),
            "sorted_pairs": torch.full((T * k,), -7, dtype=torch.int32, device=dev),
            "pair_pos": torch.full((T * k,), -7, dtype=torch.int32, device=dev)}


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _with_workspace(lg, k):
    L = i8h.lib()
    T, E = lg.shape
    o = _outputs(T, E, k)
    need = L.moe_route_permute_workspace_size(T, E, k)
    ws = torch.empty((max(need, 1),), dtype=torch.uint8, device="cuda")
    rc = L.moe_route_permute(_p(lg), T, E, k, *[_p(o[key]) for key in KEYS], _p(ws), ws.numel(), _stream())
    assert rc == i8h.I8H_OK, rc
    return o


def _no_alloc(lg, k):
    L = i8h.lib()
    T, E = lg.shape
    o = _outputs(T, E, k)
    rc = L.moe_route_permute_noalloc(_p(lg), T, E, k, *[_p(o[key]) for key in KEYS], _stream())
    assert rc == i8h.I8H_OK, rc
    return o


def _logits(T, E, seed):
    g = torch.Generator().manual_seed(seed)
    lg = torch.randn((T, E), generator=g) + 0.5 * torch.randn((1, E), generator=g)   # skewed loads
    return lg.cuda()


def _same(a, b):
    torch.cuda.synchronize()
    for key in KEYS:
        assert torch.equal(a[key], b[key]), key


@pytest.mark.parametrize("sizes", [((2048, 128, 8), (300, 128, 8)),      # prefill, then fewer pairs
                                   ((1000, 1024, 32), (37, 300, 5)),     # many chunks x E, then other E and k
                                   ((200, 64, 4), (3, 64, 4))])          # then the single-block path
def test_two_calls_match_the_workspace_form(gpu_available, sizes):
    for i, (T, E, k) in enumerate(sizes):
        print(f"no-alloc route call {i}: T={T} E={E} k={k}", flush=True)
        lg = _logits(T, E, seed=T + E + k)
        want = _with_workspace(lg, k)
        got = _no_alloc(lg, k)
        _same(got, want)


def test_largest_admitted_size(gpu_available):
    # ceil(P / 256) * E * 4 bytes == 1 MiB exactly: P = 524288 pairs at E = 128
    L = i8h.lib()
    T, E, k = 65536, 128, 8
    assert L.moe_route_permute_workspace_size(T, E, k) == 1 << 20
    print(f"no-alloc route at the scratch limit: T={T} E={E} k={k}", flush=True)
    lg = _logits(T, E, seed=5)
    _same(_no_alloc(lg, k), _with_workspace(lg, k))
    # one chunk more is refused, with nothing launched
    o = _outputs(1, E, k)
    rc = L.moe_route_permute_noalloc(_p(lg), T + 32, E, k, *[_p(o[key]) for key in KEYS], _stream())
    assert rc == i8h.I8H_EUNSUPPORTED


def test_binding_name(gpu_available):
    lg = _logits(40, 128, seed=9)
    a = i8h.moe_route_permute_noalloc(lg, 8)
    b = i8h.moe_route_permute(lg, 8)
    _same(a, b)
