"""GPU parity: moe_route_gateup_i8h_decode (routing, rotation and gate_up in
one launch) against the oracle chain.

Routing outputs must match the oracle bit for bit (weights within 1e-4
relative + 1e-5 absolute); gate_up and act within 1e-4 |ref| + 1e-5, widened
only where the bf16 rotation may round either way. The same arithmetic runs
in the two-call path (moe_route_permute, then moe_gateup_i8h_grouped_fused on
the decode-shaped kernel), so the outputs must also be identical to it bit
for bit.
"""

import numpy as np
import pytest
import torch

import int8_hadamard_domain_amd as i8h
import synth
from oracle import router
from tests.gpu_util import assert_close, assert_close_nan, bf16_cuda, check_with_rotation_slack

pytestmark = pytest.mark.gpu


def _weights_for(L, used):
    codes = np.zeros((L.E, L.N, L.K), dtype=np.int8)
    sbits = np.zeros((L.E, L.N, L.G), dtype=np.uint16)
    if used:
        c, s = synth.synthetic_i8h(L, experts=used)
        codes[used], sbits[used] = c, s
    return codes, sbits


def _run(L, lg=None, what=""):
    lg = synth.router_logits(L) if lg is None else lg
    xb = synth.activations_bf16(L)
    r = router.route(lg, L.topk)
    used = sorted(set(r["ids"].reshape(-1).tolist()))
    codes, sbits = _weights_for(L, used)
    d_lg, d_x = torch.from_numpy(lg).cuda(), bf16_cuda(xb)
    d_codes, d_scales = torch.from_numpy(codes).cuda(), bf16_cuda(sbits)
    print(f"decode {what} T={L.T} K={L.K} E={L.E} k={L.topk} N={L.N}", flush=True)
    ro, gu, act = i8h.moe_route_gateup_i8h_decode(d_lg, d_x, d_codes, d_scales, L.topk)
    torch.cuda.synchronize()
    for key in ("topk_ids", "expert_off", "sorted_pairs", "pair_pos"):
        got = ro[key].cpu().numpy()
        want = r["ids" if key == "topk_ids" else key]
        assert np.array_equal(got, want.reshape(got.shape)), key
    assert_close_nan(ro["topk_w"].cpu().numpy(), r["weights"], "topk_w")
    check_with_rotation_slack(synth.bf16_bits_to_f64(xb), codes, sbits, r, L.topk, gu, act)
    # the two-call path runs the same arithmetic
    ro2 = i8h.moe_route_permute(d_lg, L.topk)
    gu2, act2 = i8h.moe_gateup_i8h_grouped_fused(d_x, d_codes, d_scales, L.topk, ro2["expert_off"],
                                                 ro2["sorted_pairs"])
    torch.cuda.synchronize()
    assert torch.equal(gu, gu2) and torch.equal(act, act2)


def test_decode_workload(gpu_available):
    _run(synth.layer("decode"), what="workload")


def test_tiny_layer(gpu_available):
    _run(synth.layer("tiny"), what="tiny")


@pytest.mark.parametrize("T,K,E,k,N", [
    (8, 2048, 128, 8, 1536),   # 64 pairs: the limit of one wave
    (2, 2048, 256, 8, 1536),   # 4 logits per lane
    (3, 1024, 200, 5, 512),    # E not a multiple of the wavefront, one piece per lane
    (1, 4096, 64, 4, 256),     # four pieces per lane, two row pairs per wave
    (2, 384, 16, 3, 128),      # pieces past K in the last (partial) chunk
    (1, 128, 1, 1, 64),        # one expert, one group
    (5, 256, 8, 8, 192),       # every expert chosen by every token
    (4, 1024, 256, 16, 512),   # k = 16 from 16 row maxima (the threshold top-k at its limit)
    (4, 1024, 128, 16, 512),   # k above the 8 row maxima: the round-based top-k
    (2, 512, 64, 32, 128),     # one logit per lane, k = 32: the round-based top-k
])
def test_shapes(gpu_available, T, K, E, k, N):
    _run(synth.layer("verify", T=T, K=K, E=E, topk=k, N=N, bias_std=0.0), what="shape")


def test_logit_ties(gpu_available):
    # many equal logits: ties go to the lower expert index, in the same order
    # as the routing kernels
    L = synth.layer("verify", T=6, K=512, E=96, topk=6, N=256, bias_std=0.0)
    lg = np.round(synth.router_logits(L) * 2) / 2
    lg[1, :] = 0.25
    lg[2, 40:60] = 3.0
    _run(L, lg=lg.astype(np.float32), what="ties")


@pytest.mark.parametrize("case", ["rounded", "fully_tied", "signed_zeros", "top_block_tied", "minus_inf",
                                  "all_nan", "some_nan", "nan_and_minus_inf"])
def test_one_token_ties(gpu_available, case):
    # one token: the threshold/candidate top-k and its exact fallback (more
    # than 64 candidates, or a -inf threshold) against the oracle's order
    L = synth.layer("decode", K=256, N=64)
    lg = synth.router_logits(L).copy()
    if case == "rounded":
        lg = np.round(lg, 1)
    elif case == "fully_tied":
        lg[:] = 0.25
    elif case == "signed_zeros":
        lg[0, ::2] = -0.0
        lg[0, 1::2] = 0.0
        lg[0, 77] = 1.0
    elif case == "top_block_tied":
        lg[0, [3, 90, 17, 64, 120]] = 9.0
    elif case == "minus_inf":
        lg[0, :100] = -np.inf
    elif case == "all_nan":
        lg[:] = np.nan
    elif case == "some_nan":
        lg[0, ::3] = np.nan                    # NaN in every row group, the rest ranked as usual
    else:
        lg[0, :120] = np.nan
        lg[0, 120:] = -np.inf
    _run(L, lg=lg.astype(np.float32), what=f"one token {case}")


def test_nan_logits_several_tokens(gpu_available):
    # a few tokens in one launch, NaN rows among them: every id a valid
    # expert, the same grouping as the oracle
    L = synth.layer("verify", T=4, K=512, E=96, topk=6, N=256, bias_std=0.0)
    lg = synth.router_logits(L).copy()
    lg[1] = np.nan
    lg[2, ::2] = np.nan
    _run(L, lg=lg.astype(np.float32), what="nan rows")


def test_one_token_many_rows(gpu_available):
    # the decode workload's logits, many tokens one at a time
    for seed in range(24):
        L = synth.layer("decode", K=256, N=64, seed=100 + seed)
        _run(L, what=f"one token seed {100 + seed}")


def test_skewed_experts(gpu_available):
    # all tokens on the same few experts: several rows per expert
    L = synth.layer("verify", T=8, K=1024, E=128, topk=8, N=512, bias_std=0.0)
    lg = synth.router_logits(L)
    lg[:, 10:18] += 50.0
    _run(L, lg=lg, what="skewed")


def test_repeat_is_deterministic(gpu_available):
    L = synth.layer("decode")
    lg_np = synth.router_logits(L)
    lg = torch.from_numpy(lg_np).cuda()
    x = bf16_cuda(synth.activations_bf16(L))
    c, s = _weights_for(L, sorted(set(router.topk(lg_np, L.topk)[0].reshape(-1).tolist())))
    codes, scales = torch.from_numpy(c).cuda(), bf16_cuda(s)
    a = i8h.moe_route_gateup_i8h_decode(lg, x, codes, scales, L.topk)
    b = i8h.moe_route_gateup_i8h_decode(lg, x, codes, scales, L.topk)
    torch.cuda.synchronize()
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
    for key in ("topk_ids", "topk_w", "expert_off", "sorted_pairs", "pair_pos"):
        assert torch.equal(a[0][key], b[0][key])
