"""GPU: the bf16 act handoff between the gate_up calls and the down projection.

The gate_up calls can store act in bf16 (each value the float32 act rounded to
nearest even), and the down projection takes such act rows as they are, where
it would otherwise round the float32 rows itself. Both halves are checked bit
for bit against the float32 forms, whose results the other GPU tests check
against the oracle:
  - gate_up, every kernel (GEMV, the 128-pair GEMM, the tall and small-unit
    kernels; the FP8 and W8A8 forms): act_bf16 == bf16(act) and gate_up equal;
  - down, both forms: out(bf16(act)) == out(act);
  - the chain route -> gate_up -> down at the verify and prefill sizes, in the
    kernels AUTO picks: the bf16 handoff gives the float32 chain's out.
"""

import numpy as np
import pytest
import torch

import int8_hadamard_domain_amd as i8h
import synth
from tests.gpu_util import bf16_cuda

pytestmark = pytest.mark.gpu


def _layer(T, K, E, k, N, seed, fp8=False):
    L = synth.layer("decode", T=T, K=K, E=E, topk=k, N=N, seed=seed)
    codes, sbits = (synth.synthetic_fp8 if fp8 else synth.synthetic_i8h)(L)
    r = i8h.moe_route_permute(torch.from_numpy(synth.router_logits(L)).cuda(), k)
    x = bf16_cuda(synth.activations_bf16(L))
    return L, torch.from_numpy(codes).cuda(), bf16_cuda(sbits), r, x


def _assert_bf16_of(a16, a32, what):
    assert a16.dtype == torch.bfloat16 and a32.dtype == torch.float32
    want = a32.to(torch.bfloat16)
    same = a16.view(torch.int16) == want.view(torch.int16)
    assert bool(same.all()), f"{what}: {int((~same).sum())} act values differ from bf16(float32 act)"


CASES = [
    # T, K, E, k, N, seed: few pairs an expert; many (one expert above 256 pairs: two tall passes)
    (40, 512, 16, 4, 256, 0),
    (300, 256, 4, 2, 192, 1),
]


@pytest.mark.parametrize("T,K,E,k,N,seed", CASES)
@pytest.mark.parametrize("path", ["gemv", "gemm", "tall", "skinny"])
def test_i8h_act_bf16_is_the_float32_act_rounded(T, K, E, k, N, seed, path):
    L, codes, scales, r, x = _layer(T, K, E, k, N, seed)
    xr = i8h.hadamard128_rotate(x)
    g32, a32 = i8h.moe_gateup_i8h_grouped(xr, codes, scales, k, r["expert_off"], r["sorted_pairs"], path=path)
    g16, a16 = i8h.moe_gateup_i8h_grouped(xr, codes, scales, k, r["expert_off"], r["sorted_pairs"], path=path,
                                          act_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(g16, g32)
    _assert_bf16_of(a16, a32, f"i8h {path} T{T}")
    # act alone into a caller's bf16 tensor
    out = torch.full_like(a16, float("nan"))
    none, a16b = i8h.moe_gateup_i8h_grouped(xr, codes, scales, k, r["expert_off"], r["sorted_pairs"],
                                            gate_up=False, act=out, path=path)
    torch.cuda.synchronize()
    assert none is None and a16b is out and torch.equal(out.view(torch.int16), a16.view(torch.int16))


@pytest.mark.parametrize("path", ["gemm", "skinny"])
def test_fp8_act_bf16_is_the_float32_act_rounded(path):
    L, codes, scales, r, x = _layer(40, 512, 16, 4, 256, 2, fp8=True)
    g32, a32, _ = i8h.moe_gateup_fp8blk_grouped(x, codes, scales, 4, r["expert_off"], r["sorted_pairs"], path=path)
    g16, a16, _ = i8h.moe_gateup_fp8blk_grouped(x, codes, scales, 4, r["expert_off"], r["sorted_pairs"],
                                                path=path, act_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(g16, g32)
    _assert_bf16_of(a16, a32, f"fp8 {path}")


def test_i8g_act_bf16_is_the_float32_act_rounded():
    L, codes, scales, r, x = _layer(300, 256, 4, 2, 192, 3)
    g32, a32, _ = i8h.moe_gateup_i8g_grouped(x, codes, scales, 2, r["expert_off"], r["sorted_pairs"])
    g16, a16, _ = i8h.moe_gateup_i8g_grouped(x, codes, scales, 2, r["expert_off"], r["sorted_pairs"],
                                             act_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(g16, g32)
    _assert_bf16_of(a16, a32, "i8g")


def _down_case(T, I, E, k, H, seed, bias=None):
    L = synth.layer("decode", T=T, K=H, E=E, topk=k, N=2 * I, seed=seed)
    lg = synth.router_logits(L)
    if bias is not None:
        lg = (lg + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)
    r = i8h.moe_route_permute(torch.from_numpy(lg).cuda(), k)
    w = bf16_cuda(synth.down_weights_bf16(L))
    act = torch.from_numpy(synth.act_f32(L)).cuda()
    return r, w, act


@pytest.mark.parametrize("path", ["gemv", "gemm", "auto"])
@pytest.mark.parametrize("case", [(40, 256, 12, 8, 256, 10, None), (2, 1024, 16, 3, 256, 8, None),
                                  (400, 256, 6, 2, 512, 21, [3.0, 2.5, -30.0, 0.0, -30.0, 0.0])])
def test_down_on_bf16_act_equals_down_on_float32_act(case, path):
    T, I, E, k, H, seed, bias = case
    r, w, act = _down_case(T, I, E, k, H, seed, bias)
    o32 = i8h.moe_down_bf16_combine(act, w, r, path=path)
    o16 = i8h.moe_down_bf16_combine(act.to(torch.bfloat16), w, r, path=path)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32), f"down {path} T{T} I{I}: bf16-act form differs"


@pytest.mark.parametrize("name", ["verify", "prefill"])
def test_chain_with_bf16_handoff_equals_float32_chain(name):
    """route+rotate -> gate_up (AUTO) -> down (AUTO) on the workload's layer,
    with the act rows handed over in bf16, against the same chain in float32."""
    L = synth.layer(name)
    codes, sbits = synth.synthetic_i8h(L)
    codes, scales = torch.from_numpy(codes).cuda(), bf16_cuda(sbits)
    r = i8h.moe_route_permute_rotate(torch.from_numpy(synth.router_logits(L)).cuda(),
                                     bf16_cuda(synth.activations_bf16(L)), L.topk)
    used = sorted(set(r["topk_ids"].cpu().numpy().ravel().tolist()))
    wbits = np.zeros((L.E, L.K, L.I), dtype=np.uint16)
    wbits[used] = synth.down_weights_bf16(L, experts=used)
    w = bf16_cuda(wbits)
    _, a32 = i8h.moe_gateup_i8h_grouped(r["x_rot"], codes, scales, L.topk, r["expert_off"], r["sorted_pairs"],
                                        gate_up=False)
    _, a16 = i8h.moe_gateup_i8h_grouped(r["x_rot"], codes, scales, L.topk, r["expert_off"], r["sorted_pairs"],
                                        gate_up=False, act_dtype=torch.bfloat16)
    o32 = i8h.moe_down_bf16_combine(a32, w, r)
    o16 = i8h.moe_down_bf16_combine(a16, w, r)
    torch.cuda.synchronize()
    _assert_bf16_of(a16, a32, name)
    assert torch.equal(o16, o32), f"{name}: the bf16 handoff changes out"
    assert torch.isfinite(o16).all()
