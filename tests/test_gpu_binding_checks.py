"""The Python binding rejects caller-supplied tensors that do not fit the call
(wrong device, dtype or shape, or a short workspace) with TypeError or
ValueError before anything is launched: a wrong buffer never reaches a
kernel. Each case changes one tensor of an otherwise valid call."""

import pytest
import torch

import int8_hadamard_domain_amd as i8h

pytestmark = pytest.mark.gpu

T, K, E, N, k = 5, 256, 8, 128, 2


def _inputs():
    dev = torch.device("cuda")
    torch.manual_seed(0)
    x = torch.randn((T, K), device=dev).to(torch.bfloat16)
    logits = torch.randn((T, E), device=dev)
    codes = torch.randint(-127, 128, (E, N, K), device=dev, dtype=torch.int8)
    scales = torch.full((E, N, K // 128), 1e-3, device=dev).to(torch.bfloat16)
    r = i8h.moe_route_permute(logits, k)
    return x, logits, codes, scales, r


@pytest.fixture(scope="module")
def inp(gpu_available):
    return _inputs()


def _raises(fn):
    with pytest.raises((TypeError, ValueError)):
        fn()


def test_rotate_out(inp):
    x = inp[0]
    _raises(lambda: i8h.hadamard128_rotate(x, out=torch.empty((T - 1, K), dtype=torch.bfloat16, device="cuda")))
    _raises(lambda: i8h.hadamard128_rotate(x, out=torch.empty((T, K), dtype=torch.float32, device="cuda")))
    _raises(lambda: i8h.hadamard128_rotate(x, out=torch.empty((T, K), dtype=torch.bfloat16)))


def test_fp8_quantizer_outputs(inp):
    x = inp[0]
    _raises(lambda: i8h.fp8_quantize_activations(x, qx=torch.empty((T, K), dtype=torch.uint8)))
    _raises(lambda: i8h.fp8_quantize_activations(x, qx=torch.empty((T, K), dtype=torch.int8, device="cuda")))
    _raises(lambda: i8h.fp8_quantize_activations(x, qx=torch.empty((T, K - 128), dtype=torch.uint8, device="cuda")))
    _raises(lambda: i8h.fp8_quantize_activations(x, sx=torch.empty((T, K // 128), dtype=torch.float16,
                                                                  device="cuda")))
    _raises(lambda: i8h.fp8_quantize_activations(x, sx=torch.empty((T, K // 128 + 1), dtype=torch.float32,
                                                                  device="cuda")))


@pytest.mark.parametrize("key,bad", [
    ("topk_ids", lambda: torch.empty((T, k), dtype=torch.int64, device="cuda")),
    ("topk_ids", lambda: torch.empty((T, k + 1), dtype=torch.int32, device="cuda")),
    ("topk_w", lambda: torch.empty((T, k), dtype=torch.float32)),
    ("expert_off", lambda: torch.empty((E,), dtype=torch.int32, device="cuda")),
    ("sorted_pairs", lambda: torch.empty((T * k - 1,), dtype=torch.int32, device="cuda")),
    ("pair_pos", lambda: torch.empty((T * k,), dtype=torch.float32, device="cuda")),
    ("workspace", lambda: torch.empty((1,), dtype=torch.uint8, device="cuda")),
    ("workspace", lambda: torch.empty((1 << 16,), dtype=torch.int32, device="cuda")),
])
def test_routing_outputs(inp, key, bad):
    logits = inp[1]
    _raises(lambda: i8h.moe_route_permute(logits, k, out={key: bad()}))
    if key != "workspace":
        _raises(lambda: i8h.moe_route_gateup_i8h_decode(logits, inp[0], inp[2], inp[3], k, out={key: bad()}))


def test_gateup_inputs_and_outputs(inp):
    x, logits, codes, scales, r = inp
    off, sp = r["expert_off"], r["sorted_pairs"]
    _raises(lambda: i8h.moe_gateup_i8h_grouped(x, codes, scales, k, off, sp,
                                               act=torch.empty((T * k, N), device="cuda")))
    _raises(lambda: i8h.moe_gateup_i8h_grouped(x, codes, scales, k, off, sp,
                                               gate_up=torch.empty((T * k, N), dtype=torch.float64, device="cuda")))
    # act: float32 or bfloat16 only, of shape [T*k, N/2] in either
    _raises(lambda: i8h.moe_gateup_i8h_grouped(x, codes, scales, k, off, sp,
                                               act=torch.empty((T * k, N // 2), dtype=torch.float64, device="cuda")))
    _raises(lambda: i8h.moe_gateup_i8h_grouped(x, codes, scales, k, off, sp,
                                               act=torch.empty((T * k, N), dtype=torch.bfloat16, device="cuda")))
    _raises(lambda: i8h.moe_gateup_i8h_grouped(x, codes, scales, k, off, sp, act_dtype=torch.float16))
    _raises(lambda: i8h.moe_gateup_i8h_grouped(x, codes, scales, k, off[:-1].contiguous(), sp))
    _raises(lambda: i8h.moe_gateup_i8h_grouped(x, codes, scales, k + 1, off, sp))
    _raises(lambda: i8h.moe_gateup_i8h_grouped(x, codes, scales[:, :, :1].contiguous(), k, off, sp))
    _raises(lambda: i8h.moe_gateup_i8h_grouped(x, codes.cpu(), scales, k, off, sp))
    _raises(lambda: i8h.moe_gateup_i8h_grouped(x, codes, scales, k, off, sp.cpu()))
    _raises(lambda: i8h.moe_gateup_i8h_grouped_fused(x, codes, scales, k, off, sp,
                                                     workspace=torch.empty((16,), dtype=torch.int32, device="cuda")))
    fp8_codes = codes.view(torch.uint8)
    fp8_scales = torch.full((E, N // 128, K // 128), 1e-3, device="cuda").to(torch.bfloat16)
    _raises(lambda: i8h.moe_gateup_fp8blk_grouped(x, fp8_codes, fp8_scales, k, off, sp,
                                                  workspace=torch.empty((16,), dtype=torch.uint8, device="cuda")))
    _raises(lambda: i8h.moe_gateup_fp8blk_grouped(x, fp8_codes, scales, k, off, sp))
    _raises(lambda: i8h.moe_gateup_i8g_grouped(x, codes, scales, k, off, sp,
                                               workspace=torch.empty((16,), dtype=torch.uint8, device="cuda")))


def test_down_and_linear(inp):
    x, logits, codes, scales, r = inp
    I, H = N // 2, K
    act = torch.randn((T * k, I), device="cuda")
    w = torch.randn((E, H, I), device="cuda").to(torch.bfloat16)
    _raises(lambda: i8h.moe_down_bf16_combine(act[:-1].contiguous(), w, r))
    _raises(lambda: i8h.moe_down_bf16_combine(act, w, r, out=torch.empty((T, H + 8), device="cuda")))
    _raises(lambda: i8h.moe_down_bf16_combine(act, w, r, path="gemm",
                                              workspace=torch.empty((16,), dtype=torch.uint8, device="cuda")))
    _raises(lambda: i8h.moe_down_bf16_combine(act.half(), w, r))
    _raises(lambda: i8h.moe_down_bf16_combine(act.to(torch.bfloat16)[:-1].contiguous(), w, r))
    _raises(lambda: i8h.moe_down_bf16_combine(act.to(torch.bfloat16), w, r, path="gemm",
                                              workspace=torch.empty((16,), dtype=torch.uint8, device="cuda")))
    bad = dict(r)
    bad["pair_pos"] = r["pair_pos"][:-1].contiguous()
    _raises(lambda: i8h.moe_down_bf16_combine(act, w, bad))
    lin_codes = torch.randint(-127, 128, (64, K), device="cuda", dtype=torch.int8)
    lin_scales = torch.full((64, K // 128), 1e-3, device="cuda").to(torch.float16)
    _raises(lambda: i8h.linear_i8f16(x, lin_codes, lin_scales, out=torch.empty((T, 65), device="cuda")))
    _raises(lambda: i8h.linear_i8f16(x, lin_codes, lin_scales.float()))


def test_valid_calls_still_run(inp):
    # the same calls with fitting tensors go through
    x, logits, codes, scales, r = inp
    out = {key: torch.empty_like(r[key]) for key in ("topk_ids", "topk_w", "expert_off", "sorted_pairs",
                                                      "pair_pos")}
    r2 = i8h.moe_route_permute(logits, k, out=out)
    gu, act = i8h.moe_gateup_i8h_grouped(x, codes, scales, k, r2["expert_off"], r2["sorted_pairs"])
    y = i8h.hadamard128_rotate(x, out=torch.empty_like(x))
    torch.cuda.synchronize()
    assert gu.shape == (T * k, N) and act.shape == (T * k, N // 2) and y.shape == x.shape
    for key in out:
        assert torch.equal(r2[key], r[key])
