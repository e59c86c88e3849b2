"""GPU: every step form captured in a HIP graph and replayed.

The calls enqueue no allocation, synchronisation, host copy or memset, so a
caller (and bench.py) can capture them. Each test captures one step on fixed
input buffers, then replays the graph several times; before each replay the
host loads one of two input sets into those buffers with eager copies (the
program's own work between replays), and after it compares every output bit
for bit with eager calls on the same inputs. The kernels are deterministic,
so a replay must reproduce the eager bits exactly.
"""

import numpy as np
import pytest
import torch

import int8_hadamard_domain_amd as i8h
import synth
from tests.gpu_util import bf16_cuda

pytestmark = pytest.mark.gpu

ORDER = (0, 1, 1, 0, 1)   # which input set each replay runs on


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _check_replays(inputs, sets, fn, outputs):
    """inputs: the captured input buffers; sets: two lists of tensors to copy into them;
    fn: the step on the buffers; outputs(): the tensors to compare (read after each run)."""
    want = []
    for s in sets:
        for buf, src in zip(inputs, s):
            buf.copy_(src)
        fn()
        torch.cuda.synchronize()
        want.append([o.clone() for o in outputs()])
    g = _capture(fn)
    for rep, k in enumerate(ORDER):
        for buf, src in zip(inputs, sets[k]):
            buf.copy_(src)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for j, (o, w) in enumerate(zip(outputs(), want[k])):
            assert torch.equal(o, w), f"replay {rep} (input set {k}): output {j} differs from the eager call"


def _layer(name, **over):
    L = synth.layer(name, **over)
    LB = synth.layer(name, **dict(over, T=2 * L.T))
    lg = synth.router_logits(LB).reshape(2, L.T, L.E)
    x = synth.activations_bf16(LB).reshape(2, L.T, L.K)
    return L, [torch.from_numpy(lg[i]).cuda() for i in range(2)], [bf16_cuda(x[i]) for i in range(2)]


def test_decode_one_launch():
    L, lgs, xs = _layer("decode")
    codes, sbits = synth.synthetic_i8h(L)
    codes, scales = torch.from_numpy(codes).cuda(), bf16_cuda(sbits)
    lg, x = lgs[0].clone(), xs[0].clone()
    out = {}
    act = torch.empty((L.P, L.I), device="cuda")

    def fn():
        out["r"], _, _ = i8h.moe_route_gateup_i8h_decode(lg, x, codes, scales, L.topk, gate_up=False, act=act,
                                                         out=out.get("r"))
    fn()
    _check_replays([lg, x], [[lgs[0], xs[0]], [lgs[1], xs[1]]], fn,
                   lambda: [act] + [out["r"][k] for k in ("topk_ids", "topk_w", "expert_off", "sorted_pairs",
                                                          "pair_pos")])


@pytest.mark.parametrize("name,over", [("verify", {}), ("prefill", {"T": 512})])
def test_route_rotate_then_gateup(name, over):
    """verify (the small-unit kernel) and a 512-token prefill-shaped batch (the tall kernel)."""
    L, lgs, xs = _layer(name, **over)
    codes, sbits = synth.synthetic_i8h(L)
    codes, scales = torch.from_numpy(codes).cuda(), bf16_cuda(sbits)
    lg, x = lgs[0].clone(), xs[0].clone()
    r = i8h.moe_route_permute_rotate(lg, x, L.topk)
    gu = torch.empty((L.P, L.N), device="cuda")
    act = torch.empty((L.P, L.I), device="cuda")

    def fn():
        i8h.moe_route_permute_rotate(lg, x, L.topk, out=r, x_rot=r["x_rot"])
        i8h.moe_gateup_i8h_grouped(r["x_rot"], codes, scales, L.topk, r["expert_off"], r["sorted_pairs"],
                                   gate_up=gu, act=act)
    _check_replays([lg, x], [[lgs[0], xs[0]], [lgs[1], xs[1]]], fn,
                   lambda: [gu, act, r["x_rot"], r["sorted_pairs"], r["topk_w"]])


@pytest.mark.parametrize("fmt", ["fp8", "w8a8"])
def test_quantizing_variants(fmt):
    """The FP8 and W8A8 calls quantize the activations into their workspace inside the step."""
    L, lgs, xs = _layer("fp8" if fmt == "fp8" else "w8a8", **({} if fmt == "fp8" else {"T": 256}))
    codes, sbits = (synth.synthetic_fp8 if fmt == "fp8" else synth.synthetic_i8h)(L)
    codes, scales = torch.from_numpy(codes).cuda(), bf16_cuda(sbits)
    lg, x = lgs[0].clone(), xs[0].clone()
    r = i8h.moe_route_permute(lg, L.topk)
    act = torch.empty((L.P, L.I), device="cuda")
    call = i8h.moe_gateup_fp8blk_grouped if fmt == "fp8" else i8h.moe_gateup_i8g_grouped
    _, _, ws = call(x, codes, scales, L.topk, r["expert_off"], r["sorted_pairs"], gate_up=False, act=act)

    def fn():
        i8h.moe_route_permute(lg, L.topk, out=r)
        call(x, codes, scales, L.topk, r["expert_off"], r["sorted_pairs"], gate_up=False, act=act, workspace=ws)
    _check_replays([lg, x], [[lgs[0], xs[0]], [lgs[1], xs[1]]], fn, lambda: [act, ws])


@pytest.mark.parametrize("path", ["gemv", "gemm"])
def test_down_projection(path):
    L = synth.layer("verify")
    LB = synth.layer("verify", T=2 * L.T)
    lg = synth.router_logits(LB).reshape(2, L.T, L.E)
    a = synth.act_f32(LB, rows=2 * L.P).reshape(2, L.P, L.I)
    lgs = [torch.from_numpy(lg[i]).cuda() for i in range(2)]
    acts = [torch.from_numpy(a[i]).cuda() for i in range(2)]
    w = bf16_cuda(synth.down_weights_bf16(L))
    lgb, act = lgs[0].clone(), acts[0].clone()
    r = i8h.moe_route_permute(lgb, L.topk)
    out = torch.empty((L.T, L.K), device="cuda")
    ws = torch.empty((i8h.lib().moe_down_bf16_workspace_size(L.T, L.I, L.K, L.topk),), dtype=torch.uint8,
                     device="cuda")

    def fn():
        i8h.moe_route_permute(lgb, L.topk, out=r)
        i8h.moe_down_bf16_combine(act, w, r, out=out, workspace=ws, path=path)
    _check_replays([lgb, act], [[lgs[0], acts[0]], [lgs[1], acts[1]]], fn, lambda: [out])


def test_bf16_handoff_chain():
    """route + rotate -> gate_up (bf16 act) -> down (bf16 act) on a 512-token batch, one graph."""
    L, lgs, xs = _layer("prefill", T=512)
    codes, sbits = synth.synthetic_i8h(L)
    codes, scales = torch.from_numpy(codes).cuda(), bf16_cuda(sbits)
    w = bf16_cuda(synth.down_weights_bf16(L))
    lg, x = lgs[0].clone(), xs[0].clone()
    r = i8h.moe_route_permute_rotate(lg, x, L.topk)
    a16 = torch.empty((L.P, L.I), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((L.T, L.K), device="cuda")
    ws = torch.empty((i8h.lib().moe_down_bf16_act_bf16_workspace_size(L.T, L.I, L.K, L.topk),),
                     dtype=torch.uint8, device="cuda")

    def fn():
        i8h.moe_route_permute_rotate(lg, x, L.topk, out=r, x_rot=r["x_rot"])
        i8h.moe_gateup_i8h_grouped(r["x_rot"], codes, scales, L.topk, r["expert_off"], r["sorted_pairs"],
                                   gate_up=False, act=a16)
        i8h.moe_down_bf16_combine(a16, w, r, out=out, workspace=ws)
    _check_replays([lg, x], [[lgs[0], xs[0]], [lgs[1], xs[1]]], fn, lambda: [a16, out])


def test_routing_without_workspace():
    """The allocation-free routing call (its fixed per-device scratch) inside a graph."""
    L, lgs, _ = _layer("verify")
    lg = lgs[0].clone()
    r = i8h.moe_route_permute_noalloc(lg, L.topk)

    def fn():
        i8h.moe_route_permute_noalloc(lg, L.topk, out=r)
    _check_replays([lg], [[lgs[0]], [lgs[1]]], fn,
                   lambda: [r[k] for k in ("topk_ids", "topk_w", "expert_off", "sorted_pairs", "pair_pos")])


def test_decode_two_launch():
    """Decode as routing, then the gate_up call that rotates inside its GEMV (a batch of 4 tokens)."""
    L, lgs, xs = _layer("decode", T=4)
    codes, sbits = synth.synthetic_i8h(L)
    codes, scales = torch.from_numpy(codes).cuda(), bf16_cuda(sbits)
    lg, x = lgs[0].clone(), xs[0].clone()
    r = i8h.moe_route_permute(lg, L.topk)
    gu = torch.empty((L.P, L.N), device="cuda")
    act = torch.empty((L.P, L.I), device="cuda")

    def fn():
        i8h.moe_route_permute(lg, L.topk, out=r)
        i8h.moe_gateup_i8h_grouped_fused(x, codes, scales, L.topk, r["expert_off"], r["sorted_pairs"],
                                         gate_up=gu, act=act)
    _check_replays([lg, x], [[lgs[0], xs[0]], [lgs[1], xs[1]]], fn, lambda: [gu, act, r["sorted_pairs"]])


def test_drafter_linear():
    """The drafter's int8 linear (16 positions, K = 2048, N = 4096)."""
    T, K, N = 16, 2048, 4096
    codes, sbits = synth.synthetic_i8f16(N, K, seed=31)
    codes = torch.from_numpy(codes).cuda()
    scales = torch.from_numpy(sbits.view(np.float16)).cuda()
    xb = [bf16_cuda(synth.drafter_activations_bf16(T, K, seed)) for seed in (32, 33)]
    x = xb[0].clone()
    y = torch.empty((T, N), device="cuda")

    def fn():
        i8h.linear_i8f16(x, codes, scales, out=y)
    _check_replays([x], [[xb[0]], [xb[1]]], fn, lambda: [y])
