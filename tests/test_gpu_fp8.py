"""GPU parity: the FP8 E4M3 128x128-block variant against the oracle.

The activation quantizer must match bit for bit (codes and float32 scales);
the grouped product within 1e-4 relative + 1e-5 absolute on gate_up and act.
"""

import numpy as np
import pytest
import torch

import int8_hadamard_domain_amd as i8h
import synth
from oracle import gateup, numfmt, quant, router
from tests.gpu_util import assert_close, bf16_cuda

pytestmark = pytest.mark.gpu

PATHS = ("gemm", "skinny", "auto")


def _quant_compare(xb):
    print(f"fp8 act quant {xb.shape}", flush=True)
    qx, sx = i8h.fp8_quantize_activations(bf16_cuda(xb))
    torch.cuda.synchronize()
    want_q, want_s = quant.quantize_fp8_activations(numfmt.bf16_from_bits(xb))
    assert np.array_equal(sx.cpu().numpy(), want_s)
    got_q = qx.cpu().numpy()
    assert np.array_equal(got_q, want_q), np.argwhere(got_q != want_q)[:5]


def test_act_quant_workload(gpu_available):
    L = synth.layer("fp8")
    _quant_compare(synth.activations_bf16(L))


def test_act_quant_special_values(gpu_available):
    rng = np.random.default_rng(41)
    x = rng.standard_normal((8, 512)).astype(np.float32)
    x[0, :128] = 0.0                               # all-zero group
    x[1, :128] *= 1e-38                            # tiny values: subnormal codes and scales
    x[2, :128] = -0.0
    x[2, 5] = 1.0                                  # negative zeros next to a positive max
    x[3, 128:256] = 3e38                           # huge values
    x[3, 130] = -1e30
    x[4, :128] = np.linspace(-448, 448, 128)       # scale exactly 1
    x[5, 256:384] *= 1e-20
    _quant_compare(synth.to_bf16_bits(x))


def test_act_quant_ties(gpu_available):
    # build groups whose quotients x / sx land exactly on E4M3 midpoints
    grid = numfmt.e4m3_decode(np.arange(0x7E, dtype=np.uint8))
    mids = (grid[:-1] + grid[1:]) / 2
    rng = np.random.default_rng(42)
    x = np.zeros((4, 256), dtype=np.float32)
    for t in range(4):
        v = rng.choice(mids[(mids > 0.25) & (mids < 400)], 255)
        x[t, :255] = v * rng.choice([-1, 1], 255)
        x[t, 255] = 448.0                          # amax = 448 -> sx = 1
    xb = synth.to_bf16_bits(x)
    assert np.array_equal(numfmt.bf16_from_bits(xb), x.astype(np.float64))  # midpoints are bf16-exact
    _quant_compare(xb)


def _layer_fp8(L, experts_dense=True):
    if experts_dense:
        w = np.stack([synth.dense_weights(L, e) for e in range(L.E)]).astype(np.float64)
        codes, scales = quant.quantize_fp8_blocks(w)
        return codes, numfmt.bf16_to_bits(scales)
    return synth.synthetic_fp8(L)


def _run(L, codes, sbits, rows=None, what="", path="auto"):
    lg = synth.router_logits(L)
    xb = synth.activations_bf16(L)
    r = router.route(lg, L.topk)
    what = f"{what} {path}"
    print(f"fp8 gateup {what}", flush=True)
    gu, act, ws = i8h.moe_gateup_fp8blk_grouped(
        bf16_cuda(xb), torch.from_numpy(codes).cuda(), bf16_cuda(sbits), L.topk,
        torch.from_numpy(r["expert_off"]).cuda(), torch.from_numpy(r["sorted_pairs"]).cuda(), path=path)
    torch.cuda.synchronize()
    qx, sx = quant.quantize_fp8_activations(synth.bf16_bits_to_f64(xb))
    # the workspace keeps the quantized activations: bit-exact
    gq, gs, gx = i8h.fp8_workspace_views(ws, L.T, L.K)
    assert np.array_equal(gq.cpu().numpy(), qx) and np.array_equal(gs.cpu().numpy(), sx)
    # the exact bf16 values of the codes, as the product consumes them
    xq = gx.float().cpu().numpy().astype(np.float64)
    assert np.array_equal(xq, numfmt.e4m3_decode(qx))
    ref = gateup.gateup_fp8blk(qx, sx, codes, numfmt.bf16_from_bits(sbits), r["expert_off"], r["sorted_pairs"],
                               L.topk, rows=rows)
    sel = slice(None) if rows is None else rows
    assert_close(gu.cpu().numpy()[sel], ref, what + " gate_up")
    assert_close(act.cpu().numpy()[sel], gateup.epilogue(ref), what + " act")


@pytest.mark.parametrize("path", PATHS)
def test_small_layer_oracle_quantized(gpu_available, path):
    L = synth.layer("fp8", T=6, K=256, E=4, topk=2, N=256)
    codes, sbits = _layer_fp8(L)
    _run(L, codes, sbits, what="small", path=path)


@pytest.mark.parametrize("path", PATHS)
def test_mid_layer_oracle_quantized(gpu_available, path):
    L = synth.layer("fp8", T=70, E=4, topk=2)
    codes, sbits = _layer_fp8(L)
    _run(L, codes, sbits, what="mid", path=path)


@pytest.mark.parametrize("path", PATHS)
def test_full_size_sampled(gpu_available, path):
    L = synth.layer("fp8")
    codes, sbits = _layer_fp8(L, experts_dense=False)
    r = router.route(synth.router_logits(L), L.topk)
    off = r["expert_off"]
    rows = set()
    for e in range(L.E):
        if off[e + 1] > off[e]:
            rows.update([int(off[e]), int(off[e + 1] - 1)])
    rows.update(np.random.default_rng(4).integers(0, off[-1], 48).tolist())
    _run(L, codes, sbits, rows=np.array(sorted(rows)), what="full", path=path)


@pytest.mark.parametrize("path", PATHS)
def test_ragged_and_large_m(gpu_available, path):
    # one expert with 300 pairs (several m-passes), N = 128 (gate and up share a block)
    L = synth.layer("fp8", T=300, K=384, E=1, topk=1, N=128)
    codes, sbits = _layer_fp8(L)
    _run(L, codes, sbits, what="ragged", path=path)
