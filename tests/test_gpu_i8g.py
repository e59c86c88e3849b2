"""GPU parity: the W8A8 int8 g128 form against the oracle (oracle/w8a8.py).

The activation quantizer must match bit for bit (int8 codes and float32
scales); the grouped product within 1e-4 relative + 1e-5 absolute on gate_up
and act. Cases: small and mid layers with RTN-quantized dense weights, one
expert holding 400 pairs (three passes of 192, the last ragged), I = 64 and
I = 96 (column units with dead waves), unused experts, and the full prefill
layer (T = 2048, K = 2048, E = 128, top-8, N = 1536) on sampled rows.
"""

import numpy as np
import pytest
import torch

import int8_hadamard_domain_amd as i8h
import synth
from oracle import gateup, numfmt, router, w8a8
from tests.gpu_util import assert_close, bf16_cuda

pytestmark = pytest.mark.gpu


def _quant_compare(xb):
    print(f"i8 act quant {xb.shape}", flush=True)
    qx, sx = i8h.i8_quantize_activations(bf16_cuda(xb))
    torch.cuda.synchronize()
    want_q, want_s = w8a8.quantize_i8_activations(numfmt.bf16_from_bits(xb))
    assert np.array_equal(sx.cpu().numpy(), want_s)
    got_q = qx.cpu().numpy()
    assert np.array_equal(got_q, want_q), np.argwhere(got_q != want_q)[:5]


def test_act_quant_workload(gpu_available):
    _quant_compare(synth.activations_bf16(synth.layer("prefill")))


def test_act_quant_special_values(gpu_available):
    rng = np.random.default_rng(51)
    x = rng.standard_normal((8, 512)).astype(np.float32)
    x[0, :128] = 0.0                               # all-zero group
    x[1, :128] *= 1e-38                            # tiny values: subnormal scale
    x[2, :128] = -0.0
    x[2, 5] = 1.0                                  # negative zeros next to a positive max
    x[3, 128:256] = 3e38                           # huge values
    x[3, 130] = -1e30
    x[4, :128] = np.linspace(-127, 127, 128)       # scale exactly 1
    x[5, 256:384] *= 1e-20
    _quant_compare(synth.to_bf16_bits(x))


def test_act_quant_ties(gpu_available):
    # amax = 127 gives sx = 1, so every half-integer input is a tie
    rng = np.random.default_rng(52)
    x = (rng.integers(-126, 126, size=(4, 256)) + 0.5).astype(np.float32)
    x[:, 0] = 127.0
    x[:, 128] = -127.0
    _quant_compare(synth.to_bf16_bits(x))


def _layer_i8g(L):
    w = np.stack([synth.dense_weights(L, e) for e in range(L.E)]).astype(np.float64)
    codes, scales = w8a8.quantize_i8g_weights(w)
    return codes, numfmt.bf16_to_bits(scales)


def _run(L, codes, sbits, rows=None, what="", bias=None):
    lg = synth.router_logits(L)
    if bias is not None:
        lg = (lg + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)
    xb = synth.activations_bf16(L)
    r = router.route(lg, L.topk)
    print(f"i8g gateup {what}", flush=True)
    gu, act, ws = i8h.moe_gateup_i8g_grouped(
        bf16_cuda(xb), torch.from_numpy(codes).cuda(), bf16_cuda(sbits), L.topk,
        torch.from_numpy(r["expert_off"]).cuda(), torch.from_numpy(r["sorted_pairs"]).cuda())
    torch.cuda.synchronize()
    qx, sx = w8a8.quantize_i8_activations(synth.bf16_bits_to_f64(xb))
    gq, gs = i8h.i8g_workspace_views(ws, L.T, L.K)          # the workspace keeps them: bit-exact
    assert np.array_equal(gq.cpu().numpy(), qx) and np.array_equal(gs.cpu().numpy(), sx)
    ref = w8a8.gateup_i8g(qx, sx, codes, numfmt.bf16_from_bits(sbits), r["expert_off"], r["sorted_pairs"],
                          L.topk, rows=rows)
    sel = slice(None) if rows is None else rows
    assert_close(gu.cpu().numpy()[sel], ref, what + " gate_up")
    assert_close(act.cpu().numpy()[sel], gateup.epilogue(ref), what + " act")
    return r


def test_small_layer(gpu_available):
    L = synth.layer("prefill", T=6, K=256, E=4, topk=2, N=256)
    _run(L, *_layer_i8g(L), what="small")


def test_mid_layer(gpu_available):
    L = synth.layer("prefill", T=70, K=1024, E=4, topk=2, N=512)
    _run(L, *_layer_i8g(L), what="mid")


def test_one_expert_three_passes_and_half_unit(gpu_available):
    # 400 pairs on one expert: passes of 192, 192 and 16 rows; I = 64 leaves
    # half of the unit's column waves without columns
    L = synth.layer("prefill", T=400, K=384, E=1, topk=1, N=128)
    _run(L, *_layer_i8g(L), what="400 pairs, N=128")


def test_unused_experts_and_ragged_columns(gpu_available):
    # I = 96: the last 32-column slice of the unit is dead; two experts never chosen
    L = synth.layer("prefill", T=90, K=512, E=6, topk=2, N=192)
    bias = np.array([0.0, -30.0, 1.0, 0.0, -30.0, 2.0], dtype=np.float32)
    r = _run(L, *_layer_i8g(L), what="ragged", bias=bias)
    assert (np.diff(r["expert_off"]) == 0).sum() == 2


def test_full_prefill_sampled(gpu_available):
    L = synth.layer("prefill")
    codes, sbits = synth.synthetic_i8h(L)          # the same storage: int8 codes, bf16 scale per 128
    off = router.route(synth.router_logits(L), L.topk)["expert_off"]
    rows = set()
    for e in range(L.E):
        if off[e + 1] > off[e]:
            rows.update([int(off[e]), int(off[e + 1] - 1)])
    rows.update(np.random.default_rng(7).integers(0, off[-1], 64).tolist())
    _run(L, codes, sbits, rows=np.array(sorted(rows)), what="full prefill")


def test_zero_tokens_is_a_no_op(gpu_available):
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    codes = torch.zeros((4, 128, 256), dtype=torch.int8, device="cuda")
    scales = torch.zeros((4, 128, 2), dtype=torch.bfloat16, device="cuda")
    gu, act, _ = i8h.moe_gateup_i8g_grouped(x, codes, scales, 2, torch.zeros(5, dtype=torch.int32, device="cuda"),
                                            torch.empty(0, dtype=torch.int32, device="cuda"))
    assert gu.shape == (0, 128) and act.shape == (0, 64)
