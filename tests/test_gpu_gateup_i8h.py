"""GPU parity: moe_gateup_i8h_grouped (both kernels) against the oracle.

Elementwise |gpu - oracle| <= 1e-4 |oracle| + 1e-5 on gate_up and act. The
product kernels are fed the oracle's rotated activations and routing, so
each comparison checks one step. Small layers go through the oracle's own
quantizer; the full-size layers (decode, verify, prefill) use codes drawn by
the generator and are checked on sampled expert-sorted rows, covering every
column of each. An end-to-end test chains route -> rotate -> gate_up on the
GPU and widens the tolerance only by the proven near-tie bound of the bf16
rotation.
"""

import numpy as np
import pytest
import torch

import int8_hadamard_domain_amd as i8h
import synth
from oracle import gateup, hadamard, numfmt, quant, router
from tests.gpu_util import (assert_close, bf16_bits_of, bf16_cuda, check_rotation, check_with_rotation_slack,
                            fwht_tie_window, near_tie_mask)

pytestmark = pytest.mark.gpu

PATHS = ("gemv", "gemm", "tall", "skinny")


def quantized_layer(L):
    """Dense weights -> rotation -> int8 codes via the oracle quantizer."""
    w = np.stack([synth.dense_weights(L, e) for e in range(L.E)]).astype(np.float64)
    codes, scales, _ = quant.quantize_i8h(hadamard.rotate_blocks(w))
    return codes, numfmt.bf16_to_bits(scales)


def run_gpu(x_rot_bits, codes, scale_bits, off, sp, k, path, want_gu=True, want_act=True):
    return i8h.moe_gateup_i8h_grouped(
        bf16_cuda(x_rot_bits), torch.from_numpy(codes).cuda(), bf16_cuda(scale_bits), k,
        torch.from_numpy(off.astype(np.int32)).cuda(), torch.from_numpy(sp.astype(np.int32)).cuda(),
        gate_up=want_gu, act=want_act, path=path)


def compare(gu, act, x_rot, codes, scale_bits, off, sp, k, rows=None, what=""):
    torch.cuda.synchronize()
    scales = numfmt.bf16_from_bits(scale_bits)
    ref = gateup.gateup_i8h(x_rot, codes, scales, off, sp, k, rows=rows)
    sel = slice(None) if rows is None else np.asarray(rows)
    if gu is not None:
        assert_close(gu.cpu().numpy()[sel], ref, what + " gate_up")
    if act is not None:
        assert_close(act.cpu().numpy()[sel], gateup.epilogue(ref), what + " act")


def check_summation_bound(gu, act, x, codes, scales, off, sp, k, what):
    """gate_up and act against the oracle where the sums may cancel.

    gate_up: |gpu - ref| <= max(1e-4 |ref| + 1e-5, gamma * sum|terms|), with
    gamma = (K + 2G + 2) 2^-24, the textbook bound on a float32 evaluation of
    K exact products in any summation order, their G scale multiplies and the
    tall kernel's two roundings per group rescale. It equals the relative
    tolerance where sum|terms| <= 3.2 |ref| (K = 512) and takes over only
    where cancellation makes 1e-4 of the result unreachable in float32.
    Outputs with sum|terms| <= 16 |ref| must meet the relative tolerance
    itself (a float32 sum loses about sqrt(depth) 2^-24 sum|terms| there,
    under 2e-5 of the result). act: its tolerance plus those bounds carried
    through the epilogue (|gelu'| < 1.13). Returns the share of outputs where
    the summation bound is the binding one."""
    K = codes.shape[-1]
    G = K // 128
    ref = gateup.gateup_i8h(x, codes, scales, off, sp, k)
    mag = gateup.gateup_i8h(np.abs(x), np.abs(codes.astype(np.int16)).astype(np.int8), scales, off, sp, k)
    g = gu.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(g)), what + ": non-finite gate_up"
    strict = 1e-4 * np.abs(ref) + 1e-5
    lim = np.maximum(strict, (K + 2 * G + 2) * 2.0 ** -24 * mag)
    err = np.abs(g - ref)
    assert np.all(err <= lim), f"{what}: worst ratio to the bound {np.max(err / lim):.3g}"
    well = mag <= 16 * np.abs(ref)
    assert np.all(err[well] <= strict[well]), f"{what}: well-conditioned worst {np.max(err[well] / strict[well]):.3g}"
    I = codes.shape[1] // 2
    gg, uu = ref[:, :I], ref[:, I:]
    lg, lu = lim[:, :I], lim[:, I:]
    extra = 1.13 * lg * (np.abs(uu) + lu) + np.abs(gateup.gelu_tanh(gg)) * lu
    ref_act = gateup.epilogue(ref)
    a = act.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(a)), what + ": non-finite act"
    assert np.all(np.abs(a - ref_act) <= 1e-4 * np.abs(ref_act) + 1e-5 + extra), what + " act"
    return float(np.mean(lim > strict))


def oracle_inputs(L, T=None):
    lg = synth.router_logits(L)
    x = synth.bf16_bits_to_f64(synth.activations_bf16(L))
    x_rot = hadamard.rotate_activations_bf16(x)
    r = router.route(lg, L.topk)
    return x_rot, numfmt.bf16_to_bits(x_rot), r


def sample_rows(off, n_extra, seed):
    """First and last row of every non-empty expert, plus random rows."""
    off = np.asarray(off)
    rows = set()
    for e in range(off.size - 1):
        if off[e + 1] > off[e]:
            rows.add(int(off[e]))
            rows.add(int(off[e + 1] - 1))
    rng = np.random.default_rng(seed)
    rows.update(rng.integers(0, off[-1], n_extra).tolist())
    return np.array(sorted(rows))


@pytest.fixture(scope="module")
def tiny():
    L = synth.layer("tiny")
    codes, sbits = quantized_layer(L)
    x_rot, xrb, r = oracle_inputs(L)
    return L, codes, sbits, x_rot, xrb, r


@pytest.mark.parametrize("path", PATHS)
def test_tiny_layer(gpu_available, tiny, path):
    L, codes, sbits, x_rot, xrb, r = tiny
    print(f"gateup tiny {path}", flush=True)
    gu, act = run_gpu(xrb, codes, sbits, r["expert_off"], r["sorted_pairs"], L.topk, path)
    compare(gu, act, x_rot, codes, sbits, r["expert_off"], r["sorted_pairs"], L.topk, what=f"tiny/{path}")


@pytest.mark.parametrize("path", PATHS)
def test_mid_layer_oracle_quantized(gpu_available, path):
    # real K and N, several m-tiles per expert, ragged expert loads
    L = synth.layer("verify", T=40, E=8, topk=3)
    codes, sbits = quantized_layer(L)
    x_rot, xrb, r = oracle_inputs(L)
    print(f"gateup mid {path}", flush=True)
    gu, act = run_gpu(xrb, codes, sbits, r["expert_off"], r["sorted_pairs"], L.topk, path)
    compare(gu, act, x_rot, codes, sbits, r["expert_off"], r["sorted_pairs"], L.topk, what=f"mid/{path}")


_FULL = {}


def full_layer(name):
    if name not in _FULL:
        L = synth.layer(name)
        codes, sbits = synth.synthetic_i8h(L)
        x_rot, xrb, r = oracle_inputs(L)
        dev = dict(codes=torch.from_numpy(codes).cuda(), scales=bf16_cuda(sbits), x=bf16_cuda(xrb),
                   off=torch.from_numpy(r["expert_off"]).cuda(), sp=torch.from_numpy(r["sorted_pairs"]).cuda())
        _FULL.clear()   # keep one full layer resident at a time
        _FULL[name] = (L, codes, sbits, x_rot, r, dev)
    return _FULL[name]


@pytest.mark.parametrize("name", ["decode", "verify", "prefill"])
@pytest.mark.parametrize("path", ("auto",) + PATHS)
def test_full_size_sampled(gpu_available, name, path):
    L, codes, sbits, x_rot, r, d = full_layer(name)
    print(f"gateup full {name} {path}", flush=True)
    gu, act = i8h.moe_gateup_i8h_grouped(d["x"], d["codes"], d["scales"], L.topk, d["off"], d["sp"], path=path)
    rows = sample_rows(r["expert_off"], 48, seed=L.seed)
    compare(gu, act, x_rot, codes, sbits, r["expert_off"], r["sorted_pairs"], L.topk, rows=rows,
            what=f"{name}/{path}")


@pytest.mark.parametrize("name", ["verify", "prefill"])
def test_step_as_timed(gpu_available, name):
    """The verify and prefill steps as the benchmark times them, at full size:
    moe_route_permute_rotate (routing and the rotation of the token rows in
    one launch), then the grouped product with the kernel AUTO picks. The
    routing must match the oracle bit for bit and x_rot be the oracle's
    rounding of the exact rotation (one bf16 step allowed where the exact
    value sits on a rounding tie); the product on that x_rot is then held to
    the usual tolerance on sampled rows (every expert's first and last row)."""
    L, codes, sbits, _, r, d = full_layer(name)
    lg = synth.router_logits(L)
    xb = synth.activations_bf16(L)
    print(f"gateup step as timed {name}", flush=True)
    ro = i8h.moe_route_permute_rotate(torch.from_numpy(lg).cuda(), bf16_cuda(xb), L.topk)
    gu, act = i8h.moe_gateup_i8h_grouped(ro["x_rot"], d["codes"], d["scales"], L.topk, ro["expert_off"],
                                         ro["sorted_pairs"])
    torch.cuda.synchronize()
    for key, want in (("topk_ids", r["ids"]), ("expert_off", r["expert_off"]),
                      ("sorted_pairs", r["sorted_pairs"]), ("pair_pos", r["pair_pos"])):
        assert np.array_equal(ro[key].cpu().numpy(), np.asarray(want).reshape(ro[key].shape)), key
    xr_bits = ro["x_rot"].view(torch.int16).cpu().numpy().view(np.uint16)
    check_rotation(xb, xr_bits)
    rows = sample_rows(r["expert_off"], 48, seed=L.seed + 1)
    compare(gu, act, numfmt.bf16_from_bits(xr_bits), codes, sbits, r["expert_off"], r["sorted_pairs"], L.topk,
            rows=rows, what=f"step/{name}")


def _random_case(T, K, E, k, N, seed, code_range=127, xscale=1.0, scale_mag=4e-4):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    r = router.route(lg, k)
    xb = synth.to_bf16_bits((rng.standard_normal((T, K)) * xscale).astype(np.float32))
    codes = rng.integers(-code_range, code_range + 1, size=(E, N, K)).astype(np.int8)
    sb = synth.to_bf16_bits((rng.uniform(0.5, 2.0, (E, N, K // 128)) * scale_mag).astype(np.float32))
    return numfmt.bf16_from_bits(xb), xb, codes, sb, r


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("T,K,E,k,N", [
    (300, 256, 1, 1, 64),      # one expert, five m-passes, the smallest N
    (5, 128, 64, 2, 128),      # one group, many empty experts
    (7, 4096, 4, 4, 192),      # k == E, the decode kernel's largest K
    (33, 384, 3, 2, 320),      # ragged everything
    (1, 2048, 128, 8, 1536),   # one decode token
])
def test_edge_shapes(gpu_available, path, T, K, E, k, N):
    x, xb, codes, sb, r = _random_case(T, K, E, k, N, seed=T + K + E + k + N)
    print(f"gateup edge {path} T={T} K={K} E={E} k={k} N={N}", flush=True)
    gu, act = run_gpu(xb, codes, sb, r["expert_off"], r["sorted_pairs"], k, path)
    compare(gu, act, x, codes, sb, r["expert_off"], r["sorted_pairs"], k, what=f"edge/{path}")


@pytest.mark.parametrize("path", ("auto", "tall"))
def test_gemm_only_large_k(gpu_available, path):
    x, xb, codes, sb, r = _random_case(6, 8192, 3, 2, 128, seed=11)
    gu, act = run_gpu(xb, codes, sb, r["expert_off"], r["sorted_pairs"], 2, path)
    compare(gu, act, x, codes, sb, r["expert_off"], r["sorted_pairs"], 2, what=f"K8192/{path}")


@pytest.mark.parametrize("path", PATHS)
def test_zero_scales_with_nonzero_codes(gpu_available, path):
    # a zero scale removes its group whatever the codes: single groups, a
    # group zero for every row, whole rows of zeros, the first and the last
    # group (the tall kernel keeps the running result in units of the last
    # nonzero scale and masks such groups)
    x, xb, codes, sb, r = _random_case(40, 1024, 4, 2, 256, seed=13)
    s = numfmt.bf16_from_bits(sb).copy()
    rng = np.random.default_rng(14)
    s[rng.random(s.shape) < 0.1] = 0.0
    s[:, :, 0] = 0.0          # the first group of every row
    s[1, :, 7] = 0.0          # the last group of one expert
    s[2, 5, :] = 0.0          # a whole row
    s[3, 17, 1:] = 0.0        # only the first group left
    sb = numfmt.bf16_to_bits(s)
    gu, act = run_gpu(xb, codes, sb, r["expert_off"], r["sorted_pairs"], 2, path)
    compare(gu, act, x, codes, sb, r["expert_off"], r["sorted_pairs"], 2, what=f"zero-scales/{path}")


@pytest.mark.parametrize("path", PATHS)
def test_extreme_values(gpu_available, path):
    # full-range codes, large activations, scales spanning 40 octaves (2^-20
    # .. 2^20) across groups, a zero scale; sums of such terms can cancel, see
    # check_summation_bound
    rng = np.random.default_rng(12)
    T, K, E, k, N = 9, 512, 4, 2, 128
    x, xb, codes, sb, r = _random_case(T, K, E, k, N, seed=12, xscale=300.0)
    codes[:, :, :64] = 127
    codes[:, 3, :] = -127
    s = numfmt.bf16_from_bits(sb)
    s *= np.exp2(rng.integers(-20, 21, s.shape))
    s[0, 5, 1] = 0.0
    sb = numfmt.bf16_to_bits(numfmt.bf16_round(s))
    print(f"gateup extreme {path}", flush=True)
    gu, act = run_gpu(xb, codes, sb, r["expert_off"], r["sorted_pairs"], k, path)
    torch.cuda.synchronize()
    share = check_summation_bound(gu, act, x, codes, numfmt.bf16_from_bits(sb), r["expert_off"],
                                  r["sorted_pairs"], k, f"extreme/{path}")
    print(f"  summation bound binding on {100 * share:.1f}% of outputs", flush=True)


@pytest.mark.parametrize("path", ("auto",) + PATHS)
def test_scale_ratios_beyond_float_range(gpu_available, path):
    # Within single rows, group scales 2^0, 2^-60, 2^-120, a subnormal bf16
    # (2^-130) and zero, in every order, at a prefill-like load (128 pairs per
    # expert: AUTO takes the tall kernel, which keeps its running result in
    # units of the current scale). Ratios between consecutive scales reach
    # 2^130, beyond float32's range: every output must stay finite and match.
    T, K, E, k, N = 256, 1024, 4, 2, 256
    x, xb, codes, sb, r = _random_case(T, K, E, k, N, seed=17)
    rng = np.random.default_rng(18)
    G = K // 128
    levels = np.array([1.0, 2.0 ** -60, 2.0 ** -120, 2.0 ** -130, 0.0])
    pick = rng.integers(0, levels.size, (E, N, G))
    s = levels[pick] * rng.uniform(1.0, 2.0, (E, N, G))
    s[0, :, :] = levels[np.arange(N * G).reshape(N, G) % levels.size]   # every level at every group slot
    s[1, 0] = [0, 0, 2.0 ** -130, 1.0, 2.0 ** -130, 1.0, 0, 2.0 ** -120]  # subnormal first, then back and forth
    s[1, 1] = [2.0 ** -120, 2.0 ** -120, 2.0 ** -60, 2.0 ** -60, 1.0, 1.0, 2.0 ** -130, 2.0 ** -130]
    s[1, 2] = [2.0 ** -130] * G                                         # subnormal only
    s[1, 3] = [1.0, 2.0 ** -60, 2.0 ** -120, 2.0 ** -130, 0, 2.0 ** -120, 2.0 ** -60, 1.0]
    s[2, N // 2:] = 2.0 ** -125                                         # up rows all tiny, gate rows mixed
    sb = numfmt.bf16_to_bits(numfmt.bf16_round(s))
    assert numfmt.bf16_from_bits(sb)[1, 2, 0] == 2.0 ** -130            # a bf16 subnormal kept as such
    print(f"gateup scale ratios {path}", flush=True)
    gu, act = run_gpu(xb, codes, sb, r["expert_off"], r["sorted_pairs"], k, path)
    torch.cuda.synchronize()
    share = check_summation_bound(gu, act, x, codes, numfmt.bf16_from_bits(sb), r["expert_off"],
                                  r["sorted_pairs"], k, f"scale ratios/{path}")
    print(f"  summation bound binding on {100 * share:.1f}% of outputs", flush=True)


@pytest.mark.parametrize("path", PATHS)
def test_single_output(gpu_available, tiny, path):
    L, codes, sbits, x_rot, xrb, r = tiny
    gu, act = run_gpu(xrb, codes, sbits, r["expert_off"], r["sorted_pairs"], L.topk, path, want_gu=False)
    assert gu is None
    compare(None, act, x_rot, codes, sbits, r["expert_off"], r["sorted_pairs"], L.topk, what="act only")
    gu, act = run_gpu(xrb, codes, sbits, r["expert_off"], r["sorted_pairs"], L.topk, path, want_act=False)
    compare(gu, None, x_rot, codes, sbits, r["expert_off"], r["sorted_pairs"], L.topk, what="gu only")


@pytest.mark.parametrize("path", PATHS)
def test_deterministic(gpu_available, path):
    L, codes, sbits, x_rot, r, d = full_layer("verify")
    a = i8h.moe_gateup_i8h_grouped(d["x"], d["codes"], d["scales"], L.topk, d["off"], d["sp"], path=path)
    b = i8h.moe_gateup_i8h_grouped(d["x"], d["codes"], d["scales"], L.topk, d["off"], d["sp"], path=path)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("name,T", [("tiny", None), ("decode", None), ("verify", 8), ("verify", 9),
                                    ("verify", None)])
def test_fused_rotation(gpu_available, name, T):
    """moe_gateup_i8h_grouped_fused (rotation inside the call) against the
    oracle chain, with the tolerance widened only where the bf16 rotation may
    round either way (as in the end-to-end test)."""
    L = synth.layer(name) if T is None else synth.layer(name, T=T)
    lg = synth.router_logits(L)
    xb = synth.activations_bf16(L)
    x = synth.bf16_bits_to_f64(xb)
    r = router.route(lg, L.topk)
    used = sorted(set(r["ids"].reshape(-1).tolist()))
    c_used, s_used = synth.synthetic_i8h(L, experts=used)
    codes = np.zeros((L.E, L.N, L.K), dtype=np.int8)
    sbits = np.zeros((L.E, L.N, L.G), dtype=np.uint16)
    codes[used], sbits[used] = c_used, s_used
    print(f"gateup fused {name} T={L.T}", flush=True)
    gu, act = i8h.moe_gateup_i8h_grouped_fused(
        bf16_cuda(xb), torch.from_numpy(codes).cuda(), bf16_cuda(sbits), L.topk,
        torch.from_numpy(r["expert_off"]).cuda(), torch.from_numpy(r["sorted_pairs"]).cuda())
    torch.cuda.synchronize()
    check_with_rotation_slack(x, codes, sbits, r, L.topk, gu, act)


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_end_to_end_on_gpu(gpu_available, name):
    """route -> rotate -> gate_up, all on the GPU, against the oracle chain."""
    L = synth.layer(name)
    if name == "tiny":
        codes, sbits = quantized_layer(L)
    else:
        lg0 = synth.router_logits(L)
        used = sorted(set(router.topk(lg0, L.topk)[0].reshape(-1).tolist()))
        c_used, s_used = synth.synthetic_i8h(L, experts=used)
        codes = np.zeros((L.E, L.N, L.K), dtype=np.int8)
        sbits = np.zeros((L.E, L.N, L.G), dtype=np.uint16)
        codes[used], sbits[used] = c_used, s_used
    lg = synth.router_logits(L)
    xb = synth.activations_bf16(L)
    x = synth.bf16_bits_to_f64(xb)
    # oracle chain
    r = router.route(lg, L.topk)
    exact = hadamard.rotate_blocks(x)
    x_rot = numfmt.bf16_round(exact)
    scales = numfmt.bf16_from_bits(sbits)
    ref = gateup.gateup_i8h(x_rot, codes, scales, r["expert_off"], r["sorted_pairs"], L.topk)
    # GPU chain
    ro = i8h.moe_route_permute(torch.from_numpy(lg).cuda(), L.topk)
    xr = i8h.hadamard128_rotate(bf16_cuda(xb))
    gu, act = i8h.moe_gateup_i8h_grouped(xr, torch.from_numpy(codes).cuda(), bf16_cuda(sbits), L.topk,
                                         ro["expert_off"], ro["sorted_pairs"])
    torch.cuda.synchronize()
    assert np.array_equal(ro["sorted_pairs"].cpu().numpy(), r["sorted_pairs"])
    # where the rotation may round either way, allow one bf16 step of x_rot
    tie = near_tie_mask(exact, fwht_tie_window(x))
    ulp = np.ldexp(1.0, np.frexp(np.abs(x_rot) + 1e-300)[1] - 8)
    slack_x = np.where(tie, ulp, 0.0)                         # [T, K]
    off, sp = r["expert_off"], r["sorted_pairs"]
    what = quant.dequantize_i8h(codes, scales)
    slack = np.zeros_like(ref)
    for row in range(ref.shape[0]):
        e = np.searchsorted(off, row, side="right") - 1
        slack[row] = np.abs(what[e]) @ slack_x[sp[row] // L.topk]
    g = gu.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(g - ref) <= 1e-4 * np.abs(ref) + 1e-5 + slack)
    # act: bound the effect of the gate/up slack through gelu (|gelu'| < 1.13)
    I = L.N // 2
    ref_act = gateup.epilogue(ref)
    dg, du = slack[:, :I], slack[:, I:]
    act_slack = 1.13 * dg * (np.abs(ref[:, I:]) + du) + np.abs(gateup.gelu_tanh(ref[:, :I])) * du
    a = act.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(a - ref_act) <= 1e-4 * np.abs(ref_act) + 1e-5 + act_slack)
