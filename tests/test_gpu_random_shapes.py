"""GPU parity on seeded random shapes: every entry of the hot path against the oracle.

Each case draws T, K, E, topk and N from a fixed seed (small and large token
counts, K up to 5120, up to 256 experts, topk up to 32, N from 64 to 2048);
two more take 1024 experts with top-32 and top-k equal to the expert count.
Each runs, on the generator's inputs:
  - routing + rotation: ids, expert_off, sorted_pairs and pair_pos equal to
    the oracle's, weights within 1e-4 relative + 1e-5, x_rot equal up to the
    proven float32 tie window;
  - the one-launch decode form where it applies (T*topk <= 64, E <= 256,
    K <= 4096), against the oracle chain with the rotation's tie slack;
  - gate_up on every i8h kernel (GEMV, 128-pair GEMM, tall, small-unit,
    AUTO), the FP8 forms (GEMM, small-unit, AUTO; N a multiple of 128) and
    W8A8, each with float32 act and with bf16 act (bit-equal to the float32
    act rounded), on sampled expert-sorted rows (the first and last row of
    every non-empty expert plus random ones), within
    max(1e-4 |ref| + 1e-5, (K + 2G + 2) 2^-24 sum|terms|), the float32
    summation bound (the relative tolerance itself wherever
    sum|terms| <= 16 |ref|), carried through the epilogue to act;
  - the down projection + combine (GEMV and GEMM forms where they apply,
    AUTO) on float32 and bf16 act rows (bit-equal outputs), on sampled
    tokens within max(1e-4 |ref| + 1e-5, (I + topk + 4) 2^-24 sum|terms|).
The quantized activations the FP8 and W8A8 calls keep in their workspace are
compared bit for bit.
"""

import numpy as np
import pytest
import torch

import int8_hadamard_domain_amd as i8h
import synth
from oracle import down, gateup, hadamard, numfmt, quant, router, w8a8
from tests.gpu_util import assert_close, bf16_bits_of, bf16_cuda, check_rotation, check_with_rotation_slack

pytestmark = pytest.mark.gpu


def _draw_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        T = int(rng.choice([1, 2, 3, 5, 8, 16, 31, 64, 65, 127, 255, 257, 511, 1023, 1500, 2048]))
        T = max(1, T + int(rng.integers(-1, 2)))
        K = 128 * int(rng.choice([1, 2, 3, 8, 16, 24, 32, 33, 40]))
        E = int(rng.choice([1, 2, 4, 7, 8, 9, 32, 64, 128, 200, 256]))
        k = int(rng.integers(1, min(E, 32) + 1)) if rng.random() < 0.3 else int(rng.integers(1, min(E, 8) + 1))
        N = 64 * int(rng.choice([1, 2, 3, 4, 6, 8, 12, 24, 32]))
        # sized so one case's host-side generation and oracle stay near a second
        if E * N * K <= 2 ** 27 and T * K <= 2 ** 23 and T * k * N <= 2 ** 24:
            out.append((T, K, E, k, N, 7000 + len(out)))
    return out


# plus the limits the entry points accept: the most experts (1024) with the
# largest top-k (32), and top-k equal to the expert count (every token in
# every expert)
CASES = _draw_cases(32, 20261203) + [(300, 256, 1024, 32, 128, 7100), (65, 384, 32, 32, 192, 7101)]


def _sample_rows(off, rng, n=24):
    off = np.asarray(off)
    rows = set(rng.integers(0, int(off[-1]), size=min(n, int(off[-1]))).tolist())
    for e in range(len(off) - 1):
        if off[e + 1] > off[e]:
            rows.update((int(off[e]), int(off[e + 1] - 1)))
    return np.array(sorted(rows), dtype=np.int64)


def _abs_i8(c):
    a = np.abs(np.asarray(c).astype(np.int16))
    assert a.max() <= 127
    return a.astype(np.int8)


def _gateup_bound(g, ref, mag, K, what):
    G = K // 128
    g = np.asarray(g, dtype=np.float64)
    assert np.all(np.isfinite(g)), what + ": non-finite gate_up"
    strict = 1e-4 * np.abs(ref) + 1e-5
    lim = np.maximum(strict, (K + 2 * G + 2) * 2.0 ** -24 * mag)
    err = np.abs(g - ref)
    assert np.all(err <= lim), f"{what}: {(err > lim).sum()} outside, worst ratio {np.max(err / lim):.3g}"
    # where the sum hardly cancels the relative tolerance itself must hold
    well = mag <= 16 * np.abs(ref)
    assert np.all(err[well] <= strict[well]), f"{what}: well-conditioned outputs outside 1e-4 |ref| + 1e-5"
    return lim


def _act_bound(a, ref, lim, what):
    I = ref.shape[1] // 2
    extra = 1.13 * lim[:, :I] * (np.abs(ref[:, I:]) + lim[:, I:]) + np.abs(gateup.gelu_tanh(ref[:, :I])) * lim[:, I:]
    ref_act = gateup.epilogue(ref)
    a = np.asarray(a, dtype=np.float64)
    assert np.all(np.isfinite(a)), what + ": non-finite act"
    bad = np.abs(a - ref_act) > 1e-4 * np.abs(ref_act) + 1e-5 + extra
    assert not bad.any(), f"{what}: act {bad.sum()} outside"


def _both_acts(call, what):
    """call(act_dtype) -> (gate_up, act, ...); the bf16-act call must give the
    same gate_up and the float32 act rounded to nearest even."""
    r32 = call(torch.float32)
    r16 = call(torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(r16[0], r32[0]), what + ": gate_up of the bf16-act call differs"
    want = r32[1].to(torch.bfloat16).view(torch.int16)
    assert torch.equal(r16[1].view(torch.int16), want), what + ": bf16 act is not the float32 act rounded"
    return r32


@pytest.mark.parametrize("T,K,E,k,N,seed", CASES, ids=[f"T{c[0]}-K{c[1]}-E{c[2]}-k{c[3]}-N{c[4]}" for c in CASES])
def test_random_shape(T, K, E, k, N, seed):
    rng = np.random.default_rng(seed)
    L = synth.layer("decode", T=T, K=K, E=E, topk=k, N=N, seed=seed)
    lg = synth.router_logits(L)
    xb = synth.activations_bf16(L)
    x = synth.bf16_bits_to_f64(xb)
    r = router.route(lg, k)
    off, sp = r["expert_off"], r["sorted_pairs"]
    rows = _sample_rows(off, rng)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a).astype(np.int32)).cuda()
    goff, gsp = i32(off), i32(sp)
    print(f"random shape T={T} K={K} E={E} k={k} N={N}: routing", flush=True)
    gr = i8h.moe_route_permute_rotate(torch.from_numpy(lg).cuda(), bf16_cuda(xb), k)
    torch.cuda.synchronize()
    for key, want in (("topk_ids", r["ids"]), ("expert_off", off), ("sorted_pairs", sp), ("pair_pos", r["pair_pos"])):
        assert np.array_equal(gr[key].cpu().numpy(), want), key
    w32 = gr["topk_w"].cpu().numpy()
    assert_close(w32, r["weights"], "topk_w")
    check_rotation(xb, bf16_bits_of(gr["x_rot"]))

    codes, sbits = synth.synthetic_i8h(L)
    gc, gs = torch.from_numpy(codes).cuda(), bf16_cuda(sbits)
    if T * k <= 64 and E <= 256 and K <= 4096:
        print("  one-launch decode", flush=True)
        ro, gu, ac = i8h.moe_route_gateup_i8h_decode(torch.from_numpy(lg).cuda(), bf16_cuda(xb), gc, gs, k)
        torch.cuda.synchronize()
        for key in ("topk_ids", "expert_off", "sorted_pairs", "pair_pos"):
            got = ro[key].cpu().numpy()
            assert np.array_equal(got, r["ids" if key == "topk_ids" else key].reshape(got.shape)), "decode " + key
        check_with_rotation_slack(x, codes, sbits, r, k, gu, ac)

    x_rot = hadamard.rotate_activations_bf16(x)
    xrb = bf16_cuda(numfmt.bf16_to_bits(x_rot))
    scales = numfmt.bf16_from_bits(sbits)
    ref = gateup.gateup_i8h(x_rot, codes, scales, off, sp, k, rows=rows)
    mag = gateup.gateup_i8h(np.abs(x_rot), _abs_i8(codes), scales, off, sp, k, rows=rows)
    for path in ("gemv", "gemm", "tall", "skinny", "auto"):
        if path == "gemv" and K > 4096:
            continue
        print(f"  i8h {path}", flush=True)
        gu, act = _both_acts(lambda dt: i8h.moe_gateup_i8h_grouped(xrb, gc, gs, k, goff, gsp, path=path,
                                                                   act_dtype=dt), f"i8h {path}")
        lim = _gateup_bound(gu.cpu().numpy()[rows], ref, mag, K, f"i8h {path}")
        _act_bound(act.cpu().numpy()[rows], ref, lim, f"i8h {path}")

    if N % 128 == 0:
        fcodes, fsbits = synth.synthetic_fp8(L)
        fscales = numfmt.bf16_from_bits(fsbits)
        qx, sx = quant.quantize_fp8_activations(x)
        fref = gateup.gateup_fp8blk(qx, sx, fcodes, fscales, off, sp, k, rows=rows)
        fmag = gateup.gateup_fp8blk(qx & 0x7F, sx, fcodes & 0x7F, fscales, off, sp, k, rows=rows)
        gfc, gfs, gx = torch.from_numpy(fcodes).cuda(), bf16_cuda(fsbits), bf16_cuda(xb)
        for path in ("gemm", "skinny", "auto"):
            print(f"  fp8 {path}", flush=True)
            gu, act, ws = _both_acts(lambda dt: i8h.moe_gateup_fp8blk_grouped(gx, gfc, gfs, k, goff, gsp, path=path,
                                                                               act_dtype=dt), f"fp8 {path}")
            gq, gsx, _ = i8h.fp8_workspace_views(ws, T, K)
            assert np.array_equal(gq.cpu().numpy(), qx) and np.array_equal(gsx.cpu().numpy(), sx), "fp8 quantizer"
            lim = _gateup_bound(gu.cpu().numpy()[rows], fref, fmag, K, f"fp8 {path}")
            _act_bound(act.cpu().numpy()[rows], fref, lim, f"fp8 {path}")

    print("  w8a8", flush=True)
    qx, sx = w8a8.quantize_i8_activations(x)
    iref = w8a8.gateup_i8g(qx, sx, codes, scales, off, sp, k, rows=rows)
    imag = w8a8.gateup_i8g(_abs_i8(qx), sx, _abs_i8(codes), scales, off, sp, k, rows=rows)
    gx = bf16_cuda(xb)
    gu, act, ws = _both_acts(lambda dt: i8h.moe_gateup_i8g_grouped(gx, gc, gs, k, goff, gsp, act_dtype=dt), "w8a8")
    gq, gsx = i8h.i8g_workspace_views(ws, T, K)
    assert np.array_equal(gq.cpu().numpy(), qx) and np.array_equal(gsx.cpu().numpy(), sx), "w8a8 quantizer"
    lim = _gateup_bound(gu.cpu().numpy()[rows], iref, imag, K, "w8a8")
    _act_bound(act.cpu().numpy()[rows], iref, lim, "w8a8")

    # down projection: hidden size H = K, I = N / 2
    H, I = K, N // 2
    used = sorted(set(r["ids"].ravel().tolist()))
    wbits = np.zeros((E, H, I), dtype=np.uint16)
    wbits[used] = synth.down_weights_bf16(L, experts=used)
    w = synth.bf16_bits_to_f64(wbits)
    a = synth.act_f32(L)
    toks = np.unique(rng.integers(0, T, size=min(T, 16)))
    pos = np.asarray(r["pair_pos"]).reshape(T, k)[toks].ravel()
    y = down.down_grouped(a, w, off, rows=pos).reshape(toks.size, k, H)
    ya = down.down_grouped(np.abs(a), np.abs(w), off, rows=pos).reshape(toks.size, k, H)
    wts = w32.astype(np.float64)      # the router weights the GPU stored
    dref = sum(wts[toks, j:j + 1] * y[:, j] for j in range(k))
    dmag = sum(np.abs(wts[toks, j:j + 1]) * ya[:, j] for j in range(k))
    dlim = np.maximum(1e-4 * np.abs(dref) + 1e-5, (I + k + 4) * 2.0 ** -24 * dmag)
    ga = torch.from_numpy(a).cuda()
    paths = (["gemv"] if I <= 1024 else []) + (["gemm"] if I % 32 == 0 and I >= 96 and H % 256 == 0 else [])
    for path in paths + ["auto"]:
        print(f"  down {path}", flush=True)
        o32 = i8h.moe_down_bf16_combine(ga, bf16_cuda(wbits), gr, path=path)
        o16 = i8h.moe_down_bf16_combine(ga.to(torch.bfloat16), bf16_cuda(wbits), gr, path=path)
        torch.cuda.synchronize()
        o = o32.cpu().numpy()[toks].astype(np.float64)
        err = np.abs(o - dref)
        assert np.all(err <= dlim), f"down {path}: worst ratio {np.max(err / dlim):.3g}"
        assert torch.equal(o16, o32), f"down {path}: bf16-act form differs"
