"""GPU parity: moe_down_bf16_combine (both forms) against the oracle.

Elementwise |gpu - oracle| <= 1e-4 |oracle| + 1e-5 on out [T, H]. Each case
feeds both sides the same routing (the oracle router's, with the weights
rounded to float32 as the routing call stores them), the same float32 act
rows and the same bf16 down weights, so the comparison checks this step
alone. Full-size layers (decode, verify, prefill) are checked on sampled
tokens, every output column of each; smaller cases in full. Cases cover
ragged experts (empty ones, one with more than 256 pairs so the GEMM form
runs two passes), k = 1, I below one lane piece per lane, and I = 1024.
"""

import numpy as np
import pytest
import torch

import int8_hadamard_domain_amd as i8h
import synth
from oracle import down, router
from tests.gpu_util import assert_close, bf16_cuda

pytestmark = pytest.mark.gpu


def make_case(T, I, E, k, H, seed, bias=None, experts_used=None):
    L = synth.layer("decode", T=T, K=H, E=E, topk=k, N=2 * I, seed=seed)
    lg = synth.router_logits(L)
    if bias is not None:
        lg = (lg + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)
    r = router.route(lg, k)
    r["weights"] = r["weights"].astype(np.float32).astype(np.float64)    # what the routing call stores
    used = sorted(set(r["ids"].ravel().tolist())) if experts_used is None else experts_used
    wbits = np.zeros((E, H, I), dtype=np.uint16)
    wbits[used] = synth.down_weights_bf16(L, experts=used)
    act = synth.act_f32(L)
    return r, wbits, act


def gpu_routing(r):
    c = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a).astype(dt)).cuda()
    return {"topk_ids": c(r["ids"], np.int32), "topk_w": c(r["weights"], np.float32),
            "expert_off": c(r["expert_off"], np.int32), "pair_pos": c(r["pair_pos"], np.int32)}


def oracle_out(r, wbits, act, k, tokens=None):
    """out rows of the requested tokens (all by default), via sampled y rows."""
    w = synth.bf16_bits_to_f64(wbits)
    t_count = r["ids"].shape[0]
    tok = np.arange(t_count) if tokens is None else np.asarray(tokens)
    pos = np.asarray(r["pair_pos"]).reshape(t_count, k)[tok]          # [t', k] sorted rows
    y = down.down_grouped(act, w, r["expert_off"], rows=pos.ravel())
    yk = y.reshape(tok.size, k, -1)
    out = np.zeros((tok.size, yk.shape[2]))
    for j in range(k):
        out += r["weights"][tok, j:j + 1] * yk[:, j]
    return out


def run(r, wbits, act, path):
    out = i8h.moe_down_bf16_combine(torch.from_numpy(act).cuda(), bf16_cuda(wbits), gpu_routing(r), path=path)
    torch.cuda.synchronize()
    return out.cpu().numpy()


CASES = [
    # T, I, E, k, H, seed
    (4, 128, 8, 2, 256, 0),
    (1, 768, 128, 8, 2048, 1),
    (3, 96, 5, 4, 512, 7),
    (2, 1024, 16, 3, 256, 8),
    (7, 768, 12, 1, 512, 9),
    (40, 256, 12, 8, 256, 10),
]


@pytest.mark.parametrize("T,I,E,k,H,seed", CASES)
@pytest.mark.parametrize("path", ["gemv", "gemm", "auto"])
def test_down_small(T, I, E, k, H, seed, path):
    r, wbits, act = make_case(T, I, E, k, H, seed)
    ref = oracle_out(r, wbits, act, k)
    assert_close(run(r, wbits, act, path), ref, f"down {path} T{T} I{I} E{E} k{k} H{H}")


@pytest.mark.parametrize("path", ["gemm", "gemv", "auto"])
def test_down_ragged_experts_and_two_passes(path):
    # 4 experts, 2 of them never chosen; one takes more than 256 pairs
    E, k, T = 6, 2, 400
    bias = np.array([3.0, 2.5, -30.0, 0.0, -30.0, 0.0], dtype=np.float32)
    r, wbits, act = make_case(T, 256, E, k, 512, 21, bias=bias)
    counts = np.diff(r["expert_off"])
    assert counts.max() > 256 and (counts == 0).any()
    ref = oracle_out(r, wbits, act, k)
    assert_close(run(r, wbits, act, path), ref, f"down ragged {path}")


def test_forms_agree_and_repeat_bit_for_bit():
    r, wbits, act = make_case(40, 256, 12, 8, 256, 10)
    a = run(r, wbits, act, "gemm")
    b = run(r, wbits, act, "gemm")
    c = run(r, wbits, act, "gemv")
    d = run(r, wbits, act, "gemv")
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(c, d)
    assert_close(a, c.astype(np.float64), "gemm vs gemv", rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("name", ["decode", "verify", "prefill"])
def test_down_full_size(name):
    """The layer sizes of the workloads (K = H = 2048, I = 768, E = 128, top-8),
    in the form AUTO picks and bench.py times, on sampled tokens."""
    L = synth.layer(name)
    r = router.route(synth.router_logits(L), L.topk)
    r["weights"] = r["weights"].astype(np.float32).astype(np.float64)
    used = sorted(set(r["ids"].ravel().tolist()))
    wbits = np.zeros((L.E, L.K, L.I), dtype=np.uint16)
    wbits[used] = synth.down_weights_bf16(L, experts=used)
    act = synth.act_f32(L)
    got = run(r, wbits, act, "auto")
    rng = np.random.default_rng(5)
    tokens = np.unique(np.concatenate([[0, L.T - 1], rng.choice(L.T, size=min(L.T, 24), replace=False)]))
    ref = oracle_out(r, wbits, act, L.topk, tokens=tokens)
    assert_close(got[tokens], ref, f"down {name}")


def test_zero_tokens_is_a_no_op():
    out = torch.full((0, 256), 7.0, device="cuda")
    r = {"topk_ids": torch.empty((0, 2), dtype=torch.int32, device="cuda"),
         "topk_w": torch.empty((0, 2), dtype=torch.float32, device="cuda"),
         "expert_off": torch.zeros(9, dtype=torch.int32, device="cuda"),
         "pair_pos": torch.empty((0,), dtype=torch.int32, device="cuda")}
    got = i8h.moe_down_bf16_combine(torch.empty((0, 128), device="cuda"),
                                    torch.zeros((8, 256, 128), dtype=torch.bfloat16, device="cuda"), r, out=out)
    assert got.shape == (0, 256)
