"""Seeded synthetic inputs for the MoE gate_up path.

This module only draws random numbers and lays them out; it holds none of
the path's arithmetic (no rotation, no quantizer, no routing, no product).
Both the CPU oracle (through the tests) and the GPU library are fed from it.

Workloads (sizes of a routed-expert gate_up layer of Gemma 4 26B-A4B, the
model of the int8 and FP8 cards: hidden K = 2048, 128 experts, top-8, 2 x 768
gate_up rows per expert; the tiny layer is a small correctness case):

  name     T     K     E    k  N     seed  notes
  tiny     4     256   8    2  256   0     weights dense, for the quantizer
  decode   1     2048  128  8  1536  1     one decode token
  verify   128   2048  128  8  1536  2     8 sequences x (1 + 15 drafted);
                                           per-expert logit bias N(0, 0.5^2)
  prefill  2048  2048  128  8  1536  3     a prefill chunk
  fp8      128   2048  128  8  1536  4     FP8 block variant, no outliers
  w8a8     2048  2048  128  8  1536  3     W8A8 int8 g128 form at prefill sizes
                                           (the prefill chunk's tokens; codes and
                                           scales drawn as synthetic_i8h, the
                                           same storage)

Distributions: router logits N(0, 1) float32; activations N(0, 1) rounded to
bf16, with round(0.01 K) outlier channels (drawn once per layer, shared by
all tokens) scaled by 20; dense weights N(0, 0.02^2) float32.

The real checkpoints and prompts of the cards are not available; these draws
stand in for them. For the full-size layers the int8 codes and the E4M3
codes are drawn directly in the code domain (a rounded normal for int8,
normal values cast to E4M3 for FP8) with bf16 scales of the magnitude the
quantizers produce for N(0, 0.02^2) weights: the product kernels' work and
speed do not depend on how the codes were obtained.
"""

import zlib
from dataclasses import dataclass

import numpy as np

CONFIGS = {
    "tiny":    dict(T=4,    K=256,  E=8,   topk=2, N=256,  seed=0, outliers=True,  bias_std=0.0),
    "decode":  dict(T=1,    K=2048, E=128, topk=8, N=1536, seed=1, outliers=True,  bias_std=0.0),
    "verify":  dict(T=128,  K=2048, E=128, topk=8, N=1536, seed=2, outliers=True,  bias_std=0.5),
    "prefill": dict(T=2048, K=2048, E=128, topk=8, N=1536, seed=3, outliers=True,  bias_std=0.0),
    "fp8":     dict(T=128,  K=2048, E=128, topk=8, N=1536, seed=4, outliers=False, bias_std=0.0),
    "w8a8":    dict(T=2048, K=2048, E=128, topk=8, N=1536, seed=3, outliers=True,  bias_std=0.0),
}


@dataclass(frozen=True)
class Layer:
    name: str
    T: int
    K: int
    E: int
    topk: int
    N: int
    seed: int
    outliers: bool = True
    bias_std: float = 0.0

    @property
    def P(self):
        return self.T * self.topk

    @property
    def G(self):
        return self.K // 128

    @property
    def I(self):
        return self.N // 2


def layer(name, **over):
    """A named workload, optionally with sizes overridden (for test cases)."""
    d = dict(CONFIGS[name]) if name in CONFIGS else {}
    d.update(over)
    return Layer(name=name, **d)


def _rng(seed, stream, *sub):
    return np.random.default_rng([seed, zlib.crc32(stream.encode()), *sub])


def to_bf16_bits(x32):
    """Round float32 values to bf16 (nearest even) with torch's cast; return
    the uint16 bit patterns."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f64(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def router_logits(L):
    """float32 [T, E]; N(0, 1) plus an optional per-expert bias."""
    lg = _rng(L.seed, "logits").standard_normal((L.T, L.E), dtype=np.float32)
    if L.bias_std > 0:
        bias = _rng(L.seed, "bias").standard_normal(L.E, dtype=np.float32) * np.float32(L.bias_std)
        lg = lg + bias[None, :]
    return lg.astype(np.float32)


def outlier_channels(L):
    n = int(round(0.01 * L.K)) if L.outliers else 0
    return np.sort(_rng(L.seed, "outlier_channels").choice(L.K, size=n, replace=False))


def activations_bf16(L, T=None):
    """bf16 bit patterns [T, K]: N(0, 1) with the layer's outlier channels x20."""
    t_count = L.T if T is None else T
    x = _rng(L.seed, "x").standard_normal((t_count, L.K), dtype=np.float32)
    ch = outlier_channels(L)
    if ch.size:
        x[:, ch] *= np.float32(20.0)
    return to_bf16_bits(x)


def dense_weights(L, expert):
    """float32 [N, K] gate_up weights of one expert, N(0, 0.02^2)."""
    return _rng(L.seed, "W", expert).standard_normal((L.N, L.K), dtype=np.float32) * np.float32(0.02)


# Typical magnitudes of quantized N(0, 0.02^2) weights: the max of 128
# normals is about 2.6-3 sigma, so scales sit near 0.02 * 2.8 * 0.95 / 127
# and codes spread with a standard deviation near 127 / (2.8 * 0.95).
_I8_SCALE = 0.02 * 2.8 * 0.95 / 127.0
_I8_CODE_STD = 127.0 / (2.8 * 0.95)


def synthetic_i8h(L, experts=None):
    """Directly drawn int8 codes [E', N, K] (in -127..127) and bf16 scale
    bits [E', N, K/128] for the listed experts (all by default)."""
    ex = range(L.E) if experts is None else experts
    codes, scales = [], []
    for e in ex:
        r = _rng(L.seed, "i8h_codes", e)
        c = np.rint(r.standard_normal((L.N, L.K), dtype=np.float32) * np.float32(_I8_CODE_STD))
        codes.append(np.clip(c, -127, 127).astype(np.int8))
        s = _I8_SCALE * np.exp(0.1 * r.standard_normal((L.N, L.G))).astype(np.float32)
        scales.append(to_bf16_bits(s))
    return np.stack(codes), np.stack(scales)


def synthetic_fp8(L, experts=None):
    """Directly drawn E4M3 codes [E', N, K] (finite, |v| <= 448) and bf16 scale
    bits [E', N/128, K/128] for the listed experts (all by default)."""
    import torch
    ex = range(L.E) if experts is None else experts
    codes, scales = [], []
    for e in ex:
        r = _rng(L.seed, "fp8_codes", e)
        v = np.clip(r.standard_normal((L.N, L.K), dtype=np.float32) * np.float32(140.0), -448, 448)
        c = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
        codes.append(c)
        s = (0.02 * 4.0 / 448.0) * np.exp(0.1 * r.standard_normal((L.N // 128, L.G))).astype(np.float32)
        scales.append(to_bf16_bits(s))
    return np.stack(codes), np.stack(scales)


def down_weights_bf16(L, experts=None):
    """bf16 bit patterns [E', K, I] of the experts' down projections (hidden K
    rows of I = N / 2 inputs each), N(0, 0.02^2), for the listed experts (all
    by default)."""
    ex = range(L.E) if experts is None else experts
    return np.stack([to_bf16_bits(_rng(L.seed, "W_down", e).standard_normal((L.K, L.I), dtype=np.float32)
                                  * np.float32(0.02)) for e in ex])


def act_f32(L, rows=None):
    """float32 [rows, I] stand-in for the gate_up epilogue's output (the down
    projection's input), N(0, 1); P rows by default."""
    r = L.P if rows is None else rows
    return _rng(L.seed, "act").standard_normal((r, L.I), dtype=np.float32)


def f16_bits(x32):
    """float32 values -> IEEE binary16 bit patterns (nearest even), numpy's cast."""
    return np.asarray(x32, dtype=np.float32).astype(np.float16).view(np.uint16)


# Stand-in for one of the DFlash drafter's linears (int8 card, model table row
# "Speculator": it drafts 15 tokens a step, so it runs on blocks of 16
# positions): 16 tokens, hidden 2048 in, 4096 out.
DRAFTER = dict(T=16, K=2048, N=4096, seed=6)


def synthetic_i8f16(n_rows, k_dim, seed, stream="i8f16"):
    """Directly drawn int8 codes [N, K] (-127..127) and f16 scale bits
    [N, K/128] of the magnitude the RTN quantizer gives N(0, 0.02^2) rows
    (amax about 3 sigma: s near 0.02 * 3 / 127)."""
    r = _rng(seed, stream)
    c = np.rint(r.standard_normal((n_rows, k_dim), dtype=np.float32) * np.float32(127.0 / 3.0))
    codes = np.clip(c, -127, 127).astype(np.int8)
    s = (0.02 * 3.0 / 127.0) * np.exp(0.1 * r.standard_normal((n_rows, k_dim // 128))).astype(np.float32)
    return codes, f16_bits(s)


def drafter_activations_bf16(T, K, seed):
    """bf16 bit patterns [T, K], N(0, 1), for the drafter's linears."""
    return to_bf16_bits(_rng(seed, "drafter_x").standard_normal((T, K), dtype=np.float32))
