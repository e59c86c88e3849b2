"""The 128-wide Walsh-Hadamard rotation (fp64).

The int8 card stores the routed experts' gate_up codes "in the 128-wide
Hadamard domain" (model table, row "Weights") and its recipe names the
transform fwht128 (section "How this file was made"). The activations must
meet the same rotation, written by the producer of the experts' input (the
row "Needs" names the attention join that writes it).

Reading taken (the cards give no matrix): Sylvester's construction in its
natural order, H[i, j] = (-1)**popcount(i & j), normalised by 1/sqrt(128) so
that the blockwise transform is orthonormal and its own inverse. The same
normalised matrix rotates weight rows (along K) and activation rows.
"""

import numpy as np

from .numfmt import bf16_round

N = 128


def sylvester(n=N):
    """Integer Sylvester-Hadamard matrix of order n (a power of two)."""
    i = np.arange(n)
    bits = np.bitwise_and.outer(i, i)
    # popcount of i & j, one bit at a time
    pc = np.zeros_like(bits)
    b = bits.copy()
    while b.any():
        pc += b & 1
        b >>= 1
    return np.where(pc % 2 == 0, 1, -1).astype(np.int64)


def fwht(v):
    """Unnormalised fast Walsh-Hadamard transform along the last axis.

    Butterflies (a, b) -> (a + b, a - b) on index pairs (i, i + h) with
    i & h == 0, for h = 1, 2, 4, ..., n/2. In Sylvester order this equals
    sylvester(n) @ v.
    """
    y = np.array(v, dtype=np.float64, copy=True)
    n = y.shape[-1]
    h = 1
    while h < n:
        z = y.reshape(y.shape[:-1] + (n // (2 * h), 2, h))
        a = z[..., 0, :].copy()
        b = z[..., 1, :].copy()
        z[..., 0, :] = a + b
        z[..., 1, :] = a - b
        y = z.reshape(y.shape)
        h *= 2
    return y


def rotate_blocks(x, n=N):
    """Blockwise normalised rotation along the last axis, fp64 (no rounding
    beyond fp64): every run of n consecutive values v becomes H v / sqrt(n).
    The last axis must be a multiple of n."""
    x = np.asarray(x, dtype=np.float64)
    k = x.shape[-1]
    assert k % n == 0, "length must be a multiple of the block size"
    blocks = x.reshape(x.shape[:-1] + (k // n, n))
    return (fwht(blocks) / np.sqrt(n)).reshape(x.shape)


def rotate_activations_bf16(x_bf16_values, n=N):
    """The run-time activation rotation as the path defines it: the exact
    rotated value of each bf16 input row, rounded once to bf16 (ties to
    even). Input and output are fp64 arrays holding bf16 values."""
    return bf16_round(rotate_blocks(x_bf16_values, n))
