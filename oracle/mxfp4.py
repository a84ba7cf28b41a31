"""4-bit expert weights (MXFP4) for adapters over a frozen base: the oracle.

TEST INFRASTRUCTURE ONLY: the test suite uses it; the product path never
does. Plain numpy in float64.

The pages fine-tune MoE models with adapters over 4-bit frozen weights
(sourcepulse summary, "Highlighted Details": QLoRA on the fused experts,
training over quantised models; "Quick Start & Requirements": bitsandbytes
4-bit weights; "Limitations & Caveats": the fused 4-bit dequantisation).
The 4-bit format native to this chip is the OCP microscaling FP4 one:

- Element format E2M1: 1 sign bit, 2 exponent bits with bias 1, 1 mantissa
  bit; exponent field 0 is subnormal (value m / 2), otherwise
  (1 + m / 2) 2^(e - 1). The magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6.
- Blocks of 32 consecutive elements along a row (the reduction axis of the
  weight) share one power-of-two scale, stored as a biased 8-bit exponent
  (E8M0: code c means 2^(c - 127)).
- Two elements per byte: element 2i in the low nibble, 2i + 1 in the high one.

Readings taken where the pages are silent (listed with the others in the
design notes): a block with largest magnitude amax gets the smallest
exponent X with amax / 2^X <= 6 (E2M1's largest value), clamped to
[-127, 127], -127 for an all-zero block; nothing is clipped (the OCP rule
X = floor(log2(amax)) - 2 would put the largest element in [4, 8) and clip
the part above 6). Elements are x / 2^X (exact: a power of two) rounded to
the nearest E2M1 value, ties to the even mantissa; the sign is kept, so a
negative value that rounds to zero is a negative zero.
"""
from __future__ import annotations

import numpy as np

E2M1_MAX = 6.0
BLOCK = 32
E8M0_BIAS = 127


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """4-bit codes (0..15, any integer dtype) -> float64, from the bit fields."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    sign = np.where(c & 8, -1.0, 1.0)
    e = (c >> 1) & 3
    m = (c & 1).astype(np.float64)
    mag = np.where(e == 0, m / 2.0, (1.0 + m / 2.0) * np.ldexp(1.0, e - 1))
    return sign * mag


def e2m1_encode(x: np.ndarray) -> np.ndarray:
    """float -> 4-bit codes: round |x| to the nearest E2M1 magnitude, ties to
    the even mantissa (so to the even code), saturating at 6; the sign bit
    from x's sign (negative zero included). Inputs must be finite."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    # Magnitude codes 0..7 are in increasing order; the boundary between
    # codes c and c + 1 is their midpoint, which goes to the even code.
    mags = e2m1_decode(np.arange(8))
    code = np.zeros(a.shape, dtype=np.int64)
    for c in range(7):
        mid = (mags[c] + mags[c + 1]) / 2.0
        up = (a > mid) | ((a == mid) & (c % 2 == 1))  # a tie goes to code c + 1 when c is odd
        code = code + up.astype(np.int64)
    return (code | np.where(np.signbit(x), 8, 0)).astype(np.uint8)


def block_exponent(amax: np.ndarray) -> np.ndarray:
    """Smallest X with amax / 2^X <= 6, clamped to [-127, 127]; -127 for 0.
    amax = f 2^ex with f in [0.5, 1) and 6 = 0.75 2^3: amax / 2^(ex - 3) =
    8 f is at most 6 exactly when f <= 0.75, else one more power of two."""
    amax = np.asarray(amax, dtype=np.float64)
    f, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    X = np.where(amax > 0, ex - 3 + (f > 0.75), -E8M0_BIAS)
    return np.clip(X, -E8M0_BIAS, E8M0_BIAS).astype(np.int64)


def quantize_blocks(w: np.ndarray):
    """Rows of w [R, K] (K % 32 == 0) -> (packed codes [R, K/2] uint8,
    E8M0 scales [R, K/32] uint8)."""
    w = np.asarray(w, dtype=np.float64)
    R, K = w.shape
    assert K % BLOCK == 0
    blocks = w.reshape(R, K // BLOCK, BLOCK)
    X = block_exponent(np.max(np.abs(blocks), axis=2))
    codes = e2m1_encode(np.ldexp(blocks, -X[:, :, None])).reshape(R, K)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, (X + E8M0_BIAS).astype(np.uint8)


def unpack(packed: np.ndarray) -> np.ndarray:
    """[R, K/2] bytes -> [R, K] codes (low nibble first)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def dequantize_blocks(packed: np.ndarray, e8: np.ndarray) -> np.ndarray:
    """decode(code) * 2^(e8 - 127) per element, exact in float64."""
    codes = unpack(packed)
    R, K = codes.shape
    X = np.asarray(e8, dtype=np.int64) - E8M0_BIAS
    return np.ldexp(e2m1_decode(codes).reshape(R, K // BLOCK, BLOCK), X[:, :, None]).reshape(R, K)
