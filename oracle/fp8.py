"""fp8 expert weights and activations for the inference forward: the oracle.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use it; the product path never does. Plain numpy in float64.

The pages' memory-saving path stores expert weights in fewer bits and
dequantises them inside the fused MoE linear layers (sourcepulse summary:
bitsandbytes 4-bit compatibility, "Quick Start & Requirements"; QLoRA and
training over quantised GGUF models, "Highlighted Details"; the fused 4-bit
dequantisation, "Limitations & Caveats"; torchtune PR #2820, the question on
fp8 checkpoints). On this chip the matrix cores multiply 8-bit floats
directly, so both GEMM operands are 8-bit here:

- Element format: OCP 8-bit float E4M3 (1 sign, 4 exponent bits with bias 7,
  3 mantissa bits; no infinities; all-ones exponent and mantissa is NaN;
  largest finite value 448; subnormals m * 2^-9).
- Scales: one power of two per row (a token's row of x or of the expert
  activations, an output channel's row of a weight), stored as its biased
  8-bit exponent (the E8M0 encoding: code c means 2^(c - 127)). A row with
  largest magnitude amax gets the smallest exponent X with amax / 2^X <= 448
  (E4M3's largest finite value), clamped to [-127, 127]; an all-zero row
  gets -127. The row's largest element then lands in (224, 448], so no
  element is clipped (the shared-exponent rule of the OCP microscaling
  formats, floor(log2(amax)) - 8, puts it in [256, 512) and clips the part
  above 448, up to an eighth of the element). Elements are x / 2^X (exact: a
  power of two), clamped to +-448 and rounded to the nearest E4M3 value, ties
  to the even code.
- A dequantised element is decode(code) * 2^X, exact in float64.

Readings taken where the pages are silent (listed with the others in the
design notes): E4M3 rather than E5M2 (the forward needs precision more than
range); per-row rather than per-block scales (a row's scale is constant
along K, so the matrix core applies it to every product); the expert
activations A are rounded to bf16 (as the GEMM stores them) before they are
quantised.
"""
from __future__ import annotations

from typing import Dict

import numpy as np

E4M3_MAX = 448.0
E8M0_BIAS = 127


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Codes (uint8) -> float64 values, from the bit fields."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.ldexp(1.0, e - 7)
    sub = m * 2.0 ** -9
    v = sign * np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """float -> codes: clamp to +-448, round to the nearest E4M3 value, ties to
    the even code. Inputs must be finite. Exact for every float64 input: the
    arithmetic below only scales by powers of two."""
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    # Subnormal range (below 2^-6): steps of 2^-9; q = 8 lands on the
    # smallest normal value, whose code is 8 as well.
    q_sub = np.round(a * 2.0 ** 9)  # numpy rounds halves to even
    # Normal range: a = 2^e (1 + m / 8).
    frac, ex = np.frexp(np.where(a > 0, a, 1.0))  # a = frac * 2^ex, frac in [0.5, 1)
    e = ex - 1
    mant = np.round((np.ldexp(a, -e) - 1.0) * 8.0)
    carry = mant == 8
    e = np.where(carry, e + 1, e)
    mant = np.where(carry, 0, mant)
    code_norm = ((e + 7) << 3) + mant.astype(np.int64)
    code = np.where(a < 2.0 ** -6, q_sub.astype(np.int64), code_norm)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def quantize_rows(x: np.ndarray):
    """Rows of x [R, K] -> (codes [R, K] uint8, e8 [R] uint8)."""
    x = np.asarray(x, dtype=np.float64)
    amax = np.max(np.abs(x), axis=1)
    # amax = f 2^ex with f in [0.5, 1) and 448 = 0.875 2^9: amax / 2^(ex - 9)
    # = 512 f is at most 448 exactly when f <= 0.875, else one more power of two.
    f, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    X = np.where(amax > 0, ex - 9 + (f > 0.875), -E8M0_BIAS)
    X = np.clip(X, -E8M0_BIAS, E8M0_BIAS)
    codes = e4m3_encode(np.ldexp(x, -X[:, None]))
    return codes, (X + E8M0_BIAS).astype(np.uint8)


def dequantize_rows(codes: np.ndarray, e8: np.ndarray) -> np.ndarray:
    return np.ldexp(e4m3_decode(codes), e8.astype(np.int64)[:, None] - E8M0_BIAS)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float -> the nearest bfloat16 value (ties to even), as float64."""
    f = np.asarray(x, dtype=np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def quantize_weights(w: np.ndarray):
    """Stacked weights [E, N, K] -> (codes [E, N, K], e8 [E, N]): one scale per
    output channel (a row of one expert's matrix)."""
    E, N, K = w.shape
    q, s = quantize_rows(w.reshape(E * N, K))
    return q.reshape(E, N, K), s.reshape(E, N)


def experts_fp8(x: np.ndarray, row_token: np.ndarray, row_weight: np.ndarray, offsets: np.ndarray,
                gate, up, down) -> Dict[str, np.ndarray]:
    """The fp8 expert GEMMs over the sorted rows, in float64.

    x [T, H] (the bf16 hidden states as floats); row_token, row_weight [M]
    and offsets [E+1] from the sort; gate, up = (codes [E, I, H], e8 [E, I]),
    down = (codes [E, H, I], e8 [E, H]). Per sorted row p of expert e:
      G = deq(xq[row_token[p]]) deq(Wg[e])^T,  U likewise,
      A = bf16(silu(G) U),  aq = quantize_rows(A),
      O[p] = bf16(row_weight[p] * deq(aq[p]) deq(Wd[e])^T).
    """
    def deq(w):
        q, e8 = w
        E, N, K = q.shape
        return dequantize_rows(q.reshape(E * N, K), e8.reshape(E * N)).reshape(E, N, K)
    return experts_quantized(x, row_token, row_weight, offsets, deq(gate), deq(up), deq(down))


def experts_quantized(x: np.ndarray, row_token: np.ndarray, row_weight: np.ndarray, offsets: np.ndarray,
                      wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> Dict[str, np.ndarray]:
    """experts_fp8 with the expert weights given dequantised (float64 wg, wu
    [E, I, H], wd [E, H, I]): the activations x and A are quantised to E4M3
    per row as there, whatever format the weights came in."""
    xq, xe = quantize_rows(x)
    xd = dequantize_rows(xq, xe)
    E = len(offsets) - 1
    M = len(row_token)
    I = wg.shape[1]
    H = wg.shape[2]
    G = np.zeros((M, I))
    U = np.zeros((M, I))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        rows = xd[row_token[lo:hi]]
        G[lo:hi] = rows @ wg[e].T
        U[lo:hi] = rows @ wu[e].T
    A = bf16_round(G / (1.0 + np.exp(-G)) * U)
    aq, ae = quantize_rows(A)
    ad = dequantize_rows(aq, ae)
    O = np.zeros((M, H))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        O[lo:hi] = ad[lo:hi] @ wd[e].T
    O = bf16_round(O * np.asarray(row_weight, dtype=np.float64)[:, None])
    return {"xq": xq, "xe": xe, "g": G, "u": U, "a": A, "aq": aq, "ae": ae, "o_perm": O}


def combine_sum(o_perm: np.ndarray, flat_to_sorted: np.ndarray, T: int, k: int) -> np.ndarray:
    """y[t] = sum over slots j ascending of o_perm[flat_to_sorted[t k + j]], in
    float32 as the per-token sum is defined, rounded once to bf16."""
    acc = np.zeros((T, o_perm.shape[1]), dtype=np.float32)
    for j in range(k):
        acc = acc + o_perm[flat_to_sorted.reshape(T, k)[:, j]].astype(np.float32)
    return bf16_round(acc)
