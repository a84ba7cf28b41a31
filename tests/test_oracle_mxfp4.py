"""Pins of the MXFP4 oracle (oracle/mxfp4.py): the E2M1 element format, its
rounding, the block-scale rule and the packing, each against an independent
construction (brute force over the format's values, an integer search for
the exponent, hand-built bytes) rather than against the oracle's formulas."""
import math

import numpy as np
import pytest

from oracle import lora as LO
from oracle import mxfp4 as MX

# The eight E2M1 magnitudes of the OCP microscaling specification.
SPEC_MAGS = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_decode_is_the_e2m1_format():
    vals = MX.e2m1_decode(np.arange(16))
    assert vals[:8].tolist() == SPEC_MAGS
    assert np.array_equal(vals[8:], -vals[:8])
    assert np.signbit(vals[8])                      # code 8 is negative zero
    # normal codes: (1 + m/2) 2^(e-1), e = 1..3 (an independent loop over fields)
    for e in range(1, 4):
        for m in range(2):
            assert vals[(e << 1) | m] == math.ldexp(1.0 + m / 2.0, e - 1)


def nearest_even(a: float) -> int:
    """Brute force: the magnitude code nearest to a; on a tie, the even code."""
    d = [abs(a - v) for v in SPEC_MAGS]
    best = min(d)
    cands = [c for c in range(8) if d[c] == best]
    if len(cands) == 1:
        return cands[0]
    return [c for c in cands if c % 2 == 0][0]


def test_encode_rounds_to_nearest_even_and_saturates():
    rng = np.random.default_rng(5)
    mids = [(SPEC_MAGS[i] + SPEC_MAGS[i + 1]) / 2 for i in range(7)]
    xs = np.concatenate([rng.uniform(0, 7, 4000), np.array(SPEC_MAGS + mids),
                         np.nextafter(np.array(mids), 0), np.nextafter(np.array(mids), 10), [6.5, 100.0]])
    xs = np.concatenate([xs, -xs])
    got = MX.e2m1_encode(xs)
    for x, c in zip(xs, got):
        want = min(nearest_even(abs(x)), 7) | (8 if math.copysign(1.0, x) < 0 else 0)
        assert c == want, (x, c, want)


def test_encode_decode_round_trip():
    codes = np.arange(16, dtype=np.uint8)
    assert np.array_equal(MX.e2m1_encode(MX.e2m1_decode(codes)), codes)


def test_block_exponent_is_the_smallest_that_fits():
    rng = np.random.default_rng(6)
    amax = np.concatenate([rng.uniform(0, 1, 300) * 2.0 ** rng.integers(-60, 60, 300),
                           [6.0, 6.0000001, 3.0, 12.0, 5.999, 1e-45, 0.0, 2.0 ** -130, 3e38]])
    got = MX.block_exponent(amax)
    for a, X in zip(amax, got):
        if a == 0:
            assert X == -127
            continue
        want = -127
        while want < 127 and a / math.ldexp(1.0, want) > 6.0:
            want += 1
        assert X == want, (a, X, want)


def test_packing_low_nibble_first():
    w = np.zeros((1, 32))
    w[0, 0], w[0, 1], w[0, 2] = 6.0, -0.5, 1.0   # block amax 6 -> X = 0
    q, e8 = MX.quantize_blocks(w)
    assert e8.tolist() == [[127]]
    assert q[0, 0] == (7 | (9 << 4)) and q[0, 1] == 2   # 6 -> code 7, -0.5 -> 9, 1.0 -> 2
    assert np.array_equal(MX.unpack(q)[0, :4], [7, 9, 2, 0])


def test_quantize_is_lossless_on_the_grid_and_nearest_elsewhere():
    rng = np.random.default_rng(7)
    R, K = 16, 128
    codes = rng.integers(0, 16, (R, K))
    X = rng.integers(-20, 20, (R, K // 32))
    codes[:, ::32] = 7                       # each block holds a 6: its scale is reproduced
    w = np.ldexp(MX.e2m1_decode(codes).reshape(R, K // 32, 32), X[:, :, None]).reshape(R, K)
    q, e8 = MX.quantize_blocks(w)
    assert np.array_equal(MX.dequantize_blocks(q, e8), w)
    # off-grid input: every element is the nearest grid value at its block's scale
    v = rng.normal(size=(R, K)) * 2.0 ** rng.integers(-8, 8, (R, 1))
    q, e8 = MX.quantize_blocks(v)
    d = MX.dequantize_blocks(q, e8)
    Xb = e8.astype(np.int64) - 127
    for i in range(R):
        for j in range(K):
            s = math.ldexp(1.0, int(Xb[i, j // 32]))
            want = math.copysign(SPEC_MAGS[min(nearest_even(abs(v[i, j]) / s), 7)] * s, v[i, j])
            assert d[i, j] == want


def test_mxfp4_merge_is_the_merge_over_the_decoded_base():
    rng = np.random.default_rng(8)
    E, N, K, r = 2, 8, 64, 8
    w = rng.normal(size=(E * N, K)) * 0.02
    q, e8 = MX.quantize_blocks(w)
    a, b = rng.normal(size=(E, r, K)), rng.normal(size=(E, N, r))
    deq = MX.dequantize_blocks(q, e8).reshape(E, N, K)
    got = LO.merge_mxfp4(q.reshape(E, N, K // 2), e8.reshape(E, N, K // 32), a, b, 0.5)
    want = deq + 0.5 * np.einsum("enr,erk->enk", b, a)
    assert np.allclose(got, want, rtol=0, atol=1e-12)
    assert np.array_equal(LO.merge_mxfp4(q.reshape(E, N, K // 2), e8.reshape(E, N, K // 32), a, 0 * b, 0.5), deq)


@pytest.mark.parametrize("shape", [(3, 64), (1, 32)])
def test_zero_and_tiny_blocks(shape):
    w = np.zeros(shape)
    q, e8 = MX.quantize_blocks(w)
    assert np.all(e8 == 0) and np.all(q == 0)
    w[0, 0] = -0.0
    q, _ = MX.quantize_blocks(w)
    assert q[0, 0] == 8   # negative zero keeps its sign
