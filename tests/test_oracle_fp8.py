"""Pins of the fp8 oracle (oracle/fp8.py).

* E4M3 decoding of all 256 codes equals torch's float8_e4m3fn (a library
  implementation of the same OCP format) and the format's closed-form values;
* encoding inverts decoding on every finite code, rounds to the nearest
  value with ties to the even code (checked against torch's conversion on
  random values and on every midpoint), and saturates at +-448;
* row quantisation: the scale exponent is the smallest X with
  amax / 2^X <= 448 (found by a search over integers with math.ldexp per
  row), the largest element lands in (224, 448] and no element is clipped,
  elements in the normal range come back within 2^-4 relative error, zero
  rows are zero;
* the expert GEMMs against element-by-element Python loops on tiny inputs,
  and, on inputs that quantise without loss, against the plain float32
  oracle along the whole chain: G and U equal its G and U; A is its A
  rounded once to bf16; O_perm equals its gate GEMM run on the dequantised
  codes of A and of the down weights (the oracle's G = X W^T with X := A
  and W := W_down), weighted and rounded once to bf16;
* the per-token sum against an element loop over slots in ascending order
  at k > 1 (a slot-order or reshape mistake changes the float32 sum).
"""
import math

import numpy as np
import pytest
import torch

from oracle import fp8 as F8


def torch_decode(codes):
    return torch.tensor(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_encode(x):
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours, ref = F8.e4m3_decode(codes), torch_decode(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))


def test_decode_closed_form_values():
    d = lambda c: float(F8.e4m3_decode(np.array([c]))[0])  # noqa: E731
    assert d(0x38) == 1.0
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0
    assert d(0x01) == 2.0 ** -9 and d(0x07) == 7 * 2.0 ** -9
    assert d(0x08) == 2.0 ** -6
    assert d(0x40) == 2.0 and d(0x3C) == 1.5
    assert math.isnan(d(0x7F)) and math.isnan(d(0xFF))
    assert d(0x80) == 0.0 and math.copysign(1.0, d(0x80)) == -1.0


def test_encode_inverts_decode():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(F8.e4m3_encode(F8.e4m3_decode(codes)), codes)


def test_encode_round_to_nearest_even():
    # every midpoint between neighbouring positive values goes to the even code
    vals = F8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    got = F8.e4m3_encode(mids)
    lo = np.arange(0x7E)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got, want.astype(np.uint8))
    assert np.array_equal(F8.e4m3_encode(-mids), (want | 0x80).astype(np.uint8))
    # random values in range against torch's conversion
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 2.0 ** rng.integers(-12, 8, 20000)])
    x = x.astype(np.float32)
    assert np.array_equal(F8.e4m3_encode(x), torch_encode(x))


def test_encode_saturates():
    assert list(F8.e4m3_encode(np.array([448.0, 460.0, 464.0, 500.0, 1e6, -1e6]))) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E,
                                                                                         0xFE]


def test_quantize_rows_scale_and_error():
    rng = np.random.default_rng(1)
    rows = [rng.standard_normal(96) * 2.0 ** s for s in (-20, -3, 0, 5, 30)]
    rows.append(np.zeros(96))
    rows.append(np.r_[np.zeros(95), -3.0])
    # largest magnitudes on both sides of 448 * 2^k and of 224 * 2^k
    for top in (448.0, 448.0 * (1 + 2.0 ** -7), 449.0 / 2 ** 3, 224.0, 224.0 * (1 + 2.0 ** -7), 7.99, 8.0):
        rows.append(np.r_[rng.uniform(-1, 1, 95), top])
    x = np.stack(rows).astype(np.float32).astype(np.float64)
    q, e8 = F8.quantize_rows(x)
    for r in range(len(x)):
        amax = np.max(np.abs(x[r]))
        if amax == 0:
            assert e8[r] == 0 and not q[r].any()
            continue
        X = -200
        while math.ldexp(amax, -X) > 448.0:  # the smallest X with amax / 2^X <= 448
            X += 1
        assert int(e8[r]) - 127 == X
        deq = F8.dequantize_rows(q[r:r + 1], e8[r:r + 1])[0]
        top = np.max(np.abs(F8.e4m3_decode(q[r])))
        assert 224.0 <= top <= 448.0
        normal = np.abs(x[r]) >= 2.0 ** (X - 6)
        assert np.all(np.abs(deq - x[r])[normal] <= 2.0 ** -4 * np.abs(x[r])[normal])
        # below the normal range the error is at most half a subnormal step
        assert np.all(np.abs(deq - x[r])[~normal] <= 2.0 ** (X - 10))
        # nothing clipped: the largest element is within half an E4M3 step
        i = int(np.argmax(np.abs(x[r])))
        assert abs(deq[i] - x[r, i]) <= 2.0 ** -4 * abs(x[r, i])


def test_bf16_round():
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 1.0 + 2.0 ** -9])
    assert list(F8.bf16_round(x)) == [1.0, 1.0, 1.0 + 2 * 2.0 ** -7, -2.5, 1.0]


def _tiny(seed=0, T=5, H=64, I=32, E=3, k=2):
    rng = np.random.default_rng(seed)
    x = F8.bf16_round(rng.standard_normal((T, H)))
    w = {n: F8.bf16_round(0.1 * rng.standard_normal(s)) for n, s in
         [("g", (E, I, H)), ("u", (E, I, H)), ("d", (E, H, I))]}
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
    flat_e = idx.reshape(-1)
    order = np.argsort(flat_e, kind="stable")
    counts = np.bincount(flat_e, minlength=E)
    offsets = np.r_[0, np.cumsum(counts)].astype(np.int32)
    row_token = (order // k).astype(np.int32)
    row_weight = rng.uniform(0.1, 1.0, T * k)
    return x, w, offsets, row_token, row_weight


def test_experts_fp8_against_loops():
    x, w, offsets, row_token, row_weight = _tiny()
    gate, up, down = (F8.quantize_weights(w["g"]), F8.quantize_weights(w["u"]), F8.quantize_weights(w["d"]))
    out = F8.experts_fp8(x, row_token, row_weight, offsets, gate, up, down)
    dec = lambda c, s: F8.e4m3_decode(np.array([c]))[0] * 2.0 ** (int(s) - 127)  # noqa: E731
    E = len(offsets) - 1
    H, I = x.shape[1], w["g"].shape[1]
    xq, xe = F8.quantize_rows(x)
    for e in range(E):
        for p in range(offsets[e], offsets[e + 1]):
            t = row_token[p]
            for i in range(I):
                g = sum(dec(xq[t, h], xe[t]) * dec(gate[0][e, i, h], gate[1][e, i]) for h in range(H))
                u = sum(dec(xq[t, h], xe[t]) * dec(up[0][e, i, h], up[1][e, i]) for h in range(H))
                assert abs(g - out["g"][p, i]) <= 1e-12 * max(1.0, abs(g))
                assert abs(u - out["u"][p, i]) <= 1e-12 * max(1.0, abs(u))
                a = g / (1 + math.exp(-g)) * u
                assert out["a"][p, i] == F8.bf16_round(np.array([a]))[0]
            for h in range(0, H, 7):
                o = sum(dec(out["aq"][p, i], out["ae"][p]) * dec(down[0][e, h, i], down[1][e, h]) for i in range(I))
                assert out["o_perm"][p, h] == F8.bf16_round(np.array([row_weight[p] * o]))[0]


def test_experts_fp8_lossless_inputs_match_plain_oracle():
    """Inputs whose rows are E4M3 codes times a power of two quantise without
    loss, so G and U equal the float32 oracle's on the same values; A is the
    oracle's A rounded to bf16; O_perm is the oracle's GEMM on the
    dequantised A and W_down, weighted and rounded to bf16."""
    from oracle import oracle as O
    rng = np.random.default_rng(3)
    T, H, I, E, k = 6, 64, 32, 2, 1
    def exact(shape, X):
        codes = rng.integers(0, 0x7E, size=shape).astype(np.uint8) | (rng.integers(0, 2, size=shape) << 7).astype(np.uint8)
        v = F8.e4m3_decode(codes) * 2.0 ** X
        v.reshape(-1, shape[-1])[:, 0] = 448.0 * 2.0 ** X  # every row's largest element fixes its scale at X
        return v
    x = exact((T, H), -8)
    wg, wu, wd = exact((E, I, H), -12), exact((E, I, H), -12), exact((E, H, I), -12)
    xq, xe = F8.quantize_rows(x)
    assert np.array_equal(F8.dequantize_rows(xq, xe), x)
    wr = np.zeros((E, H), dtype=np.float32)
    f = O.forward(x.astype(np.float32), wr, wg.astype(np.float32), wu.astype(np.float32), wd.astype(np.float32), k)
    offsets, s2f = f["offsets"], f["sorted_to_flat"]
    row_weight = rng.uniform(0.25, 1.0, T * k)
    out = F8.experts_fp8(x, (s2f // k).astype(np.int32), row_weight, offsets, F8.quantize_weights(wg),
                         F8.quantize_weights(wu), F8.quantize_weights(wd))
    for n in ["g", "u"]:
        ref = f[n].astype(np.float64)
        assert np.max(np.abs(out[n] - ref)) <= 1e-6 * np.max(np.abs(ref)), n
    # A: the oracle's fp32 A, rounded once to bf16 (within a rounding step of
    # it; the float32 and float64 silu may straddle a bf16 midpoint)
    a32 = f["a"].astype(np.float64)
    assert np.all(np.abs(out["a"] - a32) <= 2.0 ** -8 * np.abs(a32) + 1e-30)
    assert np.mean(out["a"] == F8.bf16_round(a32)) >= 0.99
    # O_perm: the oracle's own GEMM (its G = X W^T) on X = deq(aq), W = deq(W_down)
    ad = F8.dequantize_rows(out["aq"], out["ae"])
    wq, we = F8.quantize_weights(wd)
    wdd = F8.dequantize_rows(wq.reshape(E * H, I), we.reshape(E * H)).reshape(E, H, I)
    g2 = O.experts_fwd(ad.astype(np.float32), offsets, wdd.astype(np.float32), np.zeros((E, H, I), np.float32),
                       np.zeros((E, I, H), np.float32))[0].astype(np.float64)
    want = F8.bf16_round(g2 * row_weight[:, None])
    assert np.all(np.abs(out["o_perm"] - want) <= 2.0 ** -8 * np.abs(want) + 1e-30)
    assert np.mean(out["o_perm"] == want) >= 0.99


def test_combine_sum_slots_in_order():
    """k = 3: each token's sum, element by element, adds its slots' rows in
    ascending slot order in float32, then rounds once to bf16."""
    rng = np.random.default_rng(5)
    T, k, H = 5, 3, 8
    o = F8.bf16_round(rng.standard_normal((T * k, H)) * 2.0 ** rng.integers(-20, 20, (T * k, 1)))
    f2s = rng.permutation(T * k).astype(np.int32)
    # in the first four columns a token's slots hold 1, 2^30 and -2^30: in
    # slot order the 1 is absorbed (sum 0), in reverse order it survives
    slots = f2s.reshape(T, k)
    o[slots[:, 0], :4] = 1.0
    o[slots[:, 1], :4] = 2.0 ** 30
    o[slots[:, 2], :4] = -(2.0 ** 30)
    got = F8.combine_sum(o, f2s, T, k)
    for t in range(T):
        for h in range(H):
            acc = np.float32(0.0)
            for j in range(k):
                acc = np.float32(acc + np.float32(o[f2s[t * k + j], h]))
            assert got[t, h] == F8.bf16_round(np.array([acc]))[0], (t, h)
    # a slot-order mistake shows: the reversed order gives a different sum somewhere
    rev = np.zeros((T, H), np.float32)
    for j in reversed(range(k)):
        rev = rev + o[f2s.reshape(T, k)[:, j]].astype(np.float32)
    assert not np.array_equal(F8.bf16_round(rev), got)


def test_combine_sum_one_slot_is_the_row():
    rng = np.random.default_rng(4)
    o = F8.bf16_round(rng.standard_normal((7, 16)))
    f2s = rng.permutation(7).astype(np.int32)
    assert np.array_equal(F8.combine_sum(o, f2s, 7, 1), o[f2s])
