"""Pins of the adapter oracle (oracle/lora.py).

* merged identity: with adapters, y, dX and d_topk_w equal the float32 C++
  oracle run on the merged weights W + s B A (an independent implementation);
* B = 0: the stage equals the plain one and every dA is exactly zero;
* every adapter gradient against central finite differences of
  L = <dY, Y> in float64 along random directions (the routing does not depend
  on the adapters, so no draw changes the selection);
* 8-bit frozen weights: weights that E4M3 holds exactly (codes times a power
  of two) give the plain merge bit for bit, and any weights come back within
  E4M3's half step (2^-4 relative in its normal range) plus the subnormal
  step below it, checked element by element against the decoded codes.
"""
import numpy as np
import pytest

from mixture_experts_expert_amd import synth
from oracle import lora as LO
from oracle import oracle as O

NAMES = ["a_gate", "b_gate", "a_up", "b_up", "a_down", "b_down"]


def _setup(seed=0, T=24, H=32, E=4, k=2, I=32, r=4, zero_b=False):
    cfg = synth.MoEConfig("lora_tiny", T=T, H=H, E=E, k=k, I=I, dtype="f32", backward=True)
    inp = synth.make_inputs(cfg, seed, with_dy=True)
    f = {n: inp.f32(n).astype(np.float64) for n in inp.names()}
    rng = np.random.default_rng(seed + 10)
    ad = {"a_gate": rng.standard_normal((E, r, H)) * 0.1, "b_gate": rng.standard_normal((E, I, r)) * 0.1,
          "a_up": rng.standard_normal((E, r, H)) * 0.1, "b_up": rng.standard_normal((E, I, r)) * 0.1,
          "a_down": rng.standard_normal((E, r, I)) * 0.1, "b_down": rng.standard_normal((E, H, r)) * 0.1}
    if zero_b:
        for n in ["b_gate", "b_up", "b_down"]:
            ad[n][:] = 0.0
    _, idx, w = O.route(inp.f32("x"), inp.f32("w_router"), k)
    return f, ad, idx, w.astype(np.float64), k


def _run(f, ad, idx, w, s):
    return LO.forward_backward(f["x"], f["dy"], idx, w, f["w_gate"], f["w_up"], f["w_down"], ad, s)


def test_merged_weights_match_the_plain_oracle():
    f, ad, idx, w, k = _setup(seed=1)
    s = 0.75
    out = _run(f, ad, idx, w, s)
    wg = LO.merge(f["w_gate"], ad["a_gate"], ad["b_gate"], s).astype(np.float32)
    wu = LO.merge(f["w_up"], ad["a_up"], ad["b_up"], s).astype(np.float32)
    wd = LO.merge(f["w_down"], ad["a_down"], ad["b_down"], s).astype(np.float32)
    x32, dy32 = f["x"].astype(np.float32), f["dy"].astype(np.float32)
    ref = O.forward(x32, f["w_router"].astype(np.float32), wg, wu, wd, k)
    ref.update(O.backward(ref, dy32, wg, wu, wd))
    for n in ["y", "dx", "d_topk_w"]:
        err = np.max(np.abs(out[n] - ref[n])) / np.max(np.abs(ref[n]))
        assert err <= 1e-5, (n, err)


def test_zero_b_is_the_plain_stage():
    f, ad, idx, w, k = _setup(seed=2, zero_b=True)
    out = _run(f, ad, idx, w, 2.0)
    x32, dy32 = f["x"].astype(np.float32), f["dy"].astype(np.float32)
    wg, wu, wd = (f[n].astype(np.float32) for n in ["w_gate", "w_up", "w_down"])
    ref = O.forward(x32, f["w_router"].astype(np.float32), wg, wu, wd, k)
    ref.update(O.backward(ref, dy32, wg, wu, wd))
    for n in ["y", "dx"]:
        assert np.max(np.abs(out[n] - ref[n])) <= 1e-5 * np.max(np.abs(ref[n])), n
    for n in ["da_gate", "da_up", "da_down"]:
        assert not np.any(out[n]), n
    assert np.any(out["db_gate"]) and np.any(out["db_down"])


@pytest.mark.parametrize("name", NAMES)
def test_adapter_gradients_finite_differences(name):
    f, ad, idx, w, k = _setup(seed=3)
    s = 1.5
    out = _run(f, ad, idx, w, s)
    rng = np.random.default_rng(7)
    loss = lambda a: float(np.sum(f["dy"] * _run(f, a, idx, w, s)["y"]))  # noqa: E731
    for _ in range(3):
        v = rng.standard_normal(ad[name].shape)
        h = 1e-4 * np.linalg.norm(ad[name]) / np.linalg.norm(v)
        up = dict(ad)
        up[name] = ad[name] + h * v
        dn = dict(ad)
        dn[name] = ad[name] - h * v
        fd = (loss(up) - loss(dn)) / (2 * h)
        an = float(np.sum(out["d" + name] * v))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_fp8_base_merge_lossless_and_bounded():
    from oracle import fp8 as F8
    rng = np.random.default_rng(11)
    E, N, K, r = 3, 5, 16, 4
    a, b = rng.standard_normal((E, r, K)) * 0.1, rng.standard_normal((E, N, r)) * 0.1
    # codes times 2^-12 with every row's largest element at 448 * 2^-12:
    # quantised without loss, so the fp8 merge is the plain merge
    codes = rng.integers(0, 0x7E, size=(E, N, K)).astype(np.uint8) | (rng.integers(0, 2, (E, N, K)) << 7).astype(np.uint8)
    w = F8.e4m3_decode(codes) * 2.0 ** -12
    w[:, :, 0] = 448.0 * 2.0 ** -12
    wq, e8 = F8.quantize_weights(w)
    assert np.array_equal(LO.merge_fp8(wq, e8, a, b, 0.5), LO.merge(w, a, b, 0.5))
    # generic weights: each dequantised element within half an E4M3 step
    w = rng.standard_normal((E, N, K)) * 0.02
    wq, e8 = F8.quantize_weights(w)
    deq = LO.dequantize_weights(wq, e8)
    for e in range(E):
        for n in range(N):
            X = int(e8[e, n]) - 127
            for c in range(K):
                err = abs(deq[e, n, c] - w[e, n, c])
                bound = 2.0 ** -4 * abs(w[e, n, c]) if abs(w[e, n, c]) >= 2.0 ** (X - 6) else 2.0 ** (X - 10)
                assert err <= bound, (e, n, c)
    assert np.allclose(LO.merge_fp8(wq, e8, a, b, 0.5) - deq, 0.5 * np.matmul(b, a), rtol=0, atol=1e-15)

