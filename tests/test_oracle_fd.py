"""Central finite differences of the float64 oracle.

L = <dY, Y(theta)>; for a random direction V, (L(theta + hV) - L(theta - hV)) / 2h
must match <grad, V> from the oracle's backward. Draws where the top-k
selection changes at theta +- hV are rejected (top-k is piecewise constant).

The oracle's dX covers the expert path only; the router's own GEMM backward
is dX += d_logits Wr and dWr = d_logits^T X, so a perturbation of X checks
dX + d_logits Wr, and one of Wr checks d_logits^T X.
"""
import numpy as np
import pytest

from mixture_experts_expert_amd import synth


def _setup(seed):
    cfg = synth.MoEConfig("fd", T=12, H=10, E=5, k=2, I=7, dtype="f32", backward=True)
    inp = synth.make_inputs(cfg, seed)
    t = {n: inp.f32(n).astype(np.float64) for n in inp.names()}
    # Larger router weights so routing weights vary noticeably.
    t["w_router"] = t["w_router"] * 25.0
    return cfg, t


def _loss(oracle, t, k, bias=None):
    f = oracle.forward(t["x"], t["w_router"], t["w_gate"], t["w_up"], t["w_down"], k, logit_bias=bias)
    return float((f["y"] * t["dy"]).sum()), f["topk_idx"]


@pytest.mark.parametrize("param", ["w_gate", "w_up", "w_down", "x", "w_router", "bias"])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_directional_derivative(oracle, param, seed):
    cfg, t = _setup(seed)
    k = cfg.k
    bias = np.zeros(cfg.E)
    fwd = oracle.forward(t["x"], t["w_router"], t["w_gate"], t["w_up"], t["w_down"], k, logit_bias=bias)
    bwd = oracle.backward(fwd, t["dy"], t["w_gate"], t["w_up"], t["w_down"])
    grads = {
        "w_gate": bwd["dw_gate"], "w_up": bwd["dw_up"], "w_down": bwd["dw_down"],
        "x": bwd["dx"] + bwd["d_logits"] @ t["w_router"],
        "w_router": bwd["d_logits"].T @ t["x"],
        "bias": bwd["d_logits"].sum(0),
    }
    rng = np.random.default_rng(1000 + seed)
    theta = bias if param == "bias" else t[param]
    checked = 0
    for _ in range(8):
        v = rng.standard_normal(theta.shape)
        h = 1e-4 * max(np.linalg.norm(theta), 1.0) / np.linalg.norm(v)
        vals, sels = [], []
        for sgn in (1.0, -1.0):
            tt = dict(t)
            b = bias
            if param == "bias":
                b = bias + sgn * h * v
            else:
                tt[param] = t[param] + sgn * h * v
            val, sel = _loss(oracle, tt, k, b)
            vals.append(val)
            sels.append(sel)
        if not all((s == fwd["topk_idx"]).all() for s in sels):
            continue  # selection changed inside the step: not differentiable here
        fd = (vals[0] - vals[1]) / (2 * h)
        an = float((grads[param] * v).sum())
        assert abs(fd - an) <= 1e-6 * max(abs(an), 1e-3 * np.abs(grads[param]).sum() * np.abs(v).max()), \
            (param, fd, an)
        checked += 1
    assert checked >= 3
