"""Regression check of the oracle against its stored tiny fp32 fixture.

The fixture (tests/golden/tiny_f32_seed0.json) was written by
tests/golden/make_golden.py, which calls only the oracle; it guards the
oracle against unintended changes, not against a wrong definition (the other
oracle tests do that).
"""
import json
import os

import numpy as np

from mixture_experts_expert_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_f32_seed0.json")


def test_tiny_fixture(oracle):
    g = json.load(open(GOLDEN))
    cfg = synth.CONFIGS["tiny_f32"]
    inp = synth.make_inputs(cfg, 0, with_dy=True)
    t = {n: inp.f32(n) for n in inp.names()}
    f = oracle.forward(t["x"], t["w_router"], t["w_gate"], t["w_up"], t["w_down"], cfg.k)
    b = oracle.backward(f, t["dy"], t["w_gate"], t["w_up"], t["w_down"])
    assert f["topk_idx"].tolist() == g["topk_idx"]
    assert f["counts"].tolist() == g["counts"]
    assert f["offsets"].tolist() == g["offsets"]
    assert f["sorted_to_flat"].tolist() == g["sorted_to_flat"]
    assert [float(v) for v in f["logits"][0]] == g["logits_row0"]
    np.testing.assert_allclose(f["topk_w"][:4], g["topk_w_rows0_3"], rtol=1e-6)
    np.testing.assert_allclose(f["y"][:4, :8], g["y_rows0_3_cols0_7"], rtol=1e-5, atol=1e-7)
    np.testing.assert_allclose(b["dx"][:4, :8], g["dx_rows0_3_cols0_7"], rtol=1e-5, atol=1e-7)
    np.testing.assert_allclose(b["d_logits"][0], g["d_logits_row0"], rtol=1e-4, atol=1e-8)
    np.testing.assert_allclose(b["dw_down"][0, :4, :8], g["dw_down_e0_rows0_3_cols0_7"], rtol=1e-5, atol=1e-7)
