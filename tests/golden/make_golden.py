"""Writes tests/golden/tiny_f32_seed0.json from the CPU oracle alone.

A regression fixture for the tiny fp32 workload (T=64, H=128, E=8, k=2,
I=64), seed 0: the routing integers in full and a slice of the float outputs.
It calls nothing but ``oracle/`` and the shared input generator.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from mixture_experts_expert_amd import synth  # noqa: E402
from oracle import oracle as O  # noqa: E402


def main():
    cfg = synth.CONFIGS["tiny_f32"]
    inp = synth.make_inputs(cfg, 0, with_dy=True)
    t = {n: inp.f32(n) for n in inp.names()}
    f = O.forward(t["x"], t["w_router"], t["w_gate"], t["w_up"], t["w_down"], cfg.k)
    b = O.backward(f, t["dy"], t["w_gate"], t["w_up"], t["w_down"])
    out = {
        "workload": "tiny_f32 (T=64, H=128, E=8, k=2, I=64), seed 0, dY drawn after the weights",
        "topk_idx": f["topk_idx"].tolist(),
        "counts": f["counts"].tolist(),
        "offsets": f["offsets"].tolist(),
        "sorted_to_flat": f["sorted_to_flat"].tolist(),
        "logits_row0": [float(v) for v in f["logits"][0]],
        "topk_w_rows0_3": f["topk_w"][:4].tolist(),
        "y_rows0_3_cols0_7": f["y"][:4, :8].tolist(),
        "dx_rows0_3_cols0_7": b["dx"][:4, :8].tolist(),
        "d_logits_row0": b["d_logits"][0].tolist(),
        "dw_down_e0_rows0_3_cols0_7": b["dw_down"][0, :4, :8].tolist(),
    }
    path = os.path.join(HERE, "tiny_f32_seed0.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=0)
    print(path)


if __name__ == "__main__":
    main()
