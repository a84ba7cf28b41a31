"""The training step captured into a HIP graph (torch.cuda.CUDAGraph over the
C-ABI calls) replays to the same bits as the eager step.

The library allocates nothing, issues no memset and never synchronises, so a
whole forward + backward is capturable. Each case replays the graph several
times with eager steps and synchronisations between the replays, and checks
every replay against the eager result, bit for bit; then it changes the
inputs in place and checks that a replay follows them.
"""
import numpy as np
import pytest
import torch

from mixture_experts_expert_amd import synth

import gpu_util as U
from test_gpu_parity import SPLIT_K

pytestmark = pytest.mark.gpu

OUTS = ["logits", "topk_idx", "topk_w", "offsets", "sorted_to_flat", "y", "dx", "dw_gate", "dw_up", "dw_down",
        "d_logits"]


def bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


@pytest.mark.parametrize("cfg,gather_fused", [(SPLIT_K, False), (SPLIT_K, True),
                                              (synth.CONFIGS["qwen3_30b_a3b_train"], False)],
                         ids=["split_k", "split_k-gather_fused", "qwen3_30b_a3b_train"])
def test_captured_step_replays_bitwise(cfg, gather_fused):
    from mixture_experts_expert_amd import binding as B
    U.say(f"[graph] {cfg} gather_fused={gather_fused}")
    inp = synth.make_inputs(cfg, seed=6, with_dy=True)
    d = U.DevInputs(inp)
    T = d.t["x"].shape[0]
    st = B.MoEStage(T, cfg.H, cfg.E, cfg.k, cfg.I, torch.bfloat16, gather_fused=gather_fused)
    x = d.t["x"].clone()
    dy = d.t["dy"].clone()

    def step():
        st.forward(x, d.t["w_router"], d.t["w_gate"], d.t["w_up"], d.t["w_down"], d.bias)
        st.backward(dy)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # eager, on the capture stream: every buffer exists before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = {n: st.buf[n].clone() for n in OUTS}

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step()
    for rep in range(3):
        for n in OUTS:
            st.buf[n].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in OUTS:
            assert torch.equal(bits(st.buf[n]), bits(ref[n])), (rep, n)
        step()  # eager work between replays
        torch.cuda.synchronize()
        for n in OUTS:
            assert torch.equal(bits(st.buf[n]), bits(ref[n])), ("eager", rep, n)

    # new inputs in the captured buffers: the replay computes on them
    x.copy_(torch.flip(d.t["x"], dims=[0]))
    dy.copy_(torch.flip(d.t["dy"], dims=[0]))
    step()
    torch.cuda.synchronize()
    ref2 = {n: st.buf[n].clone() for n in OUTS}
    assert not torch.equal(bits(ref2["y"]), bits(ref["y"]))
    for n in OUTS:
        st.buf[n].zero_()
    g.replay()
    torch.cuda.synchronize()
    for n in OUTS:
        assert torch.equal(bits(st.buf[n]), bits(ref2[n])), ("new inputs", n)
