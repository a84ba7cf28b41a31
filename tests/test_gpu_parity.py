"""GPU parity of the whole stage against the CPU oracle, through the C ABI.

Small workloads are compared element by element on every output (several
GEMM tiles, ragged tails, empty experts, k = E, E = 1). The benchmark-size
workloads are compared on routing in full (bit-exact) and on sampled token
rows and whole sampled experts, which the oracle computes one by one.
"""
import numpy as np
import pytest
import torch

from mixture_experts_expert_amd import synth

import gpu_util as U

pytestmark = pytest.mark.gpu

SPLIT_K = synth.MoEConfig("bf16_split_k", T=4096, H=256, E=8, k=2, I=128, dtype="bf16", backward=True, zipf_s=4.0)

SMALL = [
    synth.CONFIGS["tiny_f32"],
    synth.MoEConfig("tiny_f32_train", T=64, H=128, E=8, k=2, I=64, dtype="f32", backward=True),
    synth.MoEConfig("bf16_tiles", T=700, H=512, E=6, k=2, I=320, dtype="bf16", backward=True),
    synth.MoEConfig("bf16_many_experts", T=333, H=256, E=40, k=5, I=128, dtype="bf16", backward=True),
    synth.MoEConfig("bf16_k_eq_E", T=97, H=128, E=4, k=4, I=192, dtype="bf16", backward=True),
    synth.MoEConfig("bf16_one_expert", T=300, H=192, E=1, k=1, I=64, dtype="bf16", backward=True),
    synth.MoEConfig("bf16_one_token", T=1, H=64, E=16, k=8, I=64, dtype="bf16", backward=True),
    synth.MoEConfig("bf16_wide_E", T=200, H=128, E=1024, k=4, I=64, dtype="bf16", backward=True),
    synth.MoEConfig("bf16_skew", T=900, H=256, E=32, k=4, I=128, dtype="bf16", backward=True, zipf_s=2.5),
    # Two experts take nearly every row (about T each): their weight gradients
    # are reduced in two chunks with a partial-tile reduction (split-K); the
    # down gradient's 128 columns make a ragged partial tile.
    SPLIT_K,
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_small_all_outputs(cfg):
    U.say(f"[parity] {cfg}")
    inp = synth.make_inputs(cfg, seed=1, with_dy=cfg.backward)
    d = U.DevInputs(inp)
    st = U.run_stage(d, cfg.backward)
    ref = U.oracle_full(inp, cfg.backward)
    U.check_routing(st, ref)
    b = st.buf
    assert np.array_equal(U.to_np(b["x_perm"]), ref["x_perm"])  # gather is a copy
    tolerance = U.tol(cfg)
    for n in ["g", "u", "a", "o_perm", "y"]:
        U.check_close(n, U.to_np(b[n]), ref[n], tolerance)
    if cfg.backward:
        for n in ["do_perm", "d_topk_w", "dx_perm", "dx", "dw_gate", "dw_up", "dw_down", "d_logits"]:
            U.check_close(n, U.to_np(b[n]), ref[n], tolerance)
        empty = np.nonzero(ref["counts"] == 0)[0]
        for n in ["dw_gate", "dw_up", "dw_down"]:
            assert not b[n][torch.from_numpy(empty).cuda()].any().item() if len(empty) else True


def test_qwen3_30b_a3b_forward_full():
    """T=4096, H=2048, E=128, k=8, I=768 forward: every output element."""
    cfg = synth.CONFIGS["qwen3_30b_a3b_fwd"]
    U.say(f"[parity] {cfg}")
    inp = synth.make_inputs(cfg, seed=0)
    d = U.DevInputs(inp)
    st = U.run_stage(d, False)
    ref = U.oracle_full(inp, False)
    U.check_routing(st, ref)
    for n in ["g", "a", "o_perm", "y"]:
        U.check_close(n, U.to_np(st.buf[n]), ref[n], U.BF16_TOL)


@pytest.mark.parametrize("name", ["qwen3_30b_a3b_train", "qwen3_30b_a3b_zipf_train", "qwen3_235b_a22b_train"])
def test_training_workloads_sampled(name):
    """Benchmark-size training steps: routing in full, sampled rows and experts."""
    cfg = synth.CONFIGS[name]
    U.say(f"[parity] {cfg}")
    inp = synth.make_inputs(cfg, seed=0)
    d = U.DevInputs(inp)
    st = U.run_stage(d, True)
    U.say("  oracle routing on all tokens")
    U.check_routing(st, U.oracle_route(inp))
    counts = U.to_np(st.buf["counts"])
    order = np.argsort(counts, kind="stable")
    experts = sorted({int(order[-1]), int(order[len(order) // 2]), int(order[0])})
    if cfg.zipf_s > 0:
        # The skewed workload leaves experts empty and gives one above 10%.
        assert (counts == 0).sum() >= 1 and counts.max() > 0.10 * cfg.M, counts
    U.check_sampled(d, st, experts)


def test_split_k_is_deterministic_and_accumulates():
    """Bitwise-identical reruns (no float atomics anywhere, split-K included),
    and accumulate_dw adds a second pass onto the first."""
    cfg = SPLIT_K
    U.say(f"[determinism] {cfg}")
    inp = synth.make_inputs(cfg, seed=3, with_dy=True)
    d = U.DevInputs(inp)
    st = U.run_stage(d, True)
    counts = U.to_np(st.buf["counts"])
    assert counts.max() > 2048, counts  # the plan splits experts above 64 k-steps of 32 rows here
    first = {n: st.buf[n].clone() for n in ["y", "dx", "dw_gate", "dw_up", "dw_down", "d_logits", "dx_perm"]}
    U.run_stage(d, True, stage=st)
    for n, v in first.items():
        assert torch.equal(st.buf[n], v), n
    U.run_stage(d, True, accumulate=True, stage=st)
    for n in ["dw_gate", "dw_up", "dw_down"]:
        U.check_close(n + " x2", U.to_np(st.buf[n]), 2.0 * U.to_np(first[n]), 1e-6)


@pytest.mark.parametrize("cfg", [SMALL[2], SPLIT_K], ids=lambda c: c.name)
def test_two_stream_backward_same_bits(cfg):
    """Weight-gradient GEMMs on a second stream: the same bits as one stream."""
    from mixture_experts_expert_amd import binding as B
    U.say(f"[two streams] {cfg}")
    inp = synth.make_inputs(cfg, seed=3, with_dy=True)
    d = U.DevInputs(inp)
    st = U.run_stage(d, True)
    names = ["dx", "dx_perm", "dw_gate", "dw_up", "dw_down", "d_logits"]
    ref = {n: st.buf[n].clone() for n in names}
    aux = torch.cuda.Stream()
    for accumulate in (False, True):
        st.backward(d.t["dy"], accumulate_dw=accumulate, aux_stream=aux)
        torch.cuda.synchronize()
        for n in names:
            if accumulate and n.startswith("dw"):
                # old + new, with split-K chunks added in order: 2x within rounding
                assert torch.allclose(st.buf[n], ref[n] * 2, rtol=1e-6, atol=1e-6), (n, accumulate)
            else:
                assert torch.equal(st.buf[n], ref[n]), (n, accumulate)


@pytest.mark.parametrize("cfg", [SMALL[1], SMALL[2], SMALL[3], SPLIT_K, synth.CONFIGS["qwen3_30b_a3b_train"]],
                         ids=lambda c: c.name)
def test_paired_backward_gemms_same_bits(cfg):
    """moe_gemm_down_bwd and moe_gemm_gate_up_bwd (a data gradient and a
    weight gradient per launch) against the four single-GEMM calls on the
    same inputs: the same bits, overwriting and accumulating."""
    from mixture_experts_expert_amd import binding as B
    U.say(f"[paired backward GEMMs] {cfg}")
    inp = synth.make_inputs(cfg, seed=4, with_dy=True)
    d = U.DevInputs(inp)
    st = U.run_stage(d, True)
    b, s = st.buf, st.s
    wg, wu, wd = d.t["w_gate"], d.t["w_up"], d.t["w_down"]
    M = b["a"].shape[0]
    out = {}
    for mode in ("single", "paired"):
        o = dict(dgu=torch.empty(M, 2 * cfg.I, dtype=b["a"].dtype, device="cuda"),
                 dx_perm=torch.empty_like(b["dx_perm"]),
                 dw_gate=torch.full_like(b["dw_gate"], 0.5), dw_up=torch.full_like(b["dw_up"], -0.25),
                 dw_down=torch.full_like(b["dw_down"], 0.125))
        for acc in (0, 1):
            if mode == "single":
                B.moe_gemm_down_dgrad(s, b["do_perm"], b["offsets"], wd, b["g"], b["u"], o["dgu"])
                B.moe_gemm_down_wgrad(s, b["do_perm"], b["a"], b["offsets"], o["dw_down"], acc, st.ws)
                B.moe_gemm_gate_up_dgrad(s, o["dgu"], b["offsets"], wg, wu, o["dx_perm"])
                B.moe_gemm_gate_up_wgrad(s, o["dgu"], b["x_perm"], b["offsets"], o["dw_gate"], o["dw_up"], acc, st.ws)
            else:
                B.moe_gemm_down_bwd(s, b["do_perm"], b["a"], b["offsets"], wd, b["g"], b["u"], o["dgu"],
                                    o["dw_down"], acc, st.ws)
                B.moe_gemm_gate_up_bwd(s, o["dgu"], b["x_perm"], None, b["offsets"], wg, wu, o["dx_perm"],
                                       o["dw_gate"], o["dw_up"], acc, st.ws)
            torch.cuda.synchronize()
            out[(mode, acc)] = {n: t.clone() for n, t in o.items()}
    for acc in (0, 1):
        for n in out[("single", acc)]:
            x, y = out[("single", acc)][n], out[("paired", acc)][n]
            if x.dtype == torch.bfloat16:
                x, y = x.view(torch.int16), y.view(torch.int16)
            assert torch.equal(x, y), (n, acc)
    # and the stage's own backward (moe_grouped_gemm_bwd chains the paired calls)
    for n in ["dx_perm", "dw_gate", "dw_up", "dw_down"]:
        assert torch.equal(b[n], out[("single", 0)][n]), n
