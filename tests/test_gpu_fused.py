"""GPU parity of the fused gather and routing weights (inside the GEMMs)
against the CPU oracle and against the unfused path, through the C ABI:
the inference forward, and the training step without x_perm.

- Routing, counts, offsets and both permutations are bit-exact against the
  oracle; row_token and row_weight are exactly sorted_to_flat // k and
  topk_w[sorted_to_flat].
- The gathered gate/up GEMM multiplies the same rows in the same order as the
  x_perm one: its G, U and A are bit-identical to the unfused GEMM's.
- Training without x_perm (gate/up and its weight gradient read x through
  row_token) gives every output of the stage bit-identical to the x_perm
  path: the same rows meet the same weights in the same order.
- The weighted down GEMM with every weight 1.0 is bit-identical to the plain
  one; with the routing weights, y is within the dtype's tolerance of the
  oracle (the weight is applied before the rounding to the activation dtype
  instead of after it, and the k-sum adds weighted rows instead of
  multiply-adding them).
"""
import numpy as np
import pytest
import torch

from mixture_experts_expert_amd import synth

import gpu_util as U
from test_gpu_parity import SMALL, SPLIT_K

pytestmark = pytest.mark.gpu


def fused_forward(d: U.DevInputs):
    from mixture_experts_expert_amd import binding as B
    c = d.cfg
    T, M = d.t["x"].shape[0], c.T * c.k
    dt = torch.bfloat16 if c.dtype == "bf16" else torch.float32
    s = B.shape(T, c.H, c.E, c.k, c.I, dt)
    dev = "cuda"
    out = dict(
        logits=torch.empty(T, c.E, device=dev), topk_idx=torch.empty(T, c.k, dtype=torch.int32, device=dev),
        topk_w=torch.empty(T, c.k, device=dev), counts=torch.empty(c.E, dtype=torch.int32, device=dev),
        offsets=torch.empty(c.E + 1, dtype=torch.int32, device=dev),
        sorted_to_flat=torch.empty(M, dtype=torch.int32, device=dev),
        flat_to_sorted=torch.empty(M, dtype=torch.int32, device=dev),
        row_token=torch.empty(M, dtype=torch.int32, device=dev), row_weight=torch.empty(M, device=dev),
        a=torch.empty(M, c.I, dtype=dt, device=dev), o_perm=torch.empty(M, c.H, dtype=dt, device=dev),
        y=torch.empty(T, c.H, dtype=dt, device=dev))
    ws = torch.empty(B.moe_workspace_bytes(s), dtype=torch.uint8, device=dev)
    B.moe_forward_fused(s, d.t["x"], d.t["w_router"], d.bias, d.t["w_gate"], d.t["w_up"], d.t["w_down"],
                        out["logits"], out["topk_idx"], out["topk_w"], out["counts"], out["offsets"],
                        out["sorted_to_flat"], out["flat_to_sorted"], out["row_token"], out["row_weight"], out["a"],
                        out["o_perm"], out["y"], ws)
    torch.cuda.synchronize()
    return s, out


def check_fused_indices(out, k: int) -> None:
    s2f = U.to_np(out["sorted_to_flat"]).astype(np.int64)
    assert np.array_equal(U.to_np(out["row_token"]), (s2f // k).astype(np.int32))
    assert U.same_bits(U.to_np(out["row_weight"]), U.to_np(out["topk_w"]).reshape(-1)[s2f])


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_fused_forward_small(cfg):
    from mixture_experts_expert_amd import binding as B
    U.say(f"[fused] {cfg}")
    U.begin("fused_forward." + cfg.name, f"{cfg}, fused inference forward")
    inp = synth.make_inputs(cfg, seed=1, with_dy=False)
    d = U.DevInputs(inp)
    s, out = fused_forward(d)
    ref = U.oracle_full(inp, False)
    b = out
    assert U.same_bits(U.to_np(b["logits"]), ref["logits"]), "logits differ"
    for n in ["topk_idx", "counts", "offsets", "sorted_to_flat", "flat_to_sorted"]:
        assert np.array_equal(U.to_np(b[n]), ref[n]), n
    check_fused_indices(out, cfg.k)
    tolerance = U.tol(cfg)
    U.check_close("a", U.to_np(b["a"]), ref["a"], tolerance)
    U.check_close("y", U.to_np(b["y"]), ref["y"], tolerance)

    # The unfused stage on the same inputs: gathered gate/up equals the x_perm
    # GEMM bit for bit; down with unit weights equals plain down bit for bit.
    st = U.run_stage(d, False)
    ub = st.buf
    dt = ub["g"].dtype
    g = torch.empty_like(ub["g"])
    u = torch.empty_like(ub["u"])
    a = torch.empty_like(ub["a"])
    B.moe_gemm_gate_up_gathered(s, d.t["x"], out["row_token"], out["offsets"], d.t["w_gate"], d.t["w_up"], g, u, a)
    ones = torch.ones_like(out["row_weight"])
    o1 = torch.empty_like(ub["o_perm"])
    B.moe_gemm_down_weighted(s, ub["a"], out["offsets"], d.t["w_down"], ones, o1)
    torch.cuda.synchronize()
    for n, t in [("g", g), ("u", u), ("a", a)]:
        assert torch.equal(t.view(torch.int16) if dt == torch.bfloat16 else t,
                           ub[n].view(torch.int16) if dt == torch.bfloat16 else ub[n]), n
    assert torch.equal(o1.view(torch.int16) if dt == torch.bfloat16 else o1,
                       ub["o_perm"].view(torch.int16) if dt == torch.bfloat16 else ub["o_perm"])


def test_fused_forward_qwen3_30b_a3b_full():
    """T=4096, H=2048, E=128, k=8, I=768, the fused inference forward: every output element."""
    cfg = synth.CONFIGS["qwen3_30b_a3b_fwd"]
    U.say(f"[fused] {cfg}")
    U.begin("fused_forward." + cfg.name, f"{cfg} seed 0, fused inference forward")
    inp = synth.make_inputs(cfg, seed=0)
    d = U.DevInputs(inp)
    s, out = fused_forward(d)
    ref = U.oracle_full(inp, False)
    assert U.same_bits(U.to_np(out["logits"]), ref["logits"]), "logits differ"
    for n in ["topk_idx", "counts", "offsets", "sorted_to_flat", "flat_to_sorted"]:
        assert np.array_equal(U.to_np(out[n]), ref[n]), n
    check_fused_indices(out, cfg.k)
    for n in ["a", "y"]:
        U.check_close(n, U.to_np(out[n]), ref[n], U.BF16_TOL)


STAGE_OUT = ["logits", "topk_idx", "topk_w", "counts", "offsets", "sorted_to_flat", "flat_to_sorted", "g", "u", "a",
             "o_perm", "y", "do_perm", "d_topk_w", "dx_perm", "dx", "dw_gate", "dw_up", "dw_down", "d_logits"]


def same_tensor(a: torch.Tensor, b: torch.Tensor) -> bool:
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    return torch.equal(a, b)


def gather_fused_stage(d: U.DevInputs):
    from mixture_experts_expert_amd import binding as B
    c = d.cfg
    return B.MoEStage(d.t["x"].shape[0], c.H, c.E, c.k, c.I, torch.bfloat16 if c.dtype == "bf16" else torch.float32,
                      gather_fused=True)


@pytest.mark.parametrize("cfg", [c for c in SMALL if c.backward] + [SPLIT_K], ids=lambda c: c.name)
def test_gather_fused_training_small(cfg):
    """Training step without x_perm: every output bit-identical to the x_perm
    path (overwrite and accumulate, one and two streams), and within the
    tolerance of the oracle."""
    U.say(f"[gather-fused training] {cfg}")
    U.begin("gather_fused." + cfg.name, f"{cfg} seed 2, training without x_perm")
    inp = synth.make_inputs(cfg, seed=2, with_dy=True)
    d = U.DevInputs(inp)
    plain = U.run_stage(d, True)
    st = U.run_stage(d, True, stage=gather_fused_stage(d))
    assert "x_perm" not in st.buf
    check_fused_indices(st.buf, cfg.k)
    for n in STAGE_OUT:
        assert same_tensor(st.buf[n], plain.buf[n]), n
    ref = U.oracle_full(inp, True)
    tolerance = U.tol(cfg)
    for n in ["y", "dx", "dw_gate", "dw_up", "dw_down", "d_logits"]:
        U.check_output(n, U.to_np(st.buf[n]), ref, tolerance)
    # accumulate_dw on both, then the two-stream backward (overwrite).
    U.run_stage(d, True, accumulate=True, stage=plain)
    U.run_stage(d, True, accumulate=True, stage=st)
    for n in ["dw_gate", "dw_up", "dw_down"]:
        assert same_tensor(st.buf[n], plain.buf[n]), (n, "accumulate")
    aux = torch.cuda.Stream()
    U.run_stage(d, False, stage=st)
    st.backward(d.t["dy"], aux_stream=aux)
    U.run_stage(d, True, stage=plain)
    torch.cuda.synchronize()
    for n in ["dx", "dw_gate", "dw_up", "dw_down", "d_logits"]:
        assert same_tensor(st.buf[n], plain.buf[n]), (n, "two streams")


@pytest.mark.timeout(600)
def test_gather_fused_training_qwen3_30b_a3b_full():
    """T=8192, H=2048, E=128, k=8, I=768: the training step without x_perm
    equals the x_perm path bit for bit on every output, and every element of
    y, dx, the weight gradients and d_logits is within tolerance of the
    oracle."""
    cfg = synth.CONFIGS["qwen3_30b_a3b_train"]
    U.say(f"[gather-fused training] {cfg}")
    U.begin("gather_fused." + cfg.name, f"{cfg} seed 0, training without x_perm")
    inp = synth.make_inputs(cfg, seed=0)
    d = U.DevInputs(inp)
    plain = U.run_stage(d, True)
    st = U.run_stage(d, True, stage=gather_fused_stage(d))
    check_fused_indices(st.buf, cfg.k)
    for n in STAGE_OUT:
        assert same_tensor(st.buf[n], plain.buf[n]), n
    U.say("  oracle on all tokens")
    ref = U.oracle_full(inp, True)
    for n in ["y", "dx", "dw_gate", "dw_up", "dw_down", "d_logits"]:
        U.check_output(n, U.to_np(st.buf[n]), ref, U.BF16_TOL)



@pytest.mark.timeout(600)
def test_gather_fused_weight_grads_repeat_bitwise():
    """T=8192, H=2048, E=128, k=8, I=768: the gathered gate/up backward (x
    read through the tokens, token loads among the operand loads) gives the
    x_perm path's weight gradients bit for bit in each of six runs. A wait
    one load short in the first tile of a workgroup once let a run read a
    stage before its last block landed (a whole 256 x 256 tile off)."""
    cfg = synth.CONFIGS["qwen3_30b_a3b_train"]
    U.say(f"[gather-fused weight gradients, repeated] {cfg}")
    inp = synth.make_inputs(cfg, seed=0)
    d = U.DevInputs(inp)
    plain = U.run_stage(d, True)
    ref = {n: plain.buf[n].clone() for n in ["dw_gate", "dw_up", "dw_down"]}
    del plain
    for rep in range(6):
        st = U.run_stage(d, True, stage=gather_fused_stage(d))
        for n, v in ref.items():
            assert same_tensor(st.buf[n], v), (rep, n)
        del st

# ---- training without do_perm (dy read through the sorted rows' tokens) ----

DY_SMALL = [c for c in SMALL if c.backward and c.dtype == "bf16"] + [SPLIT_K]
FWD_SAME = ["logits", "topk_idx", "topk_w", "counts", "offsets", "sorted_to_flat", "flat_to_sorted", "g", "u", "a",
            "o_perm", "y", "d_topk_w", "d_logits"]


def dy_fused_stage(d: U.DevInputs, gather_fused: bool):
    from mixture_experts_expert_amd import binding as B
    c = d.cfg
    return B.MoEStage(d.t["x"].shape[0], c.H, c.E, c.k, c.I, torch.bfloat16, gather_fused=gather_fused,
                      dy_fused=True)


def check_dy_fused(d: U.DevInputs, st, plain, ref, tolerance):
    """Forward, d_topk_w and d_logits bit-identical to the do_perm path (same
    kernels and sums); a_w, dx_perm, dx and the weight gradients within
    tolerance of the oracle."""
    c = d.cfg
    for n in FWD_SAME:
        assert same_tensor(st.buf[n], plain.buf[n]), n
    check_fused_indices(st.buf, c.k)
    assert "do_perm" not in st.buf
    # a_w = bf16(w a): the oracle's fp32 a times the sorted row's routing weight
    s2f = ref["sorted_to_flat"].astype(np.int64)
    a_w = ref["a"].astype(np.float64) * ref["topk_w"].reshape(-1)[s2f][:, None]
    U.check_close("a_w", U.to_np(st.buf["a_w"]), a_w, tolerance)
    for n in ["dx_perm", "dx", "dw_gate", "dw_up", "dw_down"]:
        U.check_output(n, U.to_np(st.buf[n]), ref, tolerance)
    empty = np.nonzero(ref["counts"] == 0)[0]
    if len(empty):
        idx = torch.from_numpy(empty).cuda()
        for n in ["dw_gate", "dw_up", "dw_down"]:
            assert not st.buf[n][idx].any().item(), n


@pytest.mark.parametrize("gather", [False, True], ids=["x_perm", "gathered_x"])
@pytest.mark.parametrize("cfg", DY_SMALL, ids=lambda c: c.name)
def test_dy_fused_training_small(cfg, gather):
    """Training step without do_perm (moe_permute_rows or moe_permute_fused,
    moe_gemm_gate_up_aw, moe_combine_bwd without do_perm,
    moe_gemm_down_bwd_dy): against the do_perm path and the oracle, then
    accumulate_dw adding a second pass onto the first."""
    U.say(f"[dy-fused training] {cfg} gathered x={gather}")
    U.begin(f"dy_fused{'_gathered' if gather else ''}.{cfg.name}", f"{cfg} seed 2, training without do_perm")
    inp = synth.make_inputs(cfg, seed=2, with_dy=True)
    d = U.DevInputs(inp)
    plain = U.run_stage(d, True)
    st = U.run_stage(d, True, stage=dy_fused_stage(d, gather))
    ref = U.oracle_full(inp, True)
    check_dy_fused(d, st, plain, ref, U.BF16_TOL)
    first = {n: st.buf[n].clone() for n in ["dw_gate", "dw_up", "dw_down", "dx"]}
    U.run_stage(d, True, stage=st)  # a rerun: the same bits
    for n, v in first.items():
        assert same_tensor(st.buf[n], v), (n, "rerun")
    st.backward(d.t["dy"], accumulate_dw=True)
    torch.cuda.synchronize()
    for n in ["dw_gate", "dw_up", "dw_down"]:
        U.check_close(n + " x2", U.to_np(st.buf[n]), 2.0 * U.to_np(first[n]), 1e-6)


@pytest.mark.timeout(600)
def test_dy_fused_training_qwen3_30b_a3b_full():
    """T=8192, H=2048, E=128, k=8, I=768, training without do_perm: every
    element against the oracle, and bit-identical to the do_perm path where
    the arithmetic is the same (forward, d_topk_w, d_logits)."""
    cfg = synth.CONFIGS["qwen3_30b_a3b_train"]
    U.say(f"[dy-fused training] {cfg}")
    U.begin("dy_fused." + cfg.name, f"{cfg} seed 0, training without do_perm")
    inp = synth.make_inputs(cfg, seed=0)
    d = U.DevInputs(inp)
    plain = U.run_stage(d, True)
    st = U.run_stage(d, True, stage=dy_fused_stage(d, False))
    U.say("  oracle on all tokens")
    ref = U.oracle_full(inp, True)
    check_dy_fused(d, st, plain, ref, U.BF16_TOL)
