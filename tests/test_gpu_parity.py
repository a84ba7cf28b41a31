"""GPU parity of the whole stage against the CPU oracle, through the C ABI.

Every workload, small (several GEMM tiles, ragged tails, empty experts,
k = E, E = 1) and benchmark-size (the 30B forward, the 30B, skewed and 235B
training steps), is compared element by element on every output: routing,
counts, offsets and both permutations bit for bit, every float output per
token, per sorted row or per expert (see gpu_util).
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


# Per-token outputs, per-sorted-row outputs and per-expert weight gradients.
FWD_ROWS = ["g", "u", "a", "o_perm"]
BWD_ROWS = ["do_perm", "dx_perm"]
BWD_TOKENS = ["d_topk_w", "dx", "d_logits"]
WGRADS = ["dw_gate", "dw_up", "dw_down"]


def check_all(st, ref, cfg, backward: bool) -> None:
    """Every output of the stage against the oracle's, element by element."""
    b = st.buf
    U.check_routing(st, ref)
    assert np.array_equal(U.to_np(b["x_perm"]), ref["x_perm"])  # gather is a copy
    tolerance = U.tol(cfg)
    for n in FWD_ROWS + ["y"]:
        U.check_output(n, U.to_np(b[n]), ref, tolerance)
    if backward:
        for n in BWD_ROWS + BWD_TOKENS + WGRADS:
            U.check_output(n, U.to_np(b[n]), ref, tolerance)
        # an expert that no token picked has an exactly zero weight gradient
        empty = np.nonzero(ref["counts"] == 0)[0]
        if len(empty):
            idx = torch.from_numpy(empty).cuda()
            for n in WGRADS:
                assert not b[n][idx].any().item(), n


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_small_all_outputs(cfg):
    U.say(f"[parity] {cfg}")
    U.begin(cfg.name, f"{cfg} seed 1")
    inp = synth.make_inputs(cfg, seed=1, with_dy=cfg.backward)
    d = U.DevInputs(inp)
    st = U.run_stage(d, cfg.backward)
    ref = U.oracle_full(inp, cfg.backward)
    check_all(st, ref, cfg, cfg.backward)


def test_qwen3_30b_a3b_forward_full():
    """T=4096, H=2048, E=128, k=8, I=768 forward: every output element."""
    cfg = synth.CONFIGS["qwen3_30b_a3b_fwd"]
    U.say(f"[parity] {cfg}")
    U.begin(cfg.name, f"{cfg} seed 0")
    inp = synth.make_inputs(cfg, seed=0)
    d = U.DevInputs(inp)
    st = U.run_stage(d, False)
    ref = U.oracle_full(inp, False)
    check_all(st, ref, cfg, False)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["qwen3_30b_a3b_train", "qwen3_30b_a3b_zipf_train", "qwen3_235b_a22b_train"])
def test_training_workloads_full(name):
    """Benchmark-size training steps: every element of every output against
    the oracle run on all tokens (about 20 s, 40 s and 80 s of CPU on 16
    threads)."""
    cfg = synth.CONFIGS[name]
    U.say(f"[parity] {cfg}")
    U.begin(cfg.name, f"{cfg} seed 0")
    inp = synth.make_inputs(cfg, seed=0)
    d = U.DevInputs(inp)
    st = U.run_stage(d, True)
    counts = U.to_np(st.buf["counts"])
    if cfg.zipf_s > 0:
        # The skewed workload leaves experts empty and gives one above 10%.
        assert (counts == 0).sum() >= 1 and counts.max() > 0.10 * cfg.M, counts
    U.say("  oracle on all tokens")
    ref = U.oracle_full(inp, True)
    check_all(st, ref, cfg, True)


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


def test_routing_with_nan_logits():
    """NaN logits (a hidden state holding a NaN; NaN and -inf biases) select
    exactly the oracle's experts: a NaN ranks below every number, equal
    logits (NaN or not) go to the lower index. The sort then places every row; route backward skips
    caller indices outside [0, E)."""
    from mixture_experts_expert_amd import binding as B
    from oracle import oracle as O
    nan, inf = float("nan"), float("inf")
    T, H, E, k, I = 40, 128, 16, 4, 64
    cfg = synth.MoEConfig("nan_routing", T=T, H=H, E=E, k=k, I=I, dtype="bf16", backward=True)
    U.say(f"[nan routing] {cfg}")
    inp = synth.make_inputs(cfg, seed=6, with_dy=True)
    x = inp.bits["x"].copy()
    x[3, 11] = 0x7FC0  # a bf16 NaN in token 3
    x[5] = 0  # token 5's logits are the bias itself: equal logits tie on the index
    bias = np.zeros(E, np.float32)
    bias[[1, 9]] = nan
    bias[[4, 12]] = -inf
    bias[[2, 7]] = 3.0
    s = B.shape(T, H, E, k, I, torch.bfloat16)
    dev = "cuda"
    logits = torch.empty(T, E, device=dev)
    idx = torch.empty(T, k, dtype=torch.int32, device=dev)
    w = torch.empty(T, k, device=dev)
    B.moe_route(s, U.to_dev(x), U.to_dev(inp.bits["w_router"]), torch.from_numpy(bias).to(dev), logits, idx, w)
    i32 = dict(dtype=torch.int32, device=dev)
    counts, offsets = torch.empty(E, **i32), torch.empty(E + 1, **i32)
    s2f, f2s = torch.empty(T * k, **i32), torch.empty(T * k, **i32)
    x_perm = torch.empty(T * k, H, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(B.moe_workspace_bytes(s), dtype=torch.uint8, device=dev)
    B.moe_permute(s, idx, U.to_dev(x), counts, offsets, s2f, f2s, x_perm, ws)
    # caller-supplied indices outside [0, E) contribute nothing to d_logits
    bad = idx.clone()
    bad[0, 0], bad[1, 1] = E + 3, -1
    gw = torch.arange(1, k + 1, dtype=torch.float32, device=dev).repeat(T, 1)
    wts = torch.full((T, k), 0.25, device=dev)
    d_logits = torch.full((T, E), 7.0, device=dev)
    B.moe_route_bwd(s, gw, wts, bad, d_logits)
    torch.cuda.synchronize()
    xf = synth.bf16_widen(x)
    rl, ri, rw = O.route(xf, inp.f32("w_router"), k, bias)
    gl = U.to_np(logits)
    assert np.array_equal(np.isnan(gl), np.isnan(rl))
    fin = ~np.isnan(rl)
    assert np.array_equal(gl[fin].view(np.uint32), rl[fin].view(np.uint32))
    assert np.array_equal(U.to_np(idx), ri)
    assert U.to_np(idx)[3].tolist() == [0, 1, 2, 3]  # every logit of token 3 is NaN
    assert U.to_np(idx)[5].tolist() == [2, 7, 0, 3]  # 3, 3, then the lowest-index zeros
    others = np.arange(T) != 3
    assert not np.isin(U.to_np(idx)[others], [1, 9]).any()  # NaN biases are never picked over numbers
    c, o, a, b = O.permute_index(ri, E)
    assert np.array_equal(U.to_np(counts), c) and np.array_equal(U.to_np(offsets), o)
    assert np.array_equal(U.to_np(s2f), a) and np.array_equal(U.to_np(f2s), b)
    dl = U.to_np(d_logits)
    ii = U.to_np(bad)
    for t in range(T):
        want = np.zeros(E, np.float32)
        for j in range(k):
            if 0 <= ii[t, j] < E:
                want[ii[t, j]] = 0.25 * ((j + 1) - 2.5)  # w (g_j - sum_i w g_i), exact in fp32
        assert np.array_equal(dl[t], want), t


SORT_CASES = [
    # (T, E, k, skewed): T*k = 131072 is 128 indexing blocks, the most whose
    # ranking blocks scan the block counts themselves; one pair more and the
    # column scan runs as a launch of its own.
    (16384, 128, 8, False),
    (16385, 128, 8, False),
    (30000, 1024, 4, True),
    (40000, 1024, 4, False),
    (5, 3, 2, False),
]


@pytest.mark.parametrize("T,E,k,skewed", SORT_CASES, ids=lambda v: str(v))
def test_sort_both_scan_forms(T, E, k, skewed):
    """The sort alone (moe_permute_fused) on either side of the block count
    where the column scan moves into the ranking blocks: counts, offsets,
    both permutations, and each sorted row's token and weight, bit for bit
    against the oracle's stable sort."""
    from mixture_experts_expert_amd import binding as B
    from oracle import oracle as O
    U.say(f"[sort] T={T} E={E} k={k} skewed={skewed}")
    rng = np.random.default_rng(T + E + k)
    p = None
    if skewed:
        p = 1.0 / np.arange(1, E + 1) ** 1.2
        p /= p.sum()
    idx = rng.choice(E, size=(T, k), p=p).astype(np.int32)
    w = rng.random((T, k), dtype=np.float32)
    s = B.shape(T, 64, E, k, 64, torch.bfloat16)
    dev = "cuda"
    i32 = dict(dtype=torch.int32, device=dev)
    counts, offsets = torch.empty(E, **i32), torch.empty(E + 1, **i32)
    s2f, f2s = torch.empty(T * k, **i32), torch.empty(T * k, **i32)
    row_token = torch.empty(T * k, **i32)
    row_weight = torch.empty(T * k, device=dev)
    ws = torch.empty(B.moe_workspace_bytes(s), dtype=torch.uint8, device=dev)
    B.moe_permute_fused(s, U.to_dev(idx), U.to_dev(w), counts, offsets, s2f, f2s, row_token, row_weight, ws)
    torch.cuda.synchronize()
    rc, ro, rs2f, rf2s = O.permute_index(idx, E)
    assert np.array_equal(U.to_np(counts), rc)
    assert np.array_equal(U.to_np(offsets), ro)
    assert np.array_equal(U.to_np(s2f), rs2f)
    assert np.array_equal(U.to_np(f2s), rf2s)
    assert np.array_equal(U.to_np(row_token), rs2f // k)
    assert np.array_equal(U.to_np(row_weight).view(np.uint32), w.reshape(-1)[rs2f].view(np.uint32))
