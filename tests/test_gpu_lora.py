"""GPU parity of the adapter (LoRA) path against the adapter oracle, through
the C ABI.

- moe_lora_merge: every element of W' = W + s B A within one bf16 rounding of
  the float64 definition, and nearly every element equal to its nearest bf16
  (ragged 128 x 128 tiles, ranks 8 to 128, in place and out of place).
- The stage with adapters (LoRAStage: merge, the forward on W', the data
  gradients, moe_lora_grads): routing bit-exact; y, dx, d_topk_w, d_logits
  and the six adapter gradients within the bf16 tolerance of the float64
  oracle. Small shapes cover a padded rank (16 -> 64) and an unpadded one,
  experts with no rows (zero gradients), many experts and a split-K
  reduction; the full 30B-A3B training shape is checked on sampled tokens
  (y, dx and the routing gradients are per token) and on whole sampled
  experts (an expert's adapter gradients depend on its own rows only).
"""
import numpy as np
import pytest
import torch

from mixture_experts_expert_amd import synth
from oracle import lora as LO
from oracle import oracle as O

import gpu_util as U
from test_gpu_parity import SPLIT_K

pytestmark = pytest.mark.gpu

NAMES = synth.ADAPTER_NAMES


def widen(bits: np.ndarray) -> np.ndarray:
    return synth.bf16_widen(bits).astype(np.float64)


@pytest.mark.parametrize("E,N,K,r", [(3, 200, 264, 8), (2, 128, 128, 16), (4, 257, 520, 40), (2, 70, 2048, 128),
                                     (1, 1, 8, 64)])
@pytest.mark.parametrize("in_place", [False, True], ids=["out", "in_place"])
def test_merge(E, N, K, r, in_place):
    from mixture_experts_expert_amd import binding as B
    U.say(f"[lora merge] E={E} N={N} K={K} r={r} in_place={in_place}")
    rng = np.random.default_rng(E * 7919 + N * 31 + K + r)
    w = synth.bf16_round(np.float32(0.02) * rng.standard_normal((E, N, K), dtype=np.float32))
    a = synth.bf16_round(np.float32(0.02) * rng.standard_normal((E, r, K), dtype=np.float32))
    b = synth.bf16_round(np.float32(0.02) * rng.standard_normal((E, N, r), dtype=np.float32))
    s = 1.75
    wd, ad, bd = U.to_dev(w), U.to_dev(a), U.to_dev(b)
    out = wd if in_place else torch.full_like(wd, float("nan"))
    B.moe_lora_merge(E, N, K, r, s, wd, ad, bd, out)
    torch.cuda.synchronize()
    got = U.to_np(out).astype(np.float64)
    ref = LO.merge(widen(w), widen(a), widen(b), s)
    lowrank = np.abs(ref - widen(w))
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -22 * (np.abs(widen(w)) + lowrank)
    assert np.all(np.abs(got - ref) <= bound), float(np.max(np.abs(got - ref) - bound))
    nearest = widen(synth.bf16_round(ref.astype(np.float32)))
    frac = float(np.mean(got == nearest))
    U.say(f"  equal to the nearest bf16: {frac:.5f}")
    assert frac >= 0.999


def lora_run(d: U.DevInputs, r: int, s: float, adapters):
    from mixture_experts_expert_amd import binding as B
    c = d.cfg
    T = d.t["x"].shape[0]
    ad = {n: U.to_dev(adapters[n]) for n in NAMES}
    st = B.LoRAStage(T, c.H, c.E, c.k, c.I, r, s)
    st.forward(d.t["x"], d.t["w_router"], d.t["w_gate"], d.t["w_up"], d.t["w_down"], ad, d.bias)
    st.backward(d.t["dy"])
    torch.cuda.synchronize()
    assert "dw_gate" not in st.buf  # the frozen weights get no gradient
    return st


def oracle_lora(inp, adapters, s, idx, w, rows=None):
    x, dy = inp.f32("x").astype(np.float64), inp.f32("dy").astype(np.float64)
    if rows is not None:
        x, dy, idx, w = x[rows], dy[rows], idx[rows], w[rows]
    ws = [inp.f32(n).astype(np.float64) for n in ["w_gate", "w_up", "w_down"]]
    return LO.forward_backward(x, dy, idx, w.astype(np.float64), *ws, {n: widen(adapters[n]) for n in NAMES}, s)


def check_tokens(st, ref_r, ref, rows=None):
    b = st.buf
    sel = (lambda t: t) if rows is None else (lambda t: t[torch.from_numpy(rows).cuda()])
    logits = ref_r["logits"] if rows is None else ref_r["logits"][rows]
    idx = ref_r["topk_idx"] if rows is None else ref_r["topk_idx"][rows]
    U.check_close("y", U.to_np(sel(b["y"])), ref["y"], U.BF16_TOL)
    U.check_close("dx", U.to_np(sel(b["dx"])), ref["dx"], U.BF16_TOL)
    U.check_close("d_topk_w", U.to_np(sel(b["d_topk_w"])), ref["d_topk_w"], U.BF16_TOL)
    d_logits = O.route_bwd(logits, idx, ref["d_topk_w"].astype(np.float32))
    U.check_close("d_logits", U.to_np(sel(b["d_logits"])), d_logits, U.BF16_TOL)


SMALL_LORA = [
    (synth.MoEConfig("bf16_tiles", T=700, H=512, E=6, k=2, I=320, dtype="bf16", backward=True), 16),
    (synth.MoEConfig("bf16_tiles", T=700, H=512, E=6, k=2, I=320, dtype="bf16", backward=True), 64),
    (synth.MoEConfig("bf16_many_experts", T=333, H=256, E=40, k=5, I=128, dtype="bf16", backward=True), 32),
    (synth.MoEConfig("bf16_one_token", T=1, H=64, E=16, k=8, I=64, dtype="bf16", backward=True), 8),
    (synth.MoEConfig("bf16_skew", T=900, H=256, E=32, k=4, I=128, dtype="bf16", backward=True, zipf_s=2.5), 128),
    (SPLIT_K, 64),
]


@pytest.mark.parametrize("cfg,r", SMALL_LORA, ids=[f"{c.name}-r{r}" for c, r in SMALL_LORA])
def test_lora_stage_small(cfg, r):
    U.say(f"[lora stage] {cfg} r={r}")
    s = 2.0 if r == 64 else 0.75
    inp = synth.make_inputs(cfg, seed=8, with_dy=True)
    adapters = synth.make_adapters(cfg, r, seed=8)
    d = U.DevInputs(inp)
    st = lora_run(d, r, s, adapters)
    ref_r = U.oracle_route(inp)
    U.check_routing(st, ref_r)
    ref = oracle_lora(inp, adapters, s, ref_r["topk_idx"], ref_r["topk_w"])
    check_tokens(st, ref_r, ref)
    counts = ref_r["counts"]
    for n in NAMES:
        got = U.to_np(st.buf["d" + n])
        U.check_close("d" + n, got, ref["d" + n], U.BF16_TOL)
        assert not np.any(got[counts == 0]), ("experts without rows", n)


def test_lora_stage_qwen3_30b_a3b_full():
    """T=8192, H=2048, E=128, k=8, I=768, r=64, s=2: sampled tokens and experts."""
    cfg = synth.CONFIGS["qwen3_30b_a3b_train"]
    r, s = 64, 2.0
    U.say(f"[lora stage] {cfg} r={r}")
    inp = synth.make_inputs(cfg, seed=0)
    adapters = synth.make_adapters(cfg, r, seed=0)
    d = U.DevInputs(inp)
    st = lora_run(d, r, s, adapters)
    ref_r = U.oracle_route(inp)
    U.check_routing(st, ref_r)
    rows = U.sample_tokens(cfg.T, 48)
    U.say(f"  oracle on {len(rows)} sampled tokens")
    check_tokens(st, ref_r, oracle_lora(inp, adapters, s, ref_r["topk_idx"], ref_r["topk_w"], rows=rows), rows)
    counts = ref_r["counts"]
    experts = sorted({0, int(np.argmax(counts)), int(np.argmin(counts)), cfg.E - 1})
    idx = np.where(np.isin(ref_r["topk_idx"], experts), ref_r["topk_idx"], -1).astype(np.int32)
    U.say(f"  oracle on experts {experts} ({[int(counts[e]) for e in experts]} rows)")
    ref = oracle_lora(inp, adapters, s, idx, ref_r["topk_w"])
    for n in NAMES:
        U.check_close("d" + n, U.to_np(st.buf["d" + n][experts]), ref["d" + n][experts], U.BF16_TOL)


def test_lora_merges_on_a_second_stream_same_bits():
    """LoRAStage.forward(aux_stream=...) runs the merges concurrently with the
    routing and the sort: every output equals the one-stream step bit for bit,
    over two steps (the second merge overwrites weights the first backward read)."""
    from mixture_experts_expert_amd import binding as B
    cfg, r, s = SPLIT_K, 64, 2.0
    U.say(f"[lora two streams] {cfg} r={r}")
    inp = synth.make_inputs(cfg, seed=9, with_dy=True)
    adapters = synth.make_adapters(cfg, r, seed=9)
    d = U.DevInputs(inp)
    ad = {n: U.to_dev(adapters[n]) for n in NAMES}
    T = d.t["x"].shape[0]
    outs = ["y", "dx", "d_logits", "topk_idx", "offsets"] + ["d" + n for n in NAMES]

    def run(aux):
        st = B.LoRAStage(T, cfg.H, cfg.E, cfg.k, cfg.I, r, s)
        for _ in range(2):
            st.forward(d.t["x"], d.t["w_router"], d.t["w_gate"], d.t["w_up"], d.t["w_down"], ad, d.bias,
                       aux_stream=aux)
            st.backward(d.t["dy"])
        torch.cuda.synchronize()
        return {n: st.buf[n].clone() for n in outs}, [w.clone() for w in st.merged]

    ref, ref_w = run(None)
    got, got_w = run(torch.cuda.Stream())
    for n in outs:
        a, b_ = ref[n], got[n]
        if a.dtype == torch.bfloat16:
            a, b_ = a.view(torch.int16), b_.view(torch.int16)
        assert torch.equal(a, b_), n
    for a, b_ in zip(ref_w, got_w):
        assert torch.equal(a.view(torch.int16), b_.view(torch.int16))
