"""GPU parity of the adapter (LoRA) path against the adapter oracle, through
the C ABI.

- moe_lora_merge: every element of W' = W + s B A within one bf16 rounding of
  the float64 definition, and nearly every element equal to its nearest bf16
  (ragged 128 x 128 tiles, ranks 8 to 128, in place and out of place).
- The stage with adapters (LoRAStage: merge, the forward on W', the data
  gradients, moe_lora_grads): routing bit-exact; y, dx, d_topk_w, d_logits
  and the six adapter gradients within the bf16 tolerance of the float64
  oracle. Small shapes cover padded ranks (8, 16 -> 32) and unpadded ones,
  experts with no rows (zero gradients), many experts, a split-K reduction
  and the ranks 72 and 96; the full 30B-A3B training shape is checked on
  every element (per token, per expert). Each also without x_perm and
  do_perm (LoRAStage(gathered=True): moe_gemm_down_dgrad_dy and
  moe_lora_grads_gathered), and without merged weights
  (LoRAStage(unmerged=True): every GEMM over its reduction extended by the
  rank, moe_lora_grads_unmerged), and with neither (the gathered calls with
  the extended reductions), against the same oracle.
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
                                     (1, 1, 8, 64), (3, 300, 200, 96), (2, 129, 136, 72)])
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


MODES = ["x_perm", "gathered", "unmerged", "gathered_unmerged"]


def lora_run(d: U.DevInputs, r: int, s: float, adapters, mode: str = "x_perm"):
    """mode: "x_perm" (merged weights), "gathered" (merged, no x_perm and
    do_perm), "unmerged" (no merged weights) or "gathered_unmerged" (neither)."""
    from mixture_experts_expert_amd import binding as B
    c = d.cfg
    T = d.t["x"].shape[0]
    ad = {n: U.to_dev(adapters[n]) for n in NAMES}
    st = B.LoRAStage(T, c.H, c.E, c.k, c.I, r, s, gathered="gathered" in mode,
                     unmerged="unmerged" in mode)
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
    U.check_close("d_topk_w", U.to_np(sel(b["d_topk_w"])), ref["d_topk_w"], U.BF16_TOL,
                  scale=U.g_scale(ref["d_topk_w"]))
    d_logits = O.route_bwd(logits, idx, ref["d_topk_w"].astype(np.float32))
    w = ref_r["topk_w"] if rows is None else ref_r["topk_w"][rows]
    U.check_close("d_logits", U.to_np(sel(b["d_logits"])), d_logits, U.BF16_TOL,
                  scale=U.d_logits_scale(w, ref["d_topk_w"]), mask=U.topk_mask(idx, d_logits.shape[1]))


SMALL_LORA = [
    (synth.MoEConfig("bf16_tiles", T=700, H=512, E=6, k=2, I=320, dtype="bf16", backward=True), 16),
    (synth.MoEConfig("bf16_tiles", T=700, H=512, E=6, k=2, I=320, dtype="bf16", backward=True), 64),
    (synth.MoEConfig("bf16_many_experts", T=333, H=256, E=40, k=5, I=128, dtype="bf16", backward=True), 32),
    (synth.MoEConfig("bf16_one_token", T=1, H=64, E=16, k=8, I=64, dtype="bf16", backward=True), 8),
    (synth.MoEConfig("bf16_skew", T=900, H=256, E=32, k=4, I=128, dtype="bf16", backward=True, zipf_s=2.5), 128),
    (SPLIT_K, 64),
    # Ranks that are not a multiple of the 32-wide blocks of the adapter
    # kernels: the odd block count of the outer products (r = 72 -> 3 blocks
    # of 32 on the rank side, an unpadded LDS row) and the padded rank
    # (r < 128 = the padded width) whose padding must be skipped.
    (synth.MoEConfig("bf16_many_experts", T=333, H=256, E=40, k=5, I=128, dtype="bf16", backward=True), 72),
    (synth.MoEConfig("bf16_tiles", T=700, H=512, E=6, k=2, I=320, dtype="bf16", backward=True), 96),
]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("cfg,r", SMALL_LORA, ids=[f"{c.name}-r{r}" for c, r in SMALL_LORA])
def test_lora_stage_small(cfg, r, mode):
    """gathered: neither x_perm nor do_perm (x and dy read through the sorted
    rows' tokens in the GEMMs and the adapter gradients); unmerged: no W'."""
    U.say(f"[lora stage] {cfg} r={r} {mode}")
    U.begin(f"lora_r{r}{'' if mode == 'x_perm' else '_' + mode}.{cfg.name}", f"{cfg} seed 8, adapters rank {r}")
    s = 2.0 if r == 64 else 0.75
    inp = synth.make_inputs(cfg, seed=8, with_dy=True)
    adapters = synth.make_adapters(cfg, r, seed=8)
    d = U.DevInputs(inp)
    st = lora_run(d, r, s, adapters, mode)
    ref_r = U.oracle_route(inp)
    U.check_routing(st, ref_r)
    ref = oracle_lora(inp, adapters, s, ref_r["topk_idx"], ref_r["topk_w"])
    check_tokens(st, ref_r, ref)
    counts = ref_r["counts"]
    for n in NAMES:
        got = U.to_np(st.buf["d" + n])
        U.check_close("d" + n, got, ref["d" + n], U.BF16_TOL)
        assert not np.any(got[counts == 0]), ("experts without rows", n)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("mode", MODES)
def test_lora_stage_qwen3_30b_a3b_full(mode):
    """T=8192, H=2048, E=128, k=8, I=768, r=64, s=2: every element of y, dx,
    d_topk_w, d_logits and of all six adapter gradients."""
    cfg = synth.CONFIGS["qwen3_30b_a3b_train"]
    r, s = 64, 2.0
    U.say(f"[lora stage] {cfg} r={r} {mode}")
    U.begin(f"lora_r64{'' if mode == 'x_perm' else '_' + mode}." + cfg.name, f"{cfg} seed 0, adapters rank {r}, scale {s}")
    inp = synth.make_inputs(cfg, seed=0)
    adapters = synth.make_adapters(cfg, r, seed=0)
    d = U.DevInputs(inp)
    st = lora_run(d, r, s, adapters, mode)
    ref_r = U.oracle_route(inp)
    U.check_routing(st, ref_r)
    U.say("  adapter oracle on all tokens")
    ref = oracle_lora(inp, adapters, s, ref_r["topk_idx"], ref_r["topk_w"])
    check_tokens(st, ref_r, ref)
    counts = ref_r["counts"]
    for n in NAMES:
        got = U.to_np(st.buf["d" + n])
        U.check_close("d" + n, got, ref["d" + n], U.BF16_TOL)
        assert not np.any(got[counts == 0]), ("experts without rows", n)


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


# ---- adapters over 8-bit frozen experts (QLoRA-style) ----

def test_merge_fp8_decodes_every_code():
    """B = 0: W' = bf16(deq(wq)) must be the decoded code times the row's
    power of two, exactly (every finite E4M3 code, scales from 2^-20 to 2^10)."""
    from mixture_experts_expert_amd import binding as B
    from oracle import fp8 as F8
    U.say("[lora merge fp8] every code")
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    E, N, K, r = 2, 16, codes.size + 2, 8  # K % 8 == 0
    rng = np.random.default_rng(3)
    wq = np.stack([np.stack([np.roll(np.r_[codes, codes[:2]], n) for n in range(N)]) for _ in range(E)])
    e8 = (127 + rng.integers(-20, 11, size=(E, N))).astype(np.uint8)
    a = np.zeros((E, r, K), np.uint16)
    b = np.zeros((E, N, r), np.uint16)
    out = torch.empty(E, N, K, dtype=torch.bfloat16, device="cuda")
    B.moe_lora_merge_fp8(E, N, K, r, 1.0, torch.from_numpy(wq).cuda(), torch.from_numpy(e8).cuda(), U.to_dev(a),
                         U.to_dev(b), out)
    torch.cuda.synchronize()
    want = F8.dequantize_rows(wq.reshape(E * N, K), e8.reshape(E * N)).reshape(E, N, K)
    assert np.array_equal(U.to_np(out).astype(np.float64), want)


@pytest.mark.parametrize("E,N,K,r", [(3, 200, 264, 8), (2, 129, 136, 72), (4, 257, 520, 40), (2, 70, 2048, 128)])
def test_merge_fp8(E, N, K, r):
    """W' = bf16(deq(wq) + s B A) against the float64 oracle on its own
    quantisation of the same weights (the GPU quantiser's codes equal it)."""
    from mixture_experts_expert_amd import binding as B
    from oracle import fp8 as F8
    U.say(f"[lora merge fp8] E={E} N={N} K={K} r={r}")
    rng = np.random.default_rng(E * 131 + N + K + r)
    w = synth.bf16_round(np.float32(0.02) * rng.standard_normal((E, N, K), dtype=np.float32))
    a = synth.bf16_round(np.float32(0.02) * rng.standard_normal((E, r, K), dtype=np.float32))
    b = synth.bf16_round(np.float32(0.02) * rng.standard_normal((E, N, r), dtype=np.float32))
    s = 1.25
    wq = torch.empty(E, N, K, dtype=torch.uint8, device="cuda")
    e8 = torch.empty(E, N, dtype=torch.uint8, device="cuda")
    B.moe_quantize_fp8_rows(E * N, K, U.to_dev(w), wq, e8)
    out = torch.full((E, N, K), float("nan"), dtype=torch.bfloat16, device="cuda")
    B.moe_lora_merge_fp8(E, N, K, r, s, wq, e8, U.to_dev(a), U.to_dev(b), out)
    torch.cuda.synchronize()
    rq, re8 = F8.quantize_weights(widen(w))
    assert np.array_equal(wq.cpu().numpy(), rq) and np.array_equal(e8.cpu().numpy(), re8)
    got = U.to_np(out).astype(np.float64)
    deq = LO.dequantize_weights(rq, re8)
    ref = LO.merge_fp8(rq, re8, widen(a), widen(b), s)
    lowrank = np.abs(ref - deq)
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -22 * (np.abs(deq) + lowrank)
    assert np.all(np.abs(got - ref) <= bound), float(np.max(np.abs(got - ref) - bound))
    frac = float(np.mean(got == widen(synth.bf16_round(ref.astype(np.float32)))))
    U.say(f"  equal to the nearest bf16: {frac:.5f}")
    assert frac >= 0.999


def oracle_mxfp4_weights(w: np.ndarray):
    """[E,N,K] float64 -> the oracle's MXFP4 (codes [E,N,K/2], scales [E,N,K/32])."""
    from oracle import mxfp4 as MX
    E, N, K = w.shape
    q, e8 = MX.quantize_blocks(w.reshape(E * N, K))
    return q.reshape(E, N, K // 2), e8.reshape(E, N, K // 32)


def fp8_lora_check(cfg, r, s, seed, full=False, fmt="fp8"):
    from mixture_experts_expert_amd import binding as B
    from oracle import fp8 as F8
    inp = synth.make_inputs(cfg, seed=seed, with_dy=True)
    adapters = synth.make_adapters(cfg, r, seed=seed)
    d = U.DevInputs(inp)
    if fmt == "fp8":
        w8 = B.FP8Weights(d.t["w_gate"], d.t["w_up"], d.t["w_down"])
    else:
        w8 = B.MXFP4Weights(d.t["w_gate"], d.t["w_up"], d.t["w_down"])
    ad = {n: U.to_dev(adapters[n]) for n in NAMES}
    T = d.t["x"].shape[0]
    st = B.LoRAStage(T, cfg.H, cfg.E, cfg.k, cfg.I, r, s)
    st.forward(d.t["x"], d.t["w_router"], w8.gate, w8.up, w8.down, ad, d.bias)
    st.backward(d.t["dy"])
    torch.cuda.synchronize()
    ref_r = U.oracle_route(inp)
    U.check_routing(st, ref_r)
    if fmt == "fp8":
        wdeq = [LO.dequantize_weights(*F8.quantize_weights(inp.f32(n).astype(np.float64)))
                for n in ["w_gate", "w_up", "w_down"]]
    else:
        wdeq = []
        for n, mine in zip(["w_gate", "w_up", "w_down"], [w8.gate, w8.up, w8.down]):
            rq, re8 = oracle_mxfp4_weights(inp.f32(n).astype(np.float64))
            # the GPU quantiser's codes and scales are the oracle's, bit for bit
            assert np.array_equal(mine[0].cpu().numpy(), rq) and np.array_equal(mine[1].cpu().numpy(), re8), n
            wdeq.append(LO.dequantize_weights_mxfp4(rq, re8))
    x, dy = inp.f32("x").astype(np.float64), inp.f32("dy").astype(np.float64)
    if full:
        U.say("  adapter oracle on all tokens")
    ref = LO.forward_backward(x, dy, ref_r["topk_idx"], ref_r["topk_w"].astype(np.float64), *wdeq,
                              {n: widen(adapters[n]) for n in NAMES}, s)
    check_tokens(st, ref_r, ref)
    counts = ref_r["counts"]
    for n in NAMES:
        got = U.to_np(st.buf["d" + n])
        U.check_close("d" + n, got, ref["d" + n], U.BF16_TOL)
        assert not np.any(got[counts == 0]), ("experts without rows", n)


@pytest.mark.parametrize("cfg,r", [SMALL_LORA[1], SMALL_LORA[2], SMALL_LORA[4]],
                         ids=[f"{c.name}-r{r}" for c, r in [SMALL_LORA[1], SMALL_LORA[2], SMALL_LORA[4]]])
def test_lora_fp8_base_small(cfg, r):
    """The adapter step over E4M3 frozen experts against the float64 oracle
    on the dequantised weights: routing bit-exact, y, dx, d_topk_w, d_logits
    and the six adapter gradients within 2e-2."""
    U.say(f"[lora fp8 base] {cfg} r={r}")
    U.begin(f"lora_fp8_r{r}.{cfg.name}", f"{cfg} seed 8, adapters rank {r} over E4M3 frozen weights")
    fp8_lora_check(cfg, r, 2.0 if r == 64 else 0.75, 8)


@pytest.mark.timeout(900)
def test_lora_fp8_base_qwen3_30b_a3b_full():
    """T=8192, H=2048, E=128, k=8, I=768, r=64, s=2 over E4M3 frozen experts:
    every element."""
    cfg = synth.CONFIGS["qwen3_30b_a3b_train"]
    U.say(f"[lora fp8 base] {cfg} r=64")
    U.begin("lora_fp8_r64." + cfg.name, f"{cfg} seed 0, adapters rank 64, scale 2, over E4M3 frozen weights")
    fp8_lora_check(cfg, 64, 2.0, 0, full=True)


def test_quantize_mxfp4_bit_exact():
    """moe_quantize_mxfp4_rows against the oracle, codes and scales bit for
    bit: normal weights, and hand-made blocks (all zeros, a lone element,
    negative zeros, magnitudes from 2^-120 to 2^100, values on the E2M1 grid
    and on every rounding midpoint at several scales)."""
    from mixture_experts_expert_amd import binding as B
    from oracle import mxfp4 as MX
    U.say("[mxfp4] quantiser")
    rng = np.random.default_rng(11)
    rows, K = 64, 256
    w = np.float32(0.02) * rng.standard_normal((rows, K), dtype=np.float32)
    w[0] = 0.0
    w[1] = 0.0
    w[1, 37] = -3.0
    w[2] = -0.0
    w[3] = w[3] * np.float32(2.0 ** -120)
    w[4] = w[4] * np.float32(2.0 ** 100)
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], np.float32)
    mids = (mags[:-1] + mags[1:]) / 2
    for i, X in enumerate([-10, 0, 7]):
        pattern = np.r_[mags, -mags, mids, -mids, 6.0, -6.0]  # 32 values: each block's largest is 6 2^X
        grid = np.ldexp(np.tile(pattern, K // 32), X).astype(np.float32)
        w[5 + i] = grid
    bits = synth.bf16_round(w)
    q = torch.empty(rows, K // 2, dtype=torch.uint8, device="cuda")
    e8 = torch.empty(rows, K // 32, dtype=torch.uint8, device="cuda")
    B.moe_quantize_mxfp4_rows(rows, K, U.to_dev(bits), q, e8)
    torch.cuda.synchronize()
    rq, re8 = MX.quantize_blocks(widen(bits))
    gq, ge8 = q.cpu().numpy(), e8.cpu().numpy()
    assert np.array_equal(ge8, re8), np.argwhere(ge8 != re8)[:5]
    assert np.array_equal(gq, rq), np.argwhere(gq != rq)[:5]


def test_merge_mxfp4_decodes_every_code():
    """B = 0: W' = bf16(deq(wq)) must be the decoded E2M1 value times its
    block's power of two, exactly (all 16 codes, scales from 2^-20 to 2^10)."""
    from mixture_experts_expert_amd import binding as B
    from oracle import mxfp4 as MX
    U.say("[lora merge mxfp4] every code")
    E, N, K, r = 2, 16, 256, 8
    rng = np.random.default_rng(4)
    codes = np.stack([np.stack([np.roll(np.tile(np.arange(16), K // 16), 3 * n + 7 * e) for n in range(N)])
                      for e in range(E)]).astype(np.uint8)
    wq = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    e8 = (127 + rng.integers(-20, 11, size=(E, N, K // 32))).astype(np.uint8)
    a = np.zeros((E, r, K), np.uint16)
    b = np.zeros((E, N, r), np.uint16)
    out = torch.empty(E, N, K, dtype=torch.bfloat16, device="cuda")
    B.moe_lora_merge_mxfp4(E, N, K, r, 1.0, torch.from_numpy(wq).cuda(), torch.from_numpy(e8).cuda(), U.to_dev(a),
                           U.to_dev(b), out)
    torch.cuda.synchronize()
    want = MX.dequantize_blocks(wq.reshape(E * N, K // 2), e8.reshape(E * N, K // 32)).reshape(E, N, K)
    got = U.to_np(out).astype(np.float64)
    assert np.array_equal(got, want)


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """float64 values exact in float32 -> nearest bf16 (ties to even), as float64."""
    u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def test_merge_quantized_base_smallest_scale():
    """B = 0 with every scale byte 0 (2^-127, below the float32 normal range):
    W' = bf16(code value * 2^-127) for every E4M3 and E2M1 code, the
    subnormal results included (the decode scales by 2^-126, then halves)."""
    from mixture_experts_expert_amd import binding as B
    from oracle import fp8 as F8
    from oracle import mxfp4 as MX
    U.say("[lora merge] scale 2^-127")
    E, N, r = 2, 16, 8
    codes8 = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    K8 = codes8.size + 2
    wq8 = np.stack([np.stack([np.roll(np.r_[codes8, codes8[:2]], n) for n in range(N)]) for _ in range(E)])
    e8 = np.zeros((E, N), np.uint8)
    out = torch.empty(E, N, K8, dtype=torch.bfloat16, device="cuda")
    B.moe_lora_merge_fp8(E, N, K8, r, 1.0, torch.from_numpy(wq8).cuda(), torch.from_numpy(e8).cuda(),
                         U.to_dev(np.zeros((E, r, K8), np.uint16)), U.to_dev(np.zeros((E, N, r), np.uint16)), out)
    torch.cuda.synchronize()
    want = F8.dequantize_rows(wq8.reshape(E * N, K8), e8.reshape(E * N)).reshape(E, N, K8)
    assert np.array_equal(U.to_np(out).astype(np.float64), bf16_rne(want))
    K4 = 256
    codes4 = np.stack([np.stack([np.roll(np.tile(np.arange(16), K4 // 16), 3 * n + e) for n in range(N)])
                       for e in range(E)]).astype(np.uint8)
    wq4 = (codes4[..., 0::2] | (codes4[..., 1::2] << 4)).astype(np.uint8)
    e84 = np.zeros((E, N, K4 // 32), np.uint8)
    out4 = torch.empty(E, N, K4, dtype=torch.bfloat16, device="cuda")
    B.moe_lora_merge_mxfp4(E, N, K4, r, 1.0, torch.from_numpy(wq4).cuda(), torch.from_numpy(e84).cuda(),
                           U.to_dev(np.zeros((E, r, K4), np.uint16)), U.to_dev(np.zeros((E, N, r), np.uint16)), out4)
    torch.cuda.synchronize()
    want4 = MX.dequantize_blocks(wq4.reshape(E * N, K4 // 2), e84.reshape(E * N, K4 // 32)).reshape(E, N, K4)
    assert np.array_equal(U.to_np(out4).astype(np.float64), bf16_rne(want4))


@pytest.mark.parametrize("E,N,K,r", [(3, 200, 256, 8), (2, 129, 160, 72), (4, 257, 544, 40), (2, 70, 2048, 128)])
def test_merge_mxfp4(E, N, K, r):
    """W' = bf16(deq(wq) + s B A) against the float64 oracle on its own
    quantisation of the same weights (the GPU quantiser's codes equal it)."""
    from mixture_experts_expert_amd import binding as B
    U.say(f"[lora merge mxfp4] E={E} N={N} K={K} r={r}")
    rng = np.random.default_rng(E * 137 + N + K + r)
    w = synth.bf16_round(np.float32(0.02) * rng.standard_normal((E, N, K), dtype=np.float32))
    a = synth.bf16_round(np.float32(0.02) * rng.standard_normal((E, r, K), dtype=np.float32))
    b = synth.bf16_round(np.float32(0.02) * rng.standard_normal((E, N, r), dtype=np.float32))
    s = 1.25
    wq = torch.empty(E, N, K // 2, dtype=torch.uint8, device="cuda")
    e8 = torch.empty(E, N, K // 32, dtype=torch.uint8, device="cuda")
    B.moe_quantize_mxfp4_rows(E * N, K, U.to_dev(w), wq, e8)
    out = torch.full((E, N, K), float("nan"), dtype=torch.bfloat16, device="cuda")
    B.moe_lora_merge_mxfp4(E, N, K, r, s, wq, e8, U.to_dev(a), U.to_dev(b), out)
    torch.cuda.synchronize()
    rq, re8 = oracle_mxfp4_weights(widen(w))
    assert np.array_equal(wq.cpu().numpy(), rq) and np.array_equal(e8.cpu().numpy(), re8)
    got = U.to_np(out).astype(np.float64)
    deq = LO.dequantize_weights_mxfp4(rq, re8)
    ref = LO.merge_mxfp4(rq, re8, widen(a), widen(b), s)
    lowrank = np.abs(ref - deq)
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -22 * (np.abs(deq) + lowrank)
    assert np.all(np.abs(got - ref) <= bound), float(np.max(np.abs(got - ref) - bound))
    frac = float(np.mean(got == widen(synth.bf16_round(ref.astype(np.float32)))))
    U.say(f"  equal to the nearest bf16: {frac:.5f}")
    assert frac >= 0.999


@pytest.mark.parametrize("cfg,r", [SMALL_LORA[1], SMALL_LORA[2], SMALL_LORA[4]],
                         ids=[f"{c.name}-r{r}" for c, r in [SMALL_LORA[1], SMALL_LORA[2], SMALL_LORA[4]]])
def test_lora_mxfp4_base_small(cfg, r):
    """The adapter step over MXFP4 frozen experts against the float64 oracle
    on the dequantised weights: routing bit-exact, y, dx, d_topk_w, d_logits
    and the six adapter gradients within 2e-2."""
    U.say(f"[lora mxfp4 base] {cfg} r={r}")
    U.begin(f"lora_mxfp4_r{r}.{cfg.name}", f"{cfg} seed 8, adapters rank {r} over MXFP4 frozen weights")
    fp8_lora_check(cfg, r, 2.0 if r == 64 else 0.75, 8, fmt="mxfp4")


@pytest.mark.timeout(900)
def test_lora_mxfp4_base_qwen3_30b_a3b_full():
    """T=8192, H=2048, E=128, k=8, I=768, r=64, s=2 over MXFP4 frozen experts:
    every element."""
    cfg = synth.CONFIGS["qwen3_30b_a3b_train"]
    U.say(f"[lora mxfp4 base] {cfg} r=64")
    U.begin("lora_mxfp4_r64." + cfg.name, f"{cfg} seed 0, adapters rank 64, scale 2, over MXFP4 frozen weights")
    fp8_lora_check(cfg, 64, 2.0, 0, full=True, fmt="mxfp4")
