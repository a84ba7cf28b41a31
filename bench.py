"""Throughput of one MoE layer's expert stage (forward + backward) on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--seeds 0,1,2]
                    [--no-cpu-baseline] [--timed-only]

One step is the whole stage on one batch of synthetic input already resident
in HBM, on one stream, every step a call of the C ABI, as the library chains
it (MoEStage with gather_fused and dy_fused; moe_grouped_gemm_fwd and
moe_grouped_gemm_bwd): route -> expert indexing (the sort also writes each
sorted row's token and routing weight) -> gate/up GEMM reading x through the
tokens (SwiGLU epilogue; it also writes the weighted activations a_w) -> down
GEMM -> combine, then combine backward (d_topk_w) -> down backward (data
gradient reading dy through the tokens, with the routing weight and the
SwiGLU backward in its epilogue, then the weight gradient, in one persistent
launch) -> gate/up backward (likewise, x read through the tokens) ->
unpermute-sum -> router backward. Neither x_perm nor do_perm is written.
--chain xperm times the chain that materialises both (the gather writes
x_perm, the combine backward writes do_perm, and the GEMMs read them). The
line also reports the other chain's time.

Each input seed (default 0, 1 and 2) gets W untimed warmup steps and K timed
steps; the line reports the seed with the median time (`ms_per_step_by_seed`
lists all three). Prints one JSON line. `value` is tokens/s of the whole stage; TFLOP/s counts
the expert GEMMs (18*T*k*H*I per step). Around every GEMM call the timed
steps also record HIP events on the stream, which give `call_ms`,
`gemm_tflops` and `roofline`; the calls without matrix work are timed each
on its own afterwards (`other_call_ms`, `hbm_frac`). `roofline` covers the
dominant kernel (the GEMM call with the largest average time): its
algorithmic flops or bytes per launch (whichever of the MFMA and HBM minimum
times is larger decides the bound) over its average launch time. `traffic` is the HBM bytes per launch that
rocprofv3's FETCH_SIZE and WRITE_SIZE counters gave for that kernel, scaled by
what they read for a plain device copy of known size (--calibrate-copy); it is
taken from the committed summary under profiles/ and reported only while the
GEMM source still hashes to the value recorded there, as are
`mfma_busy_counter` (SQ_VALU_MFMA_BUSY_CYCLES over the SIMD-cycles of the
dispatch, GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs) and `clock_ghz_counter`
(the shader clock the kernel ran at). `cpu_baseline` times
the CPU oracle on every token of the same workload (first seed), on every
host thread this job may use (the CPUs it may run on, capped by
OMP_NUM_THREADS), with the host's CPU count and model. --library-gemms prints,
for context only, the vendor library's dense bf16 GEMMs (through torch) with
the flops of the stage's grouped GEMMs at the workload's shape.

After the timed steps (and outside them): `ms_per_step_without_call_events`
times the same step without the per-call events; `graph_ms_per_step` the same
step captured once into a HIP graph and replayed; `two_stream_ms_per_step`
the step with one launch per GEMM and the weight-gradient GEMMs on a second
stream, concurrently with the data-gradient GEMMs (x_perm chain);
`xperm_chain_ms_per_step` (or `fused_chain_ms_per_step`) the chain not timed
above; `gather_fused_ms` the x_perm chain without x_perm only (gate/up and
the gate/up backward read x through the sorted rows' tokens),
`dy_fused_ms` the x_perm chain without do_perm only, and
`gather_dy_fused_ms` without both, each with its changed
calls on their own; `single_launch_ms` the step with
one launch per GEMM (the six single-GEMM entry points) and the four backward
GEMMs on their own (whose TFLOP/s join `gemm_tflops`); `inference_forward_ms`
the forward alone, unfused and fused (no x_perm, routing weights in the down
GEMM's epilogue); `lora_ms` the training step with rank-64 adapters on frozen
experts (merges, forward on the merged weights, data and adapter gradients)
and its two adapter calls, over bf16, E4M3 and MXFP4 frozen weights, the
step without x_perm and do_perm (`step_gathered`, with
`moe_lora_grads_gathered`) and the step without merged weights
(`step_unmerged`, its calls in `unmerged_call_ms`), and the step without
either (`step_gathered_unmerged`). `--timed-only` skips these and the CPU baseline, so that
under a profiler the last K launches of every kernel are the timed steps.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE expert-stage tokens/s and TFLOP/s (fwd+bwd), Qwen3-30B-A3B shape, 1 GPU"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4096 flop/clk x 2.4 GHz, dense
PEAK_HBM_GBS = 8000.0


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


GEMM_SOURCE = os.path.join(ROOT, "mixture_experts_expert_amd", "csrc", "gemm_bf16.hip")
PROFILES = os.path.join(ROOT, "profiles")


def alg_bytes(c) -> dict:
    """Algorithmic HBM bytes of every call per launch: each tensor read or
    written once (weights once per kernel), indices included."""
    T, H, E, k, I = c.T, c.H, c.E, c.k, c.I
    M = T * k
    b16, f32, i32 = 2, 4, 4
    return {
        "moe_route": T * H * b16 + E * H * b16 + T * E * f32 + 2 * M * i32,
        "moe_permute": M * i32 + T * H * b16 + 2 * M * i32 + M * H * b16,
        "moe_gemm_gate_up": M * H * b16 + 2 * E * I * H * b16 + 3 * M * I * b16,
        "moe_gemm_down": M * I * b16 + E * H * I * b16 + M * H * b16,
        "moe_combine": M * H * b16 + 2 * M * i32 + T * H * b16,
        "moe_combine_bwd": T * H * b16 + M * H * b16 + 2 * M * i32 + M * H * b16 + M * f32,
        "moe_gemm_down_dgrad": M * H * b16 + E * H * I * b16 + 2 * M * I * b16 + 2 * M * I * b16,
        "moe_gemm_down_wgrad": M * H * b16 + M * I * b16 + E * H * I * f32,
        "moe_gemm_gate_up_dgrad": 2 * M * I * b16 + 2 * E * I * H * b16 + M * H * b16,
        "moe_gemm_gate_up_wgrad": 2 * M * I * b16 + M * H * b16 + 2 * E * I * H * f32,
        "moe_unpermute_sum": M * H * b16 + M * i32 + T * H * b16,
        "moe_route_bwd": 3 * M * i32 + T * E * f32,
        # The paired backward launches: both GEMMs' tensors, the shared input once.
        "moe_gemm_down_bwd": (M * H * b16 + E * H * I * b16 + 2 * M * I * b16 + 2 * M * I * b16
                              + M * I * b16 + E * H * I * f32),
        "moe_gemm_gate_up_bwd": (2 * M * I * b16 + 2 * E * I * H * b16 + M * H * b16
                                 + M * H * b16 + 2 * E * I * H * f32),
    }


def alg_bytes_fused(c) -> dict:
    """alg_bytes of the calls that differ in the chain without x_perm and
    do_perm: x and dy are read through the sorted rows' tokens (each tensor
    once: T rows), the sort writes row_token and row_weight, gate/up also
    writes a_w, the combine backward writes d_topk_w only."""
    T, H, E, k, I = c.T, c.H, c.E, c.k, c.I
    M = T * k
    b16, f32, i32 = 2, 4, 4
    out = dict(alg_bytes(c))
    out.update({
        "moe_permute": M * i32 + M * f32 + 3 * M * i32 + M * f32,
        "moe_gemm_gate_up": T * H * b16 + 2 * M * i32 + 2 * E * I * H * b16 + 4 * M * I * b16,
        "moe_combine_bwd": T * H * b16 + M * H * b16 + 2 * M * i32 + M * f32,
        "moe_gemm_down_bwd": (T * H * b16 + M * i32 + M * f32 + E * H * I * b16 + 2 * M * I * b16
                              + 2 * M * I * b16 + M * I * b16 + E * H * I * f32),
        "moe_gemm_gate_up_bwd": (2 * M * I * b16 + 2 * E * I * H * b16 + T * H * b16 + M * i32
                                 + M * H * b16 + 2 * E * I * H * f32),
    })
    return out


def source_hash() -> str:
    with open(GEMM_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def profiled_counters(kernel: str, workload: str, chain: str) -> dict:
    """The committed counter summary of a GEMM call (HBM bytes per launch,
    MFMA busy fraction, clock): profiles/<kernel>.<workload>.traffic.txt for
    the x_perm chain, profiles/<kernel>.gathered.<workload>.traffic.txt for
    the chain without x_perm and do_perm; {} when there is none, it was taken
    on the other chain or the GEMM source changed since."""
    name = f"{kernel}.{workload}" if chain == "xperm" else f"{kernel}.gathered.{workload}"
    path = os.path.join(PROFILES, f"{name}.traffic.txt")
    if not os.path.exists(path):
        return {}
    rec = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                rec[key.strip()] = val.strip()
    if rec.get("gemm_source_sha256_16") != source_hash() or rec.get("chain", "xperm") != chain:
        return {}
    out = {}
    for key, conv in [("hbm_bytes_per_launch", int), ("mfma_busy_frac", float), ("clock_ghz", float)]:
        try:
            out[key] = conv(rec[key])
        except (KeyError, ValueError):
            pass
    return out


def calibrate_copy(nbytes: int, reps: int) -> int:
    """A plain device-to-device copy of known size, for scaling the PMC byte
    counters (run under rocprofv3 --pmc)."""
    import torch

    torch.cuda.set_device(0)
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": nbytes, "reps": reps}), flush=True)
    return 0


def gemm_flops(c) -> dict:
    """Algorithmic flops of each grouped GEMM per launch (M = T*k rows)."""
    m, h, i = c.T * c.k, c.H, c.I
    return {
        "moe_gemm_gate_up": 4.0 * m * h * i,
        "moe_gemm_down": 2.0 * m * h * i,
        "moe_gemm_down_dgrad": 2.0 * m * h * i,
        "moe_gemm_down_wgrad": 2.0 * m * h * i,
        "moe_gemm_gate_up_dgrad": 4.0 * m * h * i,
        "moe_gemm_gate_up_wgrad": 4.0 * m * h * i,
        "moe_gemm_down_bwd": 4.0 * m * h * i,
        "moe_gemm_gate_up_bwd": 8.0 * m * h * i,
    }


def host_threads() -> dict:
    """The host's CPU count, the CPUs this process may run on, and the share
    the oracle uses: all of those, capped by OMP_NUM_THREADS when it is set
    (a machine that shares its host between jobs sets it to the job's share)."""
    nproc = os.cpu_count() or 1
    try:
        allowed = len(os.sched_getaffinity(0))
    except AttributeError:
        allowed = nproc
    share = allowed
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        share = min(share, int(cap))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": nproc, "affinity": allowed, "threads": share, "cpu_model": model}


def cpu_baseline(cfg, seed: int, tokens: int) -> dict:
    """The oracle, as it stands, on the first `tokens` tokens of the workload
    (all of them by default), on every host thread this job may use."""
    import numpy as np  # noqa: F401

    from mixture_experts_expert_amd import synth
    from oracle import oracle as O

    host = host_threads()
    O.set_threads(host["threads"])
    inp = synth.make_inputs(cfg, seed, T=tokens)
    f = {n: inp.f32(n) for n in inp.names()}
    t0 = time.perf_counter()
    fwd = O.forward(f["x"], f["w_router"], f["w_gate"], f["w_up"], f["w_down"], cfg.k, logit_bias=inp.logit_bias)
    O.backward(fwd, f["dy"], f["w_gate"], f["w_up"], f["w_down"])
    dt = time.perf_counter() - t0
    what = "all" if tokens == cfg.T else f"{tokens} of {cfg.T}"
    return {"value": tokens / dt, "unit": "tokens/s", "cores": host["threads"], "kind": "oracle",
            "sample": f"{what} tokens of the workload (seed {seed}), fwd+bwd, {dt:.1f} s",
            "host": host}


def time_calls(fn, stream, reps=10) -> float:
    """Average ms of fn() over reps calls between two HIP events on stream (two untimed calls first)."""
    import torch
    for _ in range(2):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def lora_timing(cfg, seed: int, tensors, bias, stream, r: int = 64, scale: float = 2.0) -> dict:
    """The training step with rank-r adapters on the frozen experts at the
    same shape: the three merges W' = W + s B A, the forward on W', the data
    gradients and the adapter gradients (no frozen-weight gradient); then
    the merges and the adapter-gradient call on their own; the same over 8-
    and 4-bit frozen weights, without x_perm and do_perm, without merged
    weights (step_unmerged, with its calls on their own), and without both."""
    import numpy as np
    import torch

    from mixture_experts_expert_amd import binding as B
    from mixture_experts_expert_amd import synth
    x, wr, wg, wu, wd, dy = tensors
    ad = {n: torch.from_numpy(v.view(np.int16)).to("cuda").view(torch.bfloat16)
          for n, v in synth.make_adapters(cfg, r, seed).items()}
    ls = B.LoRAStage(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, r, scale)
    lb = ls.buf

    def lora_step():
        ls.forward(x, wr, wg, wu, wd, ad, bias)
        ls.backward(dy)

    out = {"rank": r, "scale": scale, "step": round(time_calls(lora_step, stream), 4)}
    aux = torch.cuda.Stream()

    def lora_step_two_streams():
        ls.forward(x, wr, wg, wu, wd, ad, bias, aux_stream=aux)
        ls.backward(dy)

    # The merges on a second stream, concurrent with the routing and the sort.
    out["step_merges_on_second_stream"] = round(time_calls(lora_step_two_streams, stream), 4)
    out["moe_lora_merge_x3"] = round(time_calls(lambda: ls.merge(wg, wu, wd, ad), stream, reps=5), 4)
    # The same step over E4M3 frozen experts (QLoRA-style; quantised once,
    # outside the timing): the merges dequantise.
    w8 = B.FP8Weights(wg, wu, wd)

    def lora_step_fp8():
        ls.forward(x, wr, w8.gate, w8.up, w8.down, ad, bias)
        ls.backward(dy)

    out["step_fp8_base"] = round(time_calls(lora_step_fp8, stream), 4)
    out["moe_lora_merge_fp8_x3"] = round(time_calls(lambda: ls.merge(w8.gate, w8.up, w8.down, ad), stream, reps=5), 4)
    del w8
    # And over MXFP4 frozen experts (E2M1, a scale per 32 elements).
    w4 = B.MXFP4Weights(wg, wu, wd)

    def lora_step_mxfp4():
        ls.forward(x, wr, w4.gate, w4.up, w4.down, ad, bias)
        ls.backward(dy)

    out["step_mxfp4_base"] = round(time_calls(lora_step_mxfp4, stream), 4)
    out["moe_lora_merge_mxfp4_x3"] = round(time_calls(lambda: ls.merge(w4.gate, w4.up, w4.down, ad), stream,
                                                      reps=5), 4)
    del w4
    out["moe_lora_grads"] = round(time_calls(lambda: B.moe_lora_grads(
        ls.s, r, scale, lb["x_perm"], lb["a"], lb["dgu"], lb["do_perm"], lb["offsets"],
        *(ad[n] for n in B.LORA_NAMES), *(lb["d" + n] for n in B.LORA_NAMES), ls.lora_ws), stream, reps=5), 4)
    del ls, lb
    torch.cuda.empty_cache()
    # The step without x_perm and do_perm: x and dy read through the sorted
    # rows' tokens in the GEMMs and in the adapter gradients.
    gs = B.LoRAStage(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, r, scale, gathered=True)
    gb = gs.buf

    def lora_step_gathered():
        gs.forward(x, wr, wg, wu, wd, ad, bias)
        gs.backward(dy)

    out["step_gathered"] = round(time_calls(lora_step_gathered, stream), 4)
    out["moe_lora_grads_gathered"] = round(time_calls(lambda: B.moe_lora_grads_gathered(
        gs.s, r, scale, x, gb["row_token"], gb["row_weight"], gb["a"], gb["dgu"], dy, gb["offsets"],
        *(ad[n] for n in B.LORA_NAMES), *(gb["d" + n] for n in B.LORA_NAMES), gs.lora_ws), stream, reps=5), 4)
    del gs, gb
    torch.cuda.empty_cache()
    # The step without merged weights: every GEMM over its reduction extended
    # by the rank; its calls on their own.
    us = B.LoRAStage(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, r, scale, unmerged=True)
    ub, uw = us.buf, us.lora_ws

    def lora_step_unmerged():
        us.forward(x, wr, wg, wu, wd, ad, bias)
        us.backward(dy)

    out["step_unmerged"] = round(time_calls(lora_step_unmerged, stream), 4)
    un_calls = {
        "moe_lora_prepare": lambda: B.moe_lora_prepare(us.s, r, scale, *(ad[n] for n in B.LORA_NAMES), uw),
        "moe_lora_gemm_gate_up": lambda: B.moe_lora_gemm_gate_up(us.s, r, ub["x_perm"], ub["offsets"], wg, wu,
                                                                 ad["b_gate"], ad["b_up"], ub["g"], ub["u"], ub["a"], uw),
        "moe_lora_gemm_down": lambda: B.moe_lora_gemm_down(us.s, r, ub["a"], ub["offsets"], wd, ad["b_down"],
                                                           ub["o_perm"], uw),
        "moe_lora_gemm_down_dgrad": lambda: B.moe_lora_gemm_down_dgrad(us.s, r, ub["do_perm"], ub["offsets"], wd,
                                                                       ad["a_down"], ub["g"], ub["u"], ub["dgu"], uw),
        "moe_lora_gemm_gate_up_dgrad": lambda: B.moe_lora_gemm_gate_up_dgrad(us.s, r, ub["dgu"], ub["offsets"], wg, wu,
                                                                             ad["a_gate"], ad["a_up"], ub["dx_perm"],
                                                                             uw),
        "moe_lora_grads_unmerged": lambda: B.moe_lora_grads_unmerged(
            us.s, r, ub["x_perm"], ub["a"], ub["dgu"], ub["do_perm"], ub["offsets"],
            *(ub["d" + n] for n in B.LORA_NAMES), uw),
    }
    out["unmerged_call_ms"] = {n: round(time_calls(f, stream, reps=5), 4) for n, f in un_calls.items()}
    del us, ub, uw
    torch.cuda.empty_cache()
    # Neither merged weights nor x_perm and do_perm.
    gu = B.LoRAStage(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, r, scale, gathered=True, unmerged=True)

    def lora_step_gathered_unmerged():
        gu.forward(x, wr, wg, wu, wd, ad, bias)
        gu.backward(dy)

    out["step_gathered_unmerged"] = round(time_calls(lora_step_gathered_unmerged, stream), 4)
    log(f"adapter step: {out}")
    del gu, ad
    torch.cuda.empty_cache()
    return out


def library_gemms(cfg, reps: int = 20) -> dict:
    """Context only, not the product path: dense bf16 GEMMs of the vendor
    library (torch.matmul / torch.bmm -> hipBLASLt) with the flops of the
    stage's grouped GEMMs at this shape: each projection as one GEMM over all
    T*k sorted rows (one weight, bf16 output), and gate/up as a batched GEMM
    over E equal groups of rows (its right operand made contiguous first)."""
    import torch
    M, H, I, E = cfg.M, cfg.H, cfg.I, cfg.E
    g = torch.Generator(device="cuda").manual_seed(0)

    def rnd(*shape):
        return torch.randn(*shape, device="cuda", dtype=torch.bfloat16, generator=g)

    x, a, dgu = rnd(M, H), rnd(M, I), rnd(M, 2 * I)
    wgu, wd = rnd(2 * I, H), rnd(H, I)
    runs = {
        "gate_up_fwd": (lambda: x @ wgu.t(), 4 * M * H * I),
        "down_fwd": (lambda: a @ wd.t(), 2 * M * H * I),
        "gate_up_dgrad": (lambda: dgu @ wgu, 4 * M * H * I),
        "gate_up_wgrad": (lambda: dgu.t() @ x, 4 * M * H * I),
    }
    if M % E == 0:
        xe = x.view(E, M // E, H)
        wge = rnd(E, H, 2 * I)  # [E, H, 2I]: contiguous
        runs["gate_up_fwd_batched"] = (lambda: torch.bmm(xe, wge), 4 * M * H * I)
    out = {}
    for name, (f, flops) in runs.items():
        for _ in range(3):
            f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            f()
        e1.record()
        e1.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name] = {"ms": round(ms, 4), "tflops": round(flops / ms / 1e9, 1)}
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3_30b_a3b_train")
    ap.add_argument("--seeds", default="0,1,2",
                    help="input seeds; each runs W warmup and K timed steps, the line reports the median")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=0, help="oracle sample (default: every token of the workload)")
    ap.add_argument("--chain", choices=["xperm", "fused"], default="fused",
                    help="the timed chain: without x_perm and do_perm (default), or materialising both")
    ap.add_argument("--timed-only", action="store_true",
                    help="launch nothing after the timed steps (for profiling): no sequential, inference or CPU pass")
    ap.add_argument("--lora-only", action="store_true",
                    help="only time the adapter (LoRA) step and its calls; prints {\"lora_ms\": ...}")
    ap.add_argument("--library-gemms", action="store_true",
                    help="only time dense vendor-library GEMMs of the same flops (context); prints {\"library_gemm_ms\": ...}")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes (PMC counter calibration)")
    args = ap.parse_args()
    if args.calibrate_copy:
        return calibrate_copy(args.calibrate_copy, 3)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from mixture_experts_expert_amd import binding as B
    from mixture_experts_expert_amd import synth

    cfg = synth.CONFIGS[args.workload]
    assert cfg.backward and cfg.dtype == "bf16", "the benchmark runs bf16 training-step workloads"
    seeds = [int(v) for v in args.seeds.split(",")]
    torch.cuda.set_device(0)
    log(f"workload {cfg}, seeds {seeds}")

    # The step's input tensors; the call lambdas below read them from here,
    # so that switching seeds swaps the tensors they see.
    cur = {}

    def load(seed):
        t0 = time.perf_counter()
        cur.clear()
        torch.cuda.empty_cache()
        inp = synth.make_inputs(cfg, seed)
        for n in inp.names():
            cur[n] = torch.from_numpy(inp.bits[n].view(np.int16)).to("cuda").view(torch.bfloat16)
        cur["bias"] = None if inp.logit_bias is None else torch.from_numpy(inp.logit_bias).to("cuda")
        torch.cuda.synchronize()
        log(f"seed {seed}: inputs ready in {time.perf_counter() - t0:.1f} s")

    if args.library_gemms:
        print(json.dumps({"library_gemm_ms": library_gemms(cfg), "config": {"workload": cfg.name}}), flush=True)
        return 0
    if args.lora_only:
        load(seeds[0])
        tensors = tuple(cur[n] for n in ["x", "w_router", "w_gate", "w_up", "w_down", "dy"])
        print(json.dumps({"lora_ms": lora_timing(cfg, seeds[0], tensors, cur["bias"], torch.cuda.current_stream()),
                          "config": {"workload": cfg.name}}), flush=True)
        return 0

    st = B.MoEStage(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, torch.bfloat16)
    st._alloc_bwd()
    b, s = st.buf, st.s
    dgu = torch.empty(cfg.M, 2 * cfg.I, dtype=torch.bfloat16, device="cuda")  # [dG | dU]
    stream = torch.cuda.current_stream()
    # The calls below read these names when they run (closures bind late), so
    # loading another seed's inputs and rebinding them switches every call.
    x = wr = wg = wu = wd = dy = bias = None
    # The 12 C-ABI calls with one launch per GEMM; the timed step runs the
    # library's own chain (what MoEStage and moe_grouped_gemm_bwd do): the
    # backward's GEMMs as the two paired launches.
    single_names = ["moe_route", "moe_permute", "moe_gemm_gate_up", "moe_gemm_down", "moe_combine",
                    "moe_combine_bwd", "moe_gemm_down_dgrad", "moe_gemm_down_wgrad", "moe_gemm_gate_up_dgrad",
                    "moe_gemm_gate_up_wgrad", "moe_unpermute_sum", "moe_route_bwd"]
    names = ["moe_route", "moe_permute", "moe_gemm_gate_up", "moe_gemm_down", "moe_combine", "moe_combine_bwd",
             "moe_gemm_down_bwd", "moe_gemm_gate_up_bwd", "moe_unpermute_sum", "moe_route_bwd"]
    calls = [
        lambda: B.moe_route(s, x, wr, bias, b["logits"], b["topk_idx"], b["topk_w"]),
        lambda: B.moe_permute(s, b["topk_idx"], x, b["counts"], b["offsets"], b["sorted_to_flat"],
                              b["flat_to_sorted"], b["x_perm"], st.ws),
        lambda: B.moe_gemm_gate_up(s, b["x_perm"], b["offsets"], wg, wu, b["g"], b["u"], b["a"]),
        lambda: B.moe_gemm_down(s, b["a"], b["offsets"], wd, b["o_perm"]),
        lambda: B.moe_combine(s, b["o_perm"], b["topk_w"], b["flat_to_sorted"], b["y"]),
        lambda: B.moe_combine_bwd(s, dy, b["o_perm"], b["topk_w"], b["flat_to_sorted"], b["do_perm"],
                                  b["d_topk_w"]),
        lambda: B.moe_gemm_down_dgrad(s, b["do_perm"], b["offsets"], wd, b["g"], b["u"], dgu),
        lambda: B.moe_gemm_down_wgrad(s, b["do_perm"], b["a"], b["offsets"], b["dw_down"], 0, st.ws),
        lambda: B.moe_gemm_gate_up_dgrad(s, dgu, b["offsets"], wg, wu, b["dx_perm"]),
        lambda: B.moe_gemm_gate_up_wgrad(s, dgu, b["x_perm"], b["offsets"], b["dw_gate"], b["dw_up"], 0, st.ws),
        lambda: B.moe_unpermute_sum(s, b["dx_perm"], b["flat_to_sorted"], b["dx"]),
        lambda: B.moe_route_bwd(s, b["d_topk_w"], b["topk_w"], b["topk_idx"], b["d_logits"]),
    ]
    by_name = dict(zip(single_names, calls))
    by_name["moe_gemm_down_bwd"] = lambda: B.moe_gemm_down_bwd(s, b["do_perm"], b["a"], b["offsets"], wd, b["g"],
                                                               b["u"], dgu, b["dw_down"], 0, st.ws)
    by_name["moe_gemm_gate_up_bwd"] = lambda: B.moe_gemm_gate_up_bwd(s, dgu, b["x_perm"], None, b["offsets"], wg,
                                                                     wu, b["dx_perm"], b["dw_gate"], b["dw_up"], 0,
                                                                     st.ws)
    # The same step without x_perm: the sort also writes each sorted row's
    # token, and gate/up and the gate/up backward pair (its weight gradient)
    # read x rows through it.
    rt = dict(row_token=torch.empty(cfg.M, dtype=torch.int32, device="cuda"),
              row_weight=torch.empty(cfg.M, device="cuda"))
    gf_calls = dict(by_name)
    gf_calls["moe_permute"] = lambda: B.moe_permute_fused(
        s, b["topk_idx"], b["topk_w"], b["counts"], b["offsets"], b["sorted_to_flat"], b["flat_to_sorted"],
        rt["row_token"], rt["row_weight"], st.ws)
    gf_calls["moe_gemm_gate_up"] = lambda: B.moe_gemm_gate_up_gathered(
        s, x, rt["row_token"], b["offsets"], wg, wu, b["g"], b["u"], b["a"])
    gf_calls["moe_gemm_gate_up_bwd"] = lambda: B.moe_gemm_gate_up_bwd(
        s, dgu, x, rt["row_token"], b["offsets"], wg, wu, b["dx_perm"], b["dw_gate"], b["dw_up"], 0, st.ws)

    # The same step without do_perm: the gate/up GEMM also writes the weighted
    # activations, the combine backward writes d_topk_w only, and the down
    # backward reads dy through the sorted rows' tokens.
    a_w = torch.empty(cfg.M, cfg.I, dtype=torch.bfloat16, device="cuda")
    dy_calls = dict(by_name)
    dy_calls["moe_permute"] = lambda: B.moe_permute_rows(
        s, b["topk_idx"], b["topk_w"], x, b["counts"], b["offsets"], b["sorted_to_flat"], b["flat_to_sorted"],
        rt["row_token"], rt["row_weight"], b["x_perm"], st.ws)
    dy_calls["moe_gemm_gate_up"] = lambda: B.moe_gemm_gate_up_aw(
        s, b["x_perm"], None, rt["row_weight"], b["offsets"], wg, wu, b["g"], b["u"], b["a"], a_w)
    dy_calls["moe_combine_bwd"] = lambda: B.moe_combine_bwd(s, dy, b["o_perm"], b["topk_w"], b["flat_to_sorted"],
                                                            None, b["d_topk_w"])
    dy_calls["moe_gemm_down_bwd"] = lambda: B.moe_gemm_down_bwd_dy(
        s, dy, rt["row_token"], rt["row_weight"], a_w, b["offsets"], wd, b["g"], b["u"], dgu, b["dw_down"], 0, st.ws)

    # The step with neither x_perm nor do_perm: the sort writes each sorted
    # row's token and weight, gate/up reads x through the token and also
    # writes the weighted activations, the down backward reads dy through the
    # token, the gate/up backward reads x through it.
    both_calls = dict(dy_calls)
    both_calls["moe_permute"] = gf_calls["moe_permute"]
    both_calls["moe_gemm_gate_up"] = lambda: B.moe_gemm_gate_up_aw(
        s, x, rt["row_token"], rt["row_weight"], b["offsets"], wg, wu, b["g"], b["u"], b["a"], a_w)
    both_calls["moe_gemm_gate_up_bwd"] = gf_calls["moe_gemm_gate_up_bwd"]

    # The timed chain: by default the one without x_perm and do_perm
    # (both_calls); --chain xperm times the one that materialises both
    # (by_name).
    chain = both_calls if args.chain == "fused" else by_name

    # HIP events in the timed steps bracket the GEMM calls only (an event
    # between two calls costs about 5 us; bracketing all ten calls added
    # 0.1 ms to a 3 ms step): one event before the first GEMM of each run of
    # consecutive GEMM calls and one after every GEMM call. The other calls
    # are timed on their own after the timed steps.
    gemm_names = [n for n in names if n.startswith("moe_gemm")]
    # The event each GEMM call's time starts at: the previous call's end when
    # that was a GEMM, else an event of its own recorded just before it.
    start_of = {}
    for i, n in enumerate(names):
        if n in gemm_names:
            start_of[n] = names[i - 1] if i > 0 and names[i - 1] in gemm_names else "start_" + n
    ev = [{e: torch.cuda.Event(enable_timing=True) for e in gemm_names + list(start_of.values())}
          for _ in range(args.steps)]

    def step(events=None):
        for n in names:
            timed = events is not None and n in gemm_names
            if timed and start_of[n].startswith("start_"):
                events[start_of[n]].record(stream)
            chain[n]()
            if timed:
                events[n].record(stream)

    # The same step with the weight-gradient GEMMs on a second stream
    # (default priority), each overlapping a data-gradient GEMM; they run one
    # after the other there, so they can share the workspace.
    aux = torch.cuda.Stream()
    on_aux = {"moe_gemm_down_wgrad", "moe_gemm_gate_up_wgrad"}
    order2 = ["moe_route", "moe_permute", "moe_gemm_gate_up", "moe_gemm_down", "moe_combine", "moe_combine_bwd",
              "moe_gemm_down_wgrad", "moe_gemm_down_dgrad", "moe_gemm_gate_up_wgrad", "moe_gemm_gate_up_dgrad",
              "moe_unpermute_sum", "moe_route_bwd"]

    def step_two_streams():
        for n in order2:
            if n in ("moe_gemm_down_wgrad", "moe_gemm_gate_up_wgrad"):  # after combine bwd / down dgrad
                e = torch.cuda.Event()
                e.record(stream)
                aux.wait_event(e)
            if n in on_aux:
                with torch.cuda.stream(aux):
                    by_name[n]()
            else:
                by_name[n]()
        e = torch.cuda.Event()  # join
        e.record(aux)
        stream.wait_event(e)

    # W warmup and K timed steps per seed; the line reports the median seed.
    runs = []
    for seed in seeds[1:] + seeds[:1]:  # the first seed last: the later measurements use its inputs
        load(seed)
        x, wr, wg, wu, wd, dy, bias = (cur[n] for n in ["x", "w_router", "w_gate", "w_up", "w_down", "dy", "bias"])
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for k in range(args.steps):
            step(ev[k])
        end.record(stream)
        torch.cuda.synchronize()
        ms_seed = start.elapsed_time(end) / args.steps
        per_call_seed = {n: sum(ev[k][start_of[n]].elapsed_time(ev[k][n]) for k in range(args.steps)) / args.steps
                         for n in gemm_names}
        runs.append((ms_seed, seed, per_call_seed))
        log(f"seed {seed}: {args.warmup} warmup, {args.steps} timed steps: {ms_seed:.3f} ms/step; "
            + ", ".join(f"{n}={v:.3f}" for n, v in per_call_seed.items()))
    ms, median_seed, per_call = sorted(runs)[len(runs) // 2]
    ms_by_seed = {str(sd): round(m, 4) for m, sd, _ in sorted(runs, key=lambda r: r[1])}

    def time_fn(fn, reps=10):
        return time_calls(fn, stream, reps)

    # The calls without matrix work, each on its own (outside the timed steps).
    other_ms = None if args.timed_only else {n: round(time_fn(chain[n]), 4) for n in names if n not in gemm_names}

    # The same step without the per-call events (what the events themselves cost).
    plain_ms = None if args.timed_only else round(time_fn(step), 4)
    # The other chain, for comparison.
    other_chain = by_name if args.chain == "fused" else both_calls
    other_chain_ms = None if args.timed_only else round(time_fn(lambda: [other_chain[n]() for n in names]), 4)
    two_stream_ms = None if args.timed_only else round(time_fn(step_two_streams), 4)
    if two_stream_ms is not None:
        log(f"two-stream backward: {two_stream_ms:.3f} ms/step")

    # The same step captured once into a HIP graph and replayed (no launch
    # gaps between the calls).
    graph_ms = None
    if not args.timed_only:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            step()
        torch.cuda.synchronize()
        graph_ms = round(time_fn(graph.replay), 4)
        log(f"graph replay: {graph_ms:.3f} ms/step")

    def step_gather_fused():
        for n in names:
            gf_calls[n]()

    gather_fused_ms = None
    if not args.timed_only:
        gather_fused_ms = {"step": round(time_fn(step_gather_fused), 4)}
        for n in ["moe_permute", "moe_gemm_gate_up", "moe_gemm_gate_up_bwd"]:
            gather_fused_ms[n] = round(time_fn(gf_calls[n], reps=5), 4)
        log(f"step without x_perm: {gather_fused_ms}")

    def step_dy_fused():
        for n in names:
            dy_calls[n]()

    dy_fused_ms = None
    if not args.timed_only:
        dy_fused_ms = {"step": round(time_fn(step_dy_fused), 4)}
        for n in ["moe_permute", "moe_gemm_gate_up", "moe_combine_bwd", "moe_gemm_down_bwd"]:
            dy_fused_ms[n] = round(time_fn(dy_calls[n], reps=5), 4)
        log(f"step without do_perm: {dy_fused_ms}")

    def step_both_fused():
        for n in names:
            both_calls[n]()

    both_fused_ms = None
    if not args.timed_only:
        both_fused_ms = {"step": round(time_fn(step_both_fused), 4)}
        for n in ["moe_permute", "moe_gemm_gate_up", "moe_combine_bwd", "moe_gemm_down_bwd", "moe_gemm_gate_up_bwd"]:
            both_fused_ms[n] = round(time_fn(both_calls[n], reps=5), 4)
        log(f"step without x_perm and do_perm: {both_fused_ms}")

    # The same step with one launch per GEMM (the six single-GEMM entry
    # points), and each backward GEMM on its own.
    single_ms = None
    if not args.timed_only:
        single_ms = {"step": round(time_fn(lambda: [by_name[n]() for n in single_names]), 4)}
        for n in ["moe_gemm_down_dgrad", "moe_gemm_down_wgrad", "moe_gemm_gate_up_dgrad", "moe_gemm_gate_up_wgrad"]:
            single_ms[n] = round(time_fn(by_name[n], reps=5), 4)
        log(f"one launch per GEMM: {single_ms}")

    # Inference forward at the same shape (outside the timed training steps):
    # the unfused chain (route, permute with the gather, the two GEMMs, the
    # weighted combine) against the fused path (no x_perm, routing weights in
    # the down GEMM's epilogue, plain per-token sum).
    fb = dict(row_token=torch.empty(cfg.M, dtype=torch.int32, device="cuda"),
              row_weight=torch.empty(cfg.M, device="cuda"))

    def infer_unfused():
        for c in calls[:5]:
            c()

    def infer_fused():
        B.moe_forward_fused(s, x, wr, bias, wg, wu, wd, b["logits"], b["topk_idx"], b["topk_w"], b["counts"],
                            b["offsets"], b["sorted_to_flat"], b["flat_to_sorted"], fb["row_token"],
                            fb["row_weight"], b["a"], b["o_perm"], b["y"], st.ws)

    infer = None
    if not args.timed_only:
        infer = {"unfused": round(time_fn(infer_unfused), 4), "fused": round(time_fn(infer_fused), 4)}
        # The same forward with E4M3 weights and activations (weights quantised
        # once, outside the timing; x and the expert activations every call).
        w8 = B.FP8Weights(wg, wu, wd)
        u8 = torch.uint8
        f8 = dict(xq=torch.empty(cfg.T, cfg.H, dtype=u8, device="cuda"), x_e8=torch.empty(cfg.M, dtype=u8, device="cuda"),
                  aq=torch.empty(cfg.M, cfg.I, dtype=u8, device="cuda"), a_e8=torch.empty(cfg.M, dtype=u8, device="cuda"))

        def infer_fp8():
            B.moe_forward_fused_fp8(s, x, wr, bias, w8.gate[0], w8.gate[1], w8.up[0], w8.up[1], w8.down[0],
                                    w8.down[1], b["logits"], b["topk_idx"], b["topk_w"], b["counts"], b["offsets"],
                                    b["sorted_to_flat"], b["flat_to_sorted"], fb["row_token"], fb["row_weight"],
                                    f8["xq"], f8["x_e8"], b["a"], f8["aq"], f8["a_e8"], b["o_perm"], b["y"], st.ws)

        infer["fp8"] = round(time_fn(infer_fp8), 4)
        gate_up8 = lambda: B.moe_gemm_gate_up_fp8(s, f8["xq"], f8["x_e8"], fb["row_token"], b["offsets"], w8.gate[0],  # noqa: E731
                                                  w8.gate[1], w8.up[0], w8.up[1], b["a"])
        down8 = lambda: B.moe_gemm_down_fp8(s, f8["aq"], f8["a_e8"], b["offsets"], w8.down[0], w8.down[1],  # noqa: E731
                                            fb["row_weight"], b["o_perm"])
        infer["fp8_gate_up"] = round(time_fn(gate_up8, reps=5), 4)
        infer["fp8_down"] = round(time_fn(down8, reps=5), 4)
        # MXFP4 weights (E2M1, one scale per 32 along K) against the same
        # fp8 activations.
        w4 = B.MXFP4GemmWeights(wg, wu, wd)

        def infer_mxfp4():
            B.moe_forward_fused_mxfp4(s, x, wr, bias, w4.gate[0], w4.gate[1], w4.up[0], w4.up[1], w4.down[0],
                                      w4.down[1], b["logits"], b["topk_idx"], b["topk_w"], b["counts"], b["offsets"],
                                      b["sorted_to_flat"], b["flat_to_sorted"], fb["row_token"], fb["row_weight"],
                                      f8["xq"], f8["x_e8"], b["a"], f8["aq"], f8["a_e8"], b["o_perm"], b["y"], st.ws)

        infer["mxfp4"] = round(time_fn(infer_mxfp4), 4)
        gate_up4 = lambda: B.moe_gemm_gate_up_mxfp4(s, f8["xq"], f8["x_e8"], fb["row_token"], b["offsets"],  # noqa: E731
                                                    w4.gate[0], w4.gate[1], w4.up[0], w4.up[1], b["a"])
        down4 = lambda: B.moe_gemm_down_mxfp4(s, f8["aq"], f8["a_e8"], b["offsets"], w4.down[0], w4.down[1],  # noqa: E731
                                              fb["row_weight"], b["o_perm"])
        infer["mxfp4_gate_up"] = round(time_fn(gate_up4, reps=5), 4)
        infer["mxfp4_down"] = round(time_fn(down4, reps=5), 4)
        del w4
        log(f"inference forward: {infer}")

    lora = None if args.timed_only else lora_timing(cfg, seeds[0], (x, wr, wg, wu, wd, dy), bias, stream)

    flops = gemm_flops(cfg)
    nbytes = alg_bytes_fused(cfg) if args.chain == "fused" else alg_bytes(cfg)
    step_flops = sum(flops[n] for n in names if n in flops)
    tflops = step_flops / (ms * 1e-3) / 1e12

    def roofline(times):
        dominant = max(times, key=times.get)
        t_mfma = flops.get(dominant, 0.0) / (PEAK_BF16_TFLOPS * 1e12)
        t_hbm = nbytes[dominant] / (PEAK_HBM_GBS * 1e9)
        secs = times[dominant] * 1e-3
        if t_mfma >= t_hbm:
            roof = {"kernel": dominant, "bound": "mfma", "achieved": round(flops[dominant] / secs / 1e12, 1),
                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
        else:
            roof = {"kernel": dominant, "bound": "hbm", "achieved": round(nbytes[dominant] / secs / 1e9, 1),
                    "peak": PEAK_HBM_GBS, "unit": "GB/s"}
        roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
        ctr = profiled_counters(dominant, cfg.name, args.chain)
        roof["traffic"] = ctr.get("hbm_bytes_per_launch")
        roof["alg_bytes"] = nbytes[dominant]
        if dominant in flops:
            roof["mfma_frac"] = round(flops[dominant] / secs / 1e12 / PEAK_BF16_TFLOPS, 4)
            # From rocprofv3 counters (same source): SIMD-cycles with the matrix
            # core busy, and the clock the kernel ran at.
            roof["mfma_busy_counter"] = ctr.get("mfma_busy_frac")
            roof["clock_ghz_counter"] = ctr.get("clock_ghz")
        return roof

    roof = roofline(per_call)
    gemm_tflops = {n: round(flops[n] / (per_call[n] * 1e-3) / 1e12, 1) for n in names if n in flops}
    if single_ms is not None:
        for n in ["moe_gemm_down_dgrad", "moe_gemm_down_wgrad", "moe_gemm_gate_up_dgrad", "moe_gemm_gate_up_wgrad"]:
            gemm_tflops[n] = round(flops[n] / (single_ms[n] * 1e-3) / 1e12, 1)
    # HBM fraction of the calls without matrix work (algorithmic bytes).
    hbm_frac = None if other_ms is None else {
        n: round(nbytes[n] / (other_ms[n] * 1e-3) / 1e9 / PEAK_HBM_GBS, 3) for n in other_ms}
    out = {
        "metric": METRIC,
        "value": round(cfg.T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded normal inputs, random-init weights of the Qwen3-30B-A3B MoE layer shape)",
        "config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "E": cfg.E, "k": cfg.k, "I": cfg.I,
                   "seeds": seeds, "pass": "fwd+bwd", "chain": args.chain},
        "ms_per_step_by_seed": ms_by_seed,
        "tflops": round(tflops, 1),
        "mfma_peak_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "gemm_tflops": gemm_tflops,
        "call_ms": {n: round(v, 4) for n, v in per_call.items()},
        "other_call_ms": other_ms,
        "hbm_frac": hbm_frac,
        "roofline": roof,
        "ms_per_step_without_call_events": plain_ms,
        ("xperm_chain_ms_per_step" if args.chain == "fused" else "fused_chain_ms_per_step"): other_chain_ms,
        "two_stream_ms_per_step": two_stream_ms,
        "graph_ms_per_step": graph_ms,
        "gather_fused_ms": gather_fused_ms,
        "dy_fused_ms": dy_fused_ms,
        "gather_dy_fused_ms": both_fused_ms,
        "single_launch_ms": single_ms,
        "inference_forward_ms": infer,
        "lora_ms": lora,
    }
    if not (args.no_cpu_baseline or args.timed_only):
        tokens = args.cpu_tokens or cfg.T
        log(f"cpu baseline: oracle on {tokens} tokens")
        out["cpu_baseline"] = cpu_baseline(cfg, seeds[0], tokens)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
