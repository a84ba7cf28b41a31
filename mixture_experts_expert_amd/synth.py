"""Seeded synthetic inputs for one MoE layer's expert stage.

This module is the only code that the HIP path and the CPU oracle share. It
holds none of the method's arithmetic: it draws random numbers, rounds them to
bf16 where a workload is bf16, and builds the per-expert logit bias that the
skewed workload feeds to the router as an input.

Recipe (every array is drawn from ``numpy.random.default_rng(seed)``, PCG64, in
this order):

* ``x``        [T, H]    standard normal
* ``w_router`` [E, H]    0.02 * standard normal (std 0.02)
* ``w_gate``   [E, I, H] 0.02 * standard normal, one [I, H] draw per expert
* ``w_up``     [E, I, H] 0.02 * standard normal, one [I, H] draw per expert
* ``w_down``   [E, H, I] 0.02 * standard normal, one [H, I] draw per expert
* ``dy``       [T, H]    standard normal (training workloads only)

Draws are float32. bf16 workloads round each draw to bf16 with
round-to-nearest-even; both sides then see the same bytes. The skewed workload
adds a Zipf(s) logit bias ``bias[e] = -s * ln(r_e)`` where ``r = 1 +
permutation(E)`` comes from ``default_rng(seed + 1)``: softmax turns it into a
Zipf prior over experts (its normaliser cancels), so a few experts take a large
share of the assignments and some receive none.

The real workloads behind these shapes are Qwen3-MoE hidden states and trained
routers (Qwen3-30B-A3B and 235B-A22B layers fine-tuned on Alpaca); no weights or
data are used, these draws stand in for them.
"""
from __future__ import annotations

from dataclasses import dataclass, asdict
from typing import Dict, Optional

import numpy as np


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int          # tokens
    H: int          # hidden size
    E: int          # experts
    k: int          # experts per token (top-k)
    I: int          # expert intermediate size
    dtype: str      # "f32" or "bf16"
    backward: bool  # training step (forward + backward) or forward only
    zipf_s: float = 0.0  # > 0: add the Zipf(s) logit bias

    @property
    def M(self) -> int:
        """Rows after expanding each token into its k (token, expert) pairs."""
        return self.T * self.k

    def gemm_flops(self) -> float:
        """Flops of the expert GEMMs: 6*M*H*I forward, 12*M*H*I more backward."""
        f = 6.0 * self.M * self.H * self.I
        return f * 3.0 if self.backward else f

    def router_flops(self) -> float:
        return 2.0 * self.T * self.H * self.E

    def asdict(self) -> dict:
        return asdict(self)


CONFIGS: Dict[str, MoEConfig] = {
    c.name: c
    for c in [
        MoEConfig("tiny_f32", T=64, H=128, E=8, k=2, I=64, dtype="f32", backward=False),
        MoEConfig("qwen3_30b_a3b_fwd", T=4096, H=2048, E=128, k=8, I=768, dtype="bf16", backward=False),
        MoEConfig("qwen3_30b_a3b_train", T=8192, H=2048, E=128, k=8, I=768, dtype="bf16", backward=True),
        MoEConfig("qwen3_30b_a3b_zipf_train", T=16384, H=2048, E=128, k=8, I=768, dtype="bf16",
                  backward=True, zipf_s=1.2),
        MoEConfig("qwen3_235b_a22b_train", T=8192, H=4096, E=128, k=8, I=1536, dtype="bf16", backward=True),
    ]
}


def bf16_round(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Finite inputs only (the generators never produce inf or NaN).
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def bf16_widen(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> the float32 values they encode (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def zipf_bias(E: int, s: float, seed: int) -> np.ndarray:
    """Per-expert logit bias -s*ln(rank), ranks a seeded permutation of 1..E."""
    r = 1 + np.random.default_rng(seed + 1).permutation(E)
    return (-s * np.log(r.astype(np.float64))).astype(np.float32)


class Inputs:
    """One workload's inputs, as the bytes both sides receive.

    For bf16 workloads each tensor is stored as uint16 bit patterns (``bits``);
    ``f32(name)`` widens it to the exact float32 values. For f32 workloads the
    tensors are float32 and ``bits`` holds them unchanged.
    """

    def __init__(self, cfg: MoEConfig, seed: int, tensors: Dict[str, np.ndarray],
                 logit_bias: Optional[np.ndarray]):
        self.cfg = cfg
        self.seed = seed
        self.bits = tensors
        self.logit_bias = logit_bias

    def f32(self, name: str) -> np.ndarray:
        a = self.bits[name]
        if a.dtype == np.uint16:
            return bf16_widen(a)
        return a

    def names(self):
        return list(self.bits.keys())


def make_inputs(cfg: MoEConfig, seed: int = 0, *, T: Optional[int] = None,
                with_dy: Optional[bool] = None, router_only: bool = False) -> Inputs:
    """Draw one workload's inputs. ``T`` overrides the token count (sub-batches).

    ``router_only`` stops after ``x`` and ``w_router``; they are the first two
    draws, so their values equal those of the full draw.
    """
    T = cfg.T if T is None else T
    with_dy = cfg.backward if with_dy is None else with_dy
    rng = np.random.default_rng(seed)
    E, H, I = cfg.E, cfg.H, cfg.I
    bf16 = cfg.dtype == "bf16"

    def fin(a: np.ndarray) -> np.ndarray:
        return bf16_round(a) if bf16 else np.ascontiguousarray(a, dtype=np.float32)

    def stacked(rows: int, cols: int) -> np.ndarray:
        out = np.empty((E, rows, cols), dtype=np.uint16 if bf16 else np.float32)
        for e in range(E):
            out[e] = fin(np.float32(0.02) * rng.standard_normal((rows, cols), dtype=np.float32))
        return out

    t = {}
    t["x"] = fin(rng.standard_normal((T, H), dtype=np.float32))
    t["w_router"] = fin(np.float32(0.02) * rng.standard_normal((E, H), dtype=np.float32))
    bias = zipf_bias(E, cfg.zipf_s, seed) if cfg.zipf_s > 0 else None
    if router_only:
        return Inputs(cfg, seed, t, bias)
    t["w_gate"] = stacked(I, H)
    t["w_up"] = stacked(I, H)
    t["w_down"] = stacked(H, I)
    if with_dy:
        t["dy"] = fin(rng.standard_normal((T, H), dtype=np.float32))
    return Inputs(cfg, seed, t, bias)


ADAPTER_NAMES = ("a_gate", "b_gate", "a_up", "b_up", "a_down", "b_down")


def make_adapters(cfg: MoEConfig, r: int, seed: int = 0) -> Dict[str, np.ndarray]:
    """Low-rank adapters of rank r for every expert projection, as bf16 bit
    patterns (uint16). Drawn from ``default_rng(seed + 2)`` in the order
    a_gate [E, r, H], b_gate [E, I, r], a_up [E, r, H], b_up [E, I, r],
    a_down [E, r, I], b_down [E, H, r], each 0.02 * standard normal float32
    rounded to bf16 (trained adapters: B is no longer zero)."""
    rng = np.random.default_rng(seed + 2)
    E, H, I = cfg.E, cfg.H, cfg.I
    shapes = {"a_gate": (E, r, H), "b_gate": (E, I, r), "a_up": (E, r, H), "b_up": (E, I, r),
              "a_down": (E, r, I), "b_down": (E, H, r)}
    return {n: bf16_round(np.float32(0.02) * rng.standard_normal(shapes[n], dtype=np.float32))
            for n in ADAPTER_NAMES}


def random_small_config(rng: np.random.Generator, dtype: str = "f32", backward: bool = True,
                        max_T: int = 24) -> MoEConfig:
    """A random tiny shape for brute-force checks (any H, I; k <= E)."""
    E = int(rng.integers(1, 7))
    k = int(rng.integers(1, E + 1))
    return MoEConfig("random_small", T=int(rng.integers(1, max_T + 1)), H=int(rng.integers(1, 20)), E=E, k=k,
                     I=int(rng.integers(1, 12)), dtype=dtype, backward=backward)
