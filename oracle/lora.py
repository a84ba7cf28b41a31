"""Low-rank adapters on the stacked experts (frozen base weights): the oracle.

TEST INFRASTRUCTURE ONLY: the test suite uses it; the product path never
does. Plain numpy in float64.

The pages fine-tune MoE models with LoRA adapters on the fused (stacked)
expert projections (sourcepulse summary, "Highlighted Details": LoRA and
QLoRA on the fused experts, fused and unfused adapter formats; torchtune PR
#2820 lists LoRA support for the Qwen3 MoE port as still to do). The
adapter itself is the usual low-rank update of a frozen weight; the pages
print no formula for it. For expert e and projection P in {gate, up, down}
with frozen W_P[e] [N, K], adapters A_P[e] [r, K] and B_P[e] [N, r], and
scale s:
    W'_P[e] = W_P[e] + s * B_P[e] @ A_P[e]
and the stage computes exactly the plain expert MLP with W' in place of W.
The base weights get no gradient; the adapters get (p ranging over expert
e's sorted rows, X the gathered hidden states, Act = silu(G) * U):
    dB_gate[e] = s * dG^T (X A_gate^T)      dA_gate[e] = s * (dG B_gate)^T X
    dB_up[e]   = s * dU^T (X A_up^T)        dA_up[e]   = s * (dU B_up)^T X
    dB_down[e] = s * dO^T (Act A_down^T)    dA_down[e] = s * (dO B_down)^T Act
dX, dG, dU and d_logits follow the plain backward with W' (the chain rule
through W' = W + s B A gives dW' = (the plain dW) and dA = s B^T dW',
dB = s dW' A^T, which the formulas above restate without forming dW').
"""
from __future__ import annotations

from typing import Dict

import numpy as np


def merge(w: np.ndarray, a: np.ndarray, b: np.ndarray, s: float) -> np.ndarray:
    """W' = W + s B A for stacked [E, N, K] weights, a [E, r, K], b [E, N, r]."""
    return np.asarray(w, np.float64) + s * np.matmul(np.asarray(b, np.float64), np.asarray(a, np.float64))


def dequantize_weights(wq: np.ndarray, e8: np.ndarray) -> np.ndarray:
    """Frozen expert weights kept in 8 bits (the QLoRA-style base of the
    sourcepulse summary, "Highlighted Details" and "Quick Start &
    Requirements"; taken to E4M3 here): codes wq [E, N, K] with one E8M0
    scale per row e8 [E, N] -> float64 values decode(code) * 2^(e8 - 127)."""
    from oracle import fp8 as F8
    E, N, K = wq.shape
    return F8.dequantize_rows(np.asarray(wq).reshape(E * N, K), np.asarray(e8).reshape(E * N)).reshape(E, N, K)


def merge_fp8(wq: np.ndarray, e8: np.ndarray, a: np.ndarray, b: np.ndarray, s: float) -> np.ndarray:
    """W' = deq(Wq) + s B A: the adapters over the dequantised frozen weights."""
    return merge(dequantize_weights(wq, e8), a, b, s)


def dequantize_weights_mxfp4(wq: np.ndarray, e8: np.ndarray) -> np.ndarray:
    """Frozen expert weights in 4 bits (the OCP microscaling FP4 format of
    oracle/mxfp4.py): packed codes wq [E, N, K/2] with one E8M0 scale per 32
    elements of a row, e8 [E, N, K/32] -> float64 [E, N, K]."""
    from oracle import mxfp4 as MX
    E, N, K2 = wq.shape
    return MX.dequantize_blocks(np.asarray(wq).reshape(E * N, K2),
                                np.asarray(e8).reshape(E * N, -1)).reshape(E, N, 2 * K2)


def merge_mxfp4(wq: np.ndarray, e8: np.ndarray, a: np.ndarray, b: np.ndarray, s: float) -> np.ndarray:
    """W' = deq(Wq) + s B A over a 4-bit frozen base."""
    return merge(dequantize_weights_mxfp4(wq, e8), a, b, s)


def forward_backward(x, dy, topk_idx, topk_w, w_gate, w_up, w_down, ad: Dict[str, np.ndarray], s: float):
    """The stage with adapters, forward and backward, in float64.

    x [T, H], dy [T, H], routing topk_idx / topk_w [T, k] (from the router,
    which the adapters do not touch), frozen weights, adapters ad = {a_gate,
    b_gate, a_up, b_up, a_down, b_down}. Returns y, dx, d_topk_w and the six
    adapter gradients, each per the definitions in the module docstring.
    """
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    T, H = x.shape
    k = topk_idx.shape[1]
    E = w_gate.shape[0]
    wg = merge(w_gate, ad["a_gate"], ad["b_gate"], s)
    wu = merge(w_up, ad["a_up"], ad["b_up"], s)
    wd = merge(w_down, ad["a_down"], ad["b_down"], s)
    A = {n: np.asarray(ad[n], np.float64) for n in ad}
    y = np.zeros((T, H))
    dx = np.zeros((T, H))
    d_topk_w = np.zeros((T, k))
    g = {n: np.zeros_like(A[n]) for n in A}
    for e in range(E):
        tok, slot = np.nonzero(topk_idx == e)
        if len(tok) == 0:
            continue
        X = x[tok]
        w = np.asarray(topk_w, np.float64)[tok, slot][:, None]
        G = X @ wg[e].T
        U = X @ wu[e].T
        sig = 1.0 / (1.0 + np.exp(-G))
        Act = G * sig * U
        O = Act @ wd[e].T
        y[tok] += w * O
        d_topk_w[tok, slot] = np.sum(dy[tok] * O, axis=1)
        dO = w * dy[tok]
        dAct = dO @ wd[e]
        dU = dAct * G * sig
        dG = dAct * U * sig * (1.0 + G * (1.0 - sig))
        dx[tok] += dG @ wg[e] + dU @ wu[e]
        g["b_gate"][e] = s * dG.T @ (X @ A["a_gate"][e].T)
        g["a_gate"][e] = s * (dG @ A["b_gate"][e]).T @ X
        g["b_up"][e] = s * dU.T @ (X @ A["a_up"][e].T)
        g["a_up"][e] = s * (dU @ A["b_up"][e]).T @ X
        g["b_down"][e] = s * dO.T @ (Act @ A["a_down"][e].T)
        g["a_down"][e] = s * (dO @ A["b_down"][e]).T @ Act
    out = {"y": y, "dx": dx, "d_topk_w": d_topk_w}
    out.update({"d" + n: v for n, v in g.items()})
    return out
