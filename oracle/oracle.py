"""Python binding of the CPU oracle (``liboracle.so``, built from oracle.cpp).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use it; the product path never does. Every function takes and
returns numpy arrays in host memory; float arrays are all float32 (the parity
reference) or all float64 (finite differences), and the matching C symbol is
chosen from their dtype. Indices are int32.

``forward`` and ``backward`` chain the steps of the stage in order:
route -> expert indexing -> gather -> experts -> combine, and then
combine backward -> experts backward -> unpermute-sum -> router backward.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_F = {np.dtype(np.float32): "f32", np.dtype(np.float64): "f64"}


def _ensure_built():
    if not os.path.exists(_LIB_PATH):
        import importlib.util
        spec = importlib.util.spec_from_file_location("oracle_build", os.path.join(_HERE, "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()


def _l():
    global _lib
    if _lib is None:
        _ensure_built()
        _lib = ctypes.CDLL(_LIB_PATH)
    return _lib


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _suffix(*arrays) -> str:
    dts = {a.dtype for a in arrays if a is not None}
    assert len(dts) == 1, f"mixed float dtypes {dts}"
    return _F[dts.pop()]


def _c(a, dtype=None):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def set_threads(n: int) -> None:
    _l().oracle_set_threads(ctypes.c_int(n))


def threads() -> int:
    return int(_l().oracle_threads())


def route(x: np.ndarray, w_router: np.ndarray, k: int, logit_bias: Optional[np.ndarray] = None):
    """logits [T,E], topk_idx [T,k] int32, topk_w [T,k]."""
    x, w_router = _c(x), _c(w_router, x.dtype)
    logit_bias = _c(logit_bias, x.dtype)
    T, H = x.shape
    E = w_router.shape[0]
    logits = np.empty((T, E), x.dtype)
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), x.dtype)
    rc = getattr(_l(), "oracle_route_" + _suffix(x, w_router))(
        T, H, E, k, _p(x), _p(w_router), _p(logit_bias), _p(logits), _p(idx), _p(w))
    if rc != 0:
        raise ValueError(f"oracle_route rejected the shape (T={T}, H={H}, E={E}, k={k})")
    return logits, idx, w


def permute_index(topk_idx: np.ndarray, E: int):
    """counts [E], offsets [E+1], sorted_to_flat [T*k], flat_to_sorted [T*k] (int32)."""
    topk_idx = _c(topk_idx, np.int32)
    T, k = topk_idx.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    s2f = np.empty(T * k, np.int32)
    f2s = np.empty(T * k, np.int32)
    rc = _l().oracle_permute_index(T, E, k, _p(topk_idx), _p(counts), _p(offsets), _p(s2f), _p(f2s))
    if rc != 0:
        raise ValueError("oracle_permute_index: expert id out of range or bad shape")
    return counts, offsets, s2f, f2s


def gather(x: np.ndarray, sorted_to_flat: np.ndarray, k: int) -> np.ndarray:
    x = _c(x)
    s2f = _c(sorted_to_flat, np.int32)
    T, H = x.shape
    out = np.empty((s2f.shape[0], H), x.dtype)
    getattr(_l(), "oracle_gather_" + _suffix(x))(T, H, k, _p(x), _p(s2f), _p(out))
    return out


def experts_fwd(x_perm, offsets, w_gate, w_up, w_down, expert_mask=None):
    """G, U, A [M,I] and O_perm [M,H] for the sorted rows."""
    x_perm = _c(x_perm)
    dt = x_perm.dtype
    w_gate, w_up, w_down = _c(w_gate, dt), _c(w_up, dt), _c(w_down, dt)
    offsets = _c(offsets, np.int32)
    mask = _c(expert_mask, np.uint8)
    M, H = x_perm.shape
    E, I, _ = w_gate.shape
    g = np.zeros((M, I), dt)
    u = np.zeros((M, I), dt)
    a = np.zeros((M, I), dt)
    o = np.zeros((M, H), dt)
    getattr(_l(), "oracle_experts_fwd_" + _suffix(x_perm))(
        H, E, I, _p(x_perm), _p(offsets), _p(w_gate), _p(w_up), _p(w_down), _p(mask), _p(g), _p(u), _p(a), _p(o))
    return g, u, a, o


def combine(o_perm, topk_w, flat_to_sorted, T: int, k: int):
    o_perm = _c(o_perm)
    topk_w = _c(topk_w, o_perm.dtype)
    f2s = _c(flat_to_sorted, np.int32)
    H = o_perm.shape[1]
    y = np.empty((T, H), o_perm.dtype)
    getattr(_l(), "oracle_combine_" + _suffix(o_perm))(T, H, k, _p(o_perm), _p(topk_w), _p(f2s), _p(y))
    return y


def combine_bwd(dy, o_perm, topk_w, flat_to_sorted):
    dy = _c(dy)
    dt = dy.dtype
    o_perm, topk_w = _c(o_perm, dt), _c(topk_w, dt)
    f2s = _c(flat_to_sorted, np.int32)
    T, H = dy.shape
    k = topk_w.shape[1]
    do_perm = np.empty((T * k, H), dt)
    gw = np.empty((T, k), dt)
    getattr(_l(), "oracle_combine_bwd_" + _suffix(dy))(
        T, H, k, _p(dy), _p(o_perm), _p(topk_w), _p(f2s), _p(do_perm), _p(gw))
    return do_perm, gw


def experts_bwd(do_perm, x_perm, g, u, a, offsets, w_gate, w_up, w_down, expert_mask=None):
    """dX_perm [M,H], dW_gate, dW_up [E,I,H], dW_down [E,H,I]."""
    do_perm = _c(do_perm)
    dt = do_perm.dtype
    x_perm, g, u, a = (_c(v, dt) for v in (x_perm, g, u, a))
    w_gate, w_up, w_down = _c(w_gate, dt), _c(w_up, dt), _c(w_down, dt)
    offsets = _c(offsets, np.int32)
    mask = _c(expert_mask, np.uint8)
    M, H = do_perm.shape
    E, I, _ = w_gate.shape
    dx_perm = np.zeros((M, H), dt)
    dwg = np.zeros((E, I, H), dt)
    dwu = np.zeros((E, I, H), dt)
    dwd = np.zeros((E, H, I), dt)
    getattr(_l(), "oracle_experts_bwd_" + _suffix(do_perm))(
        H, E, I, _p(do_perm), _p(x_perm), _p(g), _p(u), _p(a), _p(offsets), _p(w_gate), _p(w_up), _p(w_down),
        _p(mask), _p(dx_perm), _p(dwg), _p(dwu), _p(dwd))
    return dx_perm, dwg, dwu, dwd


def unpermute_sum(dx_perm, flat_to_sorted, T: int, k: int):
    dx_perm = _c(dx_perm)
    f2s = _c(flat_to_sorted, np.int32)
    H = dx_perm.shape[1]
    dx = np.empty((T, H), dx_perm.dtype)
    getattr(_l(), "oracle_unpermute_sum_" + _suffix(dx_perm))(T, H, k, _p(dx_perm), _p(f2s), _p(dx))
    return dx


def route_bwd(logits, topk_idx, gw):
    logits = _c(logits)
    gw = _c(gw, logits.dtype)
    idx = _c(topk_idx, np.int32)
    T, E = logits.shape
    k = idx.shape[1]
    d_logits = np.empty((T, E), logits.dtype)
    getattr(_l(), "oracle_route_bwd_" + _suffix(logits))(T, E, k, _p(logits), _p(idx), _p(gw), _p(d_logits))
    return d_logits


def forward(x, w_router, w_gate, w_up, w_down, k: int, logit_bias=None, expert_mask=None) -> Dict[str, np.ndarray]:
    """The whole forward stage; returns every intermediate by name."""
    T = x.shape[0]
    E = w_router.shape[0]
    logits, idx, w = route(x, w_router, k, logit_bias)
    counts, offsets, s2f, f2s = permute_index(idx, E)
    x_perm = gather(x, s2f, k)
    g, u, a, o = experts_fwd(x_perm, offsets, w_gate, w_up, w_down, expert_mask)
    y = combine(o, w, f2s, T, k)
    return dict(logits=logits, topk_idx=idx, topk_w=w, counts=counts, offsets=offsets, sorted_to_flat=s2f,
                flat_to_sorted=f2s, x_perm=x_perm, g=g, u=u, a=a, o_perm=o, y=y)


def backward(fwd: Dict[str, np.ndarray], dy, w_gate, w_up, w_down, expert_mask=None) -> Dict[str, np.ndarray]:
    """The whole backward stage given the forward's intermediates and dY."""
    T, k = fwd["topk_idx"].shape
    do_perm, gw = combine_bwd(dy, fwd["o_perm"], fwd["topk_w"], fwd["flat_to_sorted"])
    dx_perm, dwg, dwu, dwd = experts_bwd(do_perm, fwd["x_perm"], fwd["g"], fwd["u"], fwd["a"], fwd["offsets"],
                                         w_gate, w_up, w_down, expert_mask)
    dx = unpermute_sum(dx_perm, fwd["flat_to_sorted"], T, k)
    d_logits = route_bwd(fwd["logits"], fwd["topk_idx"], gw)
    return dict(do_perm=do_perm, d_topk_w=gw, dx_perm=dx_perm, dw_gate=dwg, dw_up=dwu, dw_down=dwd, dx=dx,
                d_logits=d_logits)
