"""Python binding of libmoe's C ABI (include/moe.h), by ctypes.

Argument marshalling only: every function here has the name of a C entry
point, checks nothing the library does not check itself, passes torch CUDA
tensors as raw device pointers and the current HIP stream, and raises
``MoEError`` on a non-zero status. Every step of the stage runs in the
library's HIP kernels; there is no other code path. Importing this module on a
machine without the built library raises ImportError.

``MoEStage`` chains the calls of one forward and one backward pass, holding
the buffers (torch is used for device memory only).
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_F32, MOE_BF16 = 0, 1
STATUS = {0: "MOE_OK", 1: "MOE_EINVAL", 2: "MOE_EUNSUPPORTED", 3: "MOE_EWORKSPACE", 4: "MOE_EHIP"}


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} returned {STATUS.get(status, status)}: {msg}")
        self.status = status


class moe_shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("E", ctypes.c_int32), ("k", ctypes.c_int32),
                ("I", ctypes.c_int32), ("dtype", ctypes.c_int32)]


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run mixture_experts_expert_amd/build.py (or __graft_entry__.build())")
lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_SIGS = {
    "moe_workspace_bytes": ([moe_shape], ctypes.c_size_t),
    "moe_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "moe_route": ([moe_shape, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "moe_permute": ([moe_shape, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "moe_grouped_gemm_fwd": ([moe_shape, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "moe_combine": ([moe_shape, _P, _P, _P, _P, _P], ctypes.c_int),
    "moe_combine_bwd": ([moe_shape, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "moe_grouped_gemm_bwd": ([moe_shape, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int, _P,
                              ctypes.c_size_t, _P], ctypes.c_int),
    "moe_unpermute_sum": ([moe_shape, _P, _P, _P, _P], ctypes.c_int),
    "moe_route_bwd": ([moe_shape, _P, _P, _P, _P, _P], ctypes.c_int),
    "moe_gemm_gate_up": ([moe_shape, _P, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "moe_gemm_down": ([moe_shape, _P, _P, _P, _P, _P], ctypes.c_int),
    "moe_gemm_down_dgrad": ([moe_shape, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "moe_gemm_down_wgrad": ([moe_shape, _P, _P, _P, _P, ctypes.c_int, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "moe_gemm_gate_up_dgrad": ([moe_shape, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "moe_gemm_gate_up_wgrad": ([moe_shape, _P, _P, _P, _P, _P, ctypes.c_int, _P, ctypes.c_size_t, _P],
                               ctypes.c_int),
    "moe_permute_fused": ([moe_shape, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "moe_gemm_gate_up_gathered": ([moe_shape, _P, _P, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "moe_gemm_down_weighted": ([moe_shape, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "moe_quantize_fp8_rows": ([ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P, ctypes.c_int32, _P], ctypes.c_int),
    "moe_gemm_gate_up_fp8": ([moe_shape] + [_P] * 9 + [_P], ctypes.c_int),
    "moe_gemm_down_fp8": ([moe_shape] + [_P] * 7 + [_P], ctypes.c_int),
    "moe_forward_fused_fp8": ([moe_shape] + [_P] * 26 + [ctypes.c_size_t, _P], ctypes.c_int),
    "moe_gemm_gate_up_mxfp4": ([moe_shape] + [_P] * 9 + [_P], ctypes.c_int),
    "moe_gemm_down_mxfp4": ([moe_shape] + [_P] * 7 + [_P], ctypes.c_int),
    "moe_forward_fused_mxfp4": ([moe_shape] + [_P] * 26 + [ctypes.c_size_t, _P], ctypes.c_int),
    "moe_quantize_mxfp4_weights": ([ctypes.c_int32] * 3 + [_P] * 4, ctypes.c_int),
    "moe_gemm_down_bwd": ([moe_shape] + [_P] * 8 + [ctypes.c_int, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "moe_gemm_gate_up_bwd": ([moe_shape] + [_P] * 9 + [ctypes.c_int, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "moe_gemm_gate_up_wgrad_gathered": ([moe_shape, _P, _P, _P, _P, _P, _P, ctypes.c_int, _P, ctypes.c_size_t, _P],
                                        ctypes.c_int),
    "moe_forward_fused": ([moe_shape] + [_P] * 19 + [ctypes.c_size_t, _P], ctypes.c_int),
    "moe_forward_fused_noalloc": ([moe_shape] + [_P] * 18 + [_P], ctypes.c_int),
    "moe_permute_rows": ([moe_shape] + [_P] * 11 + [ctypes.c_size_t, _P], ctypes.c_int),
    "moe_gemm_gate_up_aw": ([moe_shape] + [_P] * 10 + [_P], ctypes.c_int),
    "moe_gemm_down_bwd_dy": ([moe_shape] + [_P] * 10 + [ctypes.c_int, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "moe_lora_workspace_bytes": ([moe_shape, ctypes.c_int32], ctypes.c_size_t),
    "moe_lora_merge": ([ctypes.c_int32] * 4 + [ctypes.c_float] + [_P] * 5, ctypes.c_int),
    "moe_lora_merge_fp8": ([ctypes.c_int32] * 4 + [ctypes.c_float] + [_P] * 6, ctypes.c_int),
    "moe_lora_grads": ([moe_shape, ctypes.c_int32, ctypes.c_float] + [_P] * 18 + [ctypes.c_size_t, _P],
                       ctypes.c_int),
    "moe_quantize_mxfp4_rows": ([ctypes.c_int32, ctypes.c_int32] + [_P] * 4, ctypes.c_int),
    "moe_lora_merge_mxfp4": ([ctypes.c_int32] * 4 + [ctypes.c_float] + [_P] * 6, ctypes.c_int),
    "moe_lora_grads_gathered": ([moe_shape, ctypes.c_int32, ctypes.c_float] + [_P] * 20 + [ctypes.c_size_t, _P],
                                ctypes.c_int),
    "moe_gemm_down_dgrad_dy": ([moe_shape] + [_P] * 9, ctypes.c_int),
    "moe_lora_unmerged_workspace_bytes": ([moe_shape, ctypes.c_int32], ctypes.c_size_t),
    "moe_lora_prepare": ([moe_shape, ctypes.c_int32, ctypes.c_float] + [_P] * 7 + [ctypes.c_size_t, _P], ctypes.c_int),
    "moe_lora_gemm_gate_up": ([moe_shape, ctypes.c_int32] + [_P] * 10 + [ctypes.c_size_t, _P], ctypes.c_int),
    "moe_lora_gemm_down": ([moe_shape, ctypes.c_int32] + [_P] * 6 + [ctypes.c_size_t, _P], ctypes.c_int),
    "moe_lora_gemm_down_dgrad": ([moe_shape, ctypes.c_int32] + [_P] * 8 + [ctypes.c_size_t, _P], ctypes.c_int),
    "moe_lora_gemm_gate_up_dgrad": ([moe_shape, ctypes.c_int32] + [_P] * 8 + [ctypes.c_size_t, _P], ctypes.c_int),
    "moe_lora_grads_unmerged": ([moe_shape, ctypes.c_int32] + [_P] * 12 + [ctypes.c_size_t, _P], ctypes.c_int),
    "moe_lora_gemm_gate_up_gathered": ([moe_shape, ctypes.c_int32] + [_P] * 11 + [ctypes.c_size_t, _P], ctypes.c_int),
    "moe_lora_gemm_down_dgrad_dy": ([moe_shape, ctypes.c_int32] + [_P] * 10 + [ctypes.c_size_t, _P], ctypes.c_int),
    "moe_lora_grads_unmerged_gathered": ([moe_shape, ctypes.c_int32] + [_P] * 14 + [ctypes.c_size_t, _P],
                                         ctypes.c_int),
}
for _name, (_args, _ret) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.argtypes = _args
    _fn.restype = _ret


def shape(T: int, H: int, E: int, k: int, I: int, dtype) -> moe_shape:
    if dtype in (torch.bfloat16, "bf16", MOE_BF16):
        dt = MOE_BF16
    elif dtype in (torch.float32, "f32", MOE_F32):
        dt = MOE_F32
    else:
        dt = int(dtype)  # passed through; the library rejects unknown codes
    return moe_shape(T, H, E, k, I, dt)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        raise MoEError(fn, rc, lib.moe_status_string(rc).decode())


def moe_workspace_bytes(s: moe_shape) -> int:
    return int(lib.moe_workspace_bytes(s))


def moe_status_string(status: int) -> str:
    return lib.moe_status_string(status).decode()


def moe_route(s, x, w_router, logit_bias, logits, topk_idx, topk_w, stream=None):
    _check("moe_route", lib.moe_route(s, _ptr(x), _ptr(w_router), _ptr(logit_bias), _ptr(logits), _ptr(topk_idx),
                                      _ptr(topk_w), _stream(stream)))


def moe_permute(s, topk_idx, x, counts, offsets, sorted_to_flat, flat_to_sorted, x_perm, ws, ws_bytes=None,
                stream=None):
    nb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("moe_permute", lib.moe_permute(s, _ptr(topk_idx), _ptr(x), _ptr(counts), _ptr(offsets),
                                          _ptr(sorted_to_flat), _ptr(flat_to_sorted), _ptr(x_perm), _ptr(ws), nb,
                                          _stream(stream)))


def moe_grouped_gemm_fwd(s, x_perm, offsets, w_gate, w_up, w_down, g, u, a, o_perm, ws=None, ws_bytes=0,
                         stream=None):
    _check("moe_grouped_gemm_fwd", lib.moe_grouped_gemm_fwd(
        s, _ptr(x_perm), _ptr(offsets), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(g), _ptr(u), _ptr(a),
        _ptr(o_perm), _ptr(ws), ws_bytes, _stream(stream)))


def moe_combine(s, o_perm, topk_w, flat_to_sorted, y, stream=None):
    _check("moe_combine", lib.moe_combine(s, _ptr(o_perm), _ptr(topk_w), _ptr(flat_to_sorted), _ptr(y),
                                          _stream(stream)))


def moe_combine_bwd(s, dy, o_perm, topk_w, flat_to_sorted, do_perm, d_topk_w, stream=None):
    _check("moe_combine_bwd", lib.moe_combine_bwd(s, _ptr(dy), _ptr(o_perm), _ptr(topk_w), _ptr(flat_to_sorted),
                                                  _ptr(do_perm), _ptr(d_topk_w), _stream(stream)))


def moe_grouped_gemm_bwd(s, do_perm, x_perm, g, u, a, offsets, w_gate, w_up, w_down, dx_perm, dw_gate, dw_up,
                         dw_down, accumulate_dw, ws, ws_bytes=None, stream=None):
    nb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("moe_grouped_gemm_bwd", lib.moe_grouped_gemm_bwd(
        s, _ptr(do_perm), _ptr(x_perm), _ptr(g), _ptr(u), _ptr(a), _ptr(offsets), _ptr(w_gate), _ptr(w_up),
        _ptr(w_down), _ptr(dx_perm), _ptr(dw_gate), _ptr(dw_up), _ptr(dw_down), int(accumulate_dw), _ptr(ws), nb,
        _stream(stream)))


def moe_unpermute_sum(s, dx_perm, flat_to_sorted, dx, stream=None):
    _check("moe_unpermute_sum", lib.moe_unpermute_sum(s, _ptr(dx_perm), _ptr(flat_to_sorted), _ptr(dx),
                                                      _stream(stream)))


def moe_route_bwd(s, d_topk_w, topk_w, topk_idx, d_logits, stream=None):
    _check("moe_route_bwd", lib.moe_route_bwd(s, _ptr(d_topk_w), _ptr(topk_w), _ptr(topk_idx), _ptr(d_logits),
                                              _stream(stream)))


def moe_gemm_gate_up(s, x_perm, offsets, w_gate, w_up, g, u, a, stream=None):
    _check("moe_gemm_gate_up", lib.moe_gemm_gate_up(s, _ptr(x_perm), _ptr(offsets), _ptr(w_gate), _ptr(w_up),
                                                    _ptr(g), _ptr(u), _ptr(a), _stream(stream)))


def moe_gemm_down(s, a, offsets, w_down, o_perm, stream=None):
    _check("moe_gemm_down", lib.moe_gemm_down(s, _ptr(a), _ptr(offsets), _ptr(w_down), _ptr(o_perm),
                                              _stream(stream)))


def moe_gemm_down_dgrad(s, do_perm, offsets, w_down, g, u, dgu, stream=None):
    _check("moe_gemm_down_dgrad", lib.moe_gemm_down_dgrad(s, _ptr(do_perm), _ptr(offsets), _ptr(w_down), _ptr(g),
                                                          _ptr(u), _ptr(dgu), _stream(stream)))


def moe_gemm_down_wgrad(s, do_perm, a, offsets, dw_down, accumulate_dw, ws, ws_bytes=None, stream=None):
    nb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("moe_gemm_down_wgrad", lib.moe_gemm_down_wgrad(s, _ptr(do_perm), _ptr(a), _ptr(offsets), _ptr(dw_down),
                                                          int(accumulate_dw), _ptr(ws), nb, _stream(stream)))


def moe_gemm_gate_up_dgrad(s, dgu, offsets, w_gate, w_up, dx_perm, stream=None):
    _check("moe_gemm_gate_up_dgrad", lib.moe_gemm_gate_up_dgrad(s, _ptr(dgu), _ptr(offsets), _ptr(w_gate),
                                                                _ptr(w_up), _ptr(dx_perm), _stream(stream)))


def moe_gemm_gate_up_wgrad(s, dgu, x_perm, offsets, dw_gate, dw_up, accumulate_dw, ws, ws_bytes=None, stream=None):
    nb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("moe_gemm_gate_up_wgrad", lib.moe_gemm_gate_up_wgrad(s, _ptr(dgu), _ptr(x_perm), _ptr(offsets),
                                                                _ptr(dw_gate), _ptr(dw_up), int(accumulate_dw),
                                                                _ptr(ws), nb, _stream(stream)))


def moe_permute_fused(s, topk_idx, topk_w, counts, offsets, sorted_to_flat, flat_to_sorted, row_token, row_weight,
                      ws, ws_bytes=None, stream=None):
    nb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("moe_permute_fused", lib.moe_permute_fused(s, _ptr(topk_idx), _ptr(topk_w), _ptr(counts), _ptr(offsets),
                                                      _ptr(sorted_to_flat), _ptr(flat_to_sorted), _ptr(row_token),
                                                      _ptr(row_weight), _ptr(ws), nb, _stream(stream)))


def moe_gemm_gate_up_gathered(s, x, row_token, offsets, w_gate, w_up, g, u, a, stream=None):
    _check("moe_gemm_gate_up_gathered", lib.moe_gemm_gate_up_gathered(
        s, _ptr(x), _ptr(row_token), _ptr(offsets), _ptr(w_gate), _ptr(w_up), _ptr(g), _ptr(u), _ptr(a),
        _stream(stream)))


def moe_quantize_fp8_rows(rows, K, x, q, e8, flat_to_sorted=None, k=0, stream=None):
    _check("moe_quantize_fp8_rows", lib.moe_quantize_fp8_rows(int(rows), int(K), _ptr(x), _ptr(q), _ptr(e8),
                                                              _ptr(flat_to_sorted), int(k), _stream(stream)))


def moe_gemm_gate_up_fp8(s, xq, x_e8, row_token, offsets, wq_gate, w_gate_e8, wq_up, w_up_e8, a, stream=None):
    _check("moe_gemm_gate_up_fp8", lib.moe_gemm_gate_up_fp8(s, _ptr(xq), _ptr(x_e8), _ptr(row_token), _ptr(offsets),
                                                            _ptr(wq_gate), _ptr(w_gate_e8), _ptr(wq_up),
                                                            _ptr(w_up_e8), _ptr(a), _stream(stream)))


def moe_gemm_down_fp8(s, aq, a_e8, offsets, wq_down, w_down_e8, row_weight, o_perm, stream=None):
    _check("moe_gemm_down_fp8", lib.moe_gemm_down_fp8(s, _ptr(aq), _ptr(a_e8), _ptr(offsets), _ptr(wq_down),
                                                      _ptr(w_down_e8), _ptr(row_weight), _ptr(o_perm),
                                                      _stream(stream)))


def moe_forward_fused_fp8(s, x, w_router, logit_bias, wq_gate, w_gate_e8, wq_up, w_up_e8, wq_down, w_down_e8, logits,
                          topk_idx, topk_w, counts, offsets, sorted_to_flat, flat_to_sorted, row_token, row_weight, xq,
                          x_e8, a, aq, a_e8, o_perm, y, ws, ws_bytes=None, stream=None):
    nb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    args = [x, w_router, logit_bias, wq_gate, w_gate_e8, wq_up, w_up_e8, wq_down, w_down_e8, logits, topk_idx,
            topk_w, counts, offsets, sorted_to_flat, flat_to_sorted, row_token, row_weight, xq, x_e8, a, aq, a_e8,
            o_perm, y, ws]
    _check("moe_forward_fused_fp8", lib.moe_forward_fused_fp8(s, *[_ptr(t) for t in args], nb, _stream(stream)))


def moe_gemm_gate_up_mxfp4(s, xq, x_e8, row_token, offsets, wq_gate, w_gate_e8, wq_up, w_up_e8, a, stream=None):
    _check("moe_gemm_gate_up_mxfp4", lib.moe_gemm_gate_up_mxfp4(
        s, _ptr(xq), _ptr(x_e8), _ptr(row_token), _ptr(offsets), _ptr(wq_gate), _ptr(w_gate_e8), _ptr(wq_up),
        _ptr(w_up_e8), _ptr(a), _stream(stream)))


def moe_gemm_down_mxfp4(s, aq, a_e8, offsets, wq_down, w_down_e8, row_weight, o_perm, stream=None):
    _check("moe_gemm_down_mxfp4", lib.moe_gemm_down_mxfp4(s, _ptr(aq), _ptr(a_e8), _ptr(offsets), _ptr(wq_down),
                                                          _ptr(w_down_e8), _ptr(row_weight), _ptr(o_perm),
                                                          _stream(stream)))


def moe_forward_fused_mxfp4(s, x, w_router, logit_bias, wq_gate, w_gate_e8, wq_up, w_up_e8, wq_down, w_down_e8,
                            logits, topk_idx, topk_w, counts, offsets, sorted_to_flat, flat_to_sorted, row_token,
                            row_weight, xq, x_e8, a, aq, a_e8, o_perm, y, ws, ws_bytes=None, stream=None):
    nb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    args = [x, w_router, logit_bias, wq_gate, w_gate_e8, wq_up, w_up_e8, wq_down, w_down_e8, logits, topk_idx,
            topk_w, counts, offsets, sorted_to_flat, flat_to_sorted, row_token, row_weight, xq, x_e8, a, aq, a_e8,
            o_perm, y, ws]
    _check("moe_forward_fused_mxfp4", lib.moe_forward_fused_mxfp4(s, *[_ptr(t) for t in args], nb, _stream(stream)))


def moe_quantize_mxfp4_weights(E, N, K, w, q, e8, stream=None):
    _check("moe_quantize_mxfp4_weights", lib.moe_quantize_mxfp4_weights(int(E), int(N), int(K), _ptr(w), _ptr(q),
                                                                        _ptr(e8), _stream(stream)))


class MXFP4GemmWeights:
    """Expert weights quantised once to MXFP4 for the fp8 x MXFP4 GEMMs of
    the inference forward (moe_quantize_mxfp4_weights): codes gate/up
    [E,I,H/2], down [E,H,I/2] (two E2M1 per byte) and their E8M0 block
    scales stored block-major, [E,H/32,I] and [E,I/32,H]."""

    def __init__(self, w_gate, w_up, w_down, stream=None):
        E, I, H = w_gate.shape
        dev = w_gate.device
        u8 = torch.uint8

        def quant(w, N, K):
            q, e8 = torch.empty(E, N, K // 2, dtype=u8, device=dev), torch.empty(E, K // 32, N, dtype=u8, device=dev)
            moe_quantize_mxfp4_weights(E, N, K, w, q, e8, stream=stream)
            return q, e8

        self.gate, self.up, self.down = quant(w_gate, I, H), quant(w_up, I, H), quant(w_down, H, I)


class FP8Weights:
    """Expert weights quantised once to E4M3 with a scale per output channel
    (moe_quantize_fp8_rows): codes gate/up [E,I,H], down [E,H,I] (uint8)
    and their E8M0 scales [E,I], [E,H]."""

    def __init__(self, w_gate, w_up, w_down, stream=None):
        E, I, H = w_gate.shape
        dev = w_gate.device
        u8 = torch.uint8
        self.gate = (torch.empty(E, I, H, dtype=u8, device=dev), torch.empty(E, I, dtype=u8, device=dev))
        self.up = (torch.empty(E, I, H, dtype=u8, device=dev), torch.empty(E, I, dtype=u8, device=dev))
        self.down = (torch.empty(E, H, I, dtype=u8, device=dev), torch.empty(E, H, dtype=u8, device=dev))
        for w, (q, e8) in ((w_gate, self.gate), (w_up, self.up)):
            moe_quantize_fp8_rows(E * I, H, w, q, e8, stream=stream)
        moe_quantize_fp8_rows(E * H, I, w_down, self.down[0], self.down[1], stream=stream)


def moe_quantize_mxfp4_rows(rows, K, inp, q, e8, stream=None):
    _check("moe_quantize_mxfp4_rows", lib.moe_quantize_mxfp4_rows(int(rows), int(K), _ptr(inp), _ptr(q), _ptr(e8),
                                                                  _stream(stream)))


def moe_lora_merge_mxfp4(E, N, K, r, scale, wq, w_e8, a, b, w_out, stream=None):
    _check("moe_lora_merge_mxfp4", lib.moe_lora_merge_mxfp4(int(E), int(N), int(K), int(r), float(scale), _ptr(wq),
                                                            _ptr(w_e8), _ptr(a), _ptr(b), _ptr(w_out),
                                                            _stream(stream)))


class MXFP4Tensor(tuple):
    """(codes [E,N,K/2] uint8, E8M0 scales [E,N,K/32] uint8) of one stacked
    weight in MXFP4 (moe_quantize_mxfp4_rows)."""


class MXFP4Weights:
    """Expert weights quantised once to MXFP4 (E2M1, one E8M0 scale per 32
    elements along the reduction axis), for adapters over a 4-bit frozen
    base: gate/up codes [E,I,H/2] and scales [E,I,H/32], down [E,H,I/2] and
    [E,H,I/32]."""

    def __init__(self, w_gate, w_up, w_down, stream=None):
        E, I, H = w_gate.shape
        dev = w_gate.device
        u8 = torch.uint8

        def quant(w, N, K):
            t = MXFP4Tensor((torch.empty(E, N, K // 2, dtype=u8, device=dev),
                             torch.empty(E, N, K // 32, dtype=u8, device=dev)))
            moe_quantize_mxfp4_rows(E * N, K, w, t[0], t[1], stream=stream)
            return t

        self.gate, self.up, self.down = quant(w_gate, I, H), quant(w_up, I, H), quant(w_down, H, I)


def moe_gemm_down_bwd(s, do_perm, a, offsets, w_down, g, u, dgu, dw_down, accumulate_dw, ws, ws_bytes=None,
                      stream=None):
    nb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("moe_gemm_down_bwd", lib.moe_gemm_down_bwd(s, _ptr(do_perm), _ptr(a), _ptr(offsets), _ptr(w_down), _ptr(g),
                                                      _ptr(u), _ptr(dgu), _ptr(dw_down), int(accumulate_dw), _ptr(ws),
                                                      nb, _stream(stream)))


def moe_gemm_gate_up_bwd(s, dgu, x_rows, row_token, offsets, w_gate, w_up, dx_perm, dw_gate, dw_up, accumulate_dw, ws,
                         ws_bytes=None, stream=None):
    """row_token None: x_rows is x_perm; else x [T,H] read through row_token."""
    nb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("moe_gemm_gate_up_bwd",
           lib.moe_gemm_gate_up_bwd(s, _ptr(dgu), _ptr(x_rows), _ptr(row_token), _ptr(offsets), _ptr(w_gate),
                                    _ptr(w_up), _ptr(dx_perm), _ptr(dw_gate), _ptr(dw_up), int(accumulate_dw),
                                    _ptr(ws), nb, _stream(stream)))


def moe_gemm_gate_up_wgrad_gathered(s, dgu, x, row_token, offsets, dw_gate, dw_up, accumulate_dw, ws, ws_bytes=None,
                                    stream=None):
    nb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("moe_gemm_gate_up_wgrad_gathered",
           lib.moe_gemm_gate_up_wgrad_gathered(s, _ptr(dgu), _ptr(x), _ptr(row_token), _ptr(offsets), _ptr(dw_gate),
                                               _ptr(dw_up), int(accumulate_dw), _ptr(ws), nb, _stream(stream)))


def moe_gemm_down_weighted(s, a, offsets, w_down, row_weight, o_perm, stream=None):
    _check("moe_gemm_down_weighted", lib.moe_gemm_down_weighted(s, _ptr(a), _ptr(offsets), _ptr(w_down),
                                                                _ptr(row_weight), _ptr(o_perm), _stream(stream)))


def moe_forward_fused(s, x, w_router, logit_bias, w_gate, w_up, w_down, logits, topk_idx, topk_w, counts, offsets,
                      sorted_to_flat, flat_to_sorted, row_token, row_weight, a, o_perm, y, ws, ws_bytes=None,
                      stream=None):
    nb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("moe_forward_fused", lib.moe_forward_fused(
        s, _ptr(x), _ptr(w_router), _ptr(logit_bias), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(logits),
        _ptr(topk_idx), _ptr(topk_w), _ptr(counts), _ptr(offsets), _ptr(sorted_to_flat), _ptr(flat_to_sorted),
        _ptr(row_token), _ptr(row_weight), _ptr(a), _ptr(o_perm), _ptr(y), _ptr(ws), nb, _stream(stream)))


def moe_permute_rows(s, topk_idx, topk_w, x, counts, offsets, sorted_to_flat, flat_to_sorted, row_token, row_weight,
                     x_perm, ws, ws_bytes=None, stream=None):
    nb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("moe_permute_rows", lib.moe_permute_rows(
        s, _ptr(topk_idx), _ptr(topk_w), _ptr(x), _ptr(counts), _ptr(offsets), _ptr(sorted_to_flat),
        _ptr(flat_to_sorted), _ptr(row_token), _ptr(row_weight), _ptr(x_perm), _ptr(ws), nb, _stream(stream)))


def moe_gemm_gate_up_aw(s, x_rows, row_token, row_weight, offsets, w_gate, w_up, g, u, a, a_w, stream=None):
    _check("moe_gemm_gate_up_aw", lib.moe_gemm_gate_up_aw(
        s, _ptr(x_rows), _ptr(row_token), _ptr(row_weight), _ptr(offsets), _ptr(w_gate), _ptr(w_up), _ptr(g), _ptr(u),
        _ptr(a), _ptr(a_w), _stream(stream)))


def moe_gemm_down_bwd_dy(s, dy, row_token, row_weight, a_w, offsets, w_down, g, u, dgu, dw_down, accumulate_dw, ws,
                         ws_bytes=None, stream=None):
    nb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("moe_gemm_down_bwd_dy", lib.moe_gemm_down_bwd_dy(
        s, _ptr(dy), _ptr(row_token), _ptr(row_weight), _ptr(a_w), _ptr(offsets), _ptr(w_down), _ptr(g), _ptr(u),
        _ptr(dgu), _ptr(dw_down), int(accumulate_dw), _ptr(ws), nb, _stream(stream)))


def moe_forward_fused_noalloc(s, x, w_router, logit_bias, w_gate, w_up, w_down, logits, topk_idx, topk_w, counts,
                              offsets, sorted_to_flat, flat_to_sorted, row_token, row_weight, a, o_perm, y,
                              stream=None):
    _check("moe_forward_fused_noalloc", lib.moe_forward_fused_noalloc(
        s, _ptr(x), _ptr(w_router), _ptr(logit_bias), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(logits),
        _ptr(topk_idx), _ptr(topk_w), _ptr(counts), _ptr(offsets), _ptr(sorted_to_flat), _ptr(flat_to_sorted),
        _ptr(row_token), _ptr(row_weight), _ptr(a), _ptr(o_perm), _ptr(y), _stream(stream)))


def moe_lora_workspace_bytes(s: moe_shape, r: int) -> int:
    return int(lib.moe_lora_workspace_bytes(s, r))


def moe_lora_merge(E, N, K, r, scale, w, a, b, w_out, stream=None):
    _check("moe_lora_merge", lib.moe_lora_merge(E, N, K, r, float(scale), _ptr(w), _ptr(a), _ptr(b), _ptr(w_out),
                                                _stream(stream)))


def moe_lora_merge_fp8(E, N, K, r, scale, wq, w_e8, a, b, w_out, stream=None):
    _check("moe_lora_merge_fp8", lib.moe_lora_merge_fp8(E, N, K, r, ctypes.c_float(scale), _ptr(wq), _ptr(w_e8), _ptr(a),
                                                        _ptr(b), _ptr(w_out), _stream(stream)))


def _merge_any(E, N, K, r, scale, w, a, b, w_out, stream=None):
    """moe_lora_merge for a bf16 frozen weight, moe_lora_merge_mxfp4 for an
    MXFP4Tensor (MXFP4Weights.gate / .up / .down), moe_lora_merge_fp8 for an
    (E4M3 codes, E8M0 row scales) pair (FP8Weights.gate / .up / .down)."""
    if isinstance(w, MXFP4Tensor):
        moe_lora_merge_mxfp4(E, N, K, r, scale, w[0], w[1], a, b, w_out, stream)
    elif isinstance(w, tuple):
        moe_lora_merge_fp8(E, N, K, r, scale, w[0], w[1], a, b, w_out, stream)
    else:
        moe_lora_merge(E, N, K, r, scale, w, a, b, w_out, stream)


def moe_lora_grads(s, r, scale, x_perm, act, dgu, do_perm, offsets, a_gate, b_gate, a_up, b_up, a_down, b_down,
                   da_gate, db_gate, da_up, db_up, da_down, db_down, ws, ws_bytes=None, stream=None):
    nb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("moe_lora_grads", lib.moe_lora_grads(
        s, r, float(scale), _ptr(x_perm), _ptr(act), _ptr(dgu), _ptr(do_perm), _ptr(offsets), _ptr(a_gate),
        _ptr(b_gate), _ptr(a_up), _ptr(b_up), _ptr(a_down), _ptr(b_down), _ptr(da_gate), _ptr(db_gate), _ptr(da_up),
        _ptr(db_up), _ptr(da_down), _ptr(db_down), _ptr(ws), nb, _stream(stream)))


def _nbytes(ws, ws_bytes):
    return ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes


def moe_lora_unmerged_workspace_bytes(s: moe_shape, r: int) -> int:
    return int(lib.moe_lora_unmerged_workspace_bytes(s, r))


def moe_lora_prepare(s, r, scale, a_gate, b_gate, a_up, b_up, a_down, b_down, ws, ws_bytes=None, stream=None):
    _check("moe_lora_prepare", lib.moe_lora_prepare(
        s, r, ctypes.c_float(scale), *[_ptr(t) for t in (a_gate, b_gate, a_up, b_up, a_down, b_down, ws)],
        _nbytes(ws, ws_bytes), _stream(stream)))


def moe_lora_gemm_gate_up(s, r, x_perm, offsets, w_gate, w_up, b_gate, b_up, g, u, a, ws, ws_bytes=None,
                          stream=None):
    _check("moe_lora_gemm_gate_up", lib.moe_lora_gemm_gate_up(
        s, r, *[_ptr(t) for t in (x_perm, offsets, w_gate, w_up, b_gate, b_up, g, u, a, ws)],
        _nbytes(ws, ws_bytes), _stream(stream)))


def moe_lora_gemm_down(s, r, a, offsets, w_down, b_down, o_perm, ws, ws_bytes=None, stream=None):
    _check("moe_lora_gemm_down", lib.moe_lora_gemm_down(
        s, r, *[_ptr(t) for t in (a, offsets, w_down, b_down, o_perm, ws)], _nbytes(ws, ws_bytes), _stream(stream)))


def moe_lora_gemm_down_dgrad(s, r, do_perm, offsets, w_down, a_down, g, u, dgu, ws, ws_bytes=None, stream=None):
    _check("moe_lora_gemm_down_dgrad", lib.moe_lora_gemm_down_dgrad(
        s, r, *[_ptr(t) for t in (do_perm, offsets, w_down, a_down, g, u, dgu, ws)], _nbytes(ws, ws_bytes),
        _stream(stream)))


def moe_lora_gemm_gate_up_dgrad(s, r, dgu, offsets, w_gate, w_up, a_gate, a_up, dx_perm, ws, ws_bytes=None,
                                stream=None):
    _check("moe_lora_gemm_gate_up_dgrad", lib.moe_lora_gemm_gate_up_dgrad(
        s, r, *[_ptr(t) for t in (dgu, offsets, w_gate, w_up, a_gate, a_up, dx_perm, ws)], _nbytes(ws, ws_bytes),
        _stream(stream)))


def moe_lora_grads_unmerged(s, r, x_perm, act, dgu, do_perm, offsets, da_gate, db_gate, da_up, db_up, da_down,
                            db_down, ws, ws_bytes=None, stream=None):
    _check("moe_lora_grads_unmerged", lib.moe_lora_grads_unmerged(
        s, r, *[_ptr(t) for t in (x_perm, act, dgu, do_perm, offsets, da_gate, db_gate, da_up, db_up, da_down,
                                  db_down, ws)], _nbytes(ws, ws_bytes), _stream(stream)))


def moe_lora_gemm_gate_up_gathered(s, r, x, row_token, offsets, w_gate, w_up, b_gate, b_up, g, u, a, ws,
                                   ws_bytes=None, stream=None):
    _check("moe_lora_gemm_gate_up_gathered", lib.moe_lora_gemm_gate_up_gathered(
        s, r, *[_ptr(t) for t in (x, row_token, offsets, w_gate, w_up, b_gate, b_up, g, u, a, ws)],
        _nbytes(ws, ws_bytes), _stream(stream)))


def moe_lora_gemm_down_dgrad_dy(s, r, dy, row_token, row_weight, offsets, w_down, a_down, g, u, dgu, ws,
                                ws_bytes=None, stream=None):
    _check("moe_lora_gemm_down_dgrad_dy", lib.moe_lora_gemm_down_dgrad_dy(
        s, r, *[_ptr(t) for t in (dy, row_token, row_weight, offsets, w_down, a_down, g, u, dgu, ws)],
        _nbytes(ws, ws_bytes), _stream(stream)))


def moe_lora_grads_unmerged_gathered(s, r, x, row_token, row_weight, act, dgu, dy, offsets, da_gate, db_gate, da_up,
                                     db_up, da_down, db_down, ws, ws_bytes=None, stream=None):
    _check("moe_lora_grads_unmerged_gathered", lib.moe_lora_grads_unmerged_gathered(
        s, r, *[_ptr(t) for t in (x, row_token, row_weight, act, dgu, dy, offsets, da_gate, db_gate, da_up, db_up,
                                  da_down, db_down, ws)], _nbytes(ws, ws_bytes), _stream(stream)))


def moe_lora_grads_gathered(s, r, scale, x, row_token, row_weight, act, dgu, dy, offsets, a_gate, b_gate, a_up,
                            b_up, a_down, b_down, da_gate, db_gate, da_up, db_up, da_down, db_down, ws, ws_bytes=None,
                            stream=None):
    nb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("moe_lora_grads_gathered", lib.moe_lora_grads_gathered(
        s, r, float(scale), _ptr(x), _ptr(row_token), _ptr(row_weight), _ptr(act), _ptr(dgu), _ptr(dy), _ptr(offsets),
        _ptr(a_gate), _ptr(b_gate), _ptr(a_up), _ptr(b_up), _ptr(a_down), _ptr(b_down), _ptr(da_gate), _ptr(db_gate),
        _ptr(da_up), _ptr(db_up), _ptr(da_down), _ptr(db_down), _ptr(ws), nb, _stream(stream)))


def moe_gemm_down_dgrad_dy(s, dy, row_token, row_weight, offsets, w_down, g, u, dgu, stream=None):
    _check("moe_gemm_down_dgrad_dy", lib.moe_gemm_down_dgrad_dy(
        s, _ptr(dy), _ptr(row_token), _ptr(row_weight), _ptr(offsets), _ptr(w_down), _ptr(g), _ptr(u), _ptr(dgu),
        _stream(stream)))


class MoEStage:
    """Buffers and call order of one MoE layer's expert stage on one GPU.

    ``weights``: x-independent tensors on the device: w_router [E,H],
    w_gate/w_up [E,I,H], w_down [E,H,I] (dtype), optional logit_bias [E]
    float32. ``forward(x)`` and ``backward(dy)`` enqueue the library calls on
    the current stream and return views of the held buffers (overwritten by
    the next call).

    ``gather_fused``: no x_perm. The sort also gives each sorted row's token
    (moe_permute_fused), and the two GEMMs that read x rows (gate/up and its
    weight gradient) read them from x through it. Same results, bit for bit.

    ``dy_fused`` (bf16): no do_perm. The forward's gate/up GEMM also writes
    the weighted activations a_w (moe_gemm_gate_up_aw), the combine backward
    writes d_topk_w only, and the down backward reads dy through the sorted
    rows' tokens (moe_gemm_down_bwd_dy). The same mathematics with the
    routing weight applied at another point: within tolerance of the oracle,
    not bit-identical to the do_perm path. Not combined with aux_stream.
    """

    def __init__(self, T: int, H: int, E: int, k: int, I: int, dtype: torch.dtype, device="cuda",
                 gather_fused: bool = False, dy_fused: bool = False):
        self.T, self.H, self.E, self.k, self.I, self.dtype = T, H, E, k, I, dtype
        self.gather_fused = gather_fused
        self.dy_fused = dy_fused
        if dy_fused and dtype != torch.bfloat16:
            raise ValueError("dy_fused needs bf16")
        self.weight_grads = True  # dw_* buffers (the adapter stage trains no frozen weight)
        self.s = shape(T, H, E, k, I, dtype)
        M = T * k
        dev = torch.device(device)
        f32, i32 = torch.float32, torch.int32
        e = lambda *sz, dt=dtype: torch.empty(*sz, dtype=dt, device=dev)  # noqa: E731
        self.buf: Dict[str, torch.Tensor] = {
            "logits": e(T, E, dt=f32), "topk_idx": e(T, k, dt=i32), "topk_w": e(T, k, dt=f32),
            "counts": e(E, dt=i32), "offsets": e(E + 1, dt=i32), "sorted_to_flat": e(M, dt=i32),
            "flat_to_sorted": e(M, dt=i32), "g": e(M, I), "u": e(M, I), "a": e(M, I),
            "o_perm": e(M, H), "y": e(T, H),
        }
        if gather_fused or dy_fused:
            self.buf.update({"row_token": e(M, dt=i32), "row_weight": e(M, dt=f32)})
        if not gather_fused:
            self.buf["x_perm"] = e(M, H)
        if dy_fused:
            self.buf["a_w"] = e(M, I)
        ws_bytes = moe_workspace_bytes(self.s)
        if ws_bytes == 0:
            raise MoEError("moe_workspace_bytes", 1, "shape rejected")
        self.ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        self._bwd_ready = False

    def _alloc_bwd(self):
        if self._bwd_ready:
            return
        T, H, E, k, I, dt = self.T, self.H, self.E, self.k, self.I, self.dtype
        dev = self.ws.device
        M = T * k
        f32 = torch.float32
        if not self.dy_fused and not getattr(self, "gathered", False):
            self.buf["do_perm"] = torch.empty(M, H, dtype=dt, device=dev)
        self.buf.update({
            "d_topk_w": torch.empty(T, k, dtype=f32, device=dev),
            "dx_perm": torch.empty(M, H, dtype=dt, device=dev), "dx": torch.empty(T, H, dtype=dt, device=dev),
            "d_logits": torch.empty(T, E, dtype=f32, device=dev),
        })
        if self.weight_grads:
            self.buf.update({
                "dw_gate": torch.empty(E, I, H, dtype=f32, device=dev),
                "dw_up": torch.empty(E, I, H, dtype=f32, device=dev),
                "dw_down": torch.empty(E, H, I, dtype=f32, device=dev),
            })
        self._bwd_ready = True

    def forward(self, x, w_router, w_gate, w_up, w_down, logit_bias=None, stream=None):
        b, s = self.buf, self.s
        self.w = (w_gate, w_up, w_down)
        self.x = x
        moe_route(s, x, w_router, logit_bias, b["logits"], b["topk_idx"], b["topk_w"], stream)
        if self.dy_fused:
            if self.gather_fused:
                moe_permute_fused(s, b["topk_idx"], b["topk_w"], b["counts"], b["offsets"], b["sorted_to_flat"],
                                  b["flat_to_sorted"], b["row_token"], b["row_weight"], self.ws, stream=stream)
                moe_gemm_gate_up_aw(s, x, b["row_token"], b["row_weight"], b["offsets"], w_gate, w_up, b["g"],
                                    b["u"], b["a"], b["a_w"], stream)
            else:
                moe_permute_rows(s, b["topk_idx"], b["topk_w"], x, b["counts"], b["offsets"], b["sorted_to_flat"],
                                 b["flat_to_sorted"], b["row_token"], b["row_weight"], b["x_perm"], self.ws,
                                 stream=stream)
                moe_gemm_gate_up_aw(s, b["x_perm"], None, b["row_weight"], b["offsets"], w_gate, w_up, b["g"],
                                    b["u"], b["a"], b["a_w"], stream)
            moe_gemm_down(s, b["a"], b["offsets"], w_down, b["o_perm"], stream)
        elif self.gather_fused:
            moe_permute_fused(s, b["topk_idx"], b["topk_w"], b["counts"], b["offsets"], b["sorted_to_flat"],
                              b["flat_to_sorted"], b["row_token"], b["row_weight"], self.ws, stream=stream)
            moe_gemm_gate_up_gathered(s, x, b["row_token"], b["offsets"], w_gate, w_up, b["g"], b["u"], b["a"],
                                      stream)
            moe_gemm_down(s, b["a"], b["offsets"], w_down, b["o_perm"], stream)
        else:
            moe_permute(s, b["topk_idx"], x, b["counts"], b["offsets"], b["sorted_to_flat"], b["flat_to_sorted"],
                        b["x_perm"], self.ws, stream=stream)
            moe_grouped_gemm_fwd(s, b["x_perm"], b["offsets"], w_gate, w_up, w_down, b["g"], b["u"], b["a"],
                                 b["o_perm"], stream=stream)
        moe_combine(s, b["o_perm"], b["topk_w"], b["flat_to_sorted"], b["y"], stream)
        return b["y"]

    def backward(self, dy, accumulate_dw: bool = False, stream=None, aux_stream=None):
        """Backward of the last forward. By default each data-gradient GEMM
        and the weight gradient that reads the same inputs run in one launch
        (moe_gemm_down_bwd, moe_gemm_gate_up_bwd). With ``aux_stream`` (a
        second stream, default priority) the six GEMMs run one per launch,
        the weight gradients there and the data gradients on ``stream``. The
        results are the same bits either way."""
        self._alloc_bwd()
        b, s = self.buf, self.s
        w_gate, w_up, w_down = self.w
        moe_combine_bwd(s, dy, b["o_perm"], b["topk_w"], b["flat_to_sorted"], b.get("do_perm"), b["d_topk_w"],
                        stream)
        acc = int(accumulate_dw)
        if self.dy_fused:
            if aux_stream is not None:
                raise ValueError("dy_fused runs the backward on one stream")
            if "dgu" not in b:
                b["dgu"] = torch.empty(self.T * self.k, 2 * self.I, dtype=self.dtype, device=self.ws.device)
            moe_gemm_down_bwd_dy(s, dy, b["row_token"], b["row_weight"], b["a_w"], b["offsets"], w_down, b["g"],
                                 b["u"], b["dgu"], b["dw_down"], acc, self.ws, stream=stream)
            if self.gather_fused:
                moe_gemm_gate_up_bwd(s, b["dgu"], self.x, b["row_token"], b["offsets"], w_gate, w_up, b["dx_perm"],
                                     b["dw_gate"], b["dw_up"], acc, self.ws, stream=stream)
            else:
                moe_gemm_gate_up_bwd(s, b["dgu"], b["x_perm"], None, b["offsets"], w_gate, w_up, b["dx_perm"],
                                     b["dw_gate"], b["dw_up"], acc, self.ws, stream=stream)
        elif aux_stream is None and not self.gather_fused:
            moe_grouped_gemm_bwd(s, b["do_perm"], b["x_perm"], b["g"], b["u"], b["a"], b["offsets"], w_gate, w_up,
                                 w_down, b["dx_perm"], b["dw_gate"], b["dw_up"], b["dw_down"], acc, self.ws,
                                 stream=stream)
        elif aux_stream is None:
            if "dgu" not in b:
                b["dgu"] = torch.empty(self.T * self.k, 2 * self.I, dtype=self.dtype, device=self.ws.device)
            moe_gemm_down_bwd(s, b["do_perm"], b["a"], b["offsets"], w_down, b["g"], b["u"], b["dgu"], b["dw_down"],
                              acc, self.ws, stream=stream)
            moe_gemm_gate_up_bwd(s, b["dgu"], self.x, b["row_token"], b["offsets"], w_gate, w_up, b["dx_perm"],
                                 b["dw_gate"], b["dw_up"], acc, self.ws, stream=stream)
        else:
            main = torch.cuda.current_stream() if stream is None else stream
            if "dgu" not in b:
                b["dgu"] = torch.empty(self.T * self.k, 2 * self.I, dtype=self.dtype, device=self.ws.device)
            forked = torch.cuda.Event()
            forked.record(main)
            aux_stream.wait_event(forked)
            moe_gemm_down_wgrad(s, b["do_perm"], b["a"], b["offsets"], b["dw_down"], acc, self.ws, stream=aux_stream)
            moe_gemm_down_dgrad(s, b["do_perm"], b["offsets"], w_down, b["g"], b["u"], b["dgu"], main)
            dgu_ready = torch.cuda.Event()
            dgu_ready.record(main)
            aux_stream.wait_event(dgu_ready)
            if self.gather_fused:
                moe_gemm_gate_up_wgrad_gathered(s, b["dgu"], self.x, b["row_token"], b["offsets"], b["dw_gate"],
                                                b["dw_up"], acc, self.ws, stream=aux_stream)
            else:
                moe_gemm_gate_up_wgrad(s, b["dgu"], b["x_perm"], b["offsets"], b["dw_gate"], b["dw_up"], acc,
                                       self.ws, stream=aux_stream)
            moe_gemm_gate_up_dgrad(s, b["dgu"], b["offsets"], w_gate, w_up, b["dx_perm"], main)
            joined = torch.cuda.Event()
            joined.record(aux_stream)
            main.wait_event(joined)
        moe_unpermute_sum(s, b["dx_perm"], b["flat_to_sorted"], b["dx"], stream)
        moe_route_bwd(s, b["d_topk_w"], b["topk_w"], b["topk_idx"], b["d_logits"], stream)
        return b["dx"]


LORA_NAMES = ("a_gate", "b_gate", "a_up", "b_up", "a_down", "b_down")


class LoRAStage(MoEStage):
    """The stage with low-rank adapters on frozen experts.

    ``forward(x, w_router, w_gate, w_up, w_down, adapters)`` merges each
    projection (moe_lora_merge into held W' buffers) and runs the plain
    forward on W'; ``backward(dy)`` runs the data gradients on W' and
    moe_lora_grads, and returns dx. The adapter gradients (float32) are in
    ``buf["d" + name]``; the frozen weights get none. ``adapters``: a_P
    [E,r,K], b_P [E,N,r] bf16 for P in gate, up, down. Each frozen weight is
    a bf16 tensor or, kept in 8 or 4 bits (QLoRA-style), the (E4M3 codes,
    E8M0 row scales) pair of FP8Weights or the MXFP4Tensor of MXFP4Weights
    (moe_lora_merge_fp8 or moe_lora_merge_mxfp4 dequantises it).

    ``gathered``: neither x_perm nor do_perm. The forward reads x through the
    sorted rows' tokens (moe_permute_fused, moe_gemm_gate_up_gathered); the
    backward's down data gradient reads dy through them and applies the
    routing weight (moe_gemm_down_dgrad_dy), and the adapter gradients read x
    and dy through them (moe_lora_grads_gathered). Within rounding of the
    default chain. Not combined with the forward's aux_stream.

    ``unmerged``: no W' at all (bf16 frozen weights only). moe_lora_prepare
    stacks the adapters; every GEMM runs over its reduction extended by the
    rank (moe_lora_gemm_gate_up, moe_lora_gemm_down, moe_lora_gemm_down_dgrad,
    moe_lora_gemm_gate_up_dgrad), and moe_lora_grads_unmerged takes the
    adapter gradients from the row projections those calls kept. Within
    rounding of the merged chain. With ``gathered`` as well, the gathered
    calls (moe_lora_gemm_gate_up_gathered, moe_lora_gemm_down_dgrad_dy,
    moe_lora_grads_unmerged_gathered) build neither x_perm nor do_perm.
    """

    def __init__(self, T: int, H: int, E: int, k: int, I: int, rank: int, scale: float, device="cuda",
                 gathered: bool = False, unmerged: bool = False):
        super().__init__(T, H, E, k, I, torch.bfloat16, device=device, gather_fused=gathered)
        self.gathered, self.unmerged = gathered, unmerged
        self.weight_grads = False
        self.rank, self.scale = rank, scale
        nb = (moe_lora_unmerged_workspace_bytes if unmerged else moe_lora_workspace_bytes)(self.s, rank)
        if nb == 0:
            raise MoEError("moe_lora_workspace_bytes", 2, "shape or rank rejected")
        dev = self.ws.device
        self.lora_ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        bf = torch.bfloat16
        self.merged = None if unmerged else (
            torch.empty(E, I, H, dtype=bf, device=dev), torch.empty(E, I, H, dtype=bf, device=dev),
            torch.empty(E, H, I, dtype=bf, device=dev))
        f32 = torch.float32
        self.buf.update({
            "da_gate": torch.empty(E, rank, H, dtype=f32, device=dev), "db_gate": torch.empty(E, I, rank, dtype=f32,
                                                                                            device=dev),
            "da_up": torch.empty(E, rank, H, dtype=f32, device=dev), "db_up": torch.empty(E, I, rank, dtype=f32,
                                                                                        device=dev),
            "da_down": torch.empty(E, rank, I, dtype=f32, device=dev), "db_down": torch.empty(E, H, rank, dtype=f32,
                                                                                            device=dev),
            "dgu": torch.empty(T * k, 2 * I, dtype=bf, device=dev),
        })

    def merge(self, w_gate, w_up, w_down, adapters, stream=None):
        if self.unmerged:
            raise ValueError("LoRAStage(unmerged=True) holds no merged weights")
        E, H, I, r = self.E, self.H, self.I, self.rank
        wg, wu, wd = self.merged
        _merge_any(E, I, H, r, self.scale, w_gate, adapters["a_gate"], adapters["b_gate"], wg, stream)
        _merge_any(E, I, H, r, self.scale, w_up, adapters["a_up"], adapters["b_up"], wu, stream)
        _merge_any(E, H, I, r, self.scale, w_down, adapters["a_down"], adapters["b_down"], wd, stream)
        return self.merged

    def forward(self, x, w_router, w_gate, w_up, w_down, adapters, logit_bias=None, stream=None, aux_stream=None):
        """With ``aux_stream`` (a second stream, default priority) the three
        merges run there, concurrently with the routing and the sort on
        ``stream``; gate/up waits for its two merges and down for its own.
        The results are the same bits either way."""
        self.adapters = adapters
        if self.unmerged:
            if aux_stream is not None:
                raise ValueError("the unmerged adapter step has no merges to move to a second stream")
            return self._forward_unmerged(x, w_router, w_gate, w_up, w_down, adapters, logit_bias, stream)
        if aux_stream is None:
            wg, wu, wd = self.merge(w_gate, w_up, w_down, adapters, stream)
            return super().forward(x, w_router, wg, wu, wd, logit_bias, stream)
        if self.gathered:
            raise ValueError("the gathered adapter step runs its merges on the forward's stream")
        E, H, I, r = self.E, self.H, self.I, self.rank
        wg, wu, wd = self.merged
        main = torch.cuda.current_stream() if stream is None else stream
        forked = torch.cuda.Event()
        forked.record(main)
        aux_stream.wait_event(forked)
        _merge_any(E, I, H, r, self.scale, w_gate, adapters["a_gate"], adapters["b_gate"], wg, aux_stream)
        _merge_any(E, I, H, r, self.scale, w_up, adapters["a_up"], adapters["b_up"], wu, aux_stream)
        gu_ready = torch.cuda.Event()
        gu_ready.record(aux_stream)
        _merge_any(E, H, I, r, self.scale, w_down, adapters["a_down"], adapters["b_down"], wd, aux_stream)
        d_ready = torch.cuda.Event()
        d_ready.record(aux_stream)
        b, s = self.buf, self.s
        self.w = (wg, wu, wd)
        self.x = x
        moe_route(s, x, w_router, logit_bias, b["logits"], b["topk_idx"], b["topk_w"], main)
        moe_permute(s, b["topk_idx"], x, b["counts"], b["offsets"], b["sorted_to_flat"], b["flat_to_sorted"],
                    b["x_perm"], self.ws, stream=main)
        main.wait_event(gu_ready)
        moe_gemm_gate_up(s, b["x_perm"], b["offsets"], wg, wu, b["g"], b["u"], b["a"], main)
        main.wait_event(d_ready)
        moe_gemm_down(s, b["a"], b["offsets"], wd, b["o_perm"], main)
        moe_combine(s, b["o_perm"], b["topk_w"], b["flat_to_sorted"], b["y"], main)
        return b["y"]

    def _forward_unmerged(self, x, w_router, w_gate, w_up, w_down, adapters, logit_bias, stream):
        b, s, r, lw = self.buf, self.s, self.rank, self.lora_ws
        if not all(isinstance(w, torch.Tensor) and w.dtype == torch.bfloat16 for w in (w_gate, w_up, w_down)):
            raise TypeError("the unmerged adapter step takes bf16 frozen weights")
        self.w = (w_gate, w_up, w_down)
        self.x = x
        moe_lora_prepare(s, r, self.scale, *(adapters[n] for n in LORA_NAMES), lw, stream=stream)
        moe_route(s, x, w_router, logit_bias, b["logits"], b["topk_idx"], b["topk_w"], stream)
        if self.gathered:
            moe_permute_fused(s, b["topk_idx"], b["topk_w"], b["counts"], b["offsets"], b["sorted_to_flat"],
                              b["flat_to_sorted"], b["row_token"], b["row_weight"], self.ws, stream=stream)
            moe_lora_gemm_gate_up_gathered(s, r, x, b["row_token"], b["offsets"], w_gate, w_up, adapters["b_gate"],
                                           adapters["b_up"], b["g"], b["u"], b["a"], lw, stream=stream)
        else:
            moe_permute(s, b["topk_idx"], x, b["counts"], b["offsets"], b["sorted_to_flat"], b["flat_to_sorted"],
                        b["x_perm"], self.ws, stream=stream)
            moe_lora_gemm_gate_up(s, r, b["x_perm"], b["offsets"], w_gate, w_up, adapters["b_gate"],
                                  adapters["b_up"], b["g"], b["u"], b["a"], lw, stream=stream)
        moe_lora_gemm_down(s, r, b["a"], b["offsets"], w_down, adapters["b_down"], b["o_perm"], lw, stream=stream)
        moe_combine(s, b["o_perm"], b["topk_w"], b["flat_to_sorted"], b["y"], stream)
        return b["y"]

    def backward(self, dy, stream=None):
        self._alloc_bwd()
        b, s = self.buf, self.s
        if self.unmerged:
            wg, wu, wd = self.w
            r, lw = self.rank, self.lora_ws
            ad = self.adapters
            if self.gathered:
                moe_combine_bwd(s, dy, b["o_perm"], b["topk_w"], b["flat_to_sorted"], None, b["d_topk_w"], stream)
                moe_lora_gemm_down_dgrad_dy(s, r, dy, b["row_token"], b["row_weight"], b["offsets"], wd, ad["a_down"],
                                            b["g"], b["u"], b["dgu"], lw, stream=stream)
            else:
                moe_combine_bwd(s, dy, b["o_perm"], b["topk_w"], b["flat_to_sorted"], b["do_perm"], b["d_topk_w"],
                                stream)
                moe_lora_gemm_down_dgrad(s, r, b["do_perm"], b["offsets"], wd, ad["a_down"], b["g"], b["u"], b["dgu"],
                                         lw, stream=stream)
            moe_lora_gemm_gate_up_dgrad(s, r, b["dgu"], b["offsets"], wg, wu, ad["a_gate"], ad["a_up"], b["dx_perm"],
                                        lw, stream=stream)
            if self.gathered:
                moe_lora_grads_unmerged_gathered(s, r, self.x, b["row_token"], b["row_weight"], b["a"], b["dgu"], dy,
                                                 b["offsets"], *(b["d" + n] for n in LORA_NAMES), lw, stream=stream)
            else:
                moe_lora_grads_unmerged(s, r, b["x_perm"], b["a"], b["dgu"], b["do_perm"], b["offsets"],
                                        *(b["d" + n] for n in LORA_NAMES), lw, stream=stream)
            moe_unpermute_sum(s, b["dx_perm"], b["flat_to_sorted"], b["dx"], stream)
            moe_route_bwd(s, b["d_topk_w"], b["topk_w"], b["topk_idx"], b["d_logits"], stream)
            return b["dx"]
        wg, wu, wd = self.merged
        ad = self.adapters
        if self.gathered:
            moe_combine_bwd(s, dy, b["o_perm"], b["topk_w"], b["flat_to_sorted"], None, b["d_topk_w"], stream)
            moe_gemm_down_dgrad_dy(s, dy, b["row_token"], b["row_weight"], b["offsets"], wd, b["g"], b["u"], b["dgu"],
                                   stream)
            moe_gemm_gate_up_dgrad(s, b["dgu"], b["offsets"], wg, wu, b["dx_perm"], stream)
            moe_lora_grads_gathered(s, self.rank, self.scale, self.x, b["row_token"], b["row_weight"], b["a"],
                                    b["dgu"], dy, b["offsets"], *(ad[n] for n in LORA_NAMES),
                                    *(b["d" + n] for n in LORA_NAMES), self.lora_ws, stream=stream)
        else:
            moe_combine_bwd(s, dy, b["o_perm"], b["topk_w"], b["flat_to_sorted"], b["do_perm"], b["d_topk_w"],
                            stream)
            moe_gemm_down_dgrad(s, b["do_perm"], b["offsets"], wd, b["g"], b["u"], b["dgu"], stream)
            moe_gemm_gate_up_dgrad(s, b["dgu"], b["offsets"], wg, wu, b["dx_perm"], stream)
            moe_lora_grads(s, self.rank, self.scale, b["x_perm"], b["a"], b["dgu"], b["do_perm"], b["offsets"],
                           *(ad[n] for n in LORA_NAMES), *(b["d" + n] for n in LORA_NAMES), self.lora_ws,
                           stream=stream)
        moe_unpermute_sum(s, b["dx_perm"], b["flat_to_sorted"], b["dx"], stream)
        moe_route_bwd(s, b["d_topk_w"], b["topk_w"], b["topk_idx"], b["d_logits"], stream)
        return b["dx"]
