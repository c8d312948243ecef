"""Python binding of the gfx950 MoE layer library (libmoe_router.so).

Argument marshalling only: every step of the layer runs in the HIP kernels
behind the C ABI declared in include/moe_router.h.  torch is used for device
memory and streams; no torch op touches the layer's arithmetic.  If the
library is missing, importing the binding's entry points raises -- there is
no fallback.

Routing follows the stage list of the fused MoE profiling plan ("Decode
吞吐专项实验分析报告", subsection "下一步 profiling 方向": gate, topk, expert
kernel, activation, sum) and the device-side grouping of "第 9 章 prefill：
最大的瓶颈" §9.9.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_router.so")

# status codes
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_DEVICE = 0, -1, -2, -3, -4, -5
# element formats
F32, BF16, MXFP4, NVFP4, MXINT8 = 0, 1, 2, 3, 4
# expert FFN kernel family
PATH_AUTO, PATH_DECODE, PATH_GROUPED = 0, 1, 2
# device error bits
DEVERR_BAD_EXPERT_ID, DEVERR_TIMEOUT = 1, 2

EXPORTS = ["moe_workspace_size", "moe_router_topk", "moe_group_tokens", "moe_expert_ffn", "moe_combine",
           "moe_forward", "moe_forward_timed", "moe_forward_stages", "moe_forward_grouping",
           "moe_check_device_error", "moe_status_string", "moe_forward_noalloc"]


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


class Shape(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("hidden", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("intermediate", ctypes.c_int32), ("renormalize", ctypes.c_int32),
                ("act_dtype", ctypes.c_int32), ("weight_dtype", ctypes.c_int32), ("path", ctypes.c_int32)]


class ExpertWeights(ctypes.Structure):
    _fields_ = [("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
                ("s_gate", ctypes.c_void_p), ("s_up", ctypes.c_void_p), ("s_down", ctypes.c_void_p),
                ("ts_gate", ctypes.c_float), ("ts_up", ctypes.c_float), ("ts_down", ctypes.c_float)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe_router.so (built by prefill_moe_router_amd/build.py); raises if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with prefill_moe_router_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
        PS, PW = ctypes.POINTER(Shape), ctypes.POINTER(ExpertWeights)
        L.moe_workspace_size.restype = sz
        L.moe_workspace_size.argtypes = [PS]
        L.moe_router_topk.restype = i32
        L.moe_router_topk.argtypes = [PS, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_group_tokens.restype = i32
        L.moe_group_tokens.argtypes = [PS, vp, vp, vp, vp, vp, sz, vp]
        L.moe_expert_ffn.restype = i32
        L.moe_expert_ffn.argtypes = [PS, vp, PW, vp, vp, vp, vp, sz, vp]
        L.moe_combine.restype = i32
        L.moe_combine.argtypes = [PS, vp, vp, vp, vp, vp]
        L.moe_forward.restype = i32
        L.moe_forward.argtypes = [PS, vp, vp, vp, PW, vp, vp, vp, vp, sz, vp]
        L.moe_forward_timed.restype = i32
        L.moe_forward_timed.argtypes = [PS, vp, vp, vp, PW, vp, vp, vp, vp, sz, vp, ctypes.POINTER(vp), i32]
        L.moe_forward_stages.restype = ctypes.c_char_p
        L.moe_forward_stages.argtypes = [PS]
        L.moe_forward_grouping.restype = i32
        L.moe_forward_grouping.argtypes = [PS, vp, sz, vp, vp, vp, vp]
        L.moe_forward_noalloc.restype = i32
        L.moe_forward_noalloc.argtypes = [PS, vp, vp, vp, PW, vp, vp, vp, vp, vp]
        L.moe_check_device_error.restype = i32
        L.moe_check_device_error.argtypes = [vp, ctypes.POINTER(i32), vp]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [i32]
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def _check(status: int, what: str):
    if status != OK:
        raise MoeError(status, what)


@dataclass
class LayerShape:
    num_tokens: int
    hidden: int
    num_experts: int
    top_k: int
    intermediate: int
    renormalize: bool = True
    act_dtype: int = BF16
    weight_dtype: int = BF16
    path: int = PATH_AUTO

    def c(self) -> Shape:
        return Shape(self.num_tokens, self.hidden, self.num_experts, self.top_k, self.intermediate,
                     int(bool(self.renormalize)), self.act_dtype, self.weight_dtype, self.path)


def _p(t) -> Optional[int]:
    """Device address of a tensor (None -> NULL)."""
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def workspace_size(shape: LayerShape) -> int:
    s = shape.c()
    return int(lib().moe_workspace_size(ctypes.byref(s)))


def alloc_workspace(shape: LayerShape, device="cuda"):
    """Zero-filled uint8 workspace tensor of the size the shape needs."""
    import torch
    n = workspace_size(shape)
    if n == 0:
        raise MoeError(ERR_INVALID_ARG, "workspace_size")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def _weights(wg, wu, wd, sg=None, su=None, sd=None, ts=(1.0, 1.0, 1.0)) -> ExpertWeights:
    """ts: the NVFP4 tensor scales of gate, up and down (ignored for other formats)."""
    return ExpertWeights(_p(wg), _p(wu), _p(wd), _p(sg), _p(su), _p(sd), float(ts[0]), float(ts[1]), float(ts[2]))


def router_topk(shape: LayerShape, x, w_router, bias, topk_ids, topk_w, ws, stream=None):
    s = shape.c()
    _check(lib().moe_router_topk(ctypes.byref(s), _p(x), _p(w_router), _p(bias), _p(topk_ids), _p(topk_w),
                                 _p(ws), ws.numel(), _stream(stream)), "moe_router_topk")


def group_tokens(shape: LayerShape, topk_ids, expert_offsets, sorted_slots, slot_pos, ws, stream=None):
    s = shape.c()
    _check(lib().moe_group_tokens(ctypes.byref(s), _p(topk_ids), _p(expert_offsets), _p(sorted_slots),
                                  _p(slot_pos), _p(ws), ws.numel(), _stream(stream)), "moe_group_tokens")


def expert_ffn(shape: LayerShape, x, weights: dict, expert_offsets, sorted_slots, expert_out, ws, stream=None):
    s = shape.c()
    w = _weights(**weights)
    _check(lib().moe_expert_ffn(ctypes.byref(s), _p(x), ctypes.byref(w), _p(expert_offsets), _p(sorted_slots),
                                _p(expert_out), _p(ws), ws.numel(), _stream(stream)), "moe_expert_ffn")


def combine(shape: LayerShape, expert_out, topk_w, slot_pos, y, stream=None):
    s = shape.c()
    _check(lib().moe_combine(ctypes.byref(s), _p(expert_out), _p(topk_w), _p(slot_pos), _p(y),
                             _stream(stream)), "moe_combine")


def forward(shape: LayerShape, x, w_router, bias, weights: dict, y, ws, topk_ids=None, topk_w=None,
            stream=None):
    s = shape.c()
    w = _weights(**weights)
    _check(lib().moe_forward(ctypes.byref(s), _p(x), _p(w_router), _p(bias), ctypes.byref(w), _p(y),
                             _p(topk_ids), _p(topk_w), _p(ws), ws.numel(), _stream(stream)), "moe_forward")


NOALLOC_SCRATCH_BYTES = 16 << 20


def forward_noalloc(shape: LayerShape, x, w_router, bias, weights: dict, y, topk_ids=None, topk_w=None,
                    device_err=None, stream=None):
    """moe_forward on the library's own per-device scratch (no workspace argument)."""
    s = shape.c()
    w = _weights(**weights)
    _check(lib().moe_forward_noalloc(ctypes.byref(s), _p(x), _p(w_router), _p(bias), ctypes.byref(w), _p(y),
                                     _p(topk_ids), _p(topk_w), _p(device_err), _stream(stream)),
           "moe_forward_noalloc")


def forward_timed(shape: LayerShape, x, w_router, bias, weights: dict, y, ws, stage_events, topk_ids=None,
                  topk_w=None, stream=None):
    """moe_forward recording stage_events[i] (hipEvent_t handles or None) before launch i and
    after the last launch."""
    s = shape.c()
    w = _weights(**weights)
    arr = (ctypes.c_void_p * max(1, len(stage_events)))(*[e for e in stage_events])
    _check(lib().moe_forward_timed(ctypes.byref(s), _p(x), _p(w_router), _p(bias), ctypes.byref(w), _p(y),
                                   _p(topk_ids), _p(topk_w), _p(ws), ws.numel(), _stream(stream), arr,
                                   len(stage_events)), "moe_forward_timed")


def forward_stages(shape: LayerShape) -> list:
    s = shape.c()
    return lib().moe_forward_stages(ctypes.byref(s)).decode().split(",")


def forward_grouping(shape: LayerShape, ws, expert_offsets, sorted_slots, slot_pos, stream=None):
    """Copies the grouping the last forward on `ws` built into the given int32 tensors."""
    s = shape.c()
    _check(lib().moe_forward_grouping(ctypes.byref(s), _p(ws), ws.numel(), _p(expert_offsets), _p(sorted_slots),
                                      _p(slot_pos), _stream(stream)), "moe_forward_grouping")


def check_device_error(ws, stream=None) -> int:
    """Synchronising read-and-clear of the workspace's device error bits."""
    bits = ctypes.c_int32(0)
    st = lib().moe_check_device_error(_p(ws), ctypes.byref(bits), _stream(stream))
    if st not in (OK, ERR_DEVICE):
        raise MoeError(st, "moe_check_device_error")
    return int(bits.value)
