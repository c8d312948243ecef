"""fp64 CPU oracle of the sparse MoE FFN layer -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke entry point and the benchmark's CPU-baseline leg may
import this package.  The HIP library never calls it and shares no code with
it.  The arithmetic lives in moe_oracle.c; this module only marshals numpy
arrays into the C calls.

What is computed (per token t, experts kept k):
  s[e]   = b[e] + sum_h x[t,h] Wr[e,h]                          (router gate)
  S_t    = k largest s by (score desc, id asc); ids ascending    (topk)
  w      = softmax(s)[S_t], renormalised to sum 1 if renorm      (topk weights)
  a      = silu(Wg[e] x_t) * (Wu[e] x_t)                         (expert kernel, activation)
  y[t]   = sum_j w_j Wd[e_j] a_j                                  (sum)
following the stage list of the fused MoE profiling plan in "Decode 吞吐专项
实验分析报告" (subsection "下一步 profiling 方向") and the device-side expert
grouping of "第 9 章 prefill：最大的瓶颈" §9.9.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

F32, BF16, MXFP4, NVFP4, MXINT8 = 0, 1, 2, 3, 4


class _Layer(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int32), ("H", ctypes.c_int32), ("E", ctypes.c_int32),
        ("K", ctypes.c_int32), ("I", ctypes.c_int32), ("renorm", ctypes.c_int32),
        ("act_dtype", ctypes.c_int32), ("w_dtype", ctypes.c_int32),
        ("x", ctypes.c_void_p), ("wr", ctypes.c_void_p), ("bias", ctypes.c_void_p),
        ("wg", ctypes.c_void_p), ("wu", ctypes.c_void_p), ("wd", ctypes.c_void_p),
        ("sg", ctypes.c_void_p), ("su", ctypes.c_void_p), ("sd", ctypes.c_void_p),
        ("tsg", ctypes.c_double), ("tsu", ctypes.c_double), ("tsd", ctypes.c_double),
    ]


_lib = None


def lib():
    """Load liboracle.so, building it with gcc if it is absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        L.orc_decode_bf16.restype = ctypes.c_double
        L.orc_decode_bf16.argtypes = [ctypes.c_uint16]
        L.orc_decode_e2m1.restype = ctypes.c_double
        L.orc_decode_e2m1.argtypes = [ctypes.c_uint]
        L.orc_decode_e8m0.restype = ctypes.c_double
        L.orc_decode_e8m0.argtypes = [ctypes.c_uint8]
        L.orc_decode_int8.restype = ctypes.c_double
        L.orc_decode_int8.argtypes = [ctypes.c_uint8]
        L.orc_decode_e4m3.restype = ctypes.c_double
        L.orc_decode_e4m3.argtypes = [ctypes.c_uint8]
        L.orc_router.restype = ctypes.c_int
        L.orc_router.argtypes = [P(_Layer), ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.orc_group.restype = ctypes.c_int
        L.orc_group.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.orc_expert_pairs.restype = ctypes.c_int
        L.orc_expert_pairs.argtypes = [P(_Layer), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                       ctypes.c_void_p]
        L.orc_forward.restype = ctypes.c_int
        L.orc_forward.argtypes = [P(_Layer), ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_void_p]
        L.orc_num_threads.restype = ctypes.c_int
        L.orc_set_num_threads.restype = None
        L.orc_set_num_threads.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


@dataclass
class Layer:
    """Host arrays of one MoE layer in the stored formats.

    x [T,H] and wr [E,H]: float32, or uint16 holding bf16 bits.
    wg, wu [E,I,H] and wd [E,H,I]: float32, uint16 (bf16 bits), or for MXFP4
    uint8 packed codes [E,I,H/2] / [E,H,I/2] with uint8 E8M0 scales sg, su
    [E,I,H/32] and sd [E,H,I/32].  fmt="nvfp4": the same codes with uint8 E4M3
    scales [E,I,H/16] / [E,H,I/16] and the tensor scales ts (gate, up, down).
    MXINT8: int8 codes [E,I,H] / [E,H,I] (OCP MX INT8 elements, implicit scale
    2^-6) with uint8 E8M0 scales as for MXFP4.
    bias [E] float32 or None.
    """
    x: np.ndarray
    wr: np.ndarray
    wg: np.ndarray
    wu: np.ndarray
    wd: np.ndarray
    top_k: int
    renorm: bool = True
    bias: Optional[np.ndarray] = None
    sg: Optional[np.ndarray] = None
    su: Optional[np.ndarray] = None
    sd: Optional[np.ndarray] = None
    fmt: Optional[str] = None
    ts: tuple = (1.0, 1.0, 1.0)

    @property
    def act_dtype(self) -> int:
        return F32 if self.x.dtype == np.float32 else BF16

    @property
    def w_dtype(self) -> int:
        if self.wg.dtype == np.float32:
            return F32
        if self.wg.dtype == np.uint16:
            return BF16
        if self.wg.dtype == np.int8:
            return MXINT8
        return NVFP4 if self.fmt == "nvfp4" else MXFP4

    @property
    def dims(self):
        T, H = self.x.shape
        E = self.wr.shape[0]
        I = self.wd.shape[2] * (2 if self.w_dtype in (MXFP4, NVFP4) else 1)
        return T, H, E, self.top_k, I

    def _struct(self) -> _Layer:
        T, H, E, K, I = self.dims
        self._keep = [self.x, self.wr, self.bias, self.wg, self.wu, self.wd, self.sg, self.su, self.sd]
        return _Layer(T, H, E, K, I, int(bool(self.renorm)), self.act_dtype, self.w_dtype,
                      _ptr(self.x), _ptr(self.wr), _ptr(self.bias), _ptr(self.wg), _ptr(self.wu),
                      _ptr(self.wd), _ptr(self.sg), _ptr(self.su), _ptr(self.sd),
                      float(self.ts[0]), float(self.ts[1]), float(self.ts[2]))


def _tokens(layer: Layer, tokens):
    if tokens is None:
        return None, layer.dims[0]
    t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
    return t, int(t.size)


def router(layer: Layer, tokens=None, want_logits: bool = False):
    """Returns dict(ids [n,k] int32, w [n,k] f64, near [n] bool, gap [n] f64, logits [n,E] f64?)."""
    T, H, E, K, I = layer.dims
    tk, n = _tokens(layer, tokens)
    ids = np.zeros((n, K), np.int32)
    w = np.zeros((n, K), np.float64)
    near = np.zeros(n, np.uint8)
    gap = np.zeros(n, np.float64)
    logits = np.zeros((n, E), np.float64) if want_logits else None
    st = layer._struct()
    rc = lib().orc_router(ctypes.byref(st), _ptr(tk), n, _ptr(logits), _ptr(ids), _ptr(w), _ptr(near), _ptr(gap))
    if rc != 0:
        raise ValueError("oracle router rejected its arguments")
    out = dict(ids=ids, w=w, near=near.astype(bool), gap=gap)
    if want_logits:
        out["logits"] = logits
    return out


def group(ids: np.ndarray, num_experts: int):
    """Stable counting sort of slots t*k+j by expert: (offsets[E+1], sorted[P], slot_pos[P])."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, K = ids.shape
    off = np.zeros(num_experts + 1, np.int32)
    srt = np.zeros(T * K, np.int32)
    pos = np.zeros(T * K, np.int32)
    rc = lib().orc_group(T, K, num_experts, _ptr(ids), _ptr(off), _ptr(srt), _ptr(pos))
    if rc != 0:
        raise ValueError("expert id out of range")
    return off, srt, pos


def expert_pairs(layer: Layer, tokens, experts) -> np.ndarray:
    """o[p] = Wd[e_p] (silu(Wg[e_p] x_t) * (Wu[e_p] x_t)) for pairs (t_p, e_p), fp64 [P,H]."""
    tk = np.ascontiguousarray(np.asarray(tokens, np.int32))
    ek = np.ascontiguousarray(np.asarray(experts, np.int32))
    H = layer.dims[1]
    o = np.zeros((tk.size, H), np.float64)
    st = layer._struct()
    rc = lib().orc_expert_pairs(ctypes.byref(st), _ptr(tk), _ptr(ek), int(tk.size), _ptr(o))
    if rc != 0:
        raise ValueError("oracle expert_pairs rejected its arguments")
    return o


def forward(layer: Layer, tokens=None, forced_ids: Optional[np.ndarray] = None):
    """Whole layer for all tokens or a subset.  Returns dict(y [n,H] f64, ids, w, near, gap)."""
    T, H, E, K, I = layer.dims
    tk, n = _tokens(layer, tokens)
    fi = None
    if forced_ids is not None:
        fi = np.ascontiguousarray(forced_ids, dtype=np.int32).reshape(n, K)
    y = np.zeros((n, H), np.float64)
    ids = np.zeros((n, K), np.int32)
    w = np.zeros((n, K), np.float64)
    near = np.zeros(n, np.uint8)
    gap = np.zeros(n, np.float64)
    st = layer._struct()
    rc = lib().orc_forward(ctypes.byref(st), _ptr(tk), n, _ptr(fi), _ptr(y), _ptr(ids), _ptr(w),
                           _ptr(near), _ptr(gap))
    if rc != 0:
        raise ValueError("oracle forward rejected its arguments")
    return dict(y=y, ids=ids, w=w, near=near.astype(bool), gap=gap)


def decode_bf16(bits: int) -> float:
    return lib().orc_decode_bf16(bits)


def decode_e2m1(code: int) -> float:
    return lib().orc_decode_e2m1(code)


def decode_e8m0(code: int) -> float:
    return lib().orc_decode_e8m0(code)


def decode_int8(code: int) -> float:
    """OCP MX INT8 element value of a code byte (before the block scale)."""
    return lib().orc_decode_int8(code)


def decode_e4m3(code: int) -> float:
    return lib().orc_decode_e4m3(code)


def num_threads() -> int:
    return lib().orc_num_threads()


def set_num_threads(n: int) -> None:
    """Thread count of later oracle calls (OpenMP)."""
    lib().orc_set_num_threads(int(n))
