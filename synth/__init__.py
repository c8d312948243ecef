"""Seeded synthetic inputs for the sparse MoE FFN layer.

This module only draws random numbers and stores them in the layer's input
formats (fp32, bf16, MXFP4).  It holds none of the layer's arithmetic: it is
the one module the oracle side and the HIP side share, so both see the same
bytes.

Workloads (the shapes of the serving deployments the pages discuss: decode
batches of at most 8 rows -- "第 9 章 prefill：最大的瓶颈" §9.5 and §9.8 --
and 8192-token prefill chunks -- the same chapter, §9.8):

  c0  tiny fp32:  T=4, H=256, E=8, top-2, I=128
  c1  decode T=1 bf16:  H=2048, E=128, top-8, I=768
  c2  decode T=8 bf16, router bias ~ N(0, 0.5) so tokens share experts
  c3  prefill T=8192 bf16, Zipf(1) expert popularity through the router bias
  c4  MXFP4 experts (E2M1, 32-element blocks, E8M0 scales), bf16 activations:
      H=4096, E=256, top-8, I=1024, at T=1, T=8 and T=4096
  c5  the same with NVFP4 experts; c6 the same with MXINT8 experts (OCP MX INT8:
      int8 elements with an implicit 2^-6, 32-element blocks, E8M0 scales)

Distributions: x ~ N(0,1); router W ~ N(0, 0.02); expert W ~ N(0, 1/sqrt(fan_in))
with fan_in = H for gate/up and I for down (the second parameter is the
standard deviation).  Draws are fp64 from numpy's PCG64, one independent
stream per (seed, tensor, expert or batch index), then rounded to fp32 (RNE)
and, for bf16 tensors, to bf16 (RNE); MXFP4 tensors are quantised from the
fp32 draws (OCP MX: shared scale 2^(floor(log2 amax) - 2), elements rounded
to nearest-even on the E2M1 grid, saturating at 6).  The stored bytes are the
truth for both sides.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

# tensor tags of the independent PCG64 streams
_TAGS = {"x": 1, "wr": 2, "bias": 3, "wg": 4, "wu": 5, "wd": 6, "perm": 7}

# Zipf temperature of the c3 router bias b[e] = beta * ln(p_e), p_e ~ rank_e^-1.
# beta = 1 is the plain reading of "Zipf(s=1.0)"; at seed 0 it leaves no expert
# empty, so beta is raised in 0.05 steps until one is (recorded, with the
# histogram, by tests/golden/make_zipf_beta.py in tests/golden/zipf_beta.json).
ZIPF_BETA = 1.05


@dataclass(frozen=True)
class Shape:
    T: int
    H: int
    E: int
    K: int
    I: int
    act: str          # "f32" | "bf16"
    w: str            # "f32" | "bf16" | "mxfp4" | "nvfp4" | "mxint8"
    bias: str = "none"  # "none" | "normal" | "zipf"
    renorm: bool = True


CONFIGS: Dict[str, Shape] = {
    "c0_tiny_f32": Shape(4, 256, 8, 2, 128, "f32", "f32"),
    "c1_decode1_bf16": Shape(1, 2048, 128, 8, 768, "bf16", "bf16"),
    "c2_decode8_bf16": Shape(8, 2048, 128, 8, 768, "bf16", "bf16", bias="normal"),
    "c3_prefill8192_bf16": Shape(8192, 2048, 128, 8, 768, "bf16", "bf16", bias="zipf"),
    # the prefill chunk with 8 decode rows appended: one call carries both
    "c3_mixed8200_bf16": Shape(8200, 2048, 128, 8, 768, "bf16", "bf16", bias="zipf"),
    "c4_mxfp4_decode1": Shape(1, 4096, 256, 8, 1024, "bf16", "mxfp4"),
    "c4_mxfp4_decode8": Shape(8, 4096, 256, 8, 1024, "bf16", "mxfp4"),
    "c4_mxfp4_prefill4096": Shape(4096, 4096, 256, 8, 1024, "bf16", "mxfp4"),
    # the MXFP4 decode shapes with NVFP4 experts (E4M3 scales per 16 elements)
    "c5_nvfp4_decode1": Shape(1, 4096, 256, 8, 1024, "bf16", "nvfp4"),
    "c5_nvfp4_decode8": Shape(8, 4096, 256, 8, 1024, "bf16", "nvfp4"),
    "c5_nvfp4_prefill4096": Shape(4096, 4096, 256, 8, 1024, "bf16", "nvfp4"),
    # the same shapes with MXINT8 experts (OCP MX INT8: int8 codes, E8M0 scale per 32)
    "c6_mxint8_decode1": Shape(1, 4096, 256, 8, 1024, "bf16", "mxint8"),
    "c6_mxint8_decode8": Shape(8, 4096, 256, 8, 1024, "bf16", "mxint8"),
    "c6_mxint8_prefill4096": Shape(4096, 4096, 256, 8, 1024, "bf16", "mxint8"),
}


def _rng(seed: int, tag: str, sub: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _TAGS[tag], sub])))


def normal(seed: int, tag: str, shape, sigma: float, sub: int = 0) -> np.ndarray:
    """fp64 N(0, sigma) draws of one stream."""
    return _rng(seed, tag, sub).standard_normal(shape) * sigma


# ---- storage formats ---------------------------------------------------------

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# E2M1 grid magnitudes by code 0..7
_E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], np.float64)


def _e2m1_code_rne(m: np.ndarray) -> np.ndarray:
    """Magnitude (already divided by the power-of-two block scale, so exact, >= 0) ->
    nearest E2M1 code with ties to the even code, saturating at 6 (code 7).

    The grid has step 0.5 on [0, 2), 1 on [2, 4) and 2 on [4, 6]; on each piece the
    code index is an affine function of m whose parity is the code's, so numpy's
    round-half-even (rint) gives ties-to-even codes."""
    m = np.minimum(m, np.float32(6.0))
    c_lo = np.rint(m * np.float32(2.0))
    c_mid = np.float32(4.0) + np.rint(m - np.float32(2.0))
    c_hi = np.float32(6.0) + np.rint((m - np.float32(4.0)) * np.float32(0.5))
    return np.where(m < 2, c_lo, np.where(m < 4, c_mid, c_hi)).astype(np.uint8)


def mxfp4_quantize(w: np.ndarray):
    """Quantise fp32 rows [R, C] (C % 32 == 0) to MXFP4 along C.

    Returns (codes [R, C/2] uint8 with the even element in the low nibble,
    scales [R, C/32] uint8 E8M0).  Block scale X = 2^(floor(log2 amax) - 2); an
    all-zero block gets scale code 0 and zero codes.
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    R, C = w.shape
    assert C % 32 == 0
    blk = w.reshape(R, C // 32, 32)
    amax = np.abs(blk).max(axis=2)
    _, ex = np.frexp(amax)                   # amax = f * 2^ex, f in [0.5, 1): floor(log2 amax) = ex - 1
    e = ex.astype(np.int64) - 1 - 2
    nz = amax > 0
    scale_code = np.where(nz, np.clip(e + 127, 0, 254), 0).astype(np.uint8)
    X = np.ldexp(np.float32(1.0), scale_code.astype(np.int32) - 127).astype(np.float32)[..., None]
    mag = np.abs(blk) / X                    # exact: X is a power of two
    code = _e2m1_code_rne(mag) | np.where(blk < 0, np.uint8(8), np.uint8(0))
    code = np.where(nz[..., None], code, np.uint8(0)).reshape(R, C)
    packed = (code[:, 0::2] & 15) | ((code[:, 1::2] & 15) << 4)
    return packed.astype(np.uint8), scale_code


def mxfp4_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Inverse storage map used by tests on the quantiser: fp64 [R, C]."""
    R = codes.shape[0]
    c = np.empty((R, codes.shape[1] * 2), np.uint8)
    c[:, 0::2] = codes & 15
    c[:, 1::2] = codes >> 4
    mag = _E2M1_GRID[c & 7]
    val = np.where(c & 8, -mag, mag)
    X = np.ldexp(1.0, scales.astype(np.int64) - 127)
    return val * np.repeat(X, 32, axis=1)


def mxint8_quantize(w: np.ndarray):
    """Quantise fp32 rows [R, C] (C % 32 == 0) to MXINT8 along C (OCP MX v1.0 INT8: an
    element is a two's complement int8 with an implicit scale of 2^-6, i.e. code / 64).

    Block scale X = 2^floor(log2 amax) (the INT8 element's largest power of two is 2^0);
    codes = v / X * 64 rounded to nearest even and clamped to [-127, 127].  An all-zero
    block gets scale code 0 and zero codes.  Returns (codes [R, C] int8, scales
    [R, C/32] uint8 E8M0).
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    R, C = w.shape
    assert C % 32 == 0
    blk = w.reshape(R, C // 32, 32)
    amax = np.abs(blk).max(axis=2)
    _, ex = np.frexp(amax)                   # floor(log2 amax) = ex - 1
    e = ex.astype(np.int64) - 1
    nz = amax > 0
    scale_code = np.where(nz, np.clip(e + 127, 0, 254), 0).astype(np.uint8)
    X = np.ldexp(np.float64(1.0), scale_code.astype(np.int32) - 127)[..., None]
    q = np.rint(blk.astype(np.float64) / X * 64.0)   # exact scaling, then ties to even
    q = np.clip(q, -127, 127)
    q = np.where(nz[..., None], q, 0).astype(np.int8).reshape(R, C)
    return q, scale_code


def mxint8_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Inverse storage map used by tests on the quantiser: fp64 [R, C]."""
    X = np.ldexp(1.0, scales.astype(np.int64) - 127)
    return codes.astype(np.float64) / 64.0 * np.repeat(X, 32, axis=1)


# NVFP4 (E2M1 codes, one E4M3 scale per 16 elements, one fp32 scale per tensor).
# Positive finite E4M3 values by code 0x00..0x7E (0x7F is NaN): exponent field 0 is
# m/8 * 2^-6, otherwise (1 + m/8) * 2^(e-7).  Ascending in the code.
_E4M3_POS = np.array([(c & 7) / 8.0 * 2.0 ** -6 if (c >> 3) == 0 else (1.0 + (c & 7) / 8.0) * 2.0 ** ((c >> 3) - 7)
                      for c in range(0x7F)], np.float64)


def nvfp4_tensor_scale(sigma: float) -> float:
    """The tensor scale the generator uses for N(0, sigma) weights: the block scales of
    blocks up to 6.5 sigma then stay within E4M3's 448."""
    return float(np.float32(sigma * 6.5 / (6.0 * 448.0)))


def nvfp4_quantize(w: np.ndarray, ts: float):
    """Quantise fp32 rows [R, C] (C % 16 == 0) to NVFP4 along C with tensor scale ts.

    Block scale: the E4M3 value nearest to amax / 6 / ts (at most 448); codes: nearest
    E2M1 value of w / (scale * ts), ties to even, saturating at 6.  An all-zero block
    gets scale code 0 and zero codes.  Returns (codes [R, C/2] uint8, even element in the
    low nibble; scales [R, C/16] uint8)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    R, C = w.shape
    assert C % 16 == 0
    blk = w.reshape(R, C // 16, 16)
    amax = np.abs(blk).max(axis=2).astype(np.float64)
    target = np.minimum(amax / 6.0 / ts, _E4M3_POS[-1])
    hi = np.clip(np.searchsorted(_E4M3_POS, target), 1, len(_E4M3_POS) - 1)
    lo = hi - 1
    pick_hi = (_E4M3_POS[hi] - target) < (target - _E4M3_POS[lo])
    scode = np.where(pick_hi, hi, lo)
    scode = np.where(amax > 0, np.maximum(scode, 1), 0).astype(np.uint8)
    S = (_E4M3_POS[scode] * ts)[..., None]
    mag = np.where(S > 0, np.abs(blk) / np.where(S > 0, S, 1.0), 0.0).astype(np.float32)
    code = _e2m1_code_rne(mag) | np.where(blk < 0, np.uint8(8), np.uint8(0))
    code = np.where((amax > 0)[..., None], code, np.uint8(0)).reshape(R, C)
    packed = (code[:, 0::2] & 15) | ((code[:, 1::2] & 15) << 4)
    return packed.astype(np.uint8), scode


def nvfp4_dequantize(codes: np.ndarray, scales: np.ndarray, ts: float) -> np.ndarray:
    """Inverse storage map used by tests on the quantiser: fp64 [R, C]."""
    R = codes.shape[0]
    c = np.empty((R, codes.shape[1] * 2), np.uint8)
    c[:, 0::2] = codes & 15
    c[:, 1::2] = codes >> 4
    mag = _E2M1_GRID[c & 7]
    val = np.where(c & 8, -mag, mag)
    return val * np.repeat(_E4M3_POS[scales] * ts, 16, axis=1)


# ---- tensors of one layer ------------------------------------------------------

@dataclass
class LayerInputs:
    shape: Shape
    x: np.ndarray            # [T,H] float32 or uint16 (bf16 bits)
    wr: np.ndarray           # [E,H]
    bias: Optional[np.ndarray]
    wg: np.ndarray
    wu: np.ndarray
    wd: np.ndarray
    sg: Optional[np.ndarray] = None
    su: Optional[np.ndarray] = None
    sd: Optional[np.ndarray] = None
    meta: dict = field(default_factory=dict)
    ts: tuple = (1.0, 1.0, 1.0)      # NVFP4 tensor scales of gate, up, down


def _store(a64: np.ndarray, fmt: str) -> np.ndarray:
    a32 = a64.astype(np.float32)
    if fmt == "f32":
        return a32
    if fmt == "bf16":
        return f32_to_bf16_bits(a32)
    raise ValueError(fmt)


def make_x(shape: Shape, seed: int = 0, batch: int = 0) -> np.ndarray:
    return _store(normal(seed, "x", (shape.T, shape.H), 1.0, sub=batch), shape.act)


def make_bias(shape: Shape, seed: int = 0, beta: Optional[float] = None) -> Optional[np.ndarray]:
    if shape.bias == "none":
        return None
    if shape.bias == "normal":
        return normal(seed, "bias", (shape.E,), 0.5).astype(np.float32)
    if shape.bias == "zipf":
        beta = ZIPF_BETA if beta is None else beta
        ranks = _rng(seed, "perm").permutation(shape.E) + 1          # a seeded ranking 1..E
        p = 1.0 / ranks
        p = p / p.sum()
        return (beta * np.log(p)).astype(np.float32)
    raise ValueError(shape.bias)


def _expert_tensor(shape: Shape, seed: int, tag: str, rows: int, cols: int, sigma: float,
                   threads: int):
    E = shape.E
    ts = nvfp4_tensor_scale(sigma)
    if shape.w in ("mxfp4", "nvfp4"):
        codes = np.empty((E, rows, cols // 2), np.uint8)
        scales = np.empty((E, rows, cols // (32 if shape.w == "mxfp4" else 16)), np.uint8)
    elif shape.w == "mxint8":
        codes = np.empty((E, rows, cols), np.int8)
        scales = np.empty((E, rows, cols // 32), np.uint8)
    else:
        out = np.empty((E, rows, cols), np.float32 if shape.w == "f32" else np.uint16)

    def one(e):
        a32 = normal(seed, tag, (rows, cols), sigma, sub=e).astype(np.float32)
        if shape.w == "mxfp4":
            codes[e], scales[e] = mxfp4_quantize(a32)
        elif shape.w == "nvfp4":
            codes[e], scales[e] = nvfp4_quantize(a32, ts)
        elif shape.w == "mxint8":
            codes[e], scales[e] = mxint8_quantize(a32)
        elif shape.w == "bf16":
            out[e] = f32_to_bf16_bits(a32)
        else:
            out[e] = a32

    if threads > 1 and E > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, range(E)))
    else:
        for e in range(E):
            one(e)
    if shape.w in ("mxfp4", "nvfp4", "mxint8"):
        return codes, scales
    return out, None


def make_layer(name_or_shape, seed: int = 0, batch: int = 0, threads: Optional[int] = None,
               beta: Optional[float] = None, **overrides) -> LayerInputs:
    """All tensors of one layer.  Expert and router weights depend only on (seed, shape
    without T); x depends on (seed, batch, T)."""
    shape = CONFIGS[name_or_shape] if isinstance(name_or_shape, str) else name_or_shape
    if overrides:
        shape = Shape(**{**shape.__dict__, **overrides})
    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    H, I = shape.H, shape.I
    x = make_x(shape, seed, batch)
    wr = _store(normal(seed, "wr", (shape.E, H), 0.02), shape.act)
    bias = make_bias(shape, seed, beta)
    wg, sg = _expert_tensor(shape, seed, "wg", I, H, 1.0 / math.sqrt(H), threads)
    wu, su = _expert_tensor(shape, seed, "wu", I, H, 1.0 / math.sqrt(H), threads)
    wd, sd = _expert_tensor(shape, seed, "wd", H, I, 1.0 / math.sqrt(I), threads)
    meta = dict(seed=seed, batch=batch, zipf_beta=(ZIPF_BETA if beta is None else beta)
                if shape.bias == "zipf" else None)
    ts = (1.0, 1.0, 1.0)
    if shape.w == "nvfp4":
        ts = (nvfp4_tensor_scale(1.0 / math.sqrt(H)), nvfp4_tensor_scale(1.0 / math.sqrt(H)),
              nvfp4_tensor_scale(1.0 / math.sqrt(I)))
    return LayerInputs(shape, x, wr, bias, wg, wu, wd, sg, su, sd, meta, ts)
