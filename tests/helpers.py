"""Shared test helpers: oracle wrapping of synthetic inputs, an independent
grouping-invariant checker, and the parity metrics."""
from __future__ import annotations

import numpy as np

import oracle
import synth


def oracle_layer(li: synth.LayerInputs, **kw) -> oracle.Layer:
    return oracle.Layer(x=li.x, wr=li.wr, wg=li.wg, wu=li.wu, wd=li.wd, top_k=kw.get("top_k", li.shape.K),
                        renorm=kw.get("renorm", li.shape.renorm), bias=li.bias,
                        sg=li.sg, su=li.su, sd=li.sd, fmt=li.shape.w if li.shape.w == "nvfp4" else None,
                        ts=li.ts)


def grouping_violations(ids: np.ndarray, E: int, off, srt, pos) -> list:
    """Check a grouping against its defining properties, written without the oracle:
    offsets are the exclusive prefix of the per-expert counts, every slot t*k+j appears
    exactly once, in the segment of its expert, in ascending slot order inside the
    segment, and slot_pos is the inverse permutation."""
    ids = np.asarray(ids).reshape(-1)
    off = np.asarray(off).reshape(-1)
    srt = np.asarray(srt).reshape(-1)
    pos = np.asarray(pos).reshape(-1)
    P = ids.size
    bad = []
    if off.size != E + 1:
        return [f"offsets has {off.size} entries, expected {E + 1}"]
    if off[0] != 0 or off[-1] != P:
        bad.append(f"offsets ends {off[0]}..{off[-1]}, expected 0..{P}")
    if np.any(np.diff(off) < 0):
        bad.append("offsets not monotone")
    counts = np.bincount(ids, minlength=E) if P else np.zeros(E, int)
    if not np.array_equal(np.diff(off), counts):
        bad.append("segment sizes differ from expert counts")
    if srt.size != P or pos.size != P:
        return bad + ["sorted/slot_pos size mismatch"]
    if P and not np.array_equal(np.sort(srt), np.arange(P)):
        bad.append("sorted_slots is not a permutation of the slots")
        return bad
    for e in range(E):
        seg = srt[off[e]:off[e + 1]] if off[e] <= off[e + 1] else np.array([], int)
        if seg.size and np.any(ids[seg] != e):
            bad.append(f"expert {e} segment holds foreign slots")
        if seg.size > 1 and np.any(np.diff(seg) <= 0):
            bad.append(f"expert {e} segment not in ascending slot order")
    if P and not np.array_equal(srt[pos], np.arange(P)):
        bad.append("slot_pos is not the inverse of sorted_slots")
    return bad


def rel_l2(a, ref) -> float:
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    n = np.linalg.norm(ref)
    return float(np.linalg.norm(a - ref) / (n if n > 0 else 1.0))


def max_abs(a, ref) -> float:
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(a - ref))) if a.size else 0.0


def decoded(a: np.ndarray) -> np.ndarray:
    """fp64 view of a stored fp32 or bf16 (uint16 bits) array, via numpy (not the oracle)."""
    if a.dtype == np.uint16:
        return synth.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)
