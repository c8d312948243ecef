"""The seeded input generator: determinism, storage rounding and the MXFP4
quantiser's defining properties (OCP MX v1.0).  CPU only."""
import json
import os

import numpy as np
import pytest
import torch

import synth

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0,
                                  3.0e38, 1e-40], np.float32)])
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.f32_to_bf16_bits(a), ref)
    # ties to even by hand: 1 + 2^-8 sits halfway between 1 and 1 + 2^-7
    assert synth.f32_to_bf16_bits(np.array([1.0 + 2 ** -8], np.float32))[0] == 0x3F80
    assert synth.f32_to_bf16_bits(np.array([1.0 + 3 * 2 ** -8], np.float32))[0] == 0x3F82


def test_generator_deterministic_and_T_independent():
    a = synth.make_layer("c0_tiny_f32")
    b = synth.make_layer("c0_tiny_f32")
    for n in ("x", "wr", "wg", "wu", "wd"):
        assert np.array_equal(getattr(a, n), getattr(b, n))
    c = synth.make_layer("c0_tiny_f32", T=9)
    for n in ("wr", "wg", "wu", "wd"):
        assert np.array_equal(getattr(a, n), getattr(c, n))
    d = synth.make_layer("c0_tiny_f32", batch=1)
    assert not np.array_equal(a.x, d.x)
    e = synth.make_layer("c0_tiny_f32", seed=1)
    assert not np.array_equal(a.wg, e.wg)


def test_generator_moments():
    li = synth.make_layer(synth.Shape(64, 512, 4, 2, 256, "f32", "f32"))
    assert abs(li.x.std() - 1.0) < 0.02
    assert abs(li.wr.std() - 0.02) < 0.001
    assert abs(li.wg.std() - 1 / np.sqrt(512)) < 0.002
    assert abs(li.wd.std() - 1 / np.sqrt(256)) < 0.002


GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_mxfp4_representable_roundtrip():
    rng = np.random.default_rng(2)
    vals = np.array(GRID + [-g for g in GRID[1:]])
    rows = []
    for s in (-9, -3, 0, 4):
        blk = rng.choice(vals, size=32) * 2.0 ** s
        blk[0] = 6.0 * 2.0 ** s                  # amax 6 * 2^s -> scale 2^s
        rows.append(blk)
    w = np.array(rows, np.float32)
    c, sc = synth.mxfp4_quantize(w)
    assert list(sc[:, 0]) == [127 - 9, 127 - 3, 127, 131]
    assert np.array_equal(synth.mxfp4_dequantize(c, sc), w.astype(np.float64))


@pytest.mark.parametrize("v,expect", [(0.25, 0.0), (0.75, 1.0), (1.25, 1.0), (1.75, 2.0),
                                      (2.5, 2.0), (3.5, 4.0), (5.0, 4.0), (7.0, 6.0), (-2.5, -2.0)])
def test_mxfp4_ties_to_even_and_saturation(v, expect):
    blk = np.zeros((1, 32), np.float32)
    blk[0, 0] = 4.0                              # amax 4 -> scale code 127 (X = 1)
    blk[0, 1] = v
    if abs(v) > 6.0:
        blk[0, 0] = 6.0
        blk[0, 2] = 4.0
    c, sc = synth.mxfp4_quantize(blk)
    X = 2.0 ** (int(sc[0, 0]) - 127)
    got = synth.mxfp4_dequantize(c, sc)[0, 1]
    if abs(v) > 6.0:
        # amax 7 -> scale 2^(floor(log2 7) - 2) = 1, 7 saturates to 6
        assert X == 1.0
    assert got == expect * X


def test_mxfp4_scale_formula_and_error_bound():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    c, sc = synth.mxfp4_quantize(w)
    blk = w.reshape(64, 8, 32).astype(np.float64)
    amax = np.abs(blk).max(axis=2)
    X = 2.0 ** (sc.astype(np.int64) - 127)
    # X = 2^(floor(log2 amax) - 2): amax / X lies in [4, 8)
    r = amax / X
    assert np.all((r >= 4) & (r < 8))
    deq = synth.mxfp4_dequantize(c, sc).reshape(64, 8, 32)
    err = np.abs(deq - blk)
    mag = np.abs(blk) / X[..., None]
    # grid step is 0.5 below 2, 1 below 4, 2 above; error <= half a step unless saturated
    step = np.where(mag < 2, 0.5, np.where(mag < 4, 1.0, 2.0))
    sat = mag > 6
    assert np.all(err[~sat] <= 0.5 * (step * X[..., None])[~sat] + 1e-30)
    assert np.all(np.abs(deq[sat]) == 6 * np.broadcast_to(X[..., None], deq.shape)[sat])


def test_mxfp4_zero_block():
    w = np.zeros((2, 64), np.float32)
    w[1, 40] = 1.0
    c, sc = synth.mxfp4_quantize(w)
    assert sc[0, 0] == 0 and sc[0, 1] == 0 and sc[1, 0] == 0 and np.all(c[0] == 0)
    assert sc[1, 1] == 125                         # amax 1 -> 2^(0-2)
    assert synth.mxfp4_dequantize(c, sc)[1, 40] == 1.0


def test_zipf_beta_matches_record():
    with open(os.path.join(GOLD, "zipf_beta.json")) as f:
        rec = json.load(f)
    assert rec["beta"] == synth.ZIPF_BETA
    h = np.array(rec["histogram"])
    assert h.sum() == 8192 * 8 and (h == 0).any() and (h > 2000).any()


def test_mxint8_quantiser():
    """The generator's MXINT8 quantiser (OCP MX INT8): block scale 2^floor(log2 amax), codes
    the nearest multiple of X/64 (ties to even) clamped to +-127, so every stored value is
    within half a step of its input unless clamped; representable values round-trip; an
    all-zero block gets scale code 0 and zero codes."""
    rng = np.random.default_rng(9)
    w = (rng.standard_normal((6, 96)) * 0.03).astype(np.float32)
    w[2, 32:64] = 0.0
    codes, scales = synth.mxint8_quantize(w)
    assert codes.dtype == np.int8 and scales.dtype == np.uint8 and codes.shape == w.shape
    assert scales[2, 1] == 0 and np.all(codes[2, 32:64] == 0)
    blk = np.abs(w.reshape(6, 3, 32)).max(axis=2)
    nz = blk > 0
    assert np.all(np.ldexp(1.0, scales[nz].astype(int) - 127) <= blk[nz])
    assert np.all(blk[nz] < np.ldexp(2.0, scales[nz].astype(int) - 127))
    d = synth.mxint8_dequantize(codes, scales)
    step = np.repeat(np.ldexp(1.0, scales.astype(int) - 127 - 6), 32, axis=1)
    assert np.all(codes >= -127) and np.all(codes <= 127)
    clamped = np.abs(codes) == 127
    assert np.all(np.abs(d - w)[~clamped] <= 0.5 * step[~clamped] + 1e-12)
    # values on the grid come back exactly; a value just under 2 X clamps to 127/64 X
    grid = np.array([[0.5, -0.25, 1.984375, -1.0] + [1.0] * 28], np.float32)
    c2, s2 = synth.mxint8_quantize(grid)
    assert s2[0, 0] == 127 and np.array_equal(synth.mxint8_dequantize(c2, s2), grid.astype(np.float64))
    c3, _ = synth.mxint8_quantize(np.array([[1.999] + [0.0] * 31], np.float32))
    assert c3[0, 0] == 127
    # ties to even: 0.5/64 and 1.5/64 above an exact grid value of a block with X = 1
    c4, s4 = synth.mxint8_quantize(np.array([[1.0, 1.0 / 128, 3.0 / 128, -1.0 / 128] + [0.0] * 28], np.float32))
    assert s4[0, 0] == 127 and list(c4[0, :4]) == [64, 0, 2, 0]
