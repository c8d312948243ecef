"""Pins of the fp64 oracle against facts fixed outside it: format definitions,
hand-worked values, closed forms, invariants, library routines on special
cases and brute force on tiny inputs.  CPU only."""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import decoded, grouping_violations, oracle_layer

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _table(name):
    rows = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _f32_layer(rng, T, H, E, K, I, renorm=True, bias=True, wr_sigma=0.3):
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = (rng.standard_normal((E, H)) * wr_sigma).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32) if bias else None
    wg = (rng.standard_normal((E, I, H)) / math.sqrt(H)).astype(np.float32)
    wu = (rng.standard_normal((E, I, H)) / math.sqrt(H)).astype(np.float32)
    wd = (rng.standard_normal((E, H, I)) / math.sqrt(I)).astype(np.float32)
    return oracle.Layer(x=x, wr=wr, wg=wg, wu=wu, wd=wd, top_k=K, renorm=renorm, bias=b)


# ---- stored-format decoders ---------------------------------------------------------

def test_bf16_decode_exhaustive():
    """All 65,536 bf16 patterns against the IEEE binary32 reading of bits<<16."""
    L = oracle.lib()
    bits = np.arange(65536, dtype=np.uint32)
    ref = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    got = np.array([L.orc_decode_bf16(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # a few by hand
    assert oracle.decode_bf16(0x3F80) == 1.0
    assert oracle.decode_bf16(0xC000) == -2.0
    assert oracle.decode_bf16(0x3F01) == 1.0 / 2 + 2.0 ** -8
    assert math.isinf(oracle.decode_bf16(0x7F80))


def test_e2m1_table():
    for code, val in _table("e2m1_table.txt"):
        got = oracle.decode_e2m1(int(code))
        assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val)), code


def test_e8m0_table():
    for code, val in _table("e8m0_cases.txt"):
        got = oracle.decode_e8m0(int(code))
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val), code


# ---- router: logits, top-k, weights ------------------------------------------------

@pytest.mark.parametrize("seed", range(4))
def test_router_logits_match_numpy(seed):
    rng = np.random.default_rng(100 + seed)
    T, H, E = 5, 24, 7
    L = _f32_layer(rng, T, H, E, 3, 4)
    r = oracle.router(L, want_logits=True)
    ref = L.x.astype(np.float64) @ L.wr.astype(np.float64).T + L.bias.astype(np.float64)
    np.testing.assert_allclose(r["logits"], ref, rtol=1e-13, atol=1e-13)


def test_router_logits_bf16_dyadic_exact():
    """bf16 inputs on a dyadic grid: every product and partial sum is exact in fp64, so the
    logits equal the integer arithmetic result exactly."""
    rng = np.random.default_rng(7)
    T, H, E = 3, 32, 6
    xi = rng.integers(-8, 9, size=(T, H))          # x = xi / 4
    wi = rng.integers(-8, 9, size=(E, H))          # wr = wi / 8
    x = synth.f32_to_bf16_bits((xi / 4.0).astype(np.float32))
    wr = synth.f32_to_bf16_bits((wi / 8.0).astype(np.float32))
    z = np.zeros((E, 1, H), np.uint16)
    L = oracle.Layer(x=x, wr=wr, wg=z, wu=z, wd=np.zeros((E, H, 1), np.uint16), top_k=2)
    r = oracle.router(L, want_logits=True)
    exact = (xi @ wi.T) / 32.0
    assert np.array_equal(r["logits"], exact)


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_full_sort(seed):
    rng = np.random.default_rng(200 + seed)
    T, H, E, K = 9, 16, 11, 1 + seed % 5
    L = _f32_layer(rng, T, H, E, K, 4)
    r = oracle.router(L, want_logits=True)
    s = L.x.astype(np.float64) @ L.wr.astype(np.float64).T + L.bias
    for t in range(T):
        order = np.lexsort((np.arange(E), -s[t]))       # score desc, id asc
        assert list(r["ids"][t]) == sorted(order[:K].tolist())


def test_router_closed_forms():
    H, E = 8, 4
    z = np.zeros((E, 1, H), np.float32)
    zd = np.zeros((E, H, 1), np.float32)
    x = np.ones((1, H), np.float32)
    wr = np.zeros((E, H), np.float32)
    b = np.array([3, 2, 1, 0], np.float32)
    L = oracle.Layer(x=x, wr=wr, wg=z, wu=z, wd=zd, top_k=2, renorm=True, bias=b)
    r = oracle.router(L)
    assert list(r["ids"][0]) == [0, 1]
    np.testing.assert_allclose(r["w"][0], [0.7310585786300049, 0.2689414213699951], rtol=1e-15)
    L.renorm = False
    r = oracle.router(L)
    np.testing.assert_allclose(r["w"][0], [0.6439142598879722, 0.23688281808991013], rtol=1e-14)
    # reversed bias: selection follows the scores, ids still reported ascending
    L.bias = np.array([0, 1, 2, 3], np.float32)
    L.renorm = True
    r = oracle.router(L)
    assert list(r["ids"][0]) == [2, 3]
    np.testing.assert_allclose(r["w"][0], [0.2689414213699951, 0.7310585786300049], rtol=1e-15)
    # equal scores: the lower id wins, weights exactly 1/k
    E5 = 5
    L5 = oracle.Layer(x=x, wr=np.zeros((E5, H), np.float32), wg=np.zeros((E5, 1, H), np.float32),
                      wu=np.zeros((E5, 1, H), np.float32), wd=np.zeros((E5, H, 1), np.float32),
                      top_k=3, bias=np.full(E5, 0.25, np.float32))
    r = oracle.router(L5)
    assert list(r["ids"][0]) == [0, 1, 2]
    assert np.all(r["w"][0] == 1.0 / 3.0)
    assert r["near"][0]                      # k-th and (k+1)-th scores tie


@pytest.mark.parametrize("seed", range(4))
def test_weights_closed_form_and_sum(seed):
    """With renorm the kept weights equal a softmax over the kept logits alone; without
    renorm they equal the full softmax at the kept ids."""
    rng = np.random.default_rng(300 + seed)
    T, H, E, K = 7, 12, 9, 4
    for renorm in (True, False):
        L = _f32_layer(rng, T, H, E, K, 4, renorm=renorm)
        r = oracle.router(L, want_logits=True)
        s = r["logits"]
        for t in range(T):
            ids = r["ids"][t]
            if renorm:
                v = np.exp(s[t, ids] - s[t, ids].max())
                np.testing.assert_allclose(r["w"][t], v / v.sum(), rtol=1e-13)
                assert abs(r["w"][t].sum() - 1.0) < 1e-12
            else:
                v = np.exp(s[t] - s[t].max())
                np.testing.assert_allclose(r["w"][t], (v / v.sum())[ids], rtol=1e-13)
    L = _f32_layer(rng, 3, 8, 5, 1, 4)
    assert np.all(oracle.router(L)["w"] == 1.0)


def test_near_tie_flag():
    H, E = 4, 6
    x = np.ones((2, H), np.float32)
    wr = np.zeros((E, H), np.float32)
    z, zd = np.zeros((E, 1, H), np.float32), np.zeros((E, H, 1), np.float32)
    # token-independent logits = bias; k=2: 2nd and 3rd ranked scores 1.0 and 1.0 + 5e-6
    b = np.array([2.0, 1.0, 1.0 + 4e-6, 0.0, -1.0, -2.0], np.float32)
    L = oracle.Layer(x=x, wr=wr, wg=z, wu=z, wd=zd, top_k=2, bias=b)
    assert oracle.router(L)["near"].all()
    b2 = np.array([2.0, 1.0, 1.0 + 1e-3, 0.0, -1.0, -2.0], np.float32)
    L.bias = b2
    r = oracle.router(L)
    assert not r["near"].any()
    np.testing.assert_allclose(r["gap"], float(b2[2]) - float(b2[1]), rtol=1e-12)
    # k == E: no (k+1)-th score, never a near tie
    L3 = oracle.Layer(x=x, wr=wr, wg=z, wu=z, wd=zd, top_k=E, bias=b)
    assert not oracle.router(L3)["near"].any()


# ---- grouping -----------------------------------------------------------------------

def _group_bruteforce(ids, E):
    T, K = ids.shape
    srt, off = [], [0]
    for e in range(E):
        for t in range(T):
            for j in range(K):
                if ids[t, j] == e:
                    srt.append(t * K + j)
        off.append(len(srt))
    pos = np.empty(T * K, np.int64)
    for p, s in enumerate(srt):
        pos[s] = p
    return np.array(off), np.array(srt), pos


@pytest.mark.parametrize("seed", range(8))
def test_group_bruteforce_and_invariants(seed):
    rng = np.random.default_rng(400 + seed)
    T, E, K = int(rng.integers(0, 40)), int(rng.integers(1, 20)), 0
    K = int(rng.integers(1, E + 1))
    ids = np.stack([np.sort(rng.choice(E, K, replace=False)) for _ in range(T)]) if T else np.zeros((0, K), np.int32)
    ids = ids.astype(np.int32).reshape(T, K)
    off, srt, pos = oracle.group(ids, E)
    boff, bsrt, bpos = _group_bruteforce(ids, E)
    assert np.array_equal(off, boff) and np.array_equal(srt, bsrt) and np.array_equal(pos, bpos)
    assert grouping_violations(ids, E, off, srt, pos) == []


def test_group_rejects_bad_ids():
    with pytest.raises(ValueError):
        oracle.group(np.array([[0, 9]], np.int32), 4)
    with pytest.raises(ValueError):
        oracle.group(np.array([[-1, 2]], np.int32), 4)


@pytest.mark.parametrize("mutation", ["swap", "drop", "dup", "order", "offset", "pos"])
def test_grouping_checker_catches_mutations(mutation):
    """The invariant checker used on GPU output must reject planted mistakes."""
    rng = np.random.default_rng(5)
    T, E, K = 12, 6, 3
    ids = np.stack([np.sort(rng.choice(E, K, replace=False)) for _ in range(T)]).astype(np.int32)
    off, srt, pos = [a.copy() for a in oracle.group(ids, E)]
    assert grouping_violations(ids, E, off, srt, pos) == []
    if mutation == "swap":          # slot moved to another expert's segment
        i, j = off[0], off[-2]
        srt[i], srt[j] = srt[j], srt[i]
    elif mutation == "drop":        # one slot lost, another duplicated
        srt[1] = srt[0]
    elif mutation == "dup":
        srt[-1] = srt[-2]
    elif mutation == "order":       # unstable order inside a segment
        e = int(np.argmax(np.diff(off)))
        a = off[e]
        srt[a], srt[a + 1] = srt[a + 1], srt[a]
    elif mutation == "offset":
        off[2] += 1
    elif mutation == "pos":
        pos[0], pos[1] = pos[1], pos[0]
    assert grouping_violations(ids, E, off, srt, pos) != []


# ---- SwiGLU experts -------------------------------------------------------------------

def test_expert_hand_cases():
    for x, wg, wu, wd, o in [list(map(float, r)) for r in _table("hand_cases.txt")]:
        L = oracle.Layer(x=np.array([[x]], np.float32), wr=np.zeros((1, 1), np.float32),
                         wg=np.array([[[wg]]], np.float32), wu=np.array([[[wu]]], np.float32),
                         wd=np.array([[[wd]]], np.float32), top_k=1)
        got = oracle.expert_pairs(L, [0], [0])[0, 0]
        assert abs(got - o) <= 1e-15 * max(1.0, abs(o)), (x, wg, wu, wd, got, o)


@pytest.mark.parametrize("seed", range(3))
def test_expert_odd_identity(seed):
    """silu(z) - silu(-z) = z, so o(x) + o(-x) = Wd (g * u) with g = Wg x, u = Wu x: a
    bilinear form with no activation in it."""
    rng = np.random.default_rng(500 + seed)
    T, H, E, I = 3, 10, 4, 6
    L = _f32_layer(rng, T, H, E, 2, I)
    L.x = np.concatenate([L.x, -L.x]).astype(np.float32)
    toks = list(range(2 * T))
    for e in range(E):
        o = oracle.expert_pairs(L, toks, [e] * len(toks))
        X = L.x[:T].astype(np.float64)
        g = X @ L.wg[e].astype(np.float64).T
        u = X @ L.wu[e].astype(np.float64).T
        ref = (g * u) @ L.wd[e].astype(np.float64).T
        np.testing.assert_allclose(o[:T] + o[T:], ref, rtol=1e-11, atol=1e-12)


def test_expert_matches_torch_library():
    """One expert through torch's own silu and matmul, in fp64."""
    rng = np.random.default_rng(600)
    T, H, E, I = 4, 16, 3, 8
    L = _f32_layer(rng, T, H, E, 2, I)
    for e in range(E):
        X = torch.from_numpy(L.x.astype(np.float64))
        ref = (torch.nn.functional.silu(X @ torch.from_numpy(L.wg[e].astype(np.float64)).T)
               * (X @ torch.from_numpy(L.wu[e].astype(np.float64)).T)) @ torch.from_numpy(L.wd[e].astype(np.float64)).T
        o = oracle.expert_pairs(L, range(T), [e] * T)
        np.testing.assert_allclose(o, ref.numpy(), rtol=1e-12, atol=1e-13)


# ---- whole layer ----------------------------------------------------------------------

def _dense_bruteforce(L: oracle.Layer, forced=None):
    """Every expert on every token (no grouping), mask from a full sort, weights from the
    full softmax -- a different loop structure written with torch fp64 primitives."""
    X = torch.from_numpy(decoded(L.x))
    Wr = torch.from_numpy(decoded(L.wr))
    s = X @ Wr.T + (torch.from_numpy(L.bias.astype(np.float64)) if L.bias is not None else 0.0)
    T, E = s.shape
    K = L.top_k
    mask = torch.zeros(T, E, dtype=torch.float64)
    for t in range(T):
        if forced is not None:
            sel = list(forced[t])
        else:
            order = sorted(range(E), key=lambda e: (-float(s[t, e]), e))
            sel = order[:K]
        mask[t, sel] = 1.0
    p = torch.softmax(s, dim=1) * mask
    if L.renorm:
        p = p / p.sum(dim=1, keepdim=True)
    y = torch.zeros(T, X.shape[1], dtype=torch.float64)
    for e in range(E):
        Wg = torch.from_numpy(decoded(L.wg[e]))
        Wu = torch.from_numpy(decoded(L.wu[e]))
        Wd = torch.from_numpy(decoded(L.wd[e]))
        o = (torch.nn.functional.silu(X @ Wg.T) * (X @ Wu.T)) @ Wd.T
        y += p[:, e:e + 1] * o
    return y.numpy()


@pytest.mark.parametrize("seed,renorm", [(0, True), (1, True), (2, False), (3, False)])
def test_forward_matches_dense_bruteforce(seed, renorm):
    rng = np.random.default_rng(700 + seed)
    T, H, E, K, I = 6, 12, 8, 3, 5
    L = _f32_layer(rng, T, H, E, K, I, renorm=renorm)
    r = oracle.forward(L)
    ref = _dense_bruteforce(L)
    np.testing.assert_allclose(r["y"], ref, rtol=1e-11, atol=1e-13)


def test_forward_c0_matches_dense_bruteforce():
    li = synth.make_layer("c0_tiny_f32")
    L = oracle_layer(li)
    r = oracle.forward(L)
    ref = _dense_bruteforce(L)
    rel = np.linalg.norm(r["y"] - ref) / np.linalg.norm(ref)
    assert rel < 1e-12


def test_forward_bf16_small_matches_dense_bruteforce():
    li = synth.make_layer(synth.Shape(5, 64, 16, 4, 32, "bf16", "bf16", bias="normal"))
    L = oracle_layer(li)
    r = oracle.forward(L)
    ref = _dense_bruteforce(L)
    assert np.linalg.norm(r["y"] - ref) / np.linalg.norm(ref) < 1e-12


def test_forward_identical_experts_equals_single_ffn():
    """All experts equal and renorm on: y = FFN(x) whatever the routing."""
    rng = np.random.default_rng(800)
    T, H, E, K, I = 5, 9, 6, 3, 7
    L = _f32_layer(rng, T, H, E, K, I)
    for W in ("wg", "wu", "wd"):
        a = getattr(L, W)
        setattr(L, W, np.ascontiguousarray(np.broadcast_to(a[:1], a.shape)))
    X = torch.from_numpy(L.x.astype(np.float64))
    ffn = (torch.nn.functional.silu(X @ torch.from_numpy(L.wg[0].astype(np.float64)).T)
           * (X @ torch.from_numpy(L.wu[0].astype(np.float64)).T)) @ torch.from_numpy(L.wd[0].astype(np.float64)).T
    np.testing.assert_allclose(oracle.forward(L)["y"], ffn.numpy(), rtol=1e-12, atol=1e-13)


def test_forward_zero_up_gives_zero():
    rng = np.random.default_rng(801)
    L = _f32_layer(rng, 4, 8, 5, 2, 6)
    L.wu = np.zeros_like(L.wu)
    assert np.all(oracle.forward(L)["y"] == 0.0)


def test_forward_subset_and_forced_ids():
    rng = np.random.default_rng(802)
    T, H, E, K, I = 7, 10, 6, 2, 4
    L = _f32_layer(rng, T, H, E, K, I)
    full = oracle.forward(L)
    sub = oracle.forward(L, tokens=[5, 1])
    np.testing.assert_array_equal(sub["y"], full["y"][[5, 1]])
    same = oracle.forward(L, forced_ids=full["ids"])
    np.testing.assert_array_equal(same["y"], full["y"])
    forced = np.array([[0, 5]] * T, np.int32)
    got = oracle.forward(L, forced_ids=forced)
    np.testing.assert_allclose(got["y"], _dense_bruteforce(L, forced=forced), rtol=1e-11, atol=1e-13)


def test_forward_mxfp4_equals_dequantised_fp32():
    """The oracle on MXFP4 storage equals the oracle on fp32 storage of the same values,
    dequantised by the generator's own (independent) inverse map."""
    li = synth.make_layer(synth.Shape(3, 64, 4, 2, 32, "bf16", "mxfp4"))
    L = oracle_layer(li)
    E = li.shape.E
    deq = {}
    for name, sname in (("wg", "sg"), ("wu", "su"), ("wd", "sd")):
        c, s = getattr(li, name), getattr(li, sname)
        deq[name] = np.stack([synth.mxfp4_dequantize(c[e], s[e]) for e in range(E)]).astype(np.float32)
        assert np.array_equal(deq[name].astype(np.float64),
                              np.stack([synth.mxfp4_dequantize(c[e], s[e]) for e in range(E)]))
    L32 = oracle.Layer(x=li.x, wr=li.wr, wg=deq["wg"], wu=deq["wu"], wd=deq["wd"], top_k=2, bias=None)
    a, b = oracle.forward(L), oracle.forward(L32)
    np.testing.assert_array_equal(a["ids"], b["ids"])
    np.testing.assert_array_equal(a["y"], b["y"])


# ---- NVFP4 (E2M1 codes, E4M3 block scales per 16 elements, fp32 tensor scale) ----------

def test_e4m3_decode_matches_torch_exhaustive():
    """All 256 E4M3 codes against torch's float8_e4m3fn (OCP FP8 E4M3), an independent
    decoder; S.1111.111 is NaN in both."""
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for code in range(256):
        got = oracle.decode_e4m3(code)
        if math.isnan(ref[code]):
            assert math.isnan(got), code
        else:
            assert got == ref[code], (code, got, ref[code])


def _nv_pack(codes: np.ndarray) -> np.ndarray:
    """[R, C] codes 0..15 -> [R, C/2] bytes, the even element in the low nibble."""
    return ((codes[:, 0::2] & 15) | ((codes[:, 1::2] & 15) << 4)).astype(np.uint8)


def test_nvfp4_hand_case():
    """One nonzero element per matrix, worked by hand from the format definition:
    gate 3.0 (E2M1 0x5) x 2.0 (E4M3 0x40) x tensor scale 0.25 = 1.5; up 1.5 (0x3) x 1.0
    (0x38) x 2.0 = 3.0; down -1.0 (0xA) x 4.0 (0x48) x 0.5 = -2.0, so with x = e_3 the
    expert output is o[7] = -2 * silu(1.5) * 3.0 and zero elsewhere."""
    H = I = 16
    x = np.zeros((1, H), np.uint16)
    x[0, 3] = 0x3F80                                   # bf16 1.0
    cg = np.zeros((I, H), np.int64); cg[2, 3] = 0x5
    cu = np.zeros((I, H), np.int64); cu[2, 3] = 0x3
    cd = np.zeros((H, I), np.int64); cd[7, 2] = 0xA
    sg = np.zeros((1, I, H // 16), np.uint8); sg[0, 2, 0] = 0x40
    su = np.zeros((1, I, H // 16), np.uint8); su[0, 2, 0] = 0x38
    sd = np.zeros((1, H, I // 16), np.uint8); sd[0, 7, 0] = 0x48
    L = oracle.Layer(x=x, wr=np.zeros((1, H), np.uint16), wg=_nv_pack(cg)[None], wu=_nv_pack(cu)[None],
                     wd=_nv_pack(cd)[None], top_k=1, sg=sg, su=su, sd=sd, fmt="nvfp4", ts=(0.25, 2.0, 0.5))
    o = oracle.expert_pairs(L, [0], [0])[0]
    want = np.zeros(H)
    want[7] = -2.0 * (1.5 / (1.0 + math.exp(-1.5))) * 3.0
    np.testing.assert_allclose(o, want, rtol=1e-15, atol=0)


def test_forward_nvfp4_matches_numpy_on_dequantised_weights():
    """The oracle's expert outputs on NVFP4 storage equal fp64 numpy matrix products on the
    weights dequantised by the generator's own (independent) inverse map."""
    li = synth.make_layer(synth.Shape(3, 64, 4, 2, 32, "bf16", "nvfp4"))
    L = oracle_layer(li)
    E, T = li.shape.E, li.shape.T
    deq = {}
    for name, sname, ts in (("wg", "sg", li.ts[0]), ("wu", "su", li.ts[1]), ("wd", "sd", li.ts[2])):
        c, s = getattr(li, name), getattr(li, sname)
        deq[name] = np.stack([synth.nvfp4_dequantize(c[e], s[e], ts) for e in range(E)])
    x = synth.bf16_bits_to_f32(li.x).astype(np.float64)
    tok = [t for t in range(T) for e in range(E)]
    exp_ = [e for t in range(T) for e in range(E)]
    got = oracle.expert_pairs(L, tok, exp_)
    for p, (t, e) in enumerate(zip(tok, exp_)):
        g = deq["wg"][e] @ x[t]
        u = deq["wu"][e] @ x[t]
        want = deq["wd"][e] @ (g / (1.0 + np.exp(-g)) * u)
        np.testing.assert_allclose(got[p], want, rtol=1e-11, atol=1e-14)


def test_nvfp4_quantiser_round_trip():
    """The generator's NVFP4 quantiser: block scales are finite E4M3 codes, the stored
    values are within half an E2M1 step (of the block's scale) of the inputs below the
    saturation point, and all-zero blocks stay zero."""
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((8, 64)) * 0.05).astype(np.float32)
    w[3, 16:32] = 0.0
    ts = synth.nvfp4_tensor_scale(0.05)
    codes, scales = synth.nvfp4_quantize(w, ts)
    assert scales.dtype == np.uint8 and np.all((scales & 0x7F) != 0x7F)
    assert scales[3, 1] == 0 and np.all(codes[3, 8:16] == 0)
    d = synth.nvfp4_dequantize(codes, scales, ts)
    blk_scale = np.repeat(np.array([[oracle.decode_e4m3(int(c)) for c in row] for row in scales]) * ts, 16, axis=1)
    ok = np.abs(w) <= 6.0 * blk_scale
    assert np.all(np.abs(d - w)[ok] <= 1.0 * blk_scale[ok] + 1e-12)


# ---- MXINT8 (OCP MX INT8 elements, E8M0 block scales per 32 elements) -------------------

def test_mxint8_table():
    """Element values of the OCP MX INT8 encoding, hand-derived from the definition."""
    rows = _table("mxint8_table.txt")
    assert len(rows) >= 12
    for code, val in rows:
        assert oracle.decode_int8(int(code, 16)) == float(val), code


def test_mxint8_decode_exhaustive_against_twos_complement():
    """All 256 codes against numpy's two's complement reading of the byte, over 64."""
    ref = np.arange(256, dtype=np.int64).astype(np.uint8).view(np.int8).astype(np.float64) / 64.0
    for code in range(256):
        assert oracle.decode_int8(code) == ref[code], code


def test_mxint8_hand_case():
    """One nonzero element per matrix, worked by hand from the format definition:
    gate 0x30 (0.75) x 2^1 (E8M0 128) = 1.5; up 0xC0 (-1.0) x 2^-2 (E8M0 125) = -0.25;
    down 0x50 (1.25) x 2^2 (E8M0 129) = 5.0, so with x = e_9 the expert output is
    o[5] = 5 * silu(1.5) * -0.25 and zero elsewhere."""
    H = I = 32
    x = np.zeros((1, H), np.uint16)
    x[0, 9] = 0x3F80                                   # bf16 1.0
    cg = np.zeros((1, I, H), np.int8); cg[0, 4, 9] = 0x30
    cu = np.zeros((1, I, H), np.int8); cu[0, 4, 9] = np.int8(-64)
    cd = np.zeros((1, H, I), np.int8); cd[0, 5, 4] = 0x50
    sg = np.zeros((1, I, 1), np.uint8); sg[0, 4, 0] = 128
    su = np.zeros((1, I, 1), np.uint8); su[0, 4, 0] = 125
    sd = np.zeros((1, H, 1), np.uint8); sd[0, 5, 0] = 129
    L = oracle.Layer(x=x, wr=np.zeros((1, H), np.uint16), wg=cg, wu=cu, wd=cd, top_k=1, sg=sg, su=su, sd=sd)
    o = oracle.expert_pairs(L, [0], [0])[0]
    want = np.zeros(H)
    want[5] = 5.0 * (1.5 / (1.0 + math.exp(-1.5))) * -0.25
    np.testing.assert_allclose(o, want, rtol=1e-15, atol=0)


def test_forward_mxint8_matches_numpy_on_dequantised_weights():
    """The oracle's expert outputs and whole layer on MXINT8 storage equal fp64 numpy
    products on the weights dequantised by the generator's own (independent) inverse map,
    and the oracle on fp32 storage of those values."""
    li = synth.make_layer(synth.Shape(3, 64, 4, 2, 32, "bf16", "mxint8", bias="normal"))
    L = oracle_layer(li)
    E, T = li.shape.E, li.shape.T
    deq = {}
    for name, sname in (("wg", "sg"), ("wu", "su"), ("wd", "sd")):
        c, s = getattr(li, name), getattr(li, sname)
        deq[name] = np.stack([synth.mxint8_dequantize(c[e], s[e]) for e in range(E)])
    x = synth.bf16_bits_to_f32(li.x).astype(np.float64)
    tok = [t for t in range(T) for e in range(E)]
    exp_ = [e for t in range(T) for e in range(E)]
    got = oracle.expert_pairs(L, tok, exp_)
    for p, (t, e) in enumerate(zip(tok, exp_)):
        g = deq["wg"][e] @ x[t]
        u = deq["wu"][e] @ x[t]
        want = deq["wd"][e] @ (g / (1.0 + np.exp(-g)) * u)
        np.testing.assert_allclose(got[p], want, rtol=1e-11, atol=1e-14)
    f32 = {k: v.astype(np.float32) for k, v in deq.items()}
    assert all(np.array_equal(f32[k].astype(np.float64), deq[k]) for k in deq)   # exact in fp32
    L32 = oracle.Layer(x=li.x, wr=li.wr, wg=f32["wg"], wu=f32["wu"], wd=f32["wd"], top_k=2, bias=li.bias)
    a, b = oracle.forward(L), oracle.forward(L32)
    np.testing.assert_array_equal(a["ids"], b["ids"])
    np.testing.assert_array_equal(a["y"], b["y"])
