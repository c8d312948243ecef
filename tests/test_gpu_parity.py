"""Parity of the HIP path (through the C ABI) with the fp64 oracle on the same
seeded inputs.  Needs an MI355X; run with -m gpu."""
import numpy as np
import pytest
import torch

import oracle
import prefill_moe_router_amd as pm
import synth
from tests.gpu_common import (W_TOL, DevLayer, canary_ok, compare_forward, forward_grouping, guarded, layer, layer_of,
                              lshape, note, run_forward, tdev, to_f64)
from tests.helpers import grouping_violations, max_abs, oracle_layer, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    pm.lib()  # loud failure when the library is missing


# ---- router ------------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["c0_tiny_f32", "c1_decode1_bf16", "c2_decode8_bf16", "c3_prefill8192_bf16",
                                  "c4_mxfp4_decode8"])
def test_router_topk_parity(name):
    note(f"router parity {name}")
    li = layer(name)
    dl = DevLayer(li)
    sh = lshape(li)
    T, K = li.shape.T, li.shape.K
    ws = pm.alloc_workspace(sh)
    ids = torch.empty(T, K, dtype=torch.int32, device="cuda")
    w = torch.empty(T, K, dtype=torch.float32, device="cuda")
    pm.router_topk(sh, dl.x, dl.wr, dl.bias, ids, w, ws)
    torch.cuda.synchronize()
    ref = oracle.router(oracle_layer(li))
    gids, gw = ids.cpu().numpy(), w.cpu().numpy()
    mism = (gids != ref["ids"]).any(1)
    assert not (mism & ~ref["near"]).any(), np.nonzero(mism & ~ref["near"])[0][:10]
    ok = ~mism
    assert max_abs(gw[ok], ref["w"][ok]) <= W_TOL
    assert np.all(np.diff(gids, axis=1) > 0)          # ascending ids
    note(f"  near-ties {int(ref['near'].sum())}, id mismatches {int(mism.sum())}")


def test_router_exact_ties_pick_lower_id():
    """Identical router rows give bit-identical logits; the lower id must win."""
    sh_ = synth.Shape(16, 256, 12, 3, 64, "bf16", "bf16")
    li = layer_of(sh_)
    popular = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(li.wr[2]) * 4)   # make 2/5/9 win often
    for e in (2, 5, 9):
        li.wr[e] = popular
    dl = DevLayer(li)
    sh = lshape(li)
    ws = pm.alloc_workspace(sh)
    ids = torch.empty(16, 3, dtype=torch.int32, device="cuda")
    w = torch.empty(16, 3, dtype=torch.float32, device="cuda")
    pm.router_topk(sh, dl.x, dl.wr, None, ids, w, ws)
    ref = oracle.router(oracle_layer(li))
    np.testing.assert_array_equal(ids.cpu().numpy(), ref["ids"])


@pytest.mark.parametrize("T,H,E,K,renorm,bias", [(1, 512, 32, 1, True, "none"), (31, 512, 32, 8, False, "normal"),
                                                 (33, 1024, 64, 8, True, "zipf"), (100, 512, 96, 32, True, "normal"),
                                                 (257, 2048, 128, 8, False, "zipf"), (64, 512, 128, 32, True, "none")])
def test_router_topk_mfma_shapes(T, H, E, K, renorm, bias):
    """Router GEMM + top-k in one MFMA kernel (E a multiple of 32 up to 128, H a multiple of
    512): ragged last token block, k from 1 to 32, with and without renormalisation and bias."""
    note(f"router mfma T={T} H={H} E={E} K={K} renorm={renorm} bias={bias}")
    li = layer_of(synth.Shape(T, H, E, K, 64, "bf16", "bf16", bias=bias, renorm=renorm), seed=T + E)
    dl = DevLayer(li)
    sh = lshape(li)
    ws = pm.alloc_workspace(sh)
    ids = torch.full((T, K), -7, dtype=torch.int32, device="cuda")
    w = torch.full((T, K), -7.0, dtype=torch.float32, device="cuda")
    pm.router_topk(sh, dl.x, dl.wr, dl.bias, ids, w, ws)
    torch.cuda.synchronize()
    ref = oracle.router(oracle_layer(li))
    gids, gw = ids.cpu().numpy(), w.cpu().numpy()
    mism = (gids != ref["ids"]).any(1)
    assert not (mism & ~ref["near"]).any(), np.nonzero(mism & ~ref["near"])[0][:10]
    ok = ~mism
    assert max_abs(gw[ok], ref["w"][ok]) <= W_TOL
    assert np.all(np.diff(gids, axis=1) > 0) and gids.min() >= 0 and gids.max() < E
    note(f"  near-ties {int(ref['near'].sum())}, id mismatches {int(mism.sum())}")


@pytest.mark.parametrize("T,H,E,K,act", [(12, 4096, 8, 2, "f32"), (9, 6144, 16, 4, "bf16"), (13, 1024, 48, 5, "bf16"),
                                         (3, 2048, 64, 8, "bf16")])
def test_router_gemv_shapes(T, H, E, K, act):
    """Router GEMV + top-k (the kernels used below the MFMA router's shapes): 1 to 16
    chunks per lane, ragged 8-token tiles, bias, ids exact away from near-ties."""
    note(f"router gemv T={T} H={H} E={E} K={K} {act}")
    w = "f32" if act == "f32" else "bf16"
    li = layer_of(synth.Shape(T, H, E, K, 64, act, w, bias="normal"), seed=H + E)
    dl = DevLayer(li)
    sh = lshape(li)
    ws = pm.alloc_workspace(sh)
    ids = torch.full((T, K), -7, dtype=torch.int32, device="cuda")
    wt = torch.full((T, K), -7.0, dtype=torch.float32, device="cuda")
    pm.router_topk(sh, dl.x, dl.wr, dl.bias, ids, wt, ws)
    torch.cuda.synchronize()
    ref = oracle.router(oracle_layer(li))
    gids, gw = ids.cpu().numpy(), wt.cpu().numpy()
    mism = (gids != ref["ids"]).any(1)
    assert not (mism & ~ref["near"]).any(), np.nonzero(mism & ~ref["near"])[0][:10]
    assert max_abs(gw[~mism], ref["w"][~mism]) <= W_TOL
    assert np.all(np.diff(gids, axis=1) > 0)


def test_router_mfma_exact_ties_pick_lower_id():
    """Identical router rows give bit-identical logits in the MFMA router too; the lower id wins."""
    sh_ = synth.Shape(40, 512, 32, 3, 64, "bf16", "bf16")
    li = layer_of(sh_)
    popular = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(li.wr[2]) * 4)
    for e in (2, 5, 9, 20):
        li.wr[e] = popular
    dl = DevLayer(li)
    sh = lshape(li)
    ws = pm.alloc_workspace(sh)
    ids = torch.empty(40, 3, dtype=torch.int32, device="cuda")
    w = torch.empty(40, 3, dtype=torch.float32, device="cuda")
    pm.router_topk(sh, dl.x, dl.wr, None, ids, w, ws)
    ref = oracle.router(oracle_layer(li))
    np.testing.assert_array_equal(ids.cpu().numpy(), ref["ids"])


# ---- grouping ----------------------------------------------------------------------------

def _group_gpu(ids_np, E, T, K):
    sh = pm.LayerShape(T, 256, E, K, 64)
    ws = pm.alloc_workspace(sh)
    P = T * K
    ids = tdev(ids_np.astype(np.int32))
    obuf, off = guarded(E + 1, torch.int32)
    sbuf, srt = guarded(P, torch.int32)
    pbuf, pos = guarded(P, torch.int32)
    pm.group_tokens(sh, ids, off, srt, pos, ws)
    torch.cuda.synchronize()
    for b, n in ((obuf, E + 1), (sbuf, P), (pbuf, P)):
        assert canary_ok(b, n, torch.int32)
    return off.cpu().numpy(), srt.cpu().numpy(), pos.cpu().numpy(), ws


@pytest.mark.parametrize("T,E,K,kind", [(1, 128, 8, "uniform"), (8, 128, 8, "uniform"), (5, 8, 8, "uniform"),
                                        (8192, 128, 8, "zipf"), (8192, 128, 8, "one_hot"),
                                        (2048, 1024, 32, "uniform"), (4096, 256, 8, "uniform"),
                                        (333, 64, 3, "zipf"), (0, 16, 2, "uniform")])
def test_group_parity(T, E, K, kind):
    note(f"group parity T={T} E={E} K={K} {kind}")
    rng = np.random.default_rng(T * 7 + E + K)
    if kind == "uniform":
        ids = np.stack([np.sort(rng.choice(E, K, replace=False)) for _ in range(T)]) if T else np.zeros((0, K))
    elif kind == "zipf":
        p = 1.0 / np.arange(1, E + 1)
        p /= p.sum()
        ids = np.stack([np.sort(rng.choice(E, K, replace=False, p=p)) for _ in range(T)])
    else:  # every token routes to experts 0..K-1: one group per expert of size T, the rest empty
        ids = np.tile(np.arange(K), (T, 1))
    ids = ids.astype(np.int32).reshape(T, K)
    off, srt, pos, _ = _group_gpu(ids, E, T, K)
    roff, rsrt, rpos = oracle.group(ids, E)
    np.testing.assert_array_equal(off, roff)
    np.testing.assert_array_equal(srt, rsrt)
    np.testing.assert_array_equal(pos, rpos)
    assert grouping_violations(ids, E, off, srt, pos) == []


def test_group_rejects_out_of_range_ids_without_oob_writes():
    T, E, K = 64, 16, 2
    rng = np.random.default_rng(3)
    ids = np.stack([np.sort(rng.choice(E, K, replace=False)) for _ in range(T)]).astype(np.int32)
    ids[5, 1] = E + 3
    ids[9, 0] = -4
    off, srt, pos, ws = _group_gpu(ids, E, T, K)
    assert pm.check_device_error(ws) & pm.DEVERR_BAD_EXPERT_ID
    assert pm.check_device_error(ws) == 0                       # read-and-clear
    assert off[-1] == T * K - 2 and pos[5 * K + 1] == -1 and pos[9 * K] == -1
    good = ids.copy()
    # the grouped part equals the oracle's grouping of the valid slots
    valid = (good >= 0) & (good < E)
    for e in range(E):
        seg = srt[off[e]:off[e + 1]]
        assert np.all(good.reshape(-1)[seg] == e)
        assert np.all(np.diff(seg) > 0)
    assert np.sum(np.diff(off)) == valid.sum()


# ---- staged expert FFN and combine ----------------------------------------------------------

@pytest.mark.parametrize("name", ["c0_tiny_f32", "c1_decode1_bf16", "c2_decode8_bf16"])
def test_staged_pipeline_parity(name):
    """router_topk -> group_tokens -> expert_ffn -> combine, each checked."""
    note(f"staged pipeline {name}")
    li = layer(name)
    dl = DevLayer(li)
    sh = lshape(li)
    T, K, E, H = li.shape.T, li.shape.K, li.shape.E, li.shape.H
    P = T * K
    ws = pm.alloc_workspace(sh)
    ids = torch.empty(T, K, dtype=torch.int32, device="cuda")
    w = torch.empty(T, K, dtype=torch.float32, device="cuda")
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    srt = torch.empty(P, dtype=torch.int32, device="cuda")
    pos = torch.empty(P, dtype=torch.int32, device="cuda")
    obuf, o = guarded(P * H, torch.float32)
    o = o.view(P, H)
    pm.router_topk(sh, dl.x, dl.wr, dl.bias, ids, w, ws)
    pm.group_tokens(sh, ids, off, srt, pos, ws)
    pm.expert_ffn(sh, dl.x, dl.weights, off, srt, o, ws)
    y = torch.empty(T, H, dtype=dl.act_torch(), device="cuda")
    pm.combine(sh, o, w, pos, y)
    torch.cuda.synchronize()
    assert canary_ok(obuf, P * H, torch.float32)
    gids = ids.cpu().numpy()
    L = oracle_layer(li)
    roff, rsrt, rpos = oracle.group(gids, E)
    np.testing.assert_array_equal(off.cpu().numpy(), roff)
    np.testing.assert_array_equal(srt.cpu().numpy(), rsrt)
    # expert outputs in sorted order against the oracle's pairs
    toks = rsrt // K
    exps = gids.reshape(-1)[rsrt]
    oref = oracle.expert_pairs(L, toks, exps)
    og = o.cpu().numpy().astype(np.float64)
    tol = 1e-5 if li.shape.act == "f32" else 1e-2
    assert rel_l2(og, oref) <= tol, rel_l2(og, oref)
    # combine of the GPU's own expert outputs: fp32 sums of k terms, one final rounding
    yref = np.zeros((T, H))
    gw = w.cpu().numpy().astype(np.float64)
    for t in range(T):
        for j in range(K):
            yref[t] += gw[t, j] * og[rpos[t * K + j]]
    yg = to_f64(y, li.shape.act)
    if li.shape.act == "f32":
        assert max_abs(yg, yref) <= 1e-5 * max(1.0, np.abs(yref).max())
    else:
        # one bf16 rounding of the fp32 sum: within 2^-8 relative of each element
        assert np.all(np.abs(yg - yref) <= np.abs(yref) * 2.0 ** -8 + 1e-6)
    compare_forward(li, dict(y=y, ids=gids, w=w.cpu().numpy()), label=f"staged {name}")


@pytest.mark.parametrize("K", [5, 10])
def test_combine_parity_random(K):
    """Random rows and weights; K = 10 takes a batch of eight rows and a tail of two.  A few
    slots are left out of the grouping (slot_pos -1, as for a bad expert id) and add
    nothing."""
    T, H = 37, 512
    rng = np.random.default_rng(11)
    o = rng.standard_normal((T * K, H)).astype(np.float32)
    w = rng.random((T, K)).astype(np.float32)
    perm = rng.permutation(T * K).astype(np.int32)
    perm[[3, 2 * K + K - 1, 5 * K + 4]] = -1
    sh = pm.LayerShape(T, H, 16, K, 64, act_dtype=pm.BF16, weight_dtype=pm.BF16)
    y = torch.empty(T, H, dtype=torch.int16, device="cuda")
    pm.combine(sh, tdev(o), tdev(w), tdev(perm), y)
    ref = np.zeros((T, H))
    for t in range(T):
        for j in range(K):
            if perm[t * K + j] >= 0:
                ref[t] += np.float64(w[t, j]) * o[perm[t * K + j]]
    yg = to_f64(y, "bf16")
    assert np.all(np.abs(yg - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-6)


def test_bf16_store_rounds_to_nearest_even():
    """The kernels store bf16 through the hardware conversion; with k = 1 and weight 1 the
    combine is a pure fp32 -> bf16 store, which must equal round-to-nearest-even bit for
    bit, ties and subnormals included."""
    rng = np.random.default_rng(5)
    T, H = 4, 512
    hi = rng.integers(0, 1 << 16, size=T * H, dtype=np.uint32)
    lo = rng.integers(0, 1 << 16, size=T * H, dtype=np.uint32)
    lo[::4] = 0x8000                      # exact ties
    lo[1::8] = 0x7fff
    lo[2::8] = 0x8001
    hi = np.where((hi & 0x7f80) == 0x7f80, hi & 0x807f, hi)   # finite values only
    hi[3::16] &= 0x807f                   # subnormals
    bits = (hi << 16) | lo
    o = bits.view(np.float32).reshape(T, H)
    sh = pm.LayerShape(T, H, 16, 1, 64, act_dtype=pm.BF16, weight_dtype=pm.BF16)
    y = torch.empty(T, H, dtype=torch.int16, device="cuda")
    pm.combine(sh, tdev(o), tdev(np.ones((T, 1), np.float32)), tdev(np.arange(T, dtype=np.int32)), y)
    torch.cuda.synchronize()
    want = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16).astype(np.uint16).reshape(T, H)
    got = y.cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want), np.argwhere(got != want)[:8]


# ---- whole layer ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["c0_tiny_f32", "c1_decode1_bf16", "c2_decode8_bf16"])
def test_forward_parity_decode_configs(name):
    note(f"forward parity {name}")
    li = layer(name)
    got = run_forward(DevLayer(li))
    compare_forward(li, got, label=name)


@pytest.mark.parametrize("name", ["c4_mxfp4_decode1", "c4_mxfp4_decode8"])
def test_forward_parity_mxfp4_decode(name):
    note(f"forward parity {name}")
    li = layer(name)
    got = run_forward(DevLayer(li))
    compare_forward(li, got, label=name)


def test_forward_parity_mxfp4_small_ragged():
    li = layer_of(synth.Shape(13, 256, 16, 4, 128, "bf16", "mxfp4"))
    got = run_forward(DevLayer(li))
    compare_forward(li, got, label="mxfp4 small")


@pytest.mark.parametrize("name", ["c5_nvfp4_decode1", "c5_nvfp4_decode8"])
def test_forward_parity_nvfp4_decode(name):
    """NVFP4 experts (E4M3 scale per 16 elements, fp32 tensor scale) on the fused decode
    launch: ids exact away from near-ties, y against the oracle."""
    note(f"forward parity {name}")
    li = layer(name)
    got = run_forward(DevLayer(li))
    compare_forward(li, got, label=name)


@pytest.mark.parametrize("T", [20, 64, 130])
def test_forward_nvfp4_streaming(T):
    """NVFP4 above 8 tokens runs on the streaming family at every T (no grouped kernels)."""
    note(f"nvfp4 streaming T={T}")
    li = layer_of(synth.Shape(T, 4096, 256, 8, 1024, "bf16", "nvfp4"), batch=90 + T)
    got = run_forward(DevLayer(li))
    compare_forward(li, got, label=f"nvfp4 T={T}")


@pytest.mark.parametrize("T,H,E,K,I,path", [(130, 1024, 32, 4, 256, pm.PATH_GROUPED),
                                            (512, 4096, 256, 8, 1024, pm.PATH_AUTO)])
def test_forward_nvfp4_grouped(T, H, E, K, I, path):
    """NVFP4 on the grouped MFMA GEMMs (codes dequantised into LDS with the split E4M3
    scale, tensor scales in the epilogues): ragged m-tiles, and AUTO's choice at 512 tokens."""
    note(f"nvfp4 grouped T={T} H={H} E={E}")
    li = layer_of(synth.Shape(T, H, E, K, I, "bf16", "nvfp4", bias="normal"), seed=7)
    sh = lshape(li, path)
    assert "router_topk" in pm.forward_stages(sh) or "router_logits" in pm.forward_stages(sh)
    assert "gate_up" in pm.forward_stages(sh)
    got = run_forward(DevLayer(li), path=path)
    compare_forward(li, got, label=f"nvfp4 grouped T={T}")


@pytest.mark.parametrize("T,H,E,K,I", [(3, 1024, 64, 4, 512), (12, 512, 32, 4, 256)])
def test_forward_nvfp4_small_shapes(T, H, E, K, I):
    """Other NVFP4 shapes: fused (T=3) and streaming (T=12, ragged rows per lane), bias."""
    li = layer_of(synth.Shape(T, H, E, K, I, "bf16", "nvfp4", bias="normal"), seed=3)
    got = run_forward(DevLayer(li))
    compare_forward(li, got, label=f"nvfp4 T={T} H={H} E={E}")


# ---- MXINT8 experts (OCP MX INT8 codes, E8M0 scale per 32 elements) --------------------------

@pytest.mark.parametrize("name", ["c6_mxint8_decode1", "c6_mxint8_decode8"])
def test_forward_parity_mxint8_decode(name):
    """MXINT8 experts on the fused decode launch (H = 4096, E = 256): ids exact away from
    near-ties, y of every token against the oracle."""
    note(f"forward parity {name}")
    li = layer(name)
    assert pm.forward_stages(lshape(li)) == ["decode_fused"]
    got = run_forward(DevLayer(li))
    compare_forward(li, got, label=name)


@pytest.mark.parametrize("T", [1, 5, 8])
def test_forward_mxint8_decode_bf16_layer_shape(T):
    """MXINT8 experts on the H = 2048, E = 128, I = 768 layer shape with a router bias."""
    li = layer_of(synth.Shape(T, 2048, 128, 8, 768, "bf16", "mxint8", bias="normal"), batch=80 + T)
    got = run_forward(DevLayer(li))
    compare_forward(li, got, label=f"mxint8 T={T} H=2048")


@pytest.mark.parametrize("T,path", [(20, pm.PATH_AUTO), (36, pm.PATH_AUTO), (40, pm.PATH_DECODE),
                                    (90, pm.PATH_DECODE)])
def test_forward_mxint8_streaming(T, path):
    """MXINT8 beyond 8 tokens on the streaming family (codes decoded once per weight row); AUTO
    keeps it below 1.25 pairs per expert (40 tokens at E = 256, k = 8)."""
    note(f"mxint8 streaming T={T}")
    li = layer_of(synth.Shape(T, 4096, 256, 8, 1024, "bf16", "mxint8"), batch=60 + T)
    sh = lshape(li, path)
    assert "router_logits" in pm.forward_stages(sh)
    got = run_forward(DevLayer(li), path=path)
    compare_forward(li, got, label=f"mxint8 streaming T={T}")


@pytest.mark.parametrize("T,H,E,K,I,path", [(130, 1024, 32, 4, 256, pm.PATH_GROUPED),
                                            (333, 512, 16, 6, 512, pm.PATH_GROUPED),
                                            (150, 1280, 16, 4, 768, pm.PATH_GROUPED),
                                            (512, 4096, 256, 8, 1024, pm.PATH_AUTO)])
def test_forward_mxint8_grouped(T, H, E, K, I, path):
    """MXINT8 on the grouped MFMA GEMMs (codes dequantised into LDS with the block's power
    of two): ragged m-tiles, skewed groups, and AUTO's choice at 512 tokens.  H and I that
    are multiples of 512 take the tile's scales from an LDS table; H = 1280 and I = 256 or
    768 load them step by step."""
    note(f"mxint8 grouped T={T} H={H} E={E}")
    li = layer_of(synth.Shape(T, H, E, K, I, "bf16", "mxint8", bias="zipf" if T == 333 else "normal"), seed=11)
    sh = lshape(li, path)
    assert "gate_up" in pm.forward_stages(sh) and "topk" not in pm.forward_stages(sh)[:1]
    got = run_forward(DevLayer(li), path=path)
    compare_forward(li, got, label=f"mxint8 grouped T={T}")


@pytest.mark.parametrize("T", [1, 2, 3, 5, 8, 9, 13])
def test_forward_token_sweep(T):
    note(f"token sweep T={T}")
    li = layer_of(synth.Shape(T, 2048, 128, 8, 768, "bf16", "bf16", bias="normal"), batch=T)
    got = run_forward(DevLayer(li))
    compare_forward(li, got, label=f"sweep T={T}")


@pytest.mark.parametrize("I", [64, 128])
@pytest.mark.parametrize("K,renorm,E", [(1, True, 8), (8, True, 8), (3, False, 16), (32, True, 64)])
def test_forward_k_and_renorm_edges(K, renorm, E, I):
    """Six tokens: I = 64 runs the staged decode kernels, I = 128 the fused kernel's per-wave top-k."""
    li = layer_of(synth.Shape(6, 256, E, K, I, "bf16", "bf16", bias="normal", renorm=renorm))
    assert pm.forward_stages(lshape(li))[0] == ("decode_fused" if I == 128 else "router_logits")
    got = run_forward(DevLayer(li))
    compare_forward(li, got, label=f"K={K} renorm={renorm} E={E} I={I}")


@pytest.mark.parametrize("K,renorm,E", [(1, True, 8), (8, True, 8), (3, False, 16), (32, True, 64), (8, False, 128),
                                         (8, True, 128), (8, False, 256), (8, True, 256), (1, True, 256),
                                         (8, True, 130), (5, False, 512), (9, True, 256), (16, False, 200)])
def test_forward_single_token_k_and_renorm(K, renorm, E):
    """One decode token: the fused kernel's one-token selections -- ranks counted over all E
    (E <= 128), ranks in two levels (E <= 512, k <= 8; E = 130 leaves its last wave two experts,
    fewer than k) and the per-wave top-k (k = 9 and 16) -- with k = 1, k = E, renorm on and off."""
    note(f"single token K={K} renorm={renorm} E={E}")
    li = layer_of(synth.Shape(1, 256, E, K, 128, "bf16", "bf16", bias="normal", renorm=renorm), batch=3)
    got = run_forward(DevLayer(li))
    assert pm.forward_stages(lshape(li)) == ["decode_fused"]
    compare_forward(li, got, label=f"T=1 K={K} renorm={renorm} E={E}")


@pytest.mark.parametrize("E,K,tied", [(12, 3, (2, 5, 9, 11)), (200, 3, (2, 5, 9, 11)), (200, 3, (199, 70, 5, 130)),
                                      (200, 12, (2, 5, 9, 11))])
def test_forward_single_token_exact_ties(E, K, tied):
    """One token whose best logits tie exactly (identical router rows): the lower ids win, in the
    fused kernel's one-token selections -- ranks over all E (E = 12), ranks in two levels with the
    tied experts in one wave's group or spread over four (E = 200, k = 3) -- and its per-wave top-k
    (k = 12)."""
    li = layer_of(synth.Shape(1, 256, E, K, 128, "bf16", "bf16"))
    assert pm.forward_stages(lshape(li)) == ["decode_fused"]
    row = synth.bf16_bits_to_f32(li.wr[2])
    s = float(synth.bf16_bits_to_f32(li.x[0]).astype(np.float64) @ row.astype(np.float64))
    popular = synth.f32_to_bf16_bits(row * (64.0 if s > 0 else -64.0))   # exact: a power of two
    for e in tied:   # four equal, largest logits for the first three places
        li.wr[e] = popular
    got = run_forward(DevLayer(li))
    ref = oracle.router(oracle_layer(li))
    kept = set(ref["ids"][0].tolist())   # ids come in ascending id order
    assert kept >= set(sorted(tied)[:3]) and (K > 3 or sorted(tied)[3] not in kept)
    np.testing.assert_array_equal(got["ids"], ref["ids"])
    np.testing.assert_allclose(got["w"], ref["w"], rtol=0, atol=W_TOL)


@pytest.mark.parametrize("T,K,renorm,E", [(6, 8, True, 130), (8, 8, False, 512), (3, 8, True, 256), (8, 1, True, 200),
                                           (2, 4, False, 64), (5, 9, True, 256)])
def test_forward_multi_token_selection(T, K, renorm, E):
    """Two to eight decode tokens in the fused kernel's per-wave top-k (arg-max rounds): E = 130
    (a 64-lane pass with two experts), E = 512 (eight logits per lane), k = 1 and 9, renorm on
    and off."""
    note(f"multi token T={T} K={K} renorm={renorm} E={E}")
    li = layer_of(synth.Shape(T, 256, E, K, 128, "bf16", "bf16", bias="normal", renorm=renorm), batch=3)
    assert pm.forward_stages(lshape(li)) == ["decode_fused"]
    got = run_forward(DevLayer(li))
    compare_forward(li, got, label=f"T={T} K={K} renorm={renorm} E={E}")


@pytest.mark.parametrize("K", [3, 9])
def test_forward_multi_token_exact_ties(K):
    """Four tokens, three of them the same, whose best logits tie exactly on experts in four
    different 64-lane passes (identical router rows): the lower ids win in the per-wave top-k,
    with the tie at the cut (k = 3) and inside the kept set (k = 9)."""
    li = layer_of(synth.Shape(4, 256, 200, K, 128, "bf16", "bf16"))
    assert pm.forward_stages(lshape(li)) == ["decode_fused"]
    li.x[1] = li.x[0]
    li.x[2] = li.x[0]
    row = synth.bf16_bits_to_f32(li.wr[2])
    s = float(synth.bf16_bits_to_f32(li.x[0]).astype(np.float64) @ row.astype(np.float64))
    popular = synth.f32_to_bf16_bits(row * (64.0 if s > 0 else -64.0))   # exact: a power of two
    for e in (199, 70, 5, 130):
        li.wr[e] = popular
    got = run_forward(DevLayer(li))
    ref = oracle.router(oracle_layer(li))
    for t in range(3):   # ids come in ascending id order
        kept = set(ref["ids"][t].tolist())
        assert kept >= {5, 70, 130} and (K > 3 or 199 not in kept)
    np.testing.assert_array_equal(got["ids"], ref["ids"])
    np.testing.assert_allclose(got["w"], ref["w"], rtol=0, atol=W_TOL)
    compare_forward(li, got, label=f"T=4 ties K={K}")


def test_forward_zero_tokens_is_noop():
    li = layer("c0_tiny_f32")
    dl = DevLayer(li)
    sh = lshape(li, T=0)
    ws = pm.alloc_workspace(sh)
    y = torch.full((4,), 3.0, device="cuda")
    pm.forward(sh, dl.x, dl.wr, None, dl.weights, y, ws)
    torch.cuda.synchronize()
    assert torch.all(y == 3.0)


def test_forward_deterministic():
    li = layer("c2_decode8_bf16")
    dl = DevLayer(li)
    a = run_forward(dl)
    b = run_forward(dl)
    assert torch.equal(a["y"], b["y"])
    np.testing.assert_array_equal(a["ids"], b["ids"])


def test_forward_identical_experts_closed_form():
    """All experts equal (renorm on): y = FFN(x) whatever the routing."""
    li = layer_of(synth.Shape(7, 256, 8, 3, 64, "bf16", "bf16", bias="normal"))
    for n in ("wg", "wu", "wd"):
        a = getattr(li, n)
        setattr(li, n, np.ascontiguousarray(np.broadcast_to(a[:1], a.shape)))
    got = run_forward(DevLayer(li))
    L1 = oracle.Layer(x=li.x, wr=li.wr[:1].copy(), wg=li.wg[:1].copy(), wu=li.wu[:1].copy(), wd=li.wd[:1].copy(),
                      top_k=1)
    ffn = oracle.forward(L1)["y"]
    assert rel_l2(to_f64(got["y"], "bf16"), ffn) <= 1e-2


def test_forward_graph_capture_replays_match_eager():
    """moe_forward makes no host synchronisation or device read: it can be captured in a
    HIP graph; every replay (with eager work and syncs between them) equals the eager run."""
    li = layer("c2_decode8_bf16")
    dl = DevLayer(li)
    sh = lshape(li)
    ws = pm.alloc_workspace(sh)
    xs = [dl.x, tdev(synth.make_x(li.shape, batch=1)), tdev(synth.make_x(li.shape, batch=2))]
    ys = [torch.empty(li.shape.T, li.shape.H, dtype=torch.int16, device="cuda") for _ in xs]
    for x, y in zip(xs, ys):
        pm.forward(sh, x, dl.wr, dl.bias, dl.weights, y, ws)
    torch.cuda.synchronize()
    eager = [y.clone() for y in ys]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for x, y in zip(xs, ys):
            pm.forward(sh, x, dl.wr, dl.bias, dl.weights, y, ws)
    for r in range(4):
        for y in ys:
            y.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for y, e in zip(ys, eager):
            assert torch.equal(y, e), f"replay {r}"
        pm.forward(sh, xs[0], dl.wr, dl.bias, dl.weights, ys[0], ws)   # eager work between replays
        torch.cuda.synchronize()


# ---- streaming GEMV family beyond 8 tokens (medium batches) -------------------------------------

@pytest.mark.parametrize("T,w,path", [(24, "bf16", pm.PATH_AUTO), (48, "bf16", pm.PATH_DECODE),
                                      (40, "mxfp4", pm.PATH_AUTO), (20, "mxfp4", pm.PATH_DECODE)])
def test_forward_medium_batch_streaming(T, w, path):
    """Tens of tokens on the streaming family (tokens staged in LDS, MXFP4 decoded once
    per row, several row passes per work-group): ids exact, y of every token against the
    oracle."""
    note(f"medium batch T={T} {w}")
    if w == "bf16":
        sh_ = synth.Shape(T, 2048, 128, 8, 768, "bf16", "bf16", bias="normal")
    else:
        sh_ = synth.Shape(T, 4096, 256, 8, 1024, "bf16", "mxfp4")
    li = layer_of(sh_, batch=70 + T)
    got = run_forward(DevLayer(li), path=path)
    compare_forward(li, got, label=f"medium T={T} {w}")


# ---- grouped MFMA family ----------------------------------------------------------------------

@pytest.mark.parametrize("T", [1, 8, 129])
def test_forward_grouped_path_forced(T):
    """The MFMA grouped family must match the oracle at any T, also decode sizes."""
    note(f"grouped forced T={T}")
    li = layer_of(synth.Shape(T, 2048, 128, 8, 768, "bf16", "bf16", bias="normal"), batch=50 + T)
    got = run_forward(DevLayer(li), path=pm.PATH_GROUPED)
    compare_forward(li, got, label=f"grouped T={T}")


def test_forward_grouped_ragged_zipf():
    """333 tokens with a strongly skewed router: partial m-tiles, empty experts."""
    sh_ = synth.Shape(333, 256, 64, 6, 256, "bf16", "bf16", bias="zipf")
    li = synth.make_layer(sh_, beta=2.0)
    got = run_forward(DevLayer(li))
    counts = np.bincount(got["ids"].ravel(), minlength=64)
    note(f"  group sizes max {counts.max()} empty {(counts == 0).sum()}")
    compare_forward(li, got, label="grouped ragged zipf")


@pytest.mark.parametrize("T,H,E,K,I,beta", [(333, 512, 16, 4, 256, 2.0), (1000, 1024, 32, 8, 512, 1.0),
                                           (200, 512, 8, 2, 128, 1.0), (150, 768, 8, 2, 384, 1.0)])
def test_forward_grouped_wide_tiles_ragged(T, H, E, K, I, beta):
    """Shapes that take the large-tile kernels for the expert GEMMs (gate/up: I a
    multiple of 128; down: H a multiple of 256): skewed groups with partial m-tiles,
    several n-tiles.  I = 128 gives the down projection the fewest 64-deep stages (two);
    H = 768 and I = 384 give three n-tiles to each GEMM."""
    note(f"grouped wide T={T} H={H} E={E} K={K} I={I}")
    sh_ = synth.Shape(T, H, E, K, I, "bf16", "bf16", bias="zipf")
    li = synth.make_layer(sh_, beta=beta)
    got = run_forward(DevLayer(li), path=pm.PATH_GROUPED)
    counts = np.bincount(got["ids"].ravel(), minlength=E)
    note(f"  group sizes max {counts.max()} empty {(counts == 0).sum()}")
    compare_forward(li, got, label=f"grouped wide T={T}")


def test_forward_grouped_top10():
    """k = 10 on the grouped path: the combine of each token's rows takes a batch of eight and
    a tail of two."""
    sh_ = synth.Shape(100, 512, 32, 10, 256, "bf16", "bf16", bias="normal")
    li = synth.make_layer(sh_)
    got = run_forward(DevLayer(li), path=pm.PATH_GROUPED)
    compare_forward(li, got, label="grouped top-10")


def test_forward_grouped_wide_persistent_tiles():
    """2048 tokens on the large-tile kernels: the gate/up grid holds one work-group per CU
    and each walks four or five of the ~1100 tiles, so the next-tile prefetch and the hand
    over of ring slots under the epilogue run many times.  Ids, y and the call's own
    grouping on every token."""
    sh_ = synth.Shape(2048, 512, 16, 8, 1024, "bf16", "bf16", bias="zipf")
    li = synth.make_layer(sh_, beta=1.0)
    note("grouped wide persistent T=2048 H=512 E=16 K=8 I=1024")
    got = run_forward(DevLayer(li), path=pm.PATH_GROUPED)
    ref = oracle.router(oracle_layer(li))
    mism = (got["ids"] != ref["ids"]).any(1)
    assert not (mism & ~ref["near"]).any()
    compare_forward(li, got, label="grouped wide persistent")
    sh = lshape(li, pm.PATH_GROUPED)
    off, srt, pos = forward_grouping(sh, got["ws"])
    roff, rsrt, rpos = oracle.group(got["ids"], li.shape.E)
    np.testing.assert_array_equal(off, roff)
    np.testing.assert_array_equal(srt, rsrt)
    np.testing.assert_array_equal(pos, rpos)


@pytest.mark.parametrize("T,H,E,K,I", [(300, 1024, 32, 4, 512), (160, 2048, 16, 8, 1024), (200, 1024, 32, 4, 512),
                                       (90, 4096, 256, 8, 1024)])
def test_forward_grouped_wide_tiles_mxfp4(T, H, E, K, I):
    """MXFP4 experts on the large-tile kernels (codes and scales loaded straight into LDS,
    decoded per operand read): skewed groups, partial m-tiles, several n-tiles.  The last two
    shapes average at most 32 pairs per expert, so they run on 64-row m-tiles."""
    note(f"grouped wide mxfp4 T={T} H={H} E={E} K={K} I={I}")
    sh_ = synth.Shape(T, H, E, K, I, "bf16", "mxfp4", bias="zipf")
    li = synth.make_layer(sh_, beta=1.0)
    got = run_forward(DevLayer(li), path=pm.PATH_GROUPED)
    compare_forward(li, got, label=f"grouped wide mxfp4 T={T}")


def test_staged_expert_ffn_grouped_path():
    """moe_expert_ffn on the grouped family: fp32 expert outputs in sorted order."""
    li = layer_of(synth.Shape(77, 256, 16, 4, 128, "bf16", "bf16", bias="normal"))
    dl = DevLayer(li)
    T, K, E, H = li.shape.T, li.shape.K, li.shape.E, li.shape.H
    sh = lshape(li, path=pm.PATH_GROUPED)
    ws = pm.alloc_workspace(sh)
    ref = oracle.router(oracle_layer(li))
    ids_np = ref["ids"]
    off, srt, pos = oracle.group(ids_np, E)
    obuf, o = guarded(T * K * H, torch.float32)
    pm.expert_ffn(sh, dl.x, dl.weights, tdev(off), tdev(srt), o.view(T * K, H), ws)
    torch.cuda.synchronize()
    assert canary_ok(obuf, T * K * H, torch.float32)
    oref = oracle.expert_pairs(oracle_layer(li), srt // K, ids_np.reshape(-1)[srt])
    r = rel_l2(o.view(T * K, H).cpu().numpy(), oref)
    assert r <= 1e-2, r


def test_forward_grouped_mxfp4_small():
    """MXFP4 experts on the grouped MFMA family (codes dequantised to bf16 in LDS)."""
    li = layer_of(synth.Shape(77, 256, 16, 4, 128, "bf16", "mxfp4", bias="normal"))
    got = run_forward(DevLayer(li), path=pm.PATH_GROUPED)
    compare_forward(li, got, label="grouped mxfp4 small")
