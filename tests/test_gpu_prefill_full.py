"""Whole prefill chunks through moe_forward, checked on every token: expert ids
against the oracle's routing, the call's own device grouping bit for bit
against the oracle's grouping of those ids, and y of every token against the
oracle within the format's tolerance.  Needs an MI355X; run with -m gpu.

The chunks are the 8192-token bf16 chunk with its Zipf-skewed routing, the
4096-token MXFP4, NVFP4 and MXINT8 chunks, and the 8192-token chunk with 8
decode rows appended in one call.  Each chunk runs once per module; the y comparison is
split in four token ranges so that no single test holds the oracle for long.
"""
import numpy as np
import pytest
import torch

import oracle
import prefill_moe_router_amd as pm
from tests.gpu_common import DevLayer, compare_forward, forward_grouping, layer, lshape, note, run_forward
from tests.helpers import grouping_violations, oracle_layer

pytestmark = pytest.mark.gpu

CHUNKS = ["c3_prefill8192_bf16", "c4_mxfp4_prefill4096", "c5_nvfp4_prefill4096", "c6_mxint8_prefill4096",
          "c3_mixed8200_bf16"]
PARTS = 4

_RUNS = {}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    pm.lib()
    yield
    _RUNS.clear()


def _run(name):
    """One moe_forward over the whole chunk; y, ids, weights and the call's grouping on the host."""
    if name not in _RUNS:
        li = layer(name)
        note(f"whole chunk {name}: T={li.shape.T} stages={','.join(pm.forward_stages(lshape(li)))}")
        dl = DevLayer(li)
        got = run_forward(dl)
        off, srt, pos = forward_grouping(lshape(li), got["ws"])
        _RUNS[name] = dict(y=got["y"].cpu(), ids=got["ids"], w=got["w"], off=off, srt=srt, pos=pos)
        del dl, got
        torch.cuda.empty_cache()
    return layer(name), _RUNS[name]


@pytest.mark.parametrize("name", CHUNKS)
def test_chunk_ids_and_device_grouping(name):
    """Ids of every token bit-exact away from the oracle's near-ties; the grouping the call
    built on the device (count, scan and placement kernels) equals the oracle's grouping
    of the call's own ids, and meets the grouping's defining properties."""
    li, got = _run(name)
    E = li.shape.E
    ref = oracle.router(oracle_layer(li))
    mism = (got["ids"] != ref["ids"]).any(1)
    assert not (mism & ~ref["near"]).any(), np.nonzero(mism & ~ref["near"])[0][:10]
    roff, rsrt, rpos = oracle.group(got["ids"], E)
    np.testing.assert_array_equal(got["off"], roff)
    np.testing.assert_array_equal(got["srt"], rsrt)
    np.testing.assert_array_equal(got["pos"], rpos)
    assert grouping_violations(got["ids"], E, got["off"], got["srt"], got["pos"]) == []
    sizes = np.diff(roff)
    note(f"  {name}: near-ties {int(ref['near'].sum())}, id mismatches {int(mism.sum())}, "
         f"groups max {sizes.max()} empty {(sizes == 0).sum()}")


@pytest.mark.parametrize("part", range(PARTS))
@pytest.mark.parametrize("name", [c for c in CHUNKS if c != "c3_mixed8200_bf16"])
def test_chunk_y_every_token(name, part):
    """y of every token against the oracle (forced to the GPU's ids on near-ties), a quarter
    of the chunk per test."""
    li, got = _run(name)
    T = li.shape.T
    toks = np.arange(part * T // PARTS, (part + 1) * T // PARTS)
    compare_forward(li, got, tokens=toks, label=f"{name} tokens {toks[0]}..{toks[-1]}")


def test_mixed_chunk_rows_equal_chunk_alone_and_decode_rows_match_oracle():
    """The 8192-token chunk with 8 decode rows appended: the first 8192 rows of x are the
    chunk's, and a token's output depends only on its own row and routing, so those rows
    of y equal the chunk-alone call's bit for bit; the 8 decode rows match the oracle."""
    li_c, chunk = _run("c3_prefill8192_bf16")
    li, got = _run("c3_mixed8200_bf16")
    Tc = li_c.shape.T
    assert np.array_equal(li.x[:Tc], li_c.x)
    np.testing.assert_array_equal(got["ids"][:Tc], chunk["ids"])
    assert torch.equal(got["y"][:Tc], chunk["y"]), "mixed call changed the chunk's rows"
    compare_forward(li, got, tokens=np.arange(Tc, li.shape.T), label="mixed: decode rows")


def test_mixed_chunk_graph_replays_match_eager():
    """The mixed call captured in one HIP graph: every replay (with eager work and
    synchronisations between them) equals the eager call, ids and weights included."""
    li = layer("c3_mixed8200_bf16")
    dl = DevLayer(li)
    sh = lshape(li)
    T = li.shape.T
    ws = pm.alloc_workspace(sh)
    y = torch.empty(T, li.shape.H, dtype=torch.int16, device="cuda")
    ids = torch.empty(T, li.shape.K, dtype=torch.int32, device="cuda")
    w = torch.empty(T, li.shape.K, dtype=torch.float32, device="cuda")
    pm.forward(sh, dl.x, dl.wr, dl.bias, dl.weights, y, ws, ids, w)
    torch.cuda.synchronize()
    eager = (y.clone(), ids.clone(), w.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pm.forward(sh, dl.x, dl.wr, dl.bias, dl.weights, y, ws, ids, w)
    for r in range(3):
        y.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager[0]) and torch.equal(ids, eager[1]) and torch.equal(w, eager[2]), f"replay {r}"
        pm.forward(sh, dl.x, dl.wr, dl.bias, dl.weights, y, ws, ids, w)
        torch.cuda.synchronize()
    if "c3_mixed8200_bf16" in _RUNS:
        assert torch.equal(y.cpu(), _RUNS["c3_mixed8200_bf16"]["y"])
