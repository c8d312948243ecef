"""moe_forward_noalloc (the entry point for callers that cannot allocate: the
workspace is the library's own per-device scratch) against moe_forward on a
caller workspace: the same kernels on the same inputs, so ids, weights and y
must agree bit for bit.  Two calls in a row, the second smaller, so the second
runs on what the first left in the scratch.  Needs an MI355X; run with -m gpu."""
import ctypes

import numpy as np
import pytest
import torch

import prefill_moe_router_amd as pm
import synth
from tests.gpu_common import DevLayer, compare_forward, layer_of, lshape, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    pm.lib()


def _both(dl, path=pm.PATH_AUTO):
    li = dl.li
    sh = lshape(li, path)
    T, K, H = li.shape.T, li.shape.K, li.shape.H
    out = []
    for noalloc in (False, True):
        y = torch.full((T, H), 7, dtype=dl.act_torch(), device="cuda")
        ids = torch.full((T, K), -7, dtype=torch.int32, device="cuda")
        w = torch.full((T, K), -7.0, dtype=torch.float32, device="cuda")
        if noalloc:
            err = torch.full((4,), -1, dtype=torch.int32, device="cuda")
            pm.forward_noalloc(sh, dl.x, dl.wr, dl.bias, dl.weights, y, ids, w, device_err=err)
            torch.cuda.synchronize()
            assert int(err[0]) == 0, f"device error bits {int(err[0])}"
        else:
            ws = pm.alloc_workspace(sh)
            pm.forward(sh, dl.x, dl.wr, dl.bias, dl.weights, y, ws, ids, w)
            torch.cuda.synchronize()
            assert pm.check_device_error(ws) == 0
        out.append(dict(y=y, ids=ids.cpu().numpy(), w=w.cpu().numpy()))
    return out


@pytest.mark.parametrize("case", ["decode_then_smaller", "medium_then_decode", "mxfp4_decode_then_smaller"])
def test_noalloc_matches_workspace_call_twice(case):
    """Two calls in a row on the scratch, the second with fewer tokens: each equals the
    caller-workspace call bit for bit and matches the oracle."""
    if case == "decode_then_smaller":
        shapes = [synth.Shape(8, 2048, 128, 8, 768, "bf16", "bf16", bias="normal"),
                  synth.Shape(3, 2048, 128, 8, 768, "bf16", "bf16", bias="normal")]
    elif case == "medium_then_decode":
        shapes = [synth.Shape(40, 2048, 128, 8, 768, "bf16", "bf16", bias="normal"),
                  synth.Shape(1, 2048, 128, 8, 768, "bf16", "bf16")]
    else:
        shapes = [synth.Shape(8, 4096, 256, 8, 1024, "bf16", "mxfp4"),
                  synth.Shape(2, 4096, 256, 8, 1024, "bf16", "mxfp4")]
    for i, shp in enumerate(shapes):
        note(f"noalloc {case} call {i}: T={shp.T} H={shp.H} E={shp.E} {shp.w}")
        li = layer_of(shp, batch=40 + i)
        dl = DevLayer(li)
        ref, got = _both(dl)
        assert torch.equal(got["y"], ref["y"]), f"call {i}: y differs from the workspace call"
        np.testing.assert_array_equal(got["ids"], ref["ids"])
        np.testing.assert_array_equal(got["w"], ref["w"])
        compare_forward(li, got, label=f"noalloc {case} call {i}")


def test_noalloc_rejects_shapes_beyond_the_scratch():
    """A shape whose workspace exceeds the scratch is refused before anything is enqueued
    (the 8192-token chunk needs ~0.7 GB)."""
    sh = pm.LayerShape(8192, 2048, 128, 8, 768)
    assert pm.workspace_size(sh) > pm.NOALLOC_SCRATCH_BYTES
    y = torch.empty(8192, 2048, dtype=torch.int16, device="cuda")
    w = dict(wg=y, wu=y, wd=y)
    with pytest.raises(pm.MoeError) as e:
        pm.forward_noalloc(sh, y, y, None, w, y)
    assert e.value.status == pm.ERR_WORKSPACE
