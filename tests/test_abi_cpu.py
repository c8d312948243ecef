"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, sizes workspaces, and rejects bad arguments on the host
before launching anything."""
import ctypes
import os
import re

import pytest

import prefill_moe_router_amd as pm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(pm.LIB_PATH), reason="libmoe_router.so not built")

FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first


def _declared_functions():
    names = []
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            src = open(os.path.join(ROOT, "include", f)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(moe_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_functions_exported():
    names = _declared_functions()
    assert set(names) == set(pm.EXPORTS), names
    L = pm.lib()
    for n in names:
        assert hasattr(L, n), n


def _shape(**kw):
    base = dict(num_tokens=4, hidden=2048, num_experts=128, top_k=8, intermediate=768)
    base.update(kw)
    return pm.LayerShape(**base)


def test_workspace_size_grows_with_tokens():
    a = pm.workspace_size(_shape(num_tokens=1))
    b = pm.workspace_size(_shape(num_tokens=8192))
    assert 0 < a < b
    assert a % 256 == 0 and b % 256 == 0


@pytest.mark.parametrize("kw", [dict(top_k=0), dict(top_k=129), dict(num_tokens=-1), dict(hidden=100),
                                dict(intermediate=12), dict(act_dtype=7), dict(weight_dtype=5),
                                dict(weight_dtype=pm.MXFP4, hidden=2048 + 16), dict(path=9)])
def test_bad_shapes_get_zero_workspace(kw):
    assert pm.workspace_size(_shape(**kw)) == 0


@pytest.mark.parametrize("kw", [dict(num_experts=2048, top_k=8), dict(top_k=64, num_experts=128),
                                dict(act_dtype=pm.F32, weight_dtype=pm.BF16)])
def test_unsupported_combinations(kw):
    s = _shape(**kw).c()
    st = pm.lib().moe_router_topk(ctypes.byref(s), FAKE, FAKE, None, FAKE, FAKE, FAKE, 1 << 40, None)
    assert st == pm.ERR_UNSUPPORTED


def _router(shape, x=FAKE, wr=FAKE, bias=None, ids=FAKE, w=FAKE, ws=FAKE, nbytes=None):
    s = shape.c()
    if nbytes is None:
        nbytes = pm.workspace_size(shape)
    return pm.lib().moe_router_topk(ctypes.byref(s), x, wr, bias, ids, w, ws, nbytes, None)


def test_router_validation():
    sh = _shape()
    assert _router(sh, x=None) == pm.ERR_INVALID_ARG
    assert _router(sh, x=FAKE + 4) == pm.ERR_INVALID_ARG          # misaligned
    assert _router(sh, bias=FAKE + 2) == pm.ERR_INVALID_ARG
    assert _router(sh, ws=None) == pm.ERR_INVALID_ARG
    assert _router(sh, nbytes=pm.workspace_size(sh) - 1) == pm.ERR_WORKSPACE
    # T == 0 is a no-op that launches nothing
    assert _router(_shape(num_tokens=0)) == pm.OK


def test_forward_validation():
    sh = _shape()
    s = sh.c()
    w = pm.ExpertWeights(FAKE, FAKE, FAKE, None, None, None)
    n = pm.workspace_size(sh)
    L = pm.lib()
    assert L.moe_forward(ctypes.byref(s), FAKE, FAKE, None, None, FAKE, None, None, FAKE, n, None) == pm.ERR_INVALID_ARG
    wbad = pm.ExpertWeights(FAKE, None, FAKE, None, None, None)
    assert L.moe_forward(ctypes.byref(s), FAKE, FAKE, None, ctypes.byref(wbad), FAKE, None, None, FAKE, n,
                         None) == pm.ERR_INVALID_ARG
    # MXFP4 needs its scale arrays
    smx = _shape(weight_dtype=pm.MXFP4).c()
    nmx = pm.workspace_size(_shape(weight_dtype=pm.MXFP4))
    assert L.moe_forward(ctypes.byref(smx), FAKE, FAKE, None, ctypes.byref(w), FAKE, None, None, FAKE, nmx,
                         None) == pm.ERR_INVALID_ARG
    s0 = _shape(num_tokens=0).c()
    assert L.moe_forward(ctypes.byref(s0), FAKE, FAKE, None, ctypes.byref(w), FAKE, None, None, FAKE,
                         pm.workspace_size(_shape(num_tokens=0)), None) == pm.OK


def test_scale_pointers_must_be_16_byte_aligned():
    """MXFP4 and NVFP4 scale arrays follow the header's 16-byte rule for device pointers."""
    L = pm.lib()
    for fmt in (pm.MXFP4, pm.NVFP4, pm.MXINT8):
        shp = _shape(weight_dtype=fmt)
        s = shp.c()
        n = pm.workspace_size(shp)
        for bad in (FAKE + 1, FAKE + 2, FAKE + 8):
            for pos in range(3):
                sc = [FAKE, FAKE, FAKE]
                sc[pos] = bad
                w = pm.ExpertWeights(FAKE, FAKE, FAKE, *sc, 1.0, 1.0, 1.0)
                assert L.moe_forward(ctypes.byref(s), FAKE, FAKE, None, ctypes.byref(w), FAKE, None, None, FAKE, n,
                                     None) == pm.ERR_INVALID_ARG, (fmt, bad, pos)


def test_forward_grouping_validation():
    """The grouping view: decode shapes keep their grouping on chip (unsupported); null
    outputs, a short workspace and bad shapes are rejected before any copy."""
    L = pm.lib()
    def grp(shp, ws=FAKE, nbytes=None, off=FAKE, srt=FAKE, pos=FAKE):
        s = shp.c()
        nb = pm.workspace_size(shp) if nbytes is None else nbytes
        return L.moe_forward_grouping(ctypes.byref(s), ws, nb, off, srt, pos, None)
    assert pm.forward_stages(_shape(num_tokens=1)) == ["decode_fused"]
    assert grp(_shape(num_tokens=1)) == pm.ERR_UNSUPPORTED
    big = _shape(num_tokens=8192)
    assert grp(big, off=None) == pm.ERR_INVALID_ARG
    assert grp(big, srt=None) == pm.ERR_INVALID_ARG
    assert grp(big, pos=FAKE + 4) == pm.ERR_INVALID_ARG
    assert grp(big, ws=None) == pm.ERR_INVALID_ARG
    assert grp(big, nbytes=pm.workspace_size(big) - 1) == pm.ERR_WORKSPACE
    assert grp(_shape(top_k=0), nbytes=1 << 30) == pm.ERR_INVALID_ARG


def test_noalloc_refuses_shapes_beyond_its_scratch_before_any_device_call():
    """moe_forward_noalloc checks the shape's workspace need against its fixed per-device
    scratch first: too large gives MOE_ERR_WORKSPACE, a bad shape MOE_ERR_INVALID_ARG, a
    misaligned error word MOE_ERR_INVALID_ARG (no device needed for any of these)."""
    L = pm.lib()
    w = pm.ExpertWeights(FAKE, FAKE, FAKE, None, None, None)
    def call(shp, err=None):
        s = shp.c()
        return L.moe_forward_noalloc(ctypes.byref(s), FAKE, FAKE, None, ctypes.byref(w), FAKE, None, None, err, None)
    big = _shape(num_tokens=8192)
    assert pm.workspace_size(big) > pm.NOALLOC_SCRATCH_BYTES
    assert call(big) == pm.ERR_WORKSPACE
    assert call(_shape(top_k=0)) == pm.ERR_INVALID_ARG
    assert call(_shape(num_tokens=1), err=FAKE + 4) == pm.ERR_INVALID_ARG
    # every decode batch of the largest supported shape fits
    assert pm.workspace_size(_shape(num_tokens=8, hidden=8192, intermediate=8192, num_experts=1024,
                                    top_k=32)) <= pm.NOALLOC_SCRATCH_BYTES


def test_nvfp4_validation():
    """NVFP4 experts: scale arrays required and 16-byte aligned, finite tensor scales; AUTO
    takes the grouped GEMMs from four pairs per expert (MXFP4: 1.5)."""
    L = pm.lib()
    shp = _shape(weight_dtype=pm.NVFP4)
    s = shp.c()
    n = pm.workspace_size(shp)
    def fwd(w, sh=s, nb=n):
        return L.moe_forward(ctypes.byref(sh), FAKE, FAKE, None, ctypes.byref(w), FAKE, None, None, FAKE, nb, None)
    assert fwd(pm.ExpertWeights(FAKE, FAKE, FAKE, None, None, None, 1.0, 1.0, 1.0)) == pm.ERR_INVALID_ARG
    assert fwd(pm.ExpertWeights(FAKE, FAKE, FAKE, FAKE, FAKE + 1, FAKE, 1.0, 1.0, 1.0)) == pm.ERR_INVALID_ARG
    assert fwd(pm.ExpertWeights(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1.0, float("inf"), 1.0)) == pm.ERR_INVALID_ARG
    assert fwd(pm.ExpertWeights(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, float("nan"), 1.0, 1.0)) == pm.ERR_INVALID_ARG
    # E = 128, k = 8: streaming below 64 tokens, grouped from 64
    for T, grouped in ((9, False), (63, False), (64, True), (4096, True)):
        stages = pm.forward_stages(_shape(weight_dtype=pm.NVFP4, num_tokens=T))
        assert ("router_topk" in stages) == grouped and "gate_up" in stages, (T, stages)
    # MXFP4 switches at 1.5 pairs per expert: 24 tokens at E = 128, k = 8
    for T, grouped in ((23, False), (24, True)):
        stages = pm.forward_stages(_shape(weight_dtype=pm.MXFP4, num_tokens=T))
        assert ("router_topk" in stages) == grouped and "gate_up" in stages, (T, stages)
    # with fp32 activations NVFP4 is not a supported pair
    assert pm.workspace_size(_shape(weight_dtype=pm.NVFP4, act_dtype=pm.F32)) == 0


def test_mxint8_validation():
    """MXINT8 experts: bf16 activations only, H and I multiples of the 32-element scale
    block, scale arrays required; AUTO takes the grouped GEMMs from 1.25 pairs per expert."""
    assert pm.workspace_size(_shape(weight_dtype=pm.MXINT8)) > 0
    assert pm.workspace_size(_shape(weight_dtype=pm.MXINT8, hidden=2048 + 16)) == 0
    assert pm.workspace_size(_shape(weight_dtype=pm.MXINT8, intermediate=768 + 8)) == 0
    assert pm.workspace_size(_shape(weight_dtype=pm.MXINT8, act_dtype=pm.F32)) == 0
    L = pm.lib()
    shp = _shape(weight_dtype=pm.MXINT8)
    s = shp.c()
    w = pm.ExpertWeights(FAKE, FAKE, FAKE, None, FAKE, FAKE)
    assert L.moe_forward(ctypes.byref(s), FAKE, FAKE, None, ctypes.byref(w), FAKE, None, None, FAKE,
                         pm.workspace_size(shp), None) == pm.ERR_INVALID_ARG
    for T, grouped in ((19, False), (20, True)):   # 1.25 pairs per expert at E = 128, k = 8
        stages = pm.forward_stages(_shape(weight_dtype=pm.MXINT8, num_tokens=T))
        assert ("router_topk" in stages) == grouped and "gate_up" in stages, (T, stages)
    assert pm.forward_stages(_shape(weight_dtype=pm.MXINT8, num_tokens=8, hidden=4096, num_experts=256,
                                    intermediate=1024)) == ["decode_fused"]


def test_status_strings():
    for st in (pm.OK, pm.ERR_INVALID_ARG, pm.ERR_UNSUPPORTED, pm.ERR_WORKSPACE, pm.ERR_HIP, pm.ERR_DEVICE):
        assert pm.status_string(st) and pm.status_string(st) != "unknown status"
    assert pm.status_string(12345) == "unknown status"
