"""Helpers for the GPU parity tests: device upload of synthetic layers, calls
through the C ABI, and comparison against the oracle."""
from __future__ import annotations

import functools
import sys

import numpy as np
import torch

import oracle
import prefill_moe_router_amd as pm
import synth
from tests.helpers import max_abs, oracle_layer, rel_l2

# tolerances of the layer output against the fp64 oracle
TOL = {"bf16": dict(rel_l2=1e-2, max_abs=3e-2), "mxfp4": dict(rel_l2=2e-2, max_abs=None),
       "nvfp4": dict(rel_l2=2e-2, max_abs=None), "mxint8": dict(rel_l2=2e-2, max_abs=None),
       "f32": dict(rel_l2=1e-5, max_abs=1e-4)}
# Gate weights, max-abs: a diagnostic (ids and y carry the acceptance bounds).  They are
# fp32 softmaxes of fp32 logits whose sum over H bf16 products differs from the oracle's
# fp64 sum by up to ~1e-5 at H = 4096 with these distributions; a weight moves by at most
# about twice its value times the largest logit error.  Any selection or normalisation
# mistake moves a weight by 1e-3 or more.
W_TOL = 1e-5


def note(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=4)
def layer(name: str, **kw) -> synth.LayerInputs:
    return synth.make_layer(name, **kw)


def layer_of(shape: synth.Shape, seed=0, batch=0) -> synth.LayerInputs:
    return synth.make_layer(shape, seed=seed, batch=batch)


def tdev(a: np.ndarray) -> torch.Tensor:
    if a is None:
        return None
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def act_code(s: synth.Shape) -> int:
    return pm.F32 if s.act == "f32" else pm.BF16


def w_code(s: synth.Shape) -> int:
    return {"f32": pm.F32, "bf16": pm.BF16, "mxfp4": pm.MXFP4, "nvfp4": pm.NVFP4, "mxint8": pm.MXINT8}[s.w]


def lshape(li: synth.LayerInputs, path=pm.PATH_AUTO, T=None, K=None, renorm=None) -> pm.LayerShape:
    s = li.shape
    return pm.LayerShape(num_tokens=s.T if T is None else T, hidden=s.H, num_experts=s.E,
                         top_k=s.K if K is None else K, intermediate=s.I,
                         renormalize=s.renorm if renorm is None else renorm,
                         act_dtype=act_code(s), weight_dtype=w_code(s), path=path)


class DevLayer:
    """Device copies of one layer's tensors."""

    def __init__(self, li: synth.LayerInputs):
        self.li = li
        self.x = tdev(li.x)
        self.wr = tdev(li.wr)
        self.bias = tdev(li.bias) if li.bias is not None else None
        self.weights = dict(wg=tdev(li.wg), wu=tdev(li.wu), wd=tdev(li.wd), sg=tdev(li.sg), su=tdev(li.su),
                            sd=tdev(li.sd), ts=li.ts)

    def act_torch(self):
        return torch.float32 if self.li.shape.act == "f32" else torch.int16


def to_f64(t: torch.Tensor, act: str) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if act == "f32":
        return a.astype(np.float64)
    return synth.bf16_bits_to_f32(a.view(np.uint16)).astype(np.float64)


CANARY = 0x5A


def guarded(n_elems: int, dtype, pad: int = 64):
    """(full buffer with canary padding after the payload, payload view)."""
    esz = torch.empty(0, dtype=dtype).element_size()
    nbytes = n_elems * esz
    buf = torch.full((nbytes + pad * 16,), CANARY, dtype=torch.uint8, device="cuda")
    return buf, buf[:nbytes].view(dtype)


def canary_ok(buf: torch.Tensor, n_elems: int, dtype) -> bool:
    esz = torch.empty(0, dtype=dtype).element_size()
    tail = buf[n_elems * esz:]
    return bool((tail == CANARY).all().item())


def run_forward(dl: DevLayer, path=pm.PATH_AUTO, T=None, x=None, K=None, renorm=None):
    li = dl.li
    sh = lshape(li, path, T=T, K=K, renorm=renorm)
    T_ = sh.num_tokens
    ws = pm.alloc_workspace(sh)
    ybuf, y = guarded(T_ * li.shape.H, dl.act_torch())
    y = y.view(T_, li.shape.H) if T_ else y
    ids = torch.full((T_, sh.top_k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((T_, sh.top_k), -7.0, dtype=torch.float32, device="cuda")
    pm.forward(sh, dl.x if x is None else x, dl.wr, dl.bias, dl.weights, y, ws, ids, w)
    torch.cuda.synchronize()
    err = pm.check_device_error(ws)
    assert err == 0, f"device error bits {err}"
    assert canary_ok(ybuf, T_ * li.shape.H, dl.act_torch()), "write past the end of y"
    return dict(y=y, ids=ids.cpu().numpy(), w=w.cpu().numpy(), ws=ws)


def forward_grouping(sh: pm.LayerShape, ws):
    """The grouping the last forward on ws built on the device: (offsets, sorted, slot_pos)."""
    E, P = sh.num_experts, sh.num_tokens * sh.top_k
    obuf, off = guarded(E + 1, torch.int32)
    sbuf, srt = guarded(P, torch.int32)
    pbuf, pos = guarded(P, torch.int32)
    pm.forward_grouping(sh, ws, off, srt, pos)
    torch.cuda.synchronize()
    for b, n in ((obuf, E + 1), (sbuf, P), (pbuf, P)):
        assert canary_ok(b, n, torch.int32), "grouping view wrote past its buffer"
    return off.cpu().numpy(), srt.cpu().numpy(), pos.cpu().numpy()


def compare_forward(li: synth.LayerInputs, got: dict, tokens=None, K=None, renorm=None, label=""):
    """Ids bit-exact except oracle near-ties; y within the format's tolerance against the
    oracle (forced to the GPU's ids on near-tie tokens that differ)."""
    L = oracle_layer(li, top_k=K or li.shape.K, renorm=li.shape.renorm if renorm is None else renorm)
    T = got["ids"].shape[0]
    toks = np.arange(T) if tokens is None else np.asarray(tokens)
    ref = oracle.forward(L, tokens=toks)
    gids = got["ids"][toks]
    gw = got["w"][toks]
    mism = (gids != ref["ids"]).any(axis=1)
    near = ref["near"]
    bad = mism & ~near
    assert not bad.any(), f"{label}: ids differ on non-near-tie tokens {toks[bad][:8]}"
    yref = ref["y"].copy()
    wref = ref["w"].copy()
    if mism.any():
        forced = oracle.forward(L, tokens=toks[mism], forced_ids=gids[mism])
        yref[mism] = forced["y"]
        wref[mism] = forced["w"]
    werr = max_abs(gw, wref)
    assert werr <= W_TOL, f"{label}: gate weights max-abs {werr:.3e}"
    fmt = li.shape.w if li.shape.w in ("mxfp4", "nvfp4", "mxint8") else li.shape.act
    y = to_f64(got["y"], li.shape.act)[toks]
    r, m = rel_l2(y, yref), max_abs(y, yref)
    tol = TOL[fmt]
    note(f"{label}: tokens={len(toks)} near_ties={int(near.sum())} id_mismatch={int(mism.sum())} "
         f"rel_l2={r:.3e} max_abs={m:.3e} w_err={werr:.2e}")
    assert r <= tol["rel_l2"], f"{label}: rel-L2 {r:.3e}"
    if tol["max_abs"] is not None:
        assert m <= tol["max_abs"], f"{label}: max-abs {m:.3e}"
    return dict(rel_l2=r, max_abs=m, near=int(near.sum()), mism=int(mism.sum()))
