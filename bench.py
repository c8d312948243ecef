"""Benchmark of the MI355X MoE layer (router top-k softmax, token->expert
grouping, SwiGLU experts, weighted combine) through the C ABI.

One step = one moe_forward over one batch of synthetic, seeded inputs that
are already resident in HBM.  Default workload (the JSON line's `value`): the
8192-token bf16 prefill chunk with Zipf-skewed routing, H=2048, E=128, top-8,
I=768 -- the largest single-GPU workload and the bf16-MFMA half of the metric.
The decode workloads of the same layer shape (1 token; 8 tokens with a router
bias) are measured in the same run and reported under `extra_workloads`, each
with its own roofline object (`--extra` selects them; `--extra none` skips).

Weights rotate over `--copies` copies (each at its own addresses: 16 x 1.2 GB
for decode, 2 for prefill) so the 256 MB Infinity Cache cannot serve repeats:
every step streams its experts from HBM.  The steps are captured once into a
HIP graph (through torch.cuda.CUDAGraph) and replayed, so host launch cost
does not hide us-scale GPU work; replays are checked against eager results
before timing.

The roofline object reports the dominant kernel (the fused decode launch, or
the expert gate/up + SwiGLU launch of the grouped path): algorithmic bytes
(decode) or flops (prefill) per launch over its average duration.  The
durations are HIP events that moe_forward_timed ties to that launch's start
and end (hipExtLaunchKernelGGL), over a second timed pass of the same steps on
torch's current stream.  The cpu_baseline object times the fp64 CPU oracle on
a bounded sample of the headline workload; each decode extra also carries a
one-thread oracle run.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s

METRIC = "MoE layer tokens/s; decode HBM GB/s % peak; prefill MFMA TFLOP/s % peak"

# HBM traffic of the dominant kernel from rocprofv3 counter passes (FETCH_SIZE, then
# WRITE_SIZE, KiB per dispatch), scaled by what the same counters read for a device copy
# of known size (FETCH_SIZE x2.0, WRITE_SIZE x1.0).  Valid only for the kernel sources
# the counters were taken on (sha1 of the listed files); otherwise traffic is null.
_SRC_DEVICE = ("prefill_moe_router_amd/csrc/moe_device.h", "83f51350610eff16eae366237d12db13d9a245a5")
_SRC_FUSED = dict([("prefill_moe_router_amd/csrc/decode_fused.hip", "5143c990fbab86e0a7a9bf0c177089fa1a3ead6b"),
                   _SRC_DEVICE])
_SRC_WIDE = dict([("prefill_moe_router_amd/csrc/grouped_gemm_wide.hip", "c7eb78ac93dcde4c73a7e9c26c4bf552fa5d66c6"),
                  _SRC_DEVICE])
_SRC_GROUPED = dict([("prefill_moe_router_amd/csrc/grouped_gemm.hip", "0d538576ed40adb102c1759b5c9614421265dea6"),
                     _SRC_DEVICE])


def _traffic(kernel, fetch_kib, write_kib, sources):
    return dict(kernel=kernel, fetch_kib=fetch_kib, write_kib=write_kib, fetch_scale=2.0, write_scale=1.0,
                sources=sources)


COUNTED_TRAFFIC = {
    "decode1": _traffic("decode_fused", 37527.0, 240.1, _SRC_FUSED),
    "decode8": _traffic("decode_fused", 197231.2, 1640.5, _SRC_FUSED),
    "mxfp4_decode1": _traffic("decode_fused", 27653.9, 344.1, _SRC_FUSED),
    "mxfp4_decode8": _traffic("decode_fused", 188483.6, 2248.5, _SRC_FUSED),
    "prefill8192": _traffic("gate_up", 1062886.1, 98309.1, _SRC_WIDE),
    "mxfp4_prefill4096": _traffic("gate_up", 993020.4, 65536.0, _SRC_GROUPED),
}


def counted_traffic(config: str, kernel: str):
    import hashlib
    rec = COUNTED_TRAFFIC.get(config)
    if not rec or rec["kernel"] != kernel:
        return None
    for path, sha in rec["sources"].items():
        with open(os.path.join(ROOT, path), "rb") as f:
            if hashlib.sha1(f.read()).hexdigest() != sha:
                return None
    return round(rec["fetch_kib"] * 1024 * rec["fetch_scale"] + rec["write_kib"] * 1024 * rec["write_scale"])

WORKLOADS = {
    "decode1": ("c1_decode1_bf16", "decode, 1 token, bf16: H=2048, E=128, top-8 renorm, I=768, SwiGLU"),
    "decode8": ("c2_decode8_bf16", "decode, 8 tokens, bf16, router bias N(0,0.5): H=2048, E=128, top-8, I=768"),
    "prefill8192": ("c3_prefill8192_bf16",
                    "prefill chunk, 8192 tokens, bf16, Zipf(1) router bias: H=2048, E=128, top-8, I=768"),
    "mixed8192_8": ("c3_mixed8200_bf16",
                    "prefill chunk of 8192 tokens plus 8 decode rows in one call, bf16, Zipf(1) router bias: "
                    "H=2048, E=128, top-8, I=768"),
    "mxfp4_decode1": ("c4_mxfp4_decode1", "decode, 1 token, MXFP4 experts, bf16 acts: H=4096, E=256, top-8, I=1024"),
    "mxfp4_decode8": ("c4_mxfp4_decode8", "decode, 8 tokens, MXFP4 experts: H=4096, E=256, top-8, I=1024"),
    "nvfp4_decode1": ("c5_nvfp4_decode1", "decode, 1 token, NVFP4 experts (E4M3 scale per 16), bf16 acts: "
                      "H=4096, E=256, top-8, I=1024"),
    "nvfp4_decode8": ("c5_nvfp4_decode8", "decode, 8 tokens, NVFP4 experts: H=4096, E=256, top-8, I=1024"),
    "nvfp4_prefill4096": ("c5_nvfp4_prefill4096",
                          "prefill chunk, 4096 tokens, NVFP4 experts: H=4096, E=256, top-8, I=1024"),
    "mxfp4_prefill4096": ("c4_mxfp4_prefill4096",
                          "prefill chunk, 4096 tokens, MXFP4 experts: H=4096, E=256, top-8, I=1024"),
    "mxint8_decode1": ("c6_mxint8_decode1", "decode, 1 token, MXINT8 experts (int8, E8M0 scale per 32), bf16 "
                       "acts: H=4096, E=256, top-8, I=1024"),
    "mxint8_decode8": ("c6_mxint8_decode8", "decode, 8 tokens, MXINT8 experts: H=4096, E=256, top-8, I=1024"),
    "mxint8_prefill4096": ("c6_mxint8_prefill4096",
                           "prefill chunk, 4096 tokens, MXINT8 experts: H=4096, E=256, top-8, I=1024"),
    "tiny": ("c0_tiny_f32", "tiny fp32: 4 tokens, H=256, E=8, top-2, I=128"),
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def weight_bytes_per_elem(w: str) -> float:
    return {"f32": 4.0, "bf16": 2.0, "mxfp4": 0.5 + 1.0 / 32.0, "nvfp4": 0.5 + 1.0 / 16.0,
            "mxint8": 1.0 + 1.0 / 32.0}[w]


def act_bytes(a: str) -> int:
    return 4 if a == "f32" else 2


HEADLINE = "prefill8192"
DEFAULT_EXTRA = "decode1,decode8"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps of the headline workload")
    ap.add_argument("--warmup", type=int, default=None, help="untimed warm-up steps of the headline workload")
    ap.add_argument("--config", default=HEADLINE, choices=sorted(WORKLOADS))
    ap.add_argument("--extra", default=None,
                    help="comma-separated extra workloads measured after the headline one ('none': skip; "
                         f"default {DEFAULT_EXTRA} with the default --config, none otherwise)")
    ap.add_argument("--copies", type=int, default=None, help="weight copies rotated over (defeats the MALL)")
    ap.add_argument("--path", default="auto", choices=["auto", "decode", "grouped"])
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def dev(a):
    import torch
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if a.dtype == np.uint16 else a)).cuda()


def measure(config: str, steps, warmup, copies, path_name: str):
    """Times exactly `steps` moe_forward calls of one workload (after `warmup` untimed ones)
    and the dominant kernel's launches; returns (line fields, layer inputs, shape)."""
    import torch
    import prefill_moe_router_amd as pm
    import synth

    name, desc = WORKLOADS[config]
    sh = synth.CONFIGS[name]
    decode = sh.T <= 8
    copies = copies or (16 if decode else 2)
    steps = steps or (1600 if decode else 20)
    warmup = warmup if warmup is not None else (160 if decode else 4)
    path = {"auto": pm.PATH_AUTO, "decode": pm.PATH_DECODE, "grouped": pm.PATH_GROUPED}[path_name]

    t0 = time.time()
    li = synth.make_layer(name)
    log(f"{config}: generated inputs in {time.time() - t0:.1f}s")
    w0 = dict(wg=dev(li.wg), wu=dev(li.wu), wd=dev(li.wd), sg=dev(li.sg), su=dev(li.su), sd=dev(li.sd), ts=li.ts)
    wcopies = [w0] + [{k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in w0.items()}
                      for _ in range(copies - 1)]
    wr, bias = dev(li.wr), dev(li.bias)
    xs = [dev(synth.make_x(sh, seed=0, batch=b)) for b in range(copies)]
    shape = pm.LayerShape(sh.T, sh.H, sh.E, sh.K, sh.I, sh.renorm,
                          pm.F32 if sh.act == "f32" else pm.BF16,
                          {"f32": pm.F32, "bf16": pm.BF16, "mxfp4": pm.MXFP4, "nvfp4": pm.NVFP4,
                           "mxint8": pm.MXINT8}[sh.w], path)
    ws = pm.alloc_workspace(shape)
    ydt = torch.float32 if sh.act == "f32" else torch.int16
    ys = [torch.empty(sh.T, sh.H, dtype=ydt, device="cuda") for _ in range(copies)]
    ids = [torch.empty(sh.T, sh.K, dtype=torch.int32, device="cuda") for _ in range(copies)]
    wts = [torch.empty(sh.T, sh.K, dtype=torch.float32, device="cuda") for _ in range(copies)]
    torch.cuda.synchronize()
    log(f"{config}: resident: {copies} weight copies, {torch.cuda.memory_allocated() / 2**30:.1f} GiB")

    def step(b, stream=None):
        pm.forward(shape, xs[b], wr, bias, wcopies[b], ys[b], ws, ids[b], wts[b], stream=stream)

    # eager reference results
    for b in range(copies):
        step(b)
    torch.cuda.synchronize()
    assert pm.check_device_error(ws) == 0
    y_eager = [y.clone() for y in ys]
    ids_eager = [i.clone() for i in ids]

    # graphs: one sweep over the copies, and partial sweeps of the first n copies (cached)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(0, stream=s)          # a warm call on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graphs = {}

    def graph_of(n):
        if n not in graphs:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for b in range(n):
                    step(b)
            graphs[n] = g
        return graphs[n]

    def replay(n):
        """Exactly n forward calls: whole sweeps, then the first n % copies copies."""
        for _ in range(n // copies):
            graph_of(copies).replay()
        if n % copies:
            graph_of(n % copies).replay()

    graph_of(copies)
    if steps % copies:
        graph_of(steps % copies)
    if warmup % copies:
        graph_of(warmup % copies)
    for r in range(3):
        for y in ys:
            y.fill_(0)
        graph_of(copies).replay()
        torch.cuda.synchronize()
        for b in range(copies):
            assert torch.equal(ys[b], y_eager[b]), f"graph replay {r} differs from eager (copy {b})"
            assert torch.equal(ids[b], ids_eager[b])
    log(f"{config}: graph replays match eager results")

    replay(warmup)
    torch.cuda.synchronize()
    # ---- timed region: exactly `steps` forward calls ----
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev0.record()
    replay(steps)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = wall * 1e3 / steps
    tokens_per_s = sh.T * steps / wall
    log(f"{config}: timed {steps} steps: {wall * 1e3:.2f} ms wall ({gpu_ms:.2f} ms GPU events), "
        f"{ms_per_step * 1e3:.2f} us/step")

    # ---- algorithmic work per step --------------------------------------------------
    bw = weight_bytes_per_elem(sh.w)
    ba = act_bytes(sh.act)
    U = [len(np.unique(i.cpu().numpy())) for i in ids_eager]
    layer_bytes = [u * 3 * sh.H * sh.I * bw + sh.E * sh.H * ba + 2 * sh.T * sh.H * ba
                   + (4 * sh.E if li.bias is not None else 0) for u in U]
    gateup_bytes = [u * 2 * sh.H * sh.I * bw + sh.T * sh.H * ba for u in U]
    layer_flops = 2 * sh.T * sh.K * 3 * sh.H * sh.I + 2 * sh.T * sh.H * sh.E
    gateup_flops = 2 * sh.T * sh.K * 2 * sh.H * sh.I

    # ---- dominant-kernel duration: start/stop events of that launch, every step ---------
    stages = pm.forward_stages(shape)
    dom_name = "decode_fused" if "decode_fused" in stages else "gate_up"
    dom = stages.index(dom_name)
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b_ in pairs:          # torch creates the underlying hipEvent_t at the first record
        a.record()
        b_.record()
    torch.cuda.synchronize()
    for k in range(steps):
        b = k % copies
        marks = [None] * (2 * len(stages))
        marks[2 * dom], marks[2 * dom + 1] = pairs[k][0].cuda_event, pairs[k][1].cuda_event
        pm.forward_timed(shape, xs[b], wr, bias, wcopies[b], ys[b], ws, marks, ids[b], wts[b])
    torch.cuda.synchronize()
    for b in range(copies):
        assert torch.equal(ys[b], y_eager[b]), "timed pass changed results"
    durs = [a.elapsed_time(b_) * 1e-3 for a, b_ in pairs]     # seconds
    kern_s = float(np.mean(durs))
    fused = dom_name == "decode_fused"
    if decode:
        kb = layer_bytes if fused else gateup_bytes
        achieved = float(np.mean(kb)) / kern_s / 1e9
        roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                        frac=round(achieved / HBM_PEAK_GBS, 4), traffic=counted_traffic(config, dom_name),
                        kernel=("decode_fused (whole layer in one launch)" if fused
                                else "gate_up (expert gate/up GEMV + SwiGLU)"),
                        kernel_us=round(kern_s * 1e6, 3), kernel_us_median=round(float(np.median(durs)) * 1e6, 3),
                        algorithmic_bytes=round(float(np.mean(kb))))
    else:
        achieved = gateup_flops / kern_s / 1e12
        roofline = dict(bound="mfma", achieved=round(achieved, 2), peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                        frac=round(achieved / BF16_PEAK_TFLOPS, 4), traffic=counted_traffic(config, dom_name),
                        kernel="gate_up (grouped expert gate/up + SwiGLU)", kernel_us=round(kern_s * 1e6, 3),
                        kernel_us_median=round(float(np.median(durs)) * 1e6, 3), algorithmic_flops=gateup_flops)
    log(f"{config}: dominant kernel {dom_name}: {kern_s * 1e6:.2f} us avg over {len(durs)} launches")

    layer_s = wall / steps
    layer = dict(layer_us=round(layer_s * 1e6, 3), unique_experts_mean=float(np.mean(U)), stages=stages)
    if decode:
        gbs = float(np.mean(layer_bytes)) / layer_s / 1e9
        layer.update(layer_bytes=round(float(np.mean(layer_bytes))), layer_gbs=round(gbs, 1),
                     layer_hbm_frac=round(gbs / HBM_PEAK_GBS, 4))
    else:
        tf = layer_flops / layer_s / 1e12
        layer.update(layer_flops=layer_flops, layer_tflops=round(tf, 2),
                     layer_mfma_frac=round(tf / BF16_PEAK_TFLOPS, 4))
    fields = dict(value=round(tokens_per_s, 1), unit="tokens/s", steps=steps, warmup=warmup,
                  ms_per_step=round(ms_per_step, 6), dtype=sh.w if sh.w != "f32" else "f32",
                  config={"workload": desc, "tokens_per_step": sh.T, "hidden": sh.H, "experts": sh.E,
                          "top_k": sh.K, "intermediate": sh.I, "weight_copies": copies,
                          "parallelism": "single GPU"},
                  roofline=roofline, layer=layer)
    del wcopies, w0, xs, ys, ws, graphs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return fields, li, sh


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "the layer is measured on one MI355X", file=sys.stderr)
        sys.exit(2)
    import torch
    torch.cuda.set_device(0)

    head, li, sh = measure(args.config, args.steps, args.warmup, args.copies, args.path)
    extra_names = args.extra if args.extra is not None else (DEFAULT_EXTRA if args.config == HEADLINE else "none")
    extras = {}
    cpu_extra = {}
    for cfg in [c for c in extra_names.split(",") if c and c != "none"]:
        f, li_x, sh_x = measure(cfg, None, None, None, "auto")
        extras[cfg] = f
        if not args.no_cpu_baseline and sh_x.T <= 8:
            cpu_extra[cfg] = (li_x, sh_x)

    out = {
        "metric": METRIC, "value": head["value"], "unit": "tokens/s", "n_gpus": 1, "steps": head["steps"],
        "warmup": head["warmup"], "ms_per_step": head["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": head["dtype"],
        "data": "synthetic (seeded N(0,1) activations, N(0,sd) random-init weights)",
        "config": head["config"], "roofline": head["roofline"], "layer": head["layer"],
    }
    if extras:
        out["extra_workloads"] = extras
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(li, sh, args.cpu_seconds)
        for cfg, (li_x, sh_x) in cpu_extra.items():
            extras[cfg]["cpu_baseline_1thread"] = cpu_baseline(li_x, sh_x, args.cpu_seconds / 3, threads=1)
    print(json.dumps(out), flush=True)


def cpu_baseline(li, sh, target_s: float, threads=None) -> dict:
    """The fp64 oracle, as it stands, on a bounded sample of the same workload."""
    import oracle
    import synth

    def layer_for(x):
        return oracle.Layer(x=x, wr=li.wr, wg=li.wg, wu=li.wu, wd=li.wd, top_k=sh.K, renorm=sh.renorm,
                            bias=li.bias, sg=li.sg, su=li.su, sd=li.sd,
                            fmt="nvfp4" if sh.w == "nvfp4" else None, ts=li.ts)

    full = oracle.num_threads()
    if threads is not None:
        oracle.set_num_threads(threads)
    try:
        nthr = oracle.num_threads()
        if sh.T <= 8:
            # independent decode steps: batches of the same shape stacked into one oracle call
            def run(nsteps):
                x = np.concatenate([synth.make_x(sh, seed=0, batch=100 + b) for b in range(nsteps)])
                t = time.perf_counter()
                oracle.forward(layer_for(x))
                return time.perf_counter() - t, nsteps * sh.T
            probe = max(1, nthr // sh.T)
            dt, n = run(probe)
            nsteps = max(1, int(probe * target_s / max(dt, 1e-3)))
            dt, n = run(nsteps)
            sample = f"{nsteps} independent {sh.T}-token decode steps ({n} token rows) in one oracle call"
        else:
            x = li.x

            def run(ntok):
                toks = np.linspace(0, sh.T - 1, ntok).astype(np.int32)
                t = time.perf_counter()
                oracle.forward(layer_for(x), tokens=toks)
                return time.perf_counter() - t, ntok
            dt, n = run(nthr)
            ntok = max(1, int(nthr * target_s / max(dt, 1e-3)))
            dt, n = run(ntok)
            sample = f"{ntok} tokens spread over the {sh.T}-token chunk (whole layer per token)"
    finally:
        oracle.set_num_threads(full)
    log(f"cpu baseline: {n} tokens in {dt:.1f}s on {min(nthr, n)} threads")
    return dict(value=round(n / dt, 3), unit="tokens/s", cores=int(min(nthr, n)), kind="oracle",
                sample=sample, seconds=round(dt, 2))


if __name__ == "__main__":
    main()
