#!/usr/bin/env python
"""Benchmark of the dynamic convolution hot path on one MI355X.

One step = the whole path over one batch of synthetic input already resident
in HBM: routing (GAP -> FC -> sigmoid/softmax) and the per-example
convolution with mixed kernels (the mixing fused into the MFMA convolution
for the ResNet-50-shaped layer, or a premix pass before it). The expert bank
is static: it is put in the convolution's weight order once, before the
timed steps (dynconv_pack_experts, once per weight update), as an inference
engine lays out its weights once. The timed steps run as replays of
HIP graphs that hold 10 whole steps each, so that one launch gap falls on ten
steps. The dominant kernel's time for the roofline comes from HIP events
around a graph of back-to-back launches of it (the timed region's sustained
load, under which the clock settles lower); eager single steps with events
around each kernel give the per-kernel times with launch gaps. Default workload: the
ResNet-50-shaped 3x3 layer, B=256, 256->256 channels, 14x14, n=4 experts,
bf16 storage with float32 accumulation.

Prints ONE JSON line with images/s (value), TFLOP/s against the bf16 MFMA
peak, the roofline of the dominant kernel (timed live with HIP events on the
stream the kernels run on) and the CPU oracle timed on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--workload KEY] [--no-cpu-baseline]
    python bench.py --profile       # short run for rocprofv3 (no CPU leg)
    python bench.py --calib-copy    # plain device copy of known size (counter calibration)
    python bench.py --backward      # training step: forward + backward (single-layer workloads)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "dynamic-conv images/s + TFLOP/s (% bf16 MFMA peak), ResNet-50 3x3 layer n=4"
PEAK_BF16_TFLOPS = 2516.6       # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 FLOP/clk)
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E
ROTATE_BYTES = 640 << 20        # rotating input/output sets larger than L2 + MALL
GRAPH_STEPS = 10                # steps per HIP graph replay in the timed loop

# HBM traffic of the dominant kernel per launch, from rocprofv3 --pmc FETCH_SIZE and
# WRITE_SIZE on the headline workload (KiB per dispatch), each scaled by what the same
# counter reads for a plain 256 MiB device copy (bench.py --calib-copy): FETCH_SIZE read
# 131085.4 KiB for 262144 KiB moved (x 2.000), WRITE_SIZE 262144 KiB (x 1.000). Valid only
# for the kernel source it was taken on (sha256 prefix over the files the dominant kernel
# is compiled from, listed below); otherwise null.
TRAFFIC = {
    "resnet50_3x3": {"source_sha": "97a3c8fc8b79f574",
                     "fetch_kib": 32312.8, "write_kib": 25088.0,
                     "fetch_scale": 262144 / 131085.4, "write_scale": 1.0},
}
KERNEL_SOURCES = [os.path.join(ROOT, "dynamic_convolution_cnn_amd", "csrc", f)
                  for f in ("conv_fused_wave.hip", "conv_common.hpp", "common.hpp")]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="resnet50_3x3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", action="store_true", help="few steps, no CPU leg")
    ap.add_argument("--calib-copy", action="store_true")
    ap.add_argument("--backward", action="store_true",
                    help="training step: forward, then the weight, input and routing gradients")
    return ap.parse_args()


def source_sha() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def calib_copy():
    """A plain device-to-device copy of 256 MiB, five times (for FETCH/WRITE_SIZE scaling)."""
    import torch
    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes": n, "copies": 5}))


def to_dev(a, dtype):
    import numpy as np
    import torch
    from dynamic_convolution_cnn_amd import inputs
    a = np.ascontiguousarray(a, np.float32)
    if dtype == "bf16":
        return torch.from_numpy(inputs.f32_to_bf16_bits(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


CPU_SAMPLE_SECONDS = 10.0  # bounded CPU sample: whole batches until this much time has passed


def cpu_baseline(w, d):
    """The oracle (route + mix + conv in fp64) on whole batches of the same
    workload, repeated until CPU_SAMPLE_SECONDS have passed, on the host's cores."""
    import oracle
    t0 = time.perf_counter()
    batches = 0
    while True:
        alpha, _, _ = oracle.route(d["x"], d["fc_w"], d["fc_b"], w.route_mode, w.temperature)
        h = d["x"]
        if w.mask_density > 0:
            L = w.layers[0]
            h = oracle.forward_sparse(h, d["experts"][0], alpha, d["mask"], L.stride, L.pad, L.groups, True)
        elif w.attention:
            a_in, _, _ = oracle.route(d["x"], d["fc_w_in"], d["fc_b_in"], oracle.SIGMOID)
            a_out, _, _ = oracle.route(d["x"], d["fc_w_out"], d["fc_b_out"], oracle.SIGMOID)
            L = w.layers[0]
            h = oracle.forward_attn(h, d["experts"][0], alpha, a_in, a_out, L.stride, L.pad, L.groups)
        else:
            for L, e in zip(w.layers, d["experts"]):
                h = oracle.forward(h, e, alpha, L.stride, L.pad, L.groups)
        batches += 1
        dt = time.perf_counter() - t0
        if dt >= CPU_SAMPLE_SECONDS:
            break
    return {"value": round(batches * w.B / dt, 3), "unit": "images/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"{batches} full batches of {w.B} examples of {w.key} (route + mix + conv, "
                      f"float64 direct loops), {dt:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU; --gpus {args.gpus} is not supported "
              "(every step is independent per example, so several GPUs would each take a share of the batch)",
              file=sys.stderr)
        sys.exit(2)
    if args.calib_copy:
        calib_copy()
        return
    if args.backward:
        train_main(args)
        return
    import numpy as np
    import torch
    from dynamic_convolution_cnn_amd import binding as bd
    from dynamic_convolution_cnn_amd import inputs

    if args.profile:
        args.steps, args.warmup, args.no_cpu_baseline = min(args.steps, 10), min(args.warmup, 3), True
    w = inputs.WORKLOADS[args.workload]
    d = inputs.make_inputs(w, seed=0)
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()

    # one static copy of the weights; R rotating sets of activations
    experts = [to_dev(e, w.dtype) for e in d["experts"]]
    fc_w, fc_b = to_dev(d["fc_w"], "f32"), to_dev(d["fc_b"], "f32")
    x0 = to_dev(d["x"], w.dtype)
    esz = 2 if w.dtype == "bf16" else 4
    set_bytes = sum(w.B * (L.Cin * L.H * L.W + L.Cout * L.Ho * L.Wo) * esz for L in w.layers)
    R = max(1, math.ceil(ROTATE_BYTES / set_bytes))
    xs = [x0] + [x0.clone() for _ in range(R - 1)]
    descs, packed, ws, outs, pols = [], [], [], [], []
    for L, e in zip(w.layers, experts):
        desc = bd.make_desc(w.B, L.Cin, L.H, L.W, L.Cout, L.k, L.k, L.stride, L.pad, L.groups, w.n,
                            bd.DYNCONV_BF16 if w.dtype == "bf16" else bd.DYNCONV_F32)
        if w.mask_density > 0:  # gated residual layer: bank packed once, W_b mixed in the step
            descs.append(desc)
            pols.append(bd.DYNCONV_POLICY_PREMIX)
            packed.append(torch.empty(bd.dynconv_packed_experts_bytes(desc), dtype=torch.uint8, device=dev))
            nb = bd.dynconv_forward_sparse_packed_workspace_bytes(desc)
            ws.append(torch.empty(max(nb, 16), dtype=torch.uint8, device=dev))
            outs.append([torch.empty((w.B, L.Cout, L.Ho, L.Wo), dtype=x0.dtype, device=dev)
                         for _ in range(R)])
            continue
        if w.attention:  # channel attentions: the forward packs its bank itself (PREMIX policy)
            descs.append(desc)
            pols.append(bd.dynconv_forward_policy(desc))  # the attentions follow the plain layer's policy
            packed.append(None)
            nb = bd.dynconv_forward_attn_workspace_bytes(desc, pols[-1])
            ws.append(torch.empty(max(nb, 16), dtype=torch.uint8, device=dev))
            outs.append([torch.empty((w.B, L.Cout, L.Ho, L.Wo), dtype=x0.dtype, device=dev)
                         for _ in range(R)])
            continue
        pol = bd.dynconv_forward_policy(desc)
        pk = bd.dynconv_packed_experts_bytes(desc)
        packed.append(torch.empty(pk, dtype=torch.uint8, device=dev) if pk else None)
        nb = (bd.dynconv_forward_packed_workspace_bytes(desc, pol) if pk
              else bd.dynconv_forward_workspace_bytes(desc, pol))
        ws.append(torch.empty(max(nb, 16), dtype=torch.uint8, device=dev))
        outs.append([torch.empty((w.B, L.Cout, L.Ho, L.Wo), dtype=x0.dtype, device=dev)
                     for _ in range(R)])
        descs.append(desc)
        pols.append(pol)
    alphas = [torch.empty((w.B, w.n), dtype=torch.float32, device=dev) for _ in range(R)]
    route_ws = torch.zeros(max(16, bd.dynconv_route_workspace_bytes(descs[0])), dtype=torch.uint8, device=dev)
    if w.attention:
        L0 = w.layers[0]
        heads = [to_dev(d[k], "f32") for k in ("fc_w_in", "fc_b_in", "fc_w_out", "fc_b_out")]
        a_ins = [torch.empty((w.B, L0.Cin), dtype=torch.float32, device=dev) for _ in range(R)]
        a_outs = [torch.empty((w.B, L0.Cout), dtype=torch.float32, device=dev) for _ in range(R)]
        route_ws = torch.empty(bd.dynconv_route_attn_workspace_bytes(descs[0]), dtype=torch.uint8,
                               device=dev)

    def route(s):
        if w.attention:
            bd.dynconv_route_attn(xs[s], w.layers[0].Cout, fc_w, fc_b, *heads, mode=w.route_mode,
                                  temperature=w.temperature, alpha=alphas[s], a_in=a_ins[s],
                                  a_out=a_outs[s], workspace=route_ws)
        else:
            bd.dynconv_route(xs[s], fc_w, fc_b, w.route_mode, w.temperature, alpha=alphas[s],
                             workspace=route_ws)

    mask_dev = torch.from_numpy(d["mask"]).to(dev) if w.mask_density > 0 else None

    def forward(li, h, s):
        L = w.layers[li]
        if w.mask_density > 0:
            bd.dynconv_forward_sparse_packed(descs[li], h, packed[li], alphas[s], mask_dev, residual=True,
                                             y=outs[li][s], workspace=ws[li])
        elif w.attention:
            bd.dynconv_forward_attn(h, experts[li], alphas[s], a_ins[s], a_outs[s], L.stride, L.pad,
                                    L.groups, policy=pols[li], y=outs[li][s], workspace=ws[li])
        elif packed[li] is not None:
            bd.dynconv_forward_packed(descs[li], h, packed[li], alphas[s], policy=pols[li],
                                      y=outs[li][s], workspace=ws[li])
        else:
            bd.dynconv_forward(h, experts[li], alphas[s], L.stride, L.pad, L.groups, policy=pols[li],
                               y=outs[li][s], workspace=ws[li])

    # the static bank in the convolution's weight order, once (timed apart)
    pev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    pev[0].record(stream)
    for li, desc in enumerate(descs):
        if packed[li] is not None:
            bd.dynconv_pack_experts(desc, experts[li], packed[li])
    pev[1].record(stream)
    torch.cuda.synchronize()
    pack_ms = pev[0].elapsed_time(pev[1])

    def step(i, ev=None):
        s = i % R
        cur = torch.cuda.current_stream()  # the capture stream inside a graph
        if ev is not None:
            ev[0].record(cur)
        route(s)
        if ev is not None:
            ev[1].record(cur)
        h = xs[s]
        for li, desc in enumerate(descs):
            forward(li, h, s)
            if ev is not None and li == 0:
                ev[2].record(cur)
            h = outs[li][s]

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # HIP graphs hold whole steps (route, pack, forward of every layer), so the
    # timed loop measures the GPU, not Python launch cost: graph g holds the G
    # steps over rotating sets g, g + 1, ..., g + G - 1 (mod R), and a few
    # one-step graphs make up the remainder, so that exactly K steps run.
    G = GRAPH_STEPS

    def capture(first, count, fn=None):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for j in range(count):
                (fn or step)(first + j)
        return g

    multi = [capture(s, G) for s in range(R)]
    single = [capture(s, 1) for s in range(R)]
    plan, i = [], 0
    while i + G <= args.steps:
        plan.append(multi[i % R]); i += G
    while i < args.steps:
        plan.append(single[i % R]); i += 1
    for g in (multi[0], single[0]):
        g.replay()
    torch.cuda.synchronize()

    # timed region: exactly K steps (graph replays)
    t0 = time.perf_counter()
    for g in plan:
        g.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    # The dominant kernel as the timed region runs it: back to back, so the
    # clock settles where sustained matrix-core load puts it. A graph of G
    # launches of the first layer's forward (rotating sets) is replayed NC
    # times between two HIP events on the launch stream.
    h0 = [xs[s] for s in range(R)]

    def fwd0(i):
        forward(0, h0[i % R], i % R)

    NC = 2 if args.profile else 20

    def back_to_back(fn):
        """ms per call of fn(i) from a graph of G calls (rotating sets), replayed NC times
        between two HIP events on the launch stream."""
        g = capture(0, G, fn)
        g.replay()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(NC):
            g.replay()
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / (NC * G)

    conv_ms = back_to_back(fwd0)
    # routing alone, back to back over the rotating inputs (no launch gaps)
    route_ms = back_to_back(lambda i: route(i % R))

    # per-kernel times of single steps (eager launches with HIP events on the
    # launch stream around route / first conv; the gaps between them let the
    # clock recover, and each event pair also holds a launch gap)
    nk = min(args.steps, 20)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(nk)]
    torch.cuda.synchronize()
    for i in range(nk):
        step(i, evs[i])
    torch.cuda.synchronize()
    route_eager_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / nk
    conv_eager_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / nk

    # standalone mixing (dynconv_mix: every W_b to memory in the natural
    # layout) of the first layer: an HBM stream of n |W| bytes in and B |W|
    # bytes out. Banks, attentions and outputs rotate over RM sets larger than
    # L2 + MALL, so the rate is HBM's; a graph of launches keeps launch cost out.
    L0 = w.layers[0]
    wbytes0 = experts[0][0].numel() * esz
    RM = max(2, math.ceil(ROTATE_BYTES / ((w.n + w.B) * wbytes0 + w.B * w.n * 4)))
    mix_sets = [(experts[0] if r == 0 else experts[0].clone(), alphas[r % R].clone(),
                 torch.empty((w.B,) + tuple(experts[0].shape[1:]), dtype=experts[0].dtype, device=dev))
                for r in range(RM)]

    def mix_call(i):
        e_r, a_r, m_r = mix_sets[i % RM]
        bd.dynconv_mix(a_r, e_r, L0.groups, mixed=m_r)
    for r in range(RM):
        mix_call(r)
    gm = capture(0, max(RM, G), mix_call)
    gm.replay()
    torch.cuda.synchronize()
    mev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    mev[0].record(stream)
    gm.replay()
    mev[1].record(stream)
    torch.cuda.synchronize()
    mix_ms = mev[0].elapsed_time(mev[1]) / max(RM, G)
    mix_bytes = (w.n + w.B) * wbytes0 + w.B * w.n * 4
    del mix_sets, gm

    # a gated layer computes only its active positions
    active = float(d["mask"].mean()) if w.mask_density > 0 else 1.0
    conv_flops0 = 2 * w.B * L0.macs_per_example() * active
    flops_all = w.conv_flops() * active
    images_s = w.B / (ms_per_step * 1e-3)
    route_bytes = w.B * L0.Cin * L0.H * L0.W * esz + w.B * w.n * 4
    conv_tflops = conv_flops0 / (conv_ms * 1e-3) / 1e12
    # algorithmic bytes of the first layer's forward: x and y once, the expert
    # bank once, and W_b written and read again when the policy materialises it
    wsize0 = experts[0][0].numel()
    conv_bytes0 = (w.B * (L0.Cin * L0.H * L0.W + L0.Cout * L0.Ho * L0.Wo) + w.n * wsize0) * esz
    if pols[0] == bd.DYNCONV_POLICY_PREMIX:
        conv_bytes0 += 2 * w.B * wsize0 * esz
    conv_gbs = conv_bytes0 / (conv_ms * 1e-3) / 1e9
    hbm_bound = conv_gbs / PEAK_HBM_GBS > conv_tflops / PEAK_BF16_TFLOPS
    traffic = None
    t = TRAFFIC.get(w.key)
    if t and t.get("source_sha") == source_sha():
        traffic = round((t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"]) * 1024)
    pol_name = {bd.DYNCONV_POLICY_FUSED: "fused", bd.DYNCONV_POLICY_PREMIX: "premix"}
    out = {
        "metric": METRIC,
        "value": round(images_s, 1),
        "unit": "images/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded numpy draws, shapes of the pages' networks; no dataset)",
        "config": {"workload": w.key, "title": w.title, "B": w.B, "n": w.n,
                   "layers": [dict(Cin=L.Cin, Cout=L.Cout, H=L.H, W=L.W, k=L.k, stride=L.stride,
                                   pad=L.pad, groups=L.groups) for L in w.layers],
                   "routing": "softmax(z/T)" if w.route_mode else "sigmoid",
                   "policy": [pol_name.get(p, str(p)) for p in pols],
                   "attention": w.attention,
                   "mask_density": w.mask_density,
                   "rotating_sets": R},
        "tflops_step": round(flops_all / (ms_per_step * 1e-3) / 1e12, 2),
        "pct_bf16_peak_step": round(100 * flops_all / (ms_per_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "kernels_us": {"route_back_to_back": round(route_ms * 1e3, 2),
                       "route_eager": round(route_eager_ms * 1e3, 2),
                       "conv_layer0": round(conv_eager_ms * 1e3, 2),
                       "conv_layer0_back_to_back": round(conv_ms * 1e3, 2),
                       "pack_once_outside_steps": round(pack_ms * 1e3, 2)},
        "route_hbm": {"us": round(route_ms * 1e3, 2), "MB": round(route_bytes / 1e6, 2),
                      "GB/s": round(route_bytes / (route_ms * 1e-3) / 1e9, 1),
                      "frac": round(route_bytes / (route_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 3)},
        "mix_hbm": {"us": round(mix_ms * 1e3, 2), "MB": round(mix_bytes / 1e6, 2), "rotating_sets": RM,
                    "GB/s": round(mix_bytes / (mix_ms * 1e-3) / 1e9, 1),
                    "frac": round(mix_bytes / (mix_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 3)},
        "roofline": ({"kernel": "conv layer 0 (" + pol_name.get(pols[0], "") + ")",
                      "bound": "hbm", "achieved": round(conv_gbs, 1),
                      "peak": PEAK_HBM_GBS, "unit": "GB/s",
                      "frac": round(conv_gbs / PEAK_HBM_GBS, 4), "traffic": traffic}
                     if hbm_bound else
                     {"kernel": "conv layer 0 (" + pol_name.get(pols[0], "") + ")",
                      "bound": "mfma", "achieved": round(conv_tflops, 2),
                      "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                      "frac": round(conv_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic}),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, d)
    print(json.dumps(out), flush=True)


def cpu_baseline_train(w, d, dy):
    """The oracle's training step (route, forward, gradients of the layer and of
    the routing, float64 direct loops) on sub-batches of the same workload until
    CPU_SAMPLE_SECONDS have passed."""
    import oracle
    L = w.layers[0]
    sub = min(w.B, 8)
    t0 = time.perf_counter()
    done = 0
    while True:
        lo = done % w.B
        hi = min(lo + sub, w.B)
        x = d["x"][lo:hi]
        alpha, _, _ = oracle.route(x, d["fc_w"], d["fc_b"], w.route_mode, w.temperature)
        oracle.forward(x, d["experts"][0], alpha, L.stride, L.pad, L.groups)
        _, da, _ = oracle.backward(x, d["experts"][0], alpha, dy[lo:hi], L.stride, L.pad, L.groups)
        oracle.route_backward(x, d["fc_w"], d["fc_b"], da, w.route_mode, w.temperature)
        done += hi - lo
        dt = time.perf_counter() - t0
        if dt >= CPU_SAMPLE_SECONDS:
            break
    return {"value": round(done / dt, 3), "unit": "images/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"{done} examples of {w.key} in sub-batches of {sub} (route, forward, dx, dalpha, "
                      f"dE and routing gradients, float64 direct loops), {dt:.1f} s"}


def train_main(args):
    """Training step of a single-layer workload: route, forward, then
    dynconv_backward_weights (dalpha, dE), dynconv_backward_data (dx) and
    dynconv_route_backward (dfc_w, dfc_b, pooling share added to dx), with the
    output gradient dy synthetic and resident like x."""
    import numpy as np
    import torch
    from dynamic_convolution_cnn_amd import binding as bd
    from dynamic_convolution_cnn_amd import inputs

    if args.profile:
        args.steps, args.warmup, args.no_cpu_baseline = min(args.steps, 10), min(args.warmup, 3), True
    w = inputs.WORKLOADS[args.workload]
    if len(w.layers) != 1 or w.attention:
        print(f"bench.py --backward: {w.key} is not a single-layer workload without channel attentions",
              file=sys.stderr)
        sys.exit(2)
    L = w.layers[0]
    d = inputs.make_inputs(w, seed=0)
    dy_host = inputs.bf16_round(np.random.default_rng(1).standard_normal((w.B, L.Cout, L.Ho, L.Wo),
                                                                         dtype=np.float32))
    if w.dtype != "bf16":
        dy_host = np.random.default_rng(1).standard_normal((w.B, L.Cout, L.Ho, L.Wo), dtype=np.float32)
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    e = to_dev(d["experts"][0], w.dtype)
    fc_w, fc_b = to_dev(d["fc_w"], "f32"), to_dev(d["fc_b"], "f32")
    x0, dy0 = to_dev(d["x"], w.dtype), to_dev(dy_host, w.dtype)
    esz = 2 if w.dtype == "bf16" else 4
    set_bytes = w.B * (2 * L.Cin * L.H * L.W + 2 * L.Cout * L.Ho * L.Wo) * esz
    R = max(1, math.ceil(ROTATE_BYTES / set_bytes))
    xs = [x0] + [x0.clone() for _ in range(R - 1)]
    dys = [dy0] + [dy0.clone() for _ in range(R - 1)]
    ys = [torch.empty((w.B, L.Cout, L.Ho, L.Wo), dtype=x0.dtype, device=dev) for _ in range(R)]
    dxs = [torch.empty_like(x0) for _ in range(R)]
    alphas = [torch.empty((w.B, w.n), dtype=torch.float32, device=dev) for _ in range(R)]
    das = [torch.empty((w.B, w.n), dtype=torch.float32, device=dev) for _ in range(R)]
    de = torch.empty(tuple(e.shape), dtype=torch.float32, device=dev)
    dfw = torch.empty((w.n, L.Cin), dtype=torch.float32, device=dev)
    dfb = torch.empty((w.n,), dtype=torch.float32, device=dev)
    desc = bd.layer_desc(x0, e, L.stride, L.pad, L.groups)
    pol = bd.dynconv_forward_policy(desc)
    ws_f = torch.empty(max(16, bd.dynconv_forward_workspace_bytes(desc, pol)), dtype=torch.uint8, device=dev)
    ws_w = torch.empty(max(16, bd.dynconv_backward_weights_workspace_bytes(desc)), dtype=torch.uint8, device=dev)
    ws_d = torch.empty(max(16, bd.dynconv_backward_data_workspace_bytes(desc)), dtype=torch.uint8, device=dev)
    rdesc = bd.make_desc(w.B, L.Cin, L.H, L.W, n=w.n, dtype=desc.dtype)
    ws_r = torch.zeros(max(16, bd.dynconv_route_workspace_bytes(rdesc)), dtype=torch.uint8, device=dev)
    ws_rb = torch.empty(max(16, bd.dynconv_route_backward_workspace_bytes(rdesc)), dtype=torch.uint8, device=dev)

    def bwd_weights(i):
        s = i % R
        bd.dynconv_backward_weights(xs[s], dys[s], e, alphas[s], L.stride, L.pad, L.groups, dalpha=das[s],
                                    dexperts=de, workspace=ws_w)

    def step(i, ev=None):
        s = i % R
        cur = torch.cuda.current_stream()
        marks = []

        def mark():
            if ev is not None:
                ev[len(marks)].record(cur)
                marks.append(1)
        mark()
        bd.dynconv_route(xs[s], fc_w, fc_b, w.route_mode, w.temperature, alpha=alphas[s], workspace=ws_r)
        mark()
        bd.dynconv_forward(xs[s], e, alphas[s], L.stride, L.pad, L.groups, policy=pol, y=ys[s], workspace=ws_f)
        mark()
        bwd_weights(s)
        mark()
        bd.dynconv_backward_data(dys[s], e, alphas[s], L.H, L.W, L.stride, L.pad, L.groups, dx=dxs[s],
                                 workspace=ws_d)
        mark()
        bd.dynconv_route_backward(xs[s], fc_w, alphas[s], das[s], w.route_mode, w.temperature, dx=dxs[s],
                                  dfc_w=dfw, dfc_b=dfb, workspace=ws_rb)
        mark()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    G = GRAPH_STEPS

    def capture(first, count, fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for j in range(count):
                fn(first + j)
        return g

    multi = [capture(s, G, step) for s in range(R)]
    single = [capture(s, 1, step) for s in range(R)]
    plan, i = [], 0
    while i + G <= args.steps:
        plan.append(multi[i % R]); i += G
    while i < args.steps:
        plan.append(single[i % R]); i += 1
    multi[0].replay(); single[0].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for g in plan:
        g.replay()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps

    # the dominant call, dynconv_backward_weights, back to back on the launch stream
    NC = 2 if args.profile else 10
    gw = capture(0, G, bwd_weights)
    gw.replay()
    torch.cuda.synchronize()
    cev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    cev[0].record(stream)
    for _ in range(NC):
        gw.replay()
    cev[1].record(stream)
    torch.cuda.synchronize()
    bw_ms = cev[0].elapsed_time(cev[1]) / (NC * G)

    # per-call times of eager steps, HIP events between the calls
    nk = min(args.steps, 20)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(nk)]
    for i in range(nk):
        step(i, evs[i])
    torch.cuda.synchronize()
    names = ["route", "forward", "backward_weights", "backward_data", "route_backward"]
    per = {nm: round(sum(ev[k].elapsed_time(ev[k + 1]) for ev in evs) / nk * 1e3, 2) for k, nm in enumerate(names)}
    per["backward_weights_back_to_back"] = round(bw_ms * 1e3, 2)

    # the kernel-gradient GEMM's work: 2 B Cout Ho Wo (Cin/g) k^2 FLOP, the same as the forward's
    gemm_flops = 2 * w.B * L.macs_per_example()
    bw_tflops = gemm_flops / (bw_ms * 1e-3) / 1e12
    step_flops = 3 * gemm_flops  # forward, kernel gradient and input gradient convolutions
    out = {
        "metric": METRIC,
        "value": round(w.B / (ms_per_step * 1e-3), 1),
        "unit": "images/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded numpy draws, shapes of the pages' networks; no dataset)",
        "config": {"workload": w.key, "title": w.title, "B": w.B, "n": w.n, "pass": "forward+backward",
                   "layers": [dict(Cin=L.Cin, Cout=L.Cout, H=L.H, W=L.W, k=L.k, stride=L.stride, pad=L.pad,
                                   groups=L.groups)],
                   "routing": "softmax(z/T)" if w.route_mode else "sigmoid", "rotating_sets": R},
        "tflops_step": round(step_flops / (ms_per_step * 1e-3) / 1e12, 2),
        "pct_bf16_peak_step": round(100 * step_flops / (ms_per_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "kernels_us": per,
        "roofline": {"kernel": "dynconv_backward_weights (kernel-gradient GEMM with its contraction into dalpha, dE)",
                     "bound": "mfma", "achieved": round(bw_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(bw_tflops / PEAK_BF16_TFLOPS, 4), "traffic": None},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_train(w, d, dy_host)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
