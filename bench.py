#!/usr/bin/env python3
"""Benchmark of the rotated W4A16 linear (ParoQuant inference hot path) on MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 4]

One step = one pass of the whole path (channel scale, pairwise rotation, AWQ
unpack, dequant, contraction, bias, output rounding) over one batch of seeded
synthetic input, through libparo's C-ABI.  The default workload is the
largest single-GPU configuration: the seven linears of a Llama-3-8B decoder
layer (q, k, v, o, gate, up, down) at 4096 tokens in bf16, run back to back.
Every timed step reads a different copy of the layers' tensors (a rotation
through at least 512 MB of distinct buffers, twice the 256 MB MALL) with
every input already resident in device memory.

Prints ONE JSON line: metric, value (decode: weight GB/s = (qweight + qzeros +
scales bytes) / step time; prefill: TFLOP/s = 2*M*I*O summed over the layers
/ step time), the step time's p10 / p50 / p90, the roofline of the dominant
kernel (its algorithmic bytes or flops per launch over its average launch
duration, timed live with HIP events on the stream it runs on, beside a
ceiling measured live on the same GPU), and the fp64 CPU oracle timed on a
bounded sample of the same workload as a baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# layer groups that read the same input in the model (one grouped call each)
SHARED_INPUT = (("q_proj", "k_proj", "v_proj"), ("gate_proj", "up_proj"))
METRIC = "ParoQuant linear: decode weight GB/s, prefill TFLOP/s, % of roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense fp16 / bf16 MFMA, published
MALL_ROTATION_BYTES = 512 << 20
MAX_BUFFER_SETS = 256
PATH_NAMES = {1: "decode_fused", 2: "decode_split", 3: "prefill"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def layer_bytes(I, O, krot, G=128, bias=True):
    """Stored-tensor bytes of one layer: weight part and rotation part."""
    weight = I * O // 2 + (I // G) * O // 2 + (I // G) * O * 2
    rot = krot * I * 2 + krot * (I // 2) * 4 + I * 4 + (O * 2 if bias else 0)
    return weight, rot


# Sources of the dominant kernel of each path (counter readings are valid
# only for the code they were taken on).
KERNEL_FILES = {1: ("decode.hip", "common.hpp"), 2: ("decode.hip", "common.hpp"),
                3: ("prefill.hip", "common.hpp", "mfma.hpp")}


def gsuffix(args):
    """Key suffix of a non-default group size in profiles/traffic.json."""
    return "" if args.group == 128 else f"-g{args.group}"


def kernel_source_hash(path):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "rotation_int4_weight_amd", "csrc")
    for fn in KERNEL_FILES[path]:
        with open(os.path.join(csrc, fn), "rb") as f:
            h.update(fn.encode() + f.read())
    return h.hexdigest()[:16]


def load_traffic(workload, kernel_hash):
    """HBM bytes per launch of the dominant kernel, from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE readings (scaled by the readings of a
    plain copy of known size), or None when they were taken on other code."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    rec = data.get("workloads", {}).get(str(workload))
    if not rec or rec.get("kernel_sources") != kernel_hash:
        return None
    cal = data["calibration"]
    return round((rec["fetch_kib"] * cal["fetch_factor"] + rec["write_kib"] * cal["write_factor"]) * 1024)


QUANT_METRIC = "ParoQuant offline transform + quantize + pack: dense weight GB/s, % of HBM roofline"
KERNEL_FILES["quantize"] = ("quantize.hip", "common.hpp")


def bench_quantize(args, paro, synth, np, torch, dev):
    """Time paro_w4_quantize_pack on the workload's first layer shape (weight
    in the workload's activation dtype, symmetric codes as the public
    configuration uses), rotating through >= 512 MB of distinct weights."""
    spec = synth.WORKLOADS[args.workload]
    lname, I, O = spec["layers"][0]
    dt = spec["act"]
    tdt = torch.float16 if dt == synth.F16 else torch.bfloat16
    host = synth.make_layer(args.workload, 0, I, O, group_size=args.group)
    w = synth.make_w(args.workload, 0, O, I, dt)
    w_bytes = O * I * 2
    nsets = min(MAX_BUFFER_SETS, max(1, -(-MALL_ROTATION_BYTES // w_bytes)))
    log(f"quantize: workload {args.workload} layer {lname} ({O} x {I}), {nsets} weight copies")
    D = paro.DeviceLayer(host, device=dev)
    wds = [torch.from_numpy(w.view(np.int16)).to(dev).view(tdt) for _ in range(nsets)]
    qw = torch.empty((I, O // 8), dtype=torch.int32, device=dev)
    qz = torch.empty((I // args.group, O // 8), dtype=torch.int32, device=dev)
    sc = torch.empty((I // args.group, O), dtype=torch.int16, device=dev)
    stream = torch.cuda.current_stream()
    step = lambda i: paro.paro_w4_quantize_pack(D, wds[i % nsets], True, qw, qz, sc, stream=stream)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / args.steps
    weight_b, rot_b = layer_bytes(I, O, host.krot, G=args.group, bias=False)
    alg = w_bytes + weight_b + rot_b           # W read once; codes, zeros, scales written; rotation read
    value = w_bytes / (us * 1e-6) / 1e9
    ach = alg / (us * 1e-6) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import ref
        rows = 64
        G = args.group
        sub = synth.Layer(I, rows, G, host.krot, host.pairs, host.theta, host.channel_scales,
                          np.zeros((I, rows // 8), np.int32), np.zeros((I // G, rows // 8), np.int32),
                          np.zeros((I // G, rows), np.uint16), None)
        n, t_start = 0, time.perf_counter()
        while True:
            wr = ref.transform_weight(sub, np.ascontiguousarray(w[:rows]), dt)
            q, z, s16, _ = ref.quantize(wr, G, True)
            ref.pack(q, z, G)
            n += 1
            el = time.perf_counter() - t_start
            if el >= args.cpu_seconds or (el / n) * (n + 1) > 3 * args.cpu_seconds:
                break
        cpu = {"value": rows * I * 2 / (el / n) / 1e9, "unit": "GB/s", "cores": ref.threads(0), "kind": "oracle",
               "sample": f"{n} oracle transform+quantize+pack call(s) on {rows} of {O} output rows of "
                         f"'{lname}', {el:.1f} s"}
    out = {
        "metric": QUANT_METRIC, "value": round(value, 3), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us / 1e3, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{lname}-weight-{O}x{I}-{'f16' if dt == synth.F16 else 'bf16'}-sym{gsuffix(args)}",
                   "group_size": args.group, "krot": host.krot, "weight_copies": nsets,
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic(f"quantize-{args.workload}{gsuffix(args)}",
                                             kernel_source_hash("quantize")),
                     "kernel": "quantize_pack_kernel",
                     "avg_launch_us": round(us, 3)},
        "cpu_baseline": cpu, "kernel_sources": kernel_source_hash("quantize"),
    }
    print(json.dumps(out), flush=True)


BWD_METRIC = "ParoQuant rotation backward (dL/dx, dL/dtheta, dL/dcs): activation GB/s, % of HBM roofline"
KERNEL_FILES["rotate_backward"] = ("rotate_backward.hip", "common.hpp", "mfma.hpp")


def bench_rotate_backward(args, paro, synth, np, torch, dev):
    """Time paro_scale_rotate_backward on the workload's first layer input
    (tokens x I; x, g = dL/dx_r and gx in the activation dtype, as autograd
    hands them over), rotating through >= 512 MB of distinct (x, g) pairs."""
    spec = synth.WORKLOADS[args.workload]
    lname, I, O = spec["layers"][0]
    M, dt = max(spec["tokens"], 64), spec["act"]
    tdt = torch.float16 if dt == synth.F16 else torch.bfloat16
    host = synth.make_layer(args.workload, 0, I, O, group_size=args.group)
    x = synth.make_x(args.workload, 0, M, I, dt)
    g = synth.make_g(args.workload, 0, M, I, dt)
    pair_bytes = 2 * M * I * 2
    nsets = min(MAX_BUFFER_SETS, max(1, -(-MALL_ROTATION_BYTES // pair_bytes)))
    log(f"rotate_backward: workload {args.workload} layer {lname} input ({M} x {I}), {nsets} (x, g) copies")
    D = paro.DeviceLayer(host, device=dev)
    up = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(tdt)
    xs = [up(x) for _ in range(nsets)]
    gs = [up(g) for _ in range(nsets)]
    gx = torch.empty((M, I), dtype=tdt, device=dev)
    gth = torch.empty((host.krot, I // 2), dtype=torch.float32, device=dev)
    gcs = torch.empty((I,), dtype=torch.float32, device=dev)
    ws = torch.empty(max(paro.paro_scale_rotate_backward_workspace_bytes(D, M), 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    step = lambda i: paro.paro_scale_rotate_backward(D, xs[i % nsets], gs[i % nsets], gx, gth, gcs, ws,
                                                     stream=stream)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / args.steps
    act_b = 3 * M * I * 2                           # x and g read, gx written
    rot_b = host.krot * I * 2 + host.krot * (I // 2) * 4 + I * 4
    alg = act_b + 2 * rot_b                         # pairs, theta, cs read; dtheta, dcs written (same sizes)
    value = act_b / (us * 1e-6) / 1e9
    ach = alg / (us * 1e-6) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import ref
        rows = min(M, 256)
        xh, gh = x[:rows], bits_to_f64_host(g[:rows], dt, np)
        n, t_start = 0, time.perf_counter()
        while True:
            ref.scale_rotate_backward(host, xh, dt, gh)
            n += 1
            el = time.perf_counter() - t_start
            if el >= args.cpu_seconds or (el / n) * (n + 1) > 3 * args.cpu_seconds:
                break
        cpu = {"value": 3 * rows * I * 2 / (el / n) / 1e9, "unit": "GB/s", "cores": ref.threads(0),
               "kind": "oracle",
               "sample": f"{n} oracle backward call(s) on {rows} of {M} tokens of '{lname}' input, {el:.1f} s"}
    wl = f"{lname}-input-backward-t{M}x{I}-{'f16' if dt == synth.F16 else 'bf16'}{gsuffix(args)}"
    out = {
        "metric": BWD_METRIC, "value": round(value, 3), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us / 1e3, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl, "group_size": args.group, "krot": host.krot, "input_copies": nsets,
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic(f"rotate_backward-{args.workload}{gsuffix(args)}",
                                             kernel_source_hash("rotate_backward")),
                     "kernel": "bwd_rrow + bwd_gram_dx + bwd_walk + bwd_theta_reduce kernels (one entry point)",
                     "avg_launch_us": round(us, 3)},
        "cpu_baseline": cpu, "kernel_sources": kernel_source_hash("rotate_backward"),
    }
    print(json.dumps(out), flush=True)


ROT_METRIC = "ParoQuant input scaling + rotation (X -> X_r): activation GB/s, % of HBM roofline"
KERNEL_FILES["rotate"] = ("scale_rotate.hip", "common.hpp", "mfma.hpp")


def bench_rotate(args, paro, synth, np, torch, dev):
    """Time the input scaling and rotation of every layer of the workload, as
    the prefill path runs it: the dense per-group matrix built once per layer
    (paro_rotation_matrix) and applied on the matrix cores into the GEMM's
    tiled layout (paro_scale_rotate_tiled), with the staged rotation
    (paro_scale_rotate: krot Givens stages in LDS, row-major X_r) timed beside
    it on the same inputs.  >= 512 MB of distinct inputs are rotated through."""
    spec = synth.WORKLOADS[args.workload]
    M, dt = spec["tokens"], spec["act"]
    tdt = torch.float16 if dt == synth.F16 else torch.bfloat16
    layers = spec["layers"]
    up = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(tdt)
    set_bytes = sum(M * I * 2 for _, I, _ in layers)
    nsets = min(MAX_BUFFER_SETS, max(1, -(-MALL_ROTATION_BYTES // set_bytes)))
    log(f"rotate: workload {args.workload}, {len(layers)} layer(s), {M} tokens, {nsets} input copies")
    Ds, hls, xts, xrs, hosts = [], [], [], [], []
    xs = [[] for _ in range(nsets)]
    for li, (lname, I, O) in enumerate(layers):
        host = synth.make_layer(args.workload, li, I, O, group_size=args.group)
        hosts.append(host)
        D = paro.DeviceLayer(host, device=dev)
        Ds.append(D)
        hl = torch.empty((paro.paro_rotation_matrix_bytes(D) // 2,), dtype=torch.int16, device=dev)
        paro.paro_rotation_matrix(D, dt, hl)
        hls.append(hl)
        xts.append(torch.empty((paro.paro_tiled_bytes(D, M) // 2,), dtype=torch.int16, device=dev))
        xrs.append(torch.empty((M, I), dtype=tdt, device=dev))
        x = up(synth.make_x(args.workload, li, M, I, dt))
        for k in range(nsets):
            xs[k].append(x.clone())
    stream = torch.cuda.current_stream()

    def dense(i):
        for li, D in enumerate(Ds):
            paro.paro_scale_rotate_tiled(D, hls[li], xs[i % nsets][li], xts[li], stream=stream)

    def staged(i):
        for li, D in enumerate(Ds):
            paro.paro_scale_rotate(D, xs[i % nsets][li], xrs[li], stream=stream)

    def timeit(step):
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for i in range(args.steps):
            step(i)
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) * 1e3 / args.steps

    us = timeit(dense)
    us_staged = timeit(staged)
    act_b = sum(2 * M * I * 2 for _, I, _ in layers)     # X read, X_r written
    mat_b = sum((I // 128) * 2 * 128 * 128 * 2 for _, I, _ in layers)  # H and L read
    value = act_b / (us * 1e-6) / 1e9
    ach = (act_b + mat_b) / (us * 1e-6) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import ref
        rows = min(M, 16)
        hx = [np.ascontiguousarray(synth.make_x(args.workload, li, M, I, dt)[:rows])
              for li, (_, I, _) in enumerate(layers)]
        n, t_start = 0, time.perf_counter()
        while True:
            for li in range(len(layers)):
                ref.scale_rotate(hosts[li], hx[li], dt)
            n += 1
            el = time.perf_counter() - t_start
            if el >= args.cpu_seconds or (el / n) * (n + 1) > 3 * args.cpu_seconds:
                break
        cpu = {"value": sum(2 * rows * I * 2 for _, I, _ in layers) / (el / n) / 1e9, "unit": "GB/s",
               "cores": ref.threads(0), "kind": "oracle",
               "sample": f"{n} round(s) of oracle scale_rotate on the first {rows} of {M} token rows of every "
                         f"layer, {el:.1f} s"}
    wl = f"{spec['name']}-input-rotation{gsuffix(args)}"
    out = {
        "metric": ROT_METRIC, "value": round(value, 3), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us / 1e3, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl, "layers": [[n, I] for n, I, _ in layers], "tokens": M,
                   "group_size": args.group, "input_copies": nsets, "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic(f"rotate-{args.workload}{gsuffix(args)}", kernel_source_hash("rotate")),
                     "kernel": "rot_apply_kernel (one launch per layer)", "avg_launch_us": round(us / len(layers), 3),
                     "launches_per_step": len(layers)},
        "staged": {"kernel": "scale_rotate_kernel (one launch per layer)", "ms_per_step": round(us_staged / 1e3, 6),
                   "value": round(act_b / (us_staged * 1e-6) / 1e9, 3), "unit": "GB/s"},
        "cpu_baseline": cpu, "kernel_sources": kernel_source_hash("rotate"),
    }
    print(json.dumps(out), flush=True)


MOE_METRIC = "ParoQuant MoE projection (shared rotation, stacked experts): TFLOP/s, % of MFMA roofline"
KERNEL_FILES["moe"] = ("prefill.hip", "scale_rotate.hip", "common.hpp", "mx.hpp", "mfma.hpp")


def bench_moe(args, paro, synth, np, torch, dev):
    """Time paro_w4a16_moe_linear on a mixture-of-experts workload (experts
    stacked in one tensor, one shared rotation, seeded skewed top-k routing),
    rotating through >= 512 MB of distinct expert weights."""
    wl = args.workload if args.workload in synth.MOE_WORKLOADS else 5
    spec = synth.MOE_WORKLOADS[wl]
    lname, I, O = spec["layer"]
    E, dt = spec["experts"], spec["act"]
    tdt = torch.float16 if dt == synth.F16 else torch.bfloat16
    host = synth.make_moe_layer(wl, E, I, O, group_size=args.group)
    offs = synth.make_routing(wl, E, spec["tokens"], spec["top_k"])
    rows = int(offs[-1])
    x = synth.make_x(wl, 0, rows, I, dt)
    w_b, r_b = layer_bytes(I, O, host.krot, G=args.group)
    set_bytes = E * w_b
    nsets = min(MAX_BUFFER_SETS, max(1, -(-MALL_ROTATION_BYTES // set_bytes)))
    log(f"moe: {spec['name']}: {E} experts of {lname} ({I} -> {O}), {rows} routed rows, loads "
        f"{np.diff(offs).tolist()}, {nsets} weight sets")
    Ds = [paro.DeviceLayer(host, device=dev) for _ in range(nsets)]
    xd = torch.from_numpy(x.view(np.int16)).to(dev).view(tdt)
    od = torch.from_numpy(offs).to(dev)
    y = torch.empty((rows, O), dtype=tdt, device=dev)
    ws = paro.make_workspace(paro.paro_w4a16_moe_linear_workspace_bytes(Ds[0], rows, dt), device=dev)
    stream = torch.cuda.current_stream()
    step = lambda i: paro.paro_w4a16_moe_linear(Ds[i % nsets], E, od, xd, y, ws, stream=stream)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / args.steps
    flops = 2.0 * rows * I * O
    value = flops / (us * 1e-6) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import ref
        e0 = int(np.argmax(np.diff(offs)))
        n_rows = min(16, int(offs[e0 + 1] - offs[e0]))
        sub = ref.expert_layer(host, e0)
        xs = np.ascontiguousarray(x[offs[e0]:offs[e0] + n_rows])
        n, t_start = 0, time.perf_counter()
        while True:
            ref.linear(sub, xs, dt)
            n += 1
            el = time.perf_counter() - t_start
            if el >= args.cpu_seconds or (el / n) * (n + 1) > 3 * args.cpu_seconds:
                break
        cpu = {"value": 2.0 * n_rows * I * O / (el / n) / 1e12, "unit": "TFLOP/s", "cores": ref.threads(0),
               "kind": "oracle", "sample": f"{n} oracle call(s) on {n_rows} rows of expert {e0}, {el:.1f} s"}
    out = {
        "metric": MOE_METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us / 1e3, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if dt == synth.BF16 else "f16", "data": "synthetic",
        "config": {"workload": spec["name"] + gsuffix(args), "experts": E, "routed_rows": rows,
                   "top_k": spec["top_k"], "group_size": args.group, "krot": host.krot, "weight_sets": nsets,
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "mfma", "achieved": round(value, 1), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(value / MFMA_PEAK_TFLOPS, 4),
                     "traffic": load_traffic(f"moe-{wl}{gsuffix(args)}", kernel_source_hash("moe")),
                     "kernel": "rot_build + rot_apply + prefill_gemm_kernel<MoE> (one entry point)",
                     "avg_launch_us": round(us, 3)},
        "cpu_baseline": cpu, "kernel_sources": kernel_source_hash("moe"),
    }
    print(json.dumps(out), flush=True)


MX_METRIC = "ParoQuant W4A4 MXFP4 linear (rotation, activation quantization, FP4 GEMM): TFLOP/s, % of FP4 MFMA roofline"
FP4_PEAK_TFLOPS = 10100.0      # MI355X dense fp4 / fp6 MFMA, published
KERNEL_FILES["mxfp4"] = ("mxfp4.hip", "common.hpp", "mx.hpp", "mfma.hpp")


def bench_mxfp4(args, paro, synth, np, torch, dev):
    """Time paro_mxfp4_linear on the workload's first layer (weights quantized
    once with paro_mxfp4_quantize_weight), rotating through >= 512 MB of
    distinct weight codes; the GEMM alone is timed the same way for its
    roofline."""
    spec = synth.WORKLOADS[args.workload]
    lname, I, O = spec["layers"][0]
    M, dt = max(spec["tokens"], 1), spec["act"]
    tdt = torch.float16 if dt == synth.F16 else torch.bfloat16
    host = synth.make_layer(args.workload, 0, I, O, group_size=args.group)
    D = paro.DeviceLayer(host, device=dev)
    x = synth.make_x(args.workload, 0, M, I, dt)
    xd = torch.from_numpy(x.view(np.int16)).to(dev).view(tdt)
    w = synth.make_w(args.workload, 0, O, I, dt)
    wd = torch.from_numpy(w.view(np.int16)).to(dev).view(tdt)
    set_bytes = O * I // 2 + O * I // 32
    nsets = min(MAX_BUFFER_SETS, max(1, -(-MALL_ROTATION_BYTES // set_bytes)))
    wcs = [torch.empty((O, I // 2), dtype=torch.uint8, device=dev) for _ in range(nsets)]
    wss = [torch.empty((O, I // 32), dtype=torch.uint8, device=dev) for _ in range(nsets)]
    for c, sc in zip(wcs, wss):
        paro.paro_mxfp4_quantize_weight(D, wd, c, sc)
    log(f"mxfp4: workload {args.workload} layer {lname} ({I} -> {O}), {M} tokens, {nsets} weight code sets")
    y = torch.empty((M, O), dtype=tdt, device=dev)
    work = torch.empty(max(paro.paro_mxfp4_linear_workspace_bytes(D, M), 16), dtype=torch.uint8, device=dev)
    ac = torch.empty((M, I // 2), dtype=torch.uint8, device=dev)
    as_ = torch.empty((M, I // 32), dtype=torch.uint8, device=dev)
    aws = torch.empty(paro.paro_mxfp4_activation_workspace_bytes(D), dtype=torch.uint8, device=dev)
    paro.paro_mxfp4_quantize_activations(D, xd, ac, as_, aws)
    bias = D.bias
    stream = torch.cuda.current_stream()

    def timed(fn, n):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for i in range(n):
            fn(i)
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) * 1e3 / n

    # The layer's dense rotation R' is built once (paro_rotation_matrix), as
    # for the W4A16 prefill bench; --rebuild-rotation builds it in every call.
    if args.rebuild_rotation:
        us = timed(lambda i: paro.paro_mxfp4_linear(D, wcs[i % nsets], wss[i % nsets], xd, y, work, stream=stream),
                   args.steps)
    else:
        hl = torch.empty((paro.paro_rotation_matrix_bytes(D) // 2,), dtype=torch.int16, device=dev)
        paro.paro_rotation_matrix(D, dt, hl, stream=stream)
        pwork = torch.empty(max(paro.paro_mxfp4_linear_prepared_workspace_bytes(D, M), 16), dtype=torch.uint8,
                            device=dev)
        us = timed(lambda i: paro.paro_mxfp4_linear_prepared(D, hl, wcs[i % nsets], wss[i % nsets], xd, y, pwork,
                                                             stream=stream), args.steps)
    g_us = None
    if not args.no_kernel_timing:
        g_us = timed(lambda i: paro.paro_mxfp4_gemm(ac, as_, wcs[i % nsets], wss[i % nsets], y, bias, stream=stream),
                     args.steps)
    flops = 2.0 * M * I * O
    value = flops / (us * 1e-6) / 1e12
    k_us = g_us if g_us is not None else us
    ach = flops / (k_us * 1e-6) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import ref
        rows = min(M, 16)
        wc_h, ws_h = ref.mxfp4_weight(host, w, dt)
        n, t_start = 0, time.perf_counter()
        while True:
            a_c, a_s = ref.mxfp4_activations(host, np.ascontiguousarray(x[:rows]), dt)
            ref.mxfp4_matmul(a_c, a_s, wc_h, ws_h, host.bias)
            n += 1
            el = time.perf_counter() - t_start
            if el >= args.cpu_seconds or (el / n) * (n + 1) > 3 * args.cpu_seconds:
                break
        cpu = {"value": 2.0 * rows * I * O / (el / n) / 1e12, "unit": "TFLOP/s", "cores": ref.threads(0),
               "kind": "oracle", "sample": f"{n} oracle call(s) (rotate, quantize, dequantized product) on {rows} "
                                          f"of {M} tokens of '{lname}', {el:.1f} s"}
    out = {
        "metric": MX_METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us / 1e3, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp4", "data": "synthetic",
        "config": {"workload": f"{spec['name']}-mxfp4{gsuffix(args)}", "tokens": M, "layer": [lname, I, O],
                   "group_size": args.group, "krot": host.krot, "weight_sets": nsets,
                   "rotation_matrix": ("built in every call" if args.rebuild_rotation
                                       else "built once (paro_rotation_matrix), applied every call"),
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "mfma", "achieved": round(ach, 1), "peak": FP4_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ach / FP4_PEAK_TFLOPS, 4),
                     "traffic": load_traffic(f"mxfp4-{args.workload}{gsuffix(args)}", kernel_source_hash("mxfp4"))
                     if g_us is not None else None,
                     "kernel": "mx_gemm_kernel" if g_us is not None else "paro_mxfp4_linear (whole entry point)",
                     "avg_launch_us": round(k_us, 3)},
        "cpu_baseline": cpu, "kernel_sources": kernel_source_hash("mxfp4"),
    }
    print(json.dumps(out), flush=True)


def measured_ceiling(decode, layers, M, tdt, torch, dev, stream, achieved):
    """What this GPU delivers, measured live beside the spec peak.
    decode (HBM-bound): a plain device-to-device copy of 512 MiB, bytes read
    plus bytes written per second.  prefill (MFMA-bound): the library's dense
    GEMM (torch.nn.functional.linear, hipBLASLt) on the workload's own shapes
    in the activation dtype, each layer's X [M][I] times a dense [O][I]
    weight -- the same flops with a weight four times larger and no
    dequantization.
    Returns {"kind", "value", "unit", "frac"} with frac = achieved / value."""
    def timed(fn, n):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n * 1e-3
    if decode:
        src = torch.ones((512 << 20) // 4, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        t = timed(lambda: dst.copy_(src), 20)
        val = 2 * src.numel() * 4 / t / 1e9
        del src, dst
        return {"kind": "device copy of 512 MiB (read + write bytes / s)", "value": round(val, 1),
                "unit": "GB/s", "frac": round(achieved / val, 4)}
    ops = []
    for _, I, O, _, _ in layers:
        a = torch.randn((M, I), device=dev).to(tdt)
        w = torch.randn((O, I), device=dev).to(tdt)  # nn.Linear layout: the library's fastest on these shapes
        ops.append((a, w))
    t = timed(lambda: [torch.nn.functional.linear(a, w) for a, w in ops], 10)
    flops = sum(2.0 * M * I * O for _, I, O, _, _ in layers)
    val = flops / t / 1e12
    del ops
    return {"kind": "dense bf16 GEMM of the library (torch.nn.functional.linear, hipBLASLt) on the same shapes",
            "value": round(val, 1), "unit": "TFLOP/s", "frac": round(achieved / val, 4)}


def bits_to_f64_host(bits, dt, np):
    """fp16 / bf16 bit patterns (uint16) -> float64 (the oracle takes g in double)."""
    if dt == 0:
        return np.asarray(bits).view(np.float16).astype(np.float64)
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", type=int, default=4,
                    help="0..4 (synth.WORKLOADS); 4, the seven linears of a Llama-3-8B decoder layer at "
                         "4096 tokens, is the largest single-GPU configuration and the default")
    ap.add_argument("--path", type=int, default=0, help="0 auto, 1 decode_fused, 2 decode_split, 3 prefill")
    ap.add_argument("--group", type=int, default=128, choices=(32, 64, 128),
                    help="rotation / quantization group size G of the synthetic layers")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of the CPU-oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true", help="skip the per-kernel timing loop")
    ap.add_argument("--rebuild-rotation", action="store_true",
                    help="prefill and --op mxfp4: rebuild each layer's dense rotation in every call (paro_w4a16_linear, "
                         "paro_mxfp4_linear) "
                         "instead of building it once per layer (paro_w4a16_linear_prepared)")
    ap.add_argument("--no-group", action="store_true",
                    help="prefill: run every layer with its own calls instead of running the layers that read "
                         "the same input (q_proj + k_proj + v_proj, gate_proj + up_proj) through "
                         "paro_w4a16_linear_prepared_multi, one GEMM launch per group")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the measured ceiling (device copy for decode, library dense GEMM for prefill)")
    ap.add_argument("--op", choices=("linear", "quantize", "rotate", "rotate_backward", "moe", "mxfp4"),
                    default="linear",
                    help="linear: the inference hot path (default); quantize: the offline W -> (qweight, "
                         "qzeros, scales) transform of the workload's first layer; rotate_backward: the "
                         "calibration-time backward of the scaling and rotation over that layer's input; "
                         "moe: the mixture-of-experts projection of workload 5 (synth.MOE_WORKLOADS); "
                         "mxfp4: the W4A4 MXFP4 linear of the workload's first layer; rotate: the input "
                         "scaling and rotation of every layer (dense prefill form, staged form beside it)")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="BYTES",
                    help="instead of the benchmark: copy BYTES between two device buffers --steps times "
                         "(reference dispatches for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the rotated W4A16 linear is measured per GPU; the multi-GPU sharding is a design "
              "note, not a measured path.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.calib_copy:
        src = torch.ones(args.calib_copy // 4, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": src.numel() * 4, "dispatches": args.steps}), flush=True)
        return

    import rotation_int4_weight_amd as paro
    import synth

    paro.load()  # raises if libparo.so is missing: there is no fallback
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    if args.op == "quantize":
        bench_quantize(args, paro, synth, np, torch, dev)
        return
    if args.op == "rotate":
        bench_rotate(args, paro, synth, np, torch, dev)
        return
    if args.op == "rotate_backward":
        bench_rotate_backward(args, paro, synth, np, torch, dev)
        return
    if args.op == "moe":
        bench_moe(args, paro, synth, np, torch, dev)
        return
    if args.op == "mxfp4":
        bench_mxfp4(args, paro, synth, np, torch, dev)
        return
    spec = synth.WORKLOADS[args.workload]
    M, act = spec["tokens"], spec["act"]
    tdt = torch.float16 if act == synth.F16 else torch.bfloat16

    # ---- one host copy per layer, replicated into distinct device buffers ----
    layers = []
    per_set = 0
    for li, (lname, I, O) in enumerate(spec["layers"]):
        host = synth.make_layer(args.workload, li, I, O, group_size=args.group)
        x = synth.make_x(args.workload, li, M, I, act)
        w_b, r_b = layer_bytes(I, O, host.krot, G=args.group)
        per_set += w_b + r_b + M * I * 2
        layers.append((lname, I, O, host, x))
    nsets = min(MAX_BUFFER_SETS, max(1, -(-MALL_ROTATION_BYTES // per_set)))
    log(f"workload {args.workload} ({spec['name']}): {len(layers)} layer(s), {nsets} buffer sets "
        f"x {per_set / 1e6:.1f} MB")
    sets = []  # sets[s][l] = (DeviceLayer, x)
    for s in range(nsets):
        row = []
        for lname, I, O, host, x in layers:
            D = paro.DeviceLayer(host, device=dev)
            xd = torch.from_numpy(x.view(np.int16)).to(dev).view(tdt)
            row.append((D, xd))
        sets.append(row)
    path = args.path or paro.paro_w4a16_linear_choose_path(sets[0][0][0], M)
    ys = [torch.empty((M, O), dtype=tdt, device=dev) for _, I, O, _, _ in layers]
    ws_bytes = max(paro.paro_w4a16_linear_workspace_bytes(sets[0][l][0], M, act, path)
                   for l in range(len(layers)))
    ws = paro.make_workspace(ws_bytes, device=dev)
    stream = torch.cuda.current_stream()

    # Prefill: each layer's dense rotation R' = diag(cs) R is built once, like
    # its packed weight (it depends on the layer alone), and every step runs
    # paro_w4a16_linear_prepared: rotation applied, then the GEMM.  With
    # --rebuild-rotation every call rebuilds it (paro_w4a16_linear).
    prepared = path == 3 and not args.rebuild_rotation
    hls = None
    if prepared:
        hls = []
        for row in sets:
            hl_row = []
            for D, _ in row:
                hl = torch.empty((paro.paro_rotation_matrix_bytes(D) // 2,), dtype=torch.int16, device=dev)
                paro.paro_rotation_matrix(D, act, hl, stream=stream)
                hl_row.append(hl)
            hls.append(hl_row)

    # Layers that read the same input (the query, key and value projections,
    # the gate and up projections) run together, one rotation each and one
    # GEMM launch per group, on the group's first input.
    names = [n for n, _, _, _, _ in layers]
    groups, li = [], 0
    while li < len(layers):
        grp = [li]
        if prepared and not args.no_group:
            for names_g in SHARED_INPUT:
                k = len(names_g)
                if (tuple(names[li:li + k]) == names_g and
                        all(layers[li + j][1] == layers[li][1] for j in range(k))):  # same in_features
                    grp = list(range(li, li + k))
        groups.append(grp)
        li += len(grp)
    for grp in groups:
        if len(grp) > 1:
            Dg = [sets[0][l][0] for l in grp]
            ws_bytes = max(ws_bytes, paro.paro_w4a16_linear_prepared_multi_workspace_bytes(Dg, M))
    if ws_bytes > ws.numel() * ws.element_size():
        ws = paro.make_workspace(ws_bytes, device=dev)

    def step(i):
        row = sets[i % nsets]
        for grp in groups:
            if len(grp) > 1:
                paro.paro_w4a16_linear_prepared_multi([row[l][0] for l in grp], [hls[i % nsets][l] for l in grp],
                                                      row[grp[0]][1], [ys[l] for l in grp], ws, stream=stream)
                continue
            l = grp[0]
            D, xd = row[l]
            if prepared:
                paro.paro_w4a16_linear_prepared(D, hls[i % nsets][l], xd, ys[l], ws, stream=stream)
            else:
                paro.paro_w4a16_linear(D, xd, ys[l], ws, stream=stream, path=path)

    # ---- whole-path timing: HIP events at block boundaries ----
    # An event recorded on the stream costs the stream about 3 us (decode
    # steps measured 10.2 against 7.1 us with one event per step), so the
    # steps are marked in blocks of at least ~100 us: ms_per_step is the
    # whole run between the first and the last mark, and the spread is that
    # of the blocks' mean step times.
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(10):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    est_ms = e0.elapsed_time(e1) / 10
    block = max(1, min(args.steps, int(np.ceil(0.1 / max(est_ms, 1e-6)))))
    bounds = list(range(0, args.steps, block)) + [args.steps]
    marks = [torch.cuda.Event(enable_timing=True) for _ in bounds]
    torch.cuda.synchronize()
    marks[0].record(stream)
    for b in range(1, len(bounds)):
        for i in range(bounds[b - 1], bounds[b]):
            step(i)
        marks[b].record(stream)
    torch.cuda.synchronize()
    ms_per_step = marks[0].elapsed_time(marks[-1]) / args.steps
    per_block = np.array([marks[b].elapsed_time(marks[b + 1]) / (bounds[b + 1] - bounds[b])
                          for b in range(len(bounds) - 1)])
    p10, p50, p90 = (float(v) for v in np.percentile(per_block, [10, 50, 90]))

    weight_bytes = sum(layer_bytes(I, O, 8, G=args.group)[0] for _, I, O, _, _ in layers)
    flops = sum(2.0 * M * I * O for _, I, O, _, _ in layers)
    alg_bytes = sum(sum(layer_bytes(I, O, h.krot, G=args.group)) + M * I * 2 + M * O * 2
                    for _, I, O, h, _ in layers)
    decode = path in (1, 2)
    if decode:
        value, unit = weight_bytes / (ms_per_step * 1e-3) / 1e9, "GB/s"
    else:
        value, unit = flops / (ms_per_step * 1e-3) / 1e12, "TFLOP/s"

    # ---- dominant kernel, timed live on its own stream ----
    # decode_fused: the step is that one kernel.  decode_split: the GEMV run
    # alone over pre-rotated activations.  prefill: the GEMM run alone over
    # X_r already in its tiled layout.
    kern = None
    if not args.no_kernel_timing:
        n_launch = max(args.steps, 20)
        if path == 1:
            launch = step
            per_launch_bytes, per_launch_flops = alg_bytes, flops
            launches_per_call = len(layers)
        elif path == 2:
            xrs = []
            for row in sets:
                xr_row = []
                for D, xd in row:
                    xr = torch.empty_like(xd)
                    paro.paro_scale_rotate(D, xd, xr, stream=stream)
                    xr_row.append(xr)
                xrs.append(xr_row)

            def launch(i):
                row = sets[i % nsets]
                for l, (D, _) in enumerate(row):
                    paro.paro_w4a16_linear_prerotated(D, xrs[i % nsets][l], ys[l], ws, stream=stream, path=path)
            per_launch_bytes, per_launch_flops = alg_bytes, flops
            launches_per_call = len(layers)
        else:  # prefill: the GEMM kernel alone, over X_r already in its tiled layout
            xts = []
            for si, row in enumerate(sets):
                xt_row = []
                for l, (D, xd) in enumerate(row):
                    if hls is not None:
                        hl = hls[si][l]
                    else:
                        hl = torch.empty((paro.paro_rotation_matrix_bytes(D) // 2,), dtype=torch.int16, device=dev)
                        paro.paro_rotation_matrix(D, act, hl, stream=stream)
                    xt = torch.empty((paro.paro_tiled_bytes(D, M) // 2,), dtype=torch.int16, device=dev)
                    paro.paro_scale_rotate_tiled(D, hl, xd, xt, stream=stream)
                    xt_row.append(xt)
                    del hl
                xts.append(xt_row)

            def launch(i):
                row = sets[i % nsets]
                for grp in groups:
                    if len(grp) > 1:
                        paro.paro_w4a16_linear_tiled_multi([row[l][0] for l in grp],
                                                           [xts[i % nsets][l] for l in grp], act, M,
                                                           [ys[l] for l in grp], stream=stream)
                    else:
                        l = grp[0]
                        paro.paro_w4a16_linear_tiled(row[l][0], xts[i % nsets][l], act, M, ys[l], stream=stream)
            per_launch_bytes, per_launch_flops = alg_bytes, flops
            launches_per_call = len(groups)
        for i in range(min(args.warmup, 20)):
            launch(i)
        torch.cuda.synchronize()
        k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        k0.record(stream)
        for i in range(n_launch):
            launch(i)
        k1.record(stream)
        torch.cuda.synchronize()
        us = k0.elapsed_time(k1) * 1e3 / (n_launch * launches_per_call)
        kern = {"name": {1: "decode_kernel<fused>", 2: "decode_kernel", 3: "prefill_gemm_kernel"}[path],
                "avg_us": us, "launches": n_launch * launches_per_call, "launches_per_step": launches_per_call,
                "bytes_per_launch": per_launch_bytes / launches_per_call,
                "flops_per_launch": per_launch_flops / launches_per_call}

    khash = kernel_source_hash(path)
    roofline = None
    if kern:
        if decode:
            ach = kern["bytes_per_launch"] / (kern["avg_us"] * 1e-6) / 1e9
            roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(ach / HBM_PEAK_GBS, 4)}
        else:
            ach = kern["flops_per_launch"] / (kern["avg_us"] * 1e-6) / 1e12
            roofline = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(ach / MFMA_PEAK_TFLOPS, 4)}
        # (the committed readings are per launch of the grouped step; an
        # ungrouped run launches other kernels)
        ungrouped = "-nogroup" if path == 3 and args.no_group else ""
        roofline["traffic"] = load_traffic(f"{args.workload}{gsuffix(args)}{ungrouped}", khash)
        roofline["kernel"] = kern["name"]
        roofline["avg_launch_us"] = round(kern["avg_us"], 3)
        roofline["launches_per_step"] = kern["launches_per_step"]
        if not args.no_ceiling:
            roofline["measured_ceiling"] = measured_ceiling(decode, layers, M, tdt, torch, dev, stream, ach)

    # ---- CPU baseline: the oracle as it stands, on a bounded sample ----
    # decode: whole calls of every layer; prefill: the first `rows` token rows
    # of every layer (rows are independent), one pass over all layers per round
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import ref
        rows = M if decode else min(M, 16)
        xs = [np.ascontiguousarray(x[:rows]) for _, _, _, _, x in layers]
        n, t_start = 0, time.perf_counter()
        while True:
            for (lname, I, O, host, _), xr in zip(layers, xs):
                ref.linear(host, xr, act)
            n += 1
            el = time.perf_counter() - t_start
            if el >= args.cpu_seconds or (el / n) * (n + 1) > 3 * args.cpu_seconds:
                break
        per_round = el / n
        layer_list = ", ".join(l[0] for l in layers)
        if decode:
            cval, cunit = weight_bytes / per_round / 1e9, "GB/s"
            sample = f"{n} round(s) of full oracle calls on {layer_list} ({rows} token(s)), {el:.1f} s"
        else:
            cval, cunit = sum(2.0 * rows * I * O for _, I, O, _, _ in layers) / per_round / 1e12, "TFLOP/s"
            sample = f"{n} round(s) of oracle calls on the first {rows} of {M} token rows of {layer_list}, {el:.1f} s"
        cpu = {"value": cval, "unit": cunit, "cores": ref.threads(0), "kind": "oracle", "sample": sample}

    out = {
        "metric": METRIC, "value": round(value, 3), "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6),
        "ms_per_step_p10_p50_p90": [round(p10, 6), round(p50, 6), round(p90, 6)],
        "spread_over": f"{len(per_block)} blocks of {block} step(s)", "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "f16" if act == synth.F16 else "bf16", "data": "synthetic",
        "config": {"workload": spec["name"] + gsuffix(args), "layers": [[n, I, O] for n, I, O, _, _ in layers], "tokens": M,
                   "group_size": args.group, "krot": 8, "path": PATH_NAMES[path], "buffer_sets": nsets,
                   "rotation_matrix": ("built once per layer (paro_rotation_matrix), applied every step"
                                       if prepared else "built in every call" if path == 3 else None),
                   "grouped": [[names[l] for l in g] for g in groups if len(g) > 1] or None,
                   "parallelism": "single-gpu"},
        "roofline": roofline, "cpu_baseline": cpu, "kernel_sources": khash,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
