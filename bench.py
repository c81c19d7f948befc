#!/usr/bin/env python3
"""Throughput of the BitLinear forward (BitNet b1.58) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the forward over one batch of synthetic inputs: for the
default workload (the 3B model's decode layers) every layer of the set
q, k, v, o (3200 x 3200), gate, up (8640 x 3200), down (3200 x 8640) at every
batch M in {1, 4, 16}: bf16 activations quantised per token to int8, the
ternary x int8 product from 2-bit packed weights, and the fp32 rescale.
Weights are ternarised and packed once, before timing (a load-time step; its
throughput is reported separately under "weight_prep").  Steps rotate over
copies of the packed weights totalling >= 1 GiB so that neither the L2 nor
the 256 MB Infinity Cache serves them.  Each step is a captured HIP graph.

--workload stack_3b_26 times one token step (batch 16) through 26 decoder
layers of the 3B model's BitLinears, 104 forwards with all weights resident:
per layer qkv (9600 x 3200), o (3200 x 3200) reading the first 3200 columns
of qkv's output, gate_up (17280 x 3200), down (3200 x 8640) reading the first
8640 columns of gate_up's output; down's output feeds the next layer.

One JSON line is printed.  'value' is packed-weight GB/s over the whole step
(wall clock around K replays); 'roofline' reports the dominant kernel from a
replay in which every launch of it is bracketed by HIP events; 'cpu_baseline'
times the CPU oracle on a bounded sample of the same work.
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

METRIC = "packed-weight GB/s + effective ternary TOPS per BitLinear (decode GEMV, prefill GEMM)"
HBM_PEAK_GBS = 8000.0
INT8_PEAK_TOPS = 5000.0
MALL_DEFEAT_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode_3b",
                    choices=["decode_3b", "prefill_3b", "llama70b_layers", "stack_3b_26"])
    ap.add_argument("--batches", default=None, help="comma list overriding the workload's batch sizes")
    ap.add_argument("--layout", default="i2", choices=["i2", "b3", "b1"],
                    help="packed weight layout; b1 runs the binary-weight variant (sign quantiser)")
    ap.add_argument("--backward", action="store_true",
                    help="time the straight-through-estimator backward (dX and dW) of the workload's forwards "
                         "instead of the forward, and print its own JSON line")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device-to-device 5 times (a plain copy of known size for scaling "
                         "the FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (got --gpus {args.gpus}); this library has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_copy": n, "copies": 5}), flush=True)
        return

    from ternary_weight_linear_forward_amd import bitlinear as bl
    from ternary_weight_linear_forward_amd import synth, workloads

    wl = workloads.ALL[args.workload]
    layout = {"i2": bl.LAYOUT_I2, "b3": bl.LAYOUT_B3, "b1": bl.LAYOUT_B1}[args.layout]
    weight_quant = bl.binarize_weights if layout == bl.LAYOUT_B1 else bl.quantize_weights
    batches = tuple(int(b) for b in args.batches.split(",")) if args.batches else wl.batches
    dev = torch.device("cuda")
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    print(f"[bench] workload={wl.name} batches={batches} layout={args.layout}", file=sys.stderr, flush=True)

    # ---- weights: quantise + pack on the GPU (timed separately) --------------
    # The stack has 4 * 26 distinct weight tensors; the other workloads one
    # tensor per named layer.
    if wl is workloads.STACK_3B:
        chain = workloads.stack_chain(workloads.STACK_DEPTH)
        weight_specs = [(link.layer, workloads.seed_for(wl, link.index, 0)) for link in chain]
    else:
        chain = None
        weight_specs = [(layer, workloads.seed_for(wl, li, 0)) for li, layer in enumerate(wl.layers)]
    layers = []
    prep_ms = 0.0
    prep_bytes = 0
    with torch.cuda.stream(stream):
        for layer, seed in weight_specs:
            w = torch.from_numpy(synth.latent_weights(layer.N, layer.K, seed=seed)).to(dev)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            T, gamma = weight_quant(w, stream=stream)
            P = bl.pack(T, layout, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            prep_ms += e0.elapsed_time(e1)
            prep_bytes += w.numel() * 4
            layers.append({"layer": layer, "gamma": gamma, "P": [P]})
            del w, T
    set_bytes = sum(L["P"][0].numel() for L in layers)
    ncopies = max(1, math.ceil(MALL_DEFEAT_BYTES / set_bytes))
    for L in layers:
        L["P"] += [L["P"][0].clone() for _ in range(ncopies - 1)]
    torch.cuda.synchronize()
    print(f"[bench] packed set {set_bytes/1e6:.1f} MB x {ncopies} copies", file=sys.stderr, flush=True)

    # ---- activations, outputs, workspaces --------------------------------------
    # A job is one bitlinear_forward: input pointer/dtype/row stride, output.
    act = synth.activations_student_t_bf16 if wl.act_dist == "student_t" else synth.activations_bf16
    keep = []

    def make_job(M, L, x_ptr, x_dtype, ldx):
        layer = L["layer"]
        nws = bl.bitlinear_forward_workspace_bytes(M, layer.N, layer.K, layout, x_dtype)
        return {"M": M, "L": L, "x_ptr": x_ptr, "x_dtype": x_dtype, "ldx": ldx,
                "ws": torch.empty(max(nws, 16), dtype=torch.uint8, device=dev), "nws": nws,
                "y": torch.empty((M, layer.N), dtype=torch.float32, device=dev)}

    def bf16_input(M, K, seed):
        xd = torch.from_numpy(act(M, K, seed=seed).view(np.int16)).to(dev).view(torch.bfloat16)
        keep.append(xd)
        return xd

    jobs = []
    if chain is not None:
        # One token step through the stack: link i reads the first K columns
        # of link i-1's fp32 output and quantises them inside its forward.
        M = batches[0]
        x0 = bf16_input(M, chain[0].layer.K, workloads.seed_for(wl, 0, 1))
        for link, L in zip(chain, layers):
            if link.index == 0:
                jobs.append(make_job(M, L, x0.data_ptr(), bl.BF16, x0.stride(0)))
            else:
                prev = jobs[-1]["y"]
                jobs.append(make_job(M, L, prev.data_ptr(), bl.F32, prev.stride(0)))
    else:
        for M in batches:
            for li, L in enumerate(layers):
                xd = bf16_input(M, L["layer"].K, workloads.seed_for(wl, li, 1) + M)
                jobs.append(make_job(M, L, xd.data_ptr(), bl.BF16, xd.stride(0)))
    torch.cuda.synchronize()

    if args.backward:
        run_backward(args, wl, jobs, layout, ncopies, stream, dev)
        return

    def launch_job(j, copy):
        """The user path: one fused bitlinear_forward (quantiser + product + rescale)."""
        L = j["L"]
        layer = L["layer"]
        st = bl.bitlinear_forward(L["P"][copy].data_ptr(), layout, L["gamma"].data_ptr(), j["M"], layer.N, layer.K,
                                  j["x_ptr"], j["x_dtype"], j["ldx"], None, j["y"].data_ptr(), bl.F32,
                                  j["y"].stride(0), j["ws"].data_ptr(), j["nws"], stream.cuda_stream)
        if st:
            raise bl.BitlinearError(st, "bitlinear_forward")

    def step(copy):
        for j in jobs:
            launch_job(j, copy)

    # ---- capture one graph per weight copy -----------------------------------
    graphs = []
    with torch.cuda.stream(stream):
        step(0)  # eager warm-up before capture
        torch.cuda.synchronize()
        for c in range(ncopies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                step(c)
            graphs.append(g)
    torch.cuda.synchronize()
    print(f"[bench] captured {len(graphs)} graphs of {len(jobs)} forwards", file=sys.stderr, flush=True)

    with torch.cuda.stream(stream):
        for k in range(args.warmup):
            graphs[k % ncopies].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for k in range(args.steps):
            graphs[(args.warmup + k) % ncopies].replay()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    step_ms = e0.elapsed_time(e1) / args.steps
    print(f"[bench] timed {args.steps} steps: {step_ms:.4f} ms/step (wall {wall*1e3/args.steps:.4f})",
          file=sys.stderr, flush=True)

    packed_per_step = sum(j["L"]["P"][0].numel() for j in jobs)
    ops_per_step = sum(2 * j["M"] * j["L"]["layer"].N * j["L"]["layer"].K for j in jobs)
    value = packed_per_step / (step_ms * 1e-3) / 1e9
    tops = ops_per_step / (step_ms * 1e-3) / 1e12

    # ---- roofline: the product kernel of every job, timed on its own ---------
    # bitlinear_forward runs the activation quantiser, then the product kernel
    # (bitlinear_product_kernel names it), or, for 1-4 tokens, one GEMV with
    # the quantiser inside.  For the first kind each job's activations are
    # quantised once through the split entry point and the product kernel is
    # timed alone; the one-launch forwards are timed as called.  A HIP graph
    # of R back-to-back launches (rotating over the weight copies) is replayed
    # between two HIP events on the launch stream; a launch's duration is the
    # replay time / R.  Durations are summed per kernel name; the kernel with
    # the most time per step is the dominant one.
    R = 16
    for j in jobs:
        layer = j["L"]["layer"]
        M = j["M"]
        algo = bl.bitlinear_auto_algo(M, layer.N, layer.K, layout, j["x_dtype"])
        j["kernel"] = bl.bitlinear_product_kernel(M, layer.N, layer.K, layout, j["x_dtype"], bl.ALGO_AUTO)
        j["fused"] = j["kernel"].startswith(("bl::k_gemv_fq<", "bl::k_gemv_persist_fq<"))
        if j["fused"]:
            with torch.cuda.stream(stream):
                launch_job(j, 0)
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    for r in range(R):
                        launch_job(j, r % ncopies)
            j["graph"] = g
            continue
        tiled = algo == bl.ALGO_GEMV_MFMA and M > 4 and layer.K <= 65536
        j["beta"] = torch.empty(M, dtype=torch.float32, device=dev)
        s_ = stream.cuda_stream
        with torch.cuda.stream(stream):
            if tiled:
                nb = bl.bitlinear_act_tiled_bytes(M, layer.K, layout)
                j["xq"], j["ldq"], xdt = torch.empty(nb, dtype=torch.int8, device=dev), 0, bl.I8_TILED
                st = bl.bitlinear_quantize_act_tiled(j["x_ptr"], j["x_dtype"], M, layer.K, j["ldx"], layout,
                                                     j["xq"].data_ptr(), nb, j["beta"].data_ptr(), s_)
            else:
                j["ldq"] = (layer.K + 63) // 64 * 64
                j["xq"], xdt = torch.empty((M, j["ldq"]), dtype=torch.int8, device=dev), bl.I8
                st = bl.bitlinear_quantize_act(j["x_ptr"], j["x_dtype"], M, layer.K, j["ldx"], j["xq"].data_ptr(),
                                               j["ldq"], j["beta"].data_ptr(), s_)
            if st:
                raise bl.BitlinearError(st, "quantize (instrumented)")
            assert bl.bitlinear_product_kernel(M, layer.N, layer.K, layout, xdt, algo) == j["kernel"]

            # int8 input needs no staging; base-3 weights for the GEMM need room
            # for their i2 rewrite (that pass is then part of the timed launch)
            nws8 = bl.bitlinear_forward_workspace_bytes(M, layer.N, layer.K, layout, xdt)
            j["ws8"] = torch.empty(max(nws8, 16), dtype=torch.uint8, device=dev)

            def product(copy, j=j, xdt=xdt, algo=algo, nws8=nws8):
                L, lay = j["L"], j["L"]["layer"]
                st = bl.bitlinear_forward_algo(L["P"][copy].data_ptr(), layout, L["gamma"].data_ptr(), j["M"],
                                               lay.N, lay.K, j["xq"].data_ptr(), xdt, j["ldq"],
                                               j["beta"].data_ptr(), j["y"].data_ptr(), bl.F32, j["y"].stride(0),
                                               j["ws8"].data_ptr() if nws8 > 0 else None, nws8, algo,
                                               stream.cuda_stream)
                if st:
                    raise bl.BitlinearError(st, "forward (instrumented)")

            product(0)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for r in range(R):
                    product(r % ncopies)
            j["graph"] = g
    torch.cuda.synchronize()

    def product_bytes(j):
        # packed weights, the activations as the kernel reads them (int8 and
        # beta, or the fp32 / bf16 rows of a one-launch forward), gamma, Y
        layer = j["L"]["layer"]
        x = j["M"] * layer.K * (4 if j["x_dtype"] == bl.F32 else 2) if j["fused"] else j["M"] * layer.K + 4 * j["M"]
        return j["L"]["P"][0].numel() + x + 4 + 4 * j["M"] * layer.N

    per_kernel = {}
    reps = 5
    with torch.cuda.stream(stream):
        for j in jobs:
            ts = []
            for _ in range(reps):
                ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                ea.record(stream)
                j["graph"].replay()
                eb.record(stream)
                ts.append((ea, eb))
            torch.cuda.synchronize()
            j["launch_ms"] = sum(a.elapsed_time(b) for a, b in ts) / (reps * R)
            d = per_kernel.setdefault(j["kernel"], {"ms": 0.0, "bytes": 0, "ops": 0, "launches": 0, "jobs": []})
            layer = j["L"]["layer"]
            d["ms"] += j["launch_ms"]
            d["bytes"] += product_bytes(j)
            d["ops"] += 2 * j["M"] * layer.N * layer.K
            d["launches"] += 1
            d["jobs"].append(f"{layer.name}@M{j['M']}")
            d.setdefault("job_us", []).append(f"{layer.name}@M{j['M']}:{j['launch_ms'] * 1e3:.1f}")
    dom_name, dom = max(per_kernel.items(), key=lambda kv: kv[1]["ms"])
    avg_us = dom["ms"] / dom["launches"] * 1e3
    bound = "mfma" if "gemm" in dom_name else "hbm"
    if bound == "hbm":
        achieved = dom["bytes"] / (dom["ms"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = dom["ops"] / (dom["ms"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": INT8_PEAK_TOPS, "unit": "TOPS",
                "frac": round(achieved / INT8_PEAK_TOPS, 4)}
    roof.update({"traffic": measured_traffic(wl.name, dom_name), "kernel": dom_name, "avg_launch_us": round(avg_us, 3),
                 "jobs": dom["jobs"],
                 "algorithmic_bytes_per_launch": dom["bytes"] // dom["launches"],
                 "algorithmic_ops_per_launch": dom["ops"] // dom["launches"]})
    kernels = {k: {"avg_us": round(v["ms"] / v["launches"] * 1e3, 3),
                   "GB/s": round(v["bytes"] / (v["ms"] * 1e-3) / 1e9, 1),
                   "TOPS": round(v["ops"] / (v["ms"] * 1e-3) / 1e12, 2), "jobs": len(v["jobs"]),
                   "us_per_job": v["job_us"]}
               for k, v in per_kernel.items()}
    print(f"[bench] per-kernel: {json.dumps(kernels)}", file=sys.stderr, flush=True)

    # ---- CPU oracle baseline --------------------------------------------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, batches, args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "layers": {L["layer"].name: [L["layer"].N, L["layer"].K] for L in layers},
            "batches": list(batches),
            "layout": args.layout,
            "weights": "binary {-1, +1}" if layout == bl.LAYOUT_B1 else "ternary {-1, 0, +1}",
            "x_dtype": "bf16" if chain is None else "bf16 stack input, fp32 between links",
            **({"depth": workloads.STACK_DEPTH,
                "glue": "qkv -> o reads qkv[:, :3200]; gate_up -> down reads gate_up[:, :8640]; "
                        "down -> next layer's qkv; per-token int8 requantisation inside every forward"}
               if chain is not None else {}),
            "bitlinears_per_step": len(jobs),
            "y_dtype": "f32",
            "weight_copies": ncopies,
            "graph_replay": True,
        },
        "effective_tops": round(tops, 2),
        "us_per_bitlinear": round(step_ms * 1e3 / len(jobs), 3),
        "kernels": kernels,
        "weight_prep": {"GB/s_latent_fp32": round(prep_bytes / (prep_ms * 1e-3) / 1e9, 1),
                        "ms": round(prep_ms, 3)},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


FP32_MFMA_PEAK_TFLOPS = 157.3


def run_backward(args, wl, jobs, layout, ncopies, stream, dev):
    """Straight-through-estimator backward of every job: dX = gamma * dY @ T
    from the packed weights and dW = dY^T @ Xhat from the job's quantised
    activations, dY ~ N(0, 1) fp32.  Each kernel is timed as a HIP graph of R
    back-to-back launches (dX rotating over the weight copies) between HIP
    events on the launch stream."""
    import torch
    from ternary_weight_linear_forward_amd import bitlinear as bl
    from ternary_weight_linear_forward_amd import synth

    R = 8
    per = {}
    total_ms = 0.0
    total_flops = 0
    for ji, j in enumerate(jobs):
        L, layer, M = j["L"], j["L"]["layer"], j["M"]
        with torch.cuda.stream(stream):
            dy = torch.from_numpy(synth.activations_f32(M, layer.N, seed=1000 + ji)).to(dev)
            x = torch.empty((M, layer.K), dtype=torch.bfloat16, device=dev)
            x.view(torch.int16).copy_(torch.from_numpy(synth.activations_bf16(M, layer.K, seed=2000 + ji)
                                                       .view(np.int16)))
            xq, beta = bl.quantize_act(x, stream=stream)
            dx = torch.empty((M, layer.K), dtype=torch.float32, device=dev)
            dw = torch.empty((layer.N, layer.K), dtype=torch.float32, device=dev)
            nws = bl.bitlinear_backward_dx_workspace_bytes(M, layer.N, layer.K, layout)
            ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=dev)

            def run_dx(c, L=L, layer=layer, M=M, dy=dy, dx=dx, ws=ws, nws=nws):
                st = bl.bitlinear_backward_dx(L["P"][c].data_ptr(), layout, L["gamma"].data_ptr(), M, layer.N,
                                              layer.K, dy.data_ptr(), dy.stride(0), dx.data_ptr(), dx.stride(0),
                                              ws.data_ptr() if nws > 0 else None, nws, stream.cuda_stream)
                if st:
                    raise bl.BitlinearError(st, "backward_dx")

            def run_dw(c, layer=layer, M=M, dy=dy, dw=dw, xq=xq, beta=beta):
                st = bl.bitlinear_backward_dw(xq.data_ptr(), xq.stride(0), beta.data_ptr(), M, layer.N, layer.K,
                                              dy.data_ptr(), dy.stride(0), dw.data_ptr(), dw.stride(0),
                                              stream.cuda_stream)
                if st:
                    raise bl.BitlinearError(st, "backward_dw")

            for name, fn, nbytes in (
                    (bl.bitlinear_backward_kernel(M, layer.N, layer.K, 0), run_dx,
                     L["P"][0].numel() + 4 * M * layer.N + 4 * M * layer.K
                     + (2 * bl.bitlinear_packed_bytes(layer.N, layer.K, bl.LAYOUT_I2) if layout != bl.LAYOUT_I2 else 0)),
                    (bl.bitlinear_backward_kernel(M, layer.N, layer.K, 1), run_dw, M * layer.K + 4 * M + 4 * M * layer.N + 4 * layer.N * layer.K)):
                fn(0)
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    for r in range(R):
                        fn(r % ncopies)
                ts = []
                for _ in range(3):
                    ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    ea.record(stream)
                    g.replay()
                    eb.record(stream)
                    ts.append((ea, eb))
                torch.cuda.synchronize()
                ms = sum(a.elapsed_time(b) for a, b in ts) / (3 * R)
                flops = 2 * M * layer.N * layer.K
                d = per.setdefault(name, {"ms": 0.0, "bytes": 0, "flops": 0, "launches": 0, "jobs": []})
                d["ms"] += ms
                d["bytes"] += nbytes
                d["flops"] += flops
                d["launches"] += 1
                d["jobs"].append(f"{layer.name}@M{M}:{ms * 1e3:.1f}us")
                total_ms += ms
                total_flops += flops
                del g
    dom_name, dom = max(per.items(), key=lambda kv: kv[1]["ms"])
    intensity = dom["flops"] / dom["bytes"]
    if intensity > FP32_MFMA_PEAK_TFLOPS / HBM_PEAK_GBS * 1e3:
        ach = dom["flops"] / (dom["ms"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / FP32_MFMA_PEAK_TFLOPS, 4)}
    else:
        ach = dom["bytes"] / (dom["ms"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4)}
    roof.update({"traffic": None, "kernel": dom_name, "avg_launch_us": round(dom["ms"] / dom["launches"] * 1e3, 3)})
    kernels = {k: {"avg_us": round(v["ms"] / v["launches"] * 1e3, 3),
                   "GB/s": round(v["bytes"] / (v["ms"] * 1e-3) / 1e9, 1),
                   "TFLOP/s": round(v["flops"] / (v["ms"] * 1e-3) / 1e12, 2), "jobs": v["jobs"]}
               for k, v in per.items()}
    out = {
        "metric": "STE backward (dX and dW) effective fp32 TFLOP/s",
        "value": round(total_flops / (total_ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "ms_per_step": round(total_ms, 5),
        "higher_is_better": True,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "layout": args.layout, "pass": "backward",
                   "dY": "N(0,1) fp32", "batches": sorted({j["M"] for j in jobs})},
        "kernels": kernels,
        "roofline": roof,
    }
    print(json.dumps(out), flush=True)


def measured_traffic(workload, kernel):
    """HBM bytes per launch of 'kernel' from the committed rocprofv3 counter
    summary (profiles/traffic_*.txt), or None when there is none for this
    workload and kernel, or when the kernel sources changed since."""
    import glob
    import hashlib

    h = hashlib.sha256()
    for f in ("gemv.hip", "gemm.hip", "common.h"):
        with open(os.path.join(ROOT, "ternary_weight_linear_forward_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    for path in glob.glob(os.path.join(ROOT, "profiles", "traffic_*.txt")):
        kv = {}
        with open(path) as fh:
            for line in fh:
                if ": " in line and not line.startswith(("#", " ")):
                    k, v = line.rstrip("\n").split(": ", 1)
                    kv[k] = v
        if kv.get("workload") == workload and kv.get("kernel") == kernel and kv.get("source_sha256") == h.hexdigest():
            return int(kv["traffic_bytes_per_launch"])
    return None


def cpu_baseline(wl, batches, seconds):
    """The CPU oracle, untuned, on a bounded sample of the same work: whole
    layers of the workload (quantise the activations, exact product, rescale),
    cycling through the step's (batch, layer) pairs until about 'seconds' of
    CPU time has passed.  Reported in the same unit (packed-weight GB/s)."""
    import oracle

    from ternary_weight_linear_forward_amd import synth, workloads
    from ternary_weight_linear_forward_amd import bitlinear as bl

    act = synth.activations_student_t_bf16 if wl.act_dist == "student_t" else synth.activations_bf16
    pairs = [(M, li) for M in batches for li in range(len(wl.layers))]
    tern = {}
    done_bytes = 0
    done = []
    t_total = 0.0
    i = 0
    while t_total < seconds and i < 400 * len(pairs):
        M, li = pairs[i % len(pairs)]
        layer = wl.layers[li]
        if li not in tern:
            w = synth.latent_weights(layer.N, layer.K, seed=workloads.seed_for(wl, li, 0))
            tern[li] = oracle.quantize_weights(w)
        t, g = tern[li]
        x = act(M, layer.K, seed=workloads.seed_for(wl, li, 1) + M)
        t0 = time.perf_counter()
        oracle.forward(t, g, x)
        t_total += time.perf_counter() - t0
        done_bytes += bl.bitlinear_packed_bytes(layer.N, layer.K, bl.LAYOUT_I2)
        done.append(f"{layer.name}@M{M}")
        i += 1
    return {"value": round(done_bytes / t_total / 1e9, 4), "unit": "GB/s", "cores": oracle.threads_used(),
            "kind": "oracle",
            "sample": f"{len(done)} BitLinear forwards ({', '.join(done[:8])}{', ...' if len(done) > 8 else ''}) "
                      f"in {t_total:.1f} s"}


if __name__ == "__main__":
    main()
