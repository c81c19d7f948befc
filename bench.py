#!/usr/bin/env python3
"""Throughput of the BitLinear forward (BitNet b1.58) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--mode grouped|single]

A step is one pass of the forward over one batch of synthetic inputs.  For the
default workload (the 3B model's decode layers) that is every layer of the set
q, k, v, o (3200 x 3200), gate, up (8640 x 3200), down (3200 x 8640) at every
batch M in {1, 4, 16}: bf16 activations quantised per token to int8, the
ternary x int8 product from 2-bit packed weights, and the fp32 rescale -- 21
BitLinear forwards.  With --mode grouped (the default) the seven layers of
one batch size are one bitlinear_forward_grouped call (3 calls per step);
--mode single issues 21 bitlinear_forward calls.

Weights are ternarised and packed once, before timing (a load-time step,
reported under "weight_prep").  Every call of a step reads its own copy of
the packed weights: the copies rotate over >= 2 GiB, so a copy is read again
only after 2 GiB of other weights, and neither the L2 nor the 256 MB Infinity
Cache can serve it.  Steps are captured HIP graphs replayed between HIP
events on the launch stream.

'roofline' reports the kernel with the most time per step, timed alone (a HIP
graph of back-to-back launches rotating over every weight copy, between HIP
events on the launch stream); 'prefill' the 3B prefill GEMM (M = 2048) the
same way, and its per-token activation quantiser alone against HBM
('prefill.quantiser'); 'cpu_baseline' the CPU oracle on a bounded sample of
the same work.

--workload stack_3b_26 times one token step (batch 16) through 26 decoder
layers of the 3B model's BitLinears (104 dependent forwards, all weights
resident; single calls only).
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
ROTATE_BYTES = 2 << 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode_3b",
                    choices=["decode_3b", "prefill_3b", "llama70b_layers", "stack_3b_26"])
    ap.add_argument("--mode", default="grouped", choices=["grouped", "single"],
                    help="grouped: the layers of one batch size in one bitlinear_forward_grouped call; "
                         "single: one bitlinear_forward per layer")
    ap.add_argument("--batches", default=None, help="comma list overriding the workload's batch sizes")
    ap.add_argument("--layers", default=None,
                    help="comma list of the workload's layer names to keep (e.g. q,k,v,o); not for the stack")
    ap.add_argument("--layout", default="i2", choices=["i2", "b3", "b1"],
                    help="packed weight layout; b1 runs the binary-weight variant (sign quantiser)")
    ap.add_argument("--backward", action="store_true",
                    help="time the straight-through-estimator backward (dX and dW) of the workload's forwards "
                         "instead of the forward, and print its own JSON line")
    ap.add_argument("--algo", default="auto", choices=["auto", "mfma", "addsub"],
                    help="the product algorithm of every forward (auto: the library's choice; mfma: the "
                         "matrix-core GEMV; addsub: the vector-ALU add/subtract GEMV, i2, M <= 16 in single mode "
                         "and M = 1 (--batches 1) in grouped mode)")
    ap.add_argument("--int8-input", action="store_true",
                    help="feed every forward activations quantised once beforehand (x_dtype I8 with beta), so a "
                         "step times the product kernels alone (not with --workload stack_3b_26)")
    ap.add_argument("--f1", action="store_true",
                    help="stack_3b_26: run every link through bitlinear_forward_chain, whose product writes the "
                         "per-token maxima of the next link's input and whose quantiser takes beta from them")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill GEMM sub-object")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device-to-device 5 times (a plain copy of known size for scaling "
                         "the FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


class Ctx:
    """Device, launch stream and the library binding."""

    def __init__(self, layout_name):
        import torch

        from ternary_weight_linear_forward_amd import bitlinear as bl

        self.torch = torch
        self.bl = bl
        self.dev = torch.device("cuda")
        torch.cuda.set_device(0)
        self.stream = torch.cuda.Stream()
        self.layout = {"i2": bl.LAYOUT_I2, "b3": bl.LAYOUT_B3, "b1": bl.LAYOUT_B1}[layout_name]
        self.layout_name = layout_name

    def events(self):
        t = self.torch
        return t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)


def prep_weights(ctx, wl, weight_specs):
    """Quantise and pack every weight tensor on the GPU (timed), then make
    copies of the packed set totalling >= ROTATE_BYTES."""
    torch, bl = ctx.torch, ctx.bl
    from ternary_weight_linear_forward_amd import synth

    weight_quant = bl.binarize_weights if ctx.layout == bl.LAYOUT_B1 else bl.quantize_weights
    layers, prep_ms, prep_bytes = [], 0.0, 0
    with torch.cuda.stream(ctx.stream):
        for layer, seed in weight_specs:
            w = torch.from_numpy(synth.latent_weights(layer.N, layer.K, seed=seed)).to(ctx.dev)
            torch.cuda.synchronize()
            e0, e1 = ctx.events()
            e0.record(ctx.stream)
            T, gamma = weight_quant(w, stream=ctx.stream)
            P = bl.pack(T, ctx.layout, stream=ctx.stream)
            e1.record(ctx.stream)
            torch.cuda.synchronize()
            prep_ms += e0.elapsed_time(e1)
            prep_bytes += w.numel() * 4
            layers.append({"layer": layer, "gamma": gamma, "P": [P]})
            del w, T
    return layers, prep_ms, prep_bytes


def add_copies(ctx, layers, ncopies):
    for L in layers:
        L["P"] += [L["P"][0].clone() for _ in range(ncopies - 1)]
    ctx.torch.cuda.synchronize()


def time_graphs(ctx, graphs, steps, warmup):
    """Replay the step graphs round robin: warm-up, then 'steps' replays
    between two HIP events on the launch stream.  Returns ms per step."""
    torch = ctx.torch
    with torch.cuda.stream(ctx.stream):
        for k in range(warmup):
            graphs[k % len(graphs)].replay()
        torch.cuda.synchronize()
        e0, e1 = ctx.events()
        e0.record(ctx.stream)
        for k in range(steps):
            graphs[(warmup + k) % len(graphs)].replay()
        e1.record(ctx.stream)
        torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def capture(ctx, fn):
    torch = ctx.torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(ctx.stream):
        with torch.cuda.graph(g, stream=ctx.stream):
            fn()
    return g


def time_launches(ctx, fn, ncalls, reps=3):
    """Average duration of one call of fn(i), i = 0 .. ncalls-1 captured back
    to back in one HIP graph, replayed 'reps' times between HIP events on the
    launch stream."""
    torch = ctx.torch
    with torch.cuda.stream(ctx.stream):
        fn(0)
        torch.cuda.synchronize()
    g = capture(ctx, lambda: [fn(i) for i in range(ncalls)])
    ts = []
    with torch.cuda.stream(ctx.stream):
        g.replay()  # warm
        for _ in range(reps):
            ea, eb = ctx.events()
            ea.record(ctx.stream)
            g.replay()
            eb.record(ctx.stream)
            ts.append((ea, eb))
        torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in ts) / (reps * ncalls)


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

    from ternary_weight_linear_forward_amd import synth, workloads

    ctx = Ctx(args.layout)
    bl = ctx.bl
    wl = workloads.ALL[args.workload]
    layout = ctx.layout
    batches = tuple(int(b) for b in args.batches.split(",")) if args.batches else wl.batches
    mode = "single" if wl is workloads.STACK_3B else args.mode
    algo = {"auto": bl.ALGO_AUTO, "mfma": bl.ALGO_GEMV_MFMA, "addsub": bl.ALGO_GEMV_ADDSUB}[args.algo]
    if algo == bl.ALGO_GEMV_ADDSUB and mode == "grouped" and (set(batches) != {1} or args.layout != "i2"):
        print("grouped calls take --algo addsub for i2 at one token only (--batches 1)", file=sys.stderr)
        sys.exit(2)
    if args.int8_input and mode != "single":
        print("--int8-input needs --mode single (a grouped call quantises its float inputs itself)", file=sys.stderr)
        sys.exit(2)
    if args.layers and wl is workloads.STACK_3B:
        print("--layers does not apply to the stack (its links follow each other)", file=sys.stderr)
        sys.exit(2)
    if args.f1 and wl is not workloads.STACK_3B:
        print("--f1 applies to --workload stack_3b_26", file=sys.stderr)
        sys.exit(2)
    if args.int8_input and wl is workloads.STACK_3B:
        print("--int8-input does not apply to the stack (its links requantise fp32 outputs)", file=sys.stderr)
        sys.exit(2)
    log(f"workload={wl.name} batches={batches} layout={args.layout} mode={mode}")

    # ---- weights ----------------------------------------------------------------
    if wl is workloads.STACK_3B:
        chain = workloads.stack_chain(workloads.STACK_DEPTH)
        specs = [(link.layer, workloads.seed_for(wl, link.index, 0)) for link in chain]
    else:
        chain = None
        names = args.layers.split(",") if args.layers else [l.name for l in wl.layers]
        unknown = set(names) - {l.name for l in wl.layers}
        if unknown:
            print(f"--layers: {sorted(unknown)} not in {wl.name}", file=sys.stderr)
            sys.exit(2)
        specs = [(layer, workloads.seed_for(wl, li, 0)) for li, layer in enumerate(wl.layers) if layer.name in names]
    layers, prep_ms, prep_bytes = prep_weights(ctx, wl, specs)
    set_bytes = sum(L["P"][0].numel() for L in layers)

    # ---- activations and the calls of a step -------------------------------------
    act = synth.activations_student_t_bf16 if wl.act_dist == "student_t" else synth.activations_bf16
    keep = []

    def bf16_input(M, K, seed):
        xd = torch.from_numpy(act(M, K, seed=seed).view(np.int16)).to(ctx.dev).view(torch.bfloat16)
        keep.append(xd)
        return xd

    # A job is one BitLinear forward; a call is what the step issues (one
    # bitlinear_forward, or one grouped call over the layers of one batch).
    jobs = []
    if chain is not None:
        M = batches[0]
        x0 = bf16_input(M, chain[0].layer.K, workloads.seed_for(wl, 0, 1))
        for link, L in zip(chain, layers):
            y = torch.empty((M, L["layer"].N), dtype=torch.float32, device=ctx.dev)
            if link.index == 0:
                jobs.append({"M": M, "L": L, "x": x0, "y": y})
            else:
                prev = jobs[-1]["y"]
                jobs.append({"M": M, "L": L, "x": prev[:, :L["layer"].K], "y": y})
    else:
        for M in batches:
            for li, L in enumerate(layers):
                jobs.append({"M": M, "L": L, "x": bf16_input(M, L["layer"].K, workloads.seed_for(wl, li, 1) + M),
                             "y": torch.empty((M, L["layer"].N), dtype=torch.float32, device=ctx.dev)})
    for j in jobs:
        lay = j["L"]["layer"]
        j["x_dtype"] = bl.F32 if j["x"].dtype == torch.float32 else bl.BF16
        j["beta"] = None
        if args.int8_input:
            with torch.cuda.stream(ctx.stream):
                j["x"], j["beta"] = bl.quantize_act(j["x"], stream=ctx.stream)
            j["x_dtype"] = bl.I8
        nws = bl.bitlinear_forward_workspace_bytes(j["M"], lay.N, lay.K, layout, j["x_dtype"])
        j["nws"] = nws
        j["ws"] = torch.empty(max(nws, 16), dtype=torch.uint8, device=ctx.dev)
    if args.f1:
        # producer-side maxima: link l's product writes them over link l+1's K
        for ji, j in enumerate(jobs):
            lay = j["L"]["layer"]
            j["parts"] = bl.bitlinear_forward_chain_parts(j["M"], lay.N, lay.K, layout)
            last = ji + 1 == len(jobs)
            j["pmax"] = None if last else torch.empty(j["parts"] * 16, dtype=torch.float32, device=ctx.dev)
            j["pmax_cols"] = 0 if last else jobs[ji + 1]["L"]["layer"].K
        for ji, j in enumerate(jobs):
            j["pmax_in"] = jobs[ji - 1]["pmax"] if ji > 0 else None
            j["nparts_in"] = jobs[ji - 1]["parts"] if ji > 0 else 0
    if mode == "grouped":
        calls = [[j for j in jobs if j["M"] == M] for M in batches]
    else:
        calls = [[j] for j in jobs]

    # Weight copies.  Independent layers: call c of step s reads copy
    # (s * ncalls + c) % ncopies, so consecutive reads of one copy are
    # ncopies calls, >= ROTATE_BYTES of weights, apart.  The stack: step s
    # reads copy s % ncopies of all 104 tensors.
    per_step = sum(j["L"]["P"][0].numel() for j in jobs)
    bytes_per_call = per_step / len(calls)
    if chain is None:
        ncopies = max(len(calls), math.ceil(ROTATE_BYTES / max(bytes_per_call, 1)))
    else:
        ncopies = max(2, math.ceil(ROTATE_BYTES / set_bytes))

    def copy_of(s, ci):
        return (s * len(calls) + ci) % ncopies if chain is None else s % ncopies

    add_copies(ctx, layers, ncopies)
    log(f"packed set {set_bytes / 1e6:.1f} MB x {ncopies} copies; {len(calls)} calls of {len(jobs)} forwards per step")

    def grouped_arrays(call, copy):
        specs_ = [(j["L"]["P"][copy], j["L"]["gamma"], j["x"], j["L"]["layer"].N, j["L"]["layer"].K) for j in call]
        arr, _ = bl.grouped_jobs(specs_, outs=[j["y"] for j in call])
        return arr

    for ci, call in enumerate(calls):
        if mode == "grouped":
            arr = grouped_arrays(call, 0)
            nws = bl.bitlinear_forward_grouped_workspace_bytes(arr, len(call), layout, call[0]["x_dtype"])
            call_ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=ctx.dev)
            for j in call:
                j["call"] = {"ws": call_ws, "nws": nws, "index": ci}

    def launch_call(ci, copy):
        call = calls[ci]
        s_ = ctx.stream.cuda_stream
        if mode == "grouped":
            arr = grouped_arrays(call, copy)
            c = call[0]["call"]
            st = bl.bitlinear_forward_grouped_algo(arr, len(call), layout, call[0]["x_dtype"], bl.F32, algo,
                                                   c["ws"].data_ptr(), c["nws"], s_)
            if st:
                raise bl.BitlinearError(st, "bitlinear_forward_grouped_algo")
            return
        j = call[0]
        L, lay = j["L"], j["L"]["layer"]
        if args.f1:
            st = bl.bitlinear_forward_chain(
                L["P"][copy].data_ptr(), layout, L["gamma"].data_ptr(), j["M"], lay.N, lay.K, j["x"].data_ptr(),
                j["x_dtype"], j["x"].stride(0), j["pmax_in"].data_ptr() if j["pmax_in"] is not None else None,
                j["nparts_in"], j["y"].data_ptr(), bl.F32, j["y"].stride(0),
                j["pmax"].data_ptr() if j["pmax"] is not None else None, j["pmax_cols"], j["ws"].data_ptr(), j["nws"],
                s_)
            if st:
                raise bl.BitlinearError(st, "bitlinear_forward_chain")
            return
        st = bl.bitlinear_forward_algo(L["P"][copy].data_ptr(), layout, L["gamma"].data_ptr(), j["M"], lay.N, lay.K,
                                       j["x"].data_ptr(), j["x_dtype"], j["x"].stride(0),
                                       j["beta"].data_ptr() if j["beta"] is not None else None, j["y"].data_ptr(),
                                       bl.F32, j["y"].stride(0), j["ws"].data_ptr() if j["nws"] > 0 else None,
                                       j["nws"], algo, s_)
        if st:
            raise bl.BitlinearError(st, "bitlinear_forward")

    def step(s):
        for ci in range(len(calls)):
            launch_call(ci, copy_of(s, ci))

    if args.backward:
        run_backward(args, wl, jobs, layout, ncopies, ctx.stream, ctx.dev)
        return

    # ---- timed steps -------------------------------------------------------------
    nsteps_distinct = ncopies // math.gcd(ncopies, len(calls)) if chain is None else ncopies
    with torch.cuda.stream(ctx.stream):
        step(0)
        torch.cuda.synchronize()
    graphs = [capture(ctx, lambda s=s: step(s)) for s in range(nsteps_distinct)]
    torch.cuda.synchronize()
    log(f"captured {len(graphs)} step graphs")
    step_ms = time_graphs(ctx, graphs, args.steps, args.warmup)
    log(f"timed {args.steps} steps: {step_ms:.4f} ms/step")
    ops_per_step = sum(2 * j["M"] * j["L"]["layer"].N * j["L"]["layer"].K for j in jobs)
    value = per_step / (step_ms * 1e-3) / 1e9
    tops = ops_per_step / (step_ms * 1e-3) / 1e12

    # ---- roofline: every call's kernels timed alone ------------------------------
    # A call of one launch (a grouped call that quantises inside, or a
    # one-launch forward) is timed as called.  A call that runs the quantiser
    # first is timed whole and, for the product kernel alone, with its
    # activations quantised once beforehand (bitlinear_product_kernel /
    # bitlinear_grouped_kernel name the kernel).  Graphs of back-to-back calls
    # rotate over every weight copy.
    per_kernel = {}
    call_us = []
    for ci, call in enumerate(calls):
        kname, one_launch = call_kernel(ctx, call, mode, layout, algo)
        ms_call = time_launches(ctx, lambda i, ci=ci: launch_call(ci, i % ncopies), ncopies)
        call_us.append(round(ms_call * 1e3, 3))
        if one_launch:
            ms = ms_call
        elif mode == "single":
            ms = time_product_only(ctx, call[0], layout, ncopies, algo)
        else:
            ms = None  # the grouped product behind a quantiser launch: counted in the call time only
        if ms is None:
            continue
        d = per_kernel.setdefault(kname, {"ms": 0.0, "bytes": 0, "ops": 0, "launches": 0, "calls": []})
        d["ms"] += ms
        d["bytes"] += sum(product_bytes(bl, j, layout, one_launch) for j in call)
        d["ops"] += sum(2 * j["M"] * j["L"]["layer"].N * j["L"]["layer"].K for j in call)
        d["launches"] += 1
        d["calls"].append(f"{'+'.join(j['L']['layer'].name for j in call)}@M{call[0]['M']}:{ms * 1e3:.2f}us")
    if not per_kernel:  # every call quantises in a launch of its own: the calls themselves
        for ci, call in enumerate(calls):
            d = per_kernel.setdefault("grouped call (quantiser + product)",
                                      {"ms": 0.0, "bytes": 0, "ops": 0, "launches": 0, "calls": []})
            d["ms"] += call_us[ci] * 1e-3
            d["bytes"] += sum(product_bytes(bl, j, layout, True) for j in call)
            d["ops"] += sum(2 * j["M"] * j["L"]["layer"].N * j["L"]["layer"].K for j in call)
            d["launches"] += 1
            d["calls"].append(f"M{call[0]['M']}:{call_us[ci]:.2f}us")
    dom_name, dom = max(per_kernel.items(), key=lambda kv: kv[1]["ms"])
    avg_us = dom["ms"] / dom["launches"] * 1e3
    bound = "mfma" if "gemm" in dom_name else "hbm"
    roof = roofline(bound, dom)
    roof.update({"traffic": measured_traffic(wl.name, dom_name), "kernel": dom_name,
                 "avg_launch_us": round(avg_us, 3), "launches_per_step": dom["launches"], "calls": dom["calls"],
                 "algorithmic_bytes_per_launch": dom["bytes"] // dom["launches"],
                 "algorithmic_ops_per_launch": dom["ops"] // dom["launches"],
                 "timing": "HIP events on the launch stream around a graph of back-to-back calls over every weight "
                           "copy"})
    kernels = {k: {"avg_us": round(v["ms"] / v["launches"] * 1e3, 3),
                   "GB/s": round(v["bytes"] / (v["ms"] * 1e-3) / 1e9, 1),
                   "TOPS": round(v["ops"] / (v["ms"] * 1e-3) / 1e12, 2), "calls": v["calls"]}
               for k, v in per_kernel.items()}
    log(f"per-kernel: {json.dumps(kernels)}")

    prefill = None
    if wl is workloads.DECODE_3B and not args.no_prefill and args.layout == "i2":
        prefill = run_prefill(ctx, args)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, batches, args.cpu_seconds, layout)

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
            "layers": {L["layer"].name: [L["layer"].N, L["layer"].K] for L in layers[:7]},
            "batches": list(batches),
            "layout": args.layout,
            "weights": "binary {-1, +1}" if layout == bl.LAYOUT_B1 else "ternary {-1, 0, +1}",
            "x_dtype": "bf16" if chain is None else "bf16 stack input, fp32 between links",
            **({"depth": workloads.STACK_DEPTH,
                "glue": "qkv -> o reads qkv[:, :3200]; gate_up -> down reads gate_up[:, :8640]; "
                        "down -> next layer's qkv; per-token int8 requantisation inside every forward"}
               if chain is not None else {}),
            "bitlinears_per_step": len(jobs),
            "calls_per_step": len(calls),
            "mode": mode,
            **({"algo": args.algo} if algo != bl.ALGO_AUTO else {}),
            **({"input": "int8 activations and beta quantised before the timed steps"} if args.int8_input else {}),
            **({"f1": "bitlinear_forward_chain: each product writes per-workgroup maxima of the next link's input, "
                      "the next quantiser takes beta from them"} if args.f1 else {}),
            "y_dtype": "f32",
            "weight_copies": ncopies,
            "rotation_bytes": int(ncopies * (bytes_per_call if chain is None else set_bytes)),
            "graph_replay": True,
        },
        "effective_tops": round(tops, 2),
        "us_per_bitlinear": round(step_ms * 1e3 / len(jobs), 3),
        "us_per_call": call_us,
        "kernels": kernels,
        "weight_prep": {"GB/s_latent_fp32": round(prep_bytes / (prep_ms * 1e-3) / 1e9, 1),
                        "ms": round(prep_ms, 3)},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if prefill is not None:
        out["prefill"] = prefill
    print(json.dumps(out), flush=True)


def roofline(bound, d):
    if bound == "hbm":
        achieved = d["bytes"] / (d["ms"] * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    achieved = d["ops"] / (d["ms"] * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 1), "peak": INT8_PEAK_TOPS, "unit": "TFLOP/s",
            "frac": round(achieved / INT8_PEAK_TOPS, 4)}


def call_kernel(ctx, call, mode, layout, algo):
    """(name of the product kernel of a call, whether the call is that one
    launch)."""
    bl = ctx.bl
    if mode == "grouped":
        specs_ = [(j["L"]["P"][0], j["L"]["gamma"], j["x"], j["L"]["layer"].N, j["L"]["layer"].K) for j in call]
        arr, _ = bl.grouped_jobs(specs_, outs=[j["y"] for j in call])
        name = bl.bitlinear_grouped_kernel_algo(arr, len(call), layout, call[0]["x_dtype"], algo)
        one = name is not None and (name.endswith(f", {call[0]['x_dtype']}>") or "_addsub<" in name)
        return name, one
    j = call[0]
    lay = j["L"]["layer"]
    name = bl.bitlinear_product_kernel(j["M"], lay.N, lay.K, layout, j["x_dtype"], algo)
    return name, j["x_dtype"] == bl.I8 or name.startswith(("bl::k_gemv_fq<", "bl::k_gemv_persist_fq<"))


def product_bytes(bl, j, layout, one_launch):
    """Algorithmic bytes of one job's product: packed weights, the activations
    as the kernel reads them (the fp32 / bf16 rows when it quantises them
    itself, else int8 and beta), gamma, and the fp32 output."""
    lay = j["L"]["layer"]
    es = 4 if j["x_dtype"] == bl.F32 else 2
    x = j["M"] * lay.K * es if one_launch and j["x_dtype"] != bl.I8 else j["M"] * lay.K + 4 * j["M"]
    return bl.bitlinear_packed_bytes(lay.N, lay.K, layout) + x + 4 + 4 * j["M"] * lay.N


def time_product_only(ctx, j, layout, ncopies, algo):
    """The product kernel of a single forward alone: its activations quantised
    once beforehand (through the split entry points), then the forward on
    int8 input, rotating over the weight copies."""
    torch, bl = ctx.torch, ctx.bl
    L, lay, M = j["L"], j["L"]["layer"], j["M"]
    if algo == bl.ALGO_AUTO:
        algo = bl.bitlinear_auto_algo(M, lay.N, lay.K, layout, j["x_dtype"])
    tiled = algo == bl.ALGO_GEMV_MFMA and M > 4 and lay.K <= 65536
    beta = torch.empty(M, dtype=torch.float32, device=ctx.dev)
    s_ = ctx.stream.cuda_stream
    with torch.cuda.stream(ctx.stream):
        if tiled:
            nb = bl.bitlinear_act_tiled_bytes(M, lay.K, layout)
            xq, ldq, xdt = torch.empty(nb, dtype=torch.int8, device=ctx.dev), 0, bl.I8_TILED
            st = bl.bitlinear_quantize_act_tiled(j["x"].data_ptr(), j["x_dtype"], M, lay.K, j["x"].stride(0), layout,
                                                 xq.data_ptr(), nb, beta.data_ptr(), s_)
        else:
            ldq = (lay.K + 63) // 64 * 64
            xq, xdt = torch.empty((M, ldq), dtype=torch.int8, device=ctx.dev), bl.I8
            st = bl.bitlinear_quantize_act(j["x"].data_ptr(), j["x_dtype"], M, lay.K, j["x"].stride(0), xq.data_ptr(),
                                           ldq, beta.data_ptr(), s_)
        if st:
            raise bl.BitlinearError(st, "quantize (instrumented)")
    nws8 = bl.bitlinear_forward_workspace_bytes(M, lay.N, lay.K, layout, xdt)
    ws8 = torch.empty(max(nws8, 16), dtype=torch.uint8, device=ctx.dev)

    def product(i):
        st = bl.bitlinear_forward_algo(L["P"][i % ncopies].data_ptr(), layout, L["gamma"].data_ptr(), M, lay.N,
                                       lay.K, xq.data_ptr(), xdt, ldq, beta.data_ptr(), j["y"].data_ptr(), bl.F32,
                                       j["y"].stride(0), ws8.data_ptr() if nws8 > 0 else None, nws8, algo, s_)
        if st:
            raise bl.BitlinearError(st, "forward (instrumented)")

    return time_launches(ctx, product, ncopies)


def run_prefill(ctx, args):
    """The 3B prefill GEMM (M = 2048, Student-t activations, i2): a step of
    its three forwards (quantiser + GEMM each), and the GEMM kernel alone on
    pre-quantised int8 activations, rotating over weight copies of >= 2 GiB."""
    torch, bl = ctx.torch, ctx.bl
    from ternary_weight_linear_forward_amd import synth, workloads

    wl = workloads.PREFILL_3B
    M = wl.batches[0]
    layers, _, _ = prep_weights(ctx, wl, [(layer, workloads.seed_for(wl, li, 0)) for li, layer in enumerate(wl.layers)])
    set_bytes = sum(L["P"][0].numel() for L in layers)
    ncopies = max(2, math.ceil(ROTATE_BYTES / set_bytes))
    add_copies(ctx, layers, ncopies)
    jobs = []
    for li, L in enumerate(layers):
        lay = L["layer"]
        x = synth.activations_student_t_bf16(M, lay.K, seed=workloads.seed_for(wl, li, 1) + M)
        xd = torch.from_numpy(x.view(np.int16)).to(ctx.dev).view(torch.bfloat16)
        nws = bl.bitlinear_forward_workspace_bytes(M, lay.N, lay.K, ctx.layout, bl.BF16)
        jobs.append({"M": M, "L": L, "x": xd, "x_dtype": bl.BF16, "nws": nws,
                     "ws": torch.empty(max(nws, 16), dtype=torch.uint8, device=ctx.dev),
                     "y": torch.empty((M, lay.N), dtype=torch.float32, device=ctx.dev)})

    def fwd(j, copy):
        L, lay = j["L"], j["L"]["layer"]
        st = bl.bitlinear_forward(L["P"][copy].data_ptr(), ctx.layout, L["gamma"].data_ptr(), M, lay.N, lay.K,
                                  j["x"].data_ptr(), bl.BF16, j["x"].stride(0), None, j["y"].data_ptr(), bl.F32,
                                  j["y"].stride(0), j["ws"].data_ptr(), j["nws"], ctx.stream.cuda_stream)
        if st:
            raise bl.BitlinearError(st, "bitlinear_forward (prefill)")

    def step(s):
        for j in jobs:
            fwd(j, s % ncopies)

    with torch.cuda.stream(ctx.stream):
        step(0)
        torch.cuda.synchronize()
    graphs = [capture(ctx, lambda s=s: step(s)) for s in range(ncopies)]
    step_ms = time_graphs(ctx, graphs, max(5, args.steps // 5), 2)
    ops = sum(2 * M * j["L"]["layer"].N * j["L"]["layer"].K for j in jobs)
    packed = sum(j["L"]["P"][0].numel() for j in jobs)
    d = {"ms": 0.0, "bytes": 0, "ops": 0, "launches": 0, "calls": []}
    kname = None
    for j in jobs:
        lay = j["L"]["layer"]
        kname = bl.bitlinear_product_kernel(M, lay.N, lay.K, ctx.layout, bl.I8, bl.ALGO_AUTO)
        ms = time_product_only(ctx, j, ctx.layout, ncopies, bl.ALGO_AUTO)
        d["ms"] += ms
        d["ops"] += 2 * M * lay.N * lay.K
        d["bytes"] += product_bytes(bl, j, ctx.layout, False)
        d["launches"] += 1
        d["calls"].append(f"{lay.name}@M{M}:{ms * 1e3:.2f}us")
    roof = roofline("mfma", d)
    roof.update({"traffic": None, "kernel": kname, "avg_launch_us": round(d["ms"] / d["launches"] * 1e3, 3),
                 "launches_per_step": d["launches"], "calls": d["calls"],
                 "algorithmic_ops_per_launch": d["ops"] // d["launches"],
                 "timing": "HIP events on the launch stream around a graph of back-to-back GEMMs over every weight "
                           "copy (activations quantised beforehand)"})
    log(f"prefill: {step_ms:.4f} ms/step, GEMM {json.dumps(roof)}")
    quant = time_prefill_quantiser(ctx, jobs, M)
    log(f"prefill quantiser: {json.dumps(quant)}")
    return {
        "workload": wl.name,
        "metric": "effective ternary TOPS of the prefill step (quantiser + GEMM + rescale per layer)",
        "value": round(ops / (step_ms * 1e-3) / 1e12, 2),
        "unit": "TOPS",
        "ms_per_step": round(step_ms, 5),
        "packed_weight_GB/s": round(packed / (step_ms * 1e-3) / 1e9, 2),
        "config": {"M": M, "layers": {j["L"]["layer"].name: [j["L"]["layer"].N, j["L"]["layer"].K] for j in jobs},
                   "activations": "Student-t(4) bf16", "layout": "i2", "weight_copies": ncopies},
        "roofline": roof,
        "quantiser": quant,
        "cpu_baseline": cpu_baseline(wl, wl.batches, max(args.cpu_seconds / 2, 3.0), ctx.layout, rows=64),
    }


def time_prefill_quantiser(ctx, jobs, M):
    """The per-token activation quantiser of each prefill forward, timed alone
    against HBM: bf16 rows in, int8 rows (K rounded up to 16) and beta out.
    A graph of back-to-back launches rotates over input and output copies of
    >= ROTATE_BYTES in all, so that neither L2 nor the Infinity Cache holds
    them between uses."""
    torch, bl = ctx.torch, ctx.bl
    d = {"ms": 0.0, "bytes": 0, "launches": 0, "calls": []}
    for j in jobs:
        K = j["L"]["layer"].K
        ldq = (K + 15) // 16 * 16
        nbytes = M * K * 2 + M * ldq + 4 * M
        nc = max(2, math.ceil(ROTATE_BYTES / nbytes))
        xs = [j["x"]] + [j["x"].clone() for _ in range(nc - 1)]
        outs = [(torch.empty((M, ldq), dtype=torch.int8, device=ctx.dev),
                 torch.empty(M, dtype=torch.float32, device=ctx.dev)) for _ in range(nc)]

        def q(i, xs=xs, outs=outs, K=K, ldq=ldq):
            x, (xq, beta) = xs[i % len(xs)], outs[i % len(outs)]
            st = bl.bitlinear_quantize_act(x.data_ptr(), bl.BF16, M, K, x.stride(0), xq.data_ptr(), ldq,
                                           beta.data_ptr(), ctx.stream.cuda_stream)
            if st:
                raise bl.BitlinearError(st, "bitlinear_quantize_act (prefill)")

        ms = time_launches(ctx, q, nc)
        d["ms"] += ms
        d["bytes"] += nbytes
        d["launches"] += 1
        d["calls"].append(f"{j['L']['layer'].name}@M{M}:{ms * 1e3:.2f}us")
        del xs, outs
    roof = roofline("hbm", d)
    roof.update({"avg_launch_us": round(d["ms"] / d["launches"] * 1e3, 3), "launches_per_step": d["launches"],
                 "calls": d["calls"], "algorithmic_bytes_per_launch": d["bytes"] // d["launches"],
                 "timing": "HIP events on the launch stream around a graph of back-to-back launches over input "
                           "and output copies of >= 2 GiB"})
    return roof


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
    for f in ("group.hip", "gemv_core.h", "fq_core.h", "gemv.hip", "gemm.hip", "common.h"):
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


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, batches, seconds, layout, rows=None):
    """The CPU oracle, untuned, on a bounded sample of the same work: whole
    layers of the workload (quantise the activations, exact product, rescale)
    -- or, with 'rows', the first 'rows' tokens of each -- cycling through the
    step's (batch, layer) pairs until about 'seconds' of CPU time has passed.
    Reported in the unit of the GPU figure it stands beside (packed-weight
    GB/s for decode, effective TOPS with rows)."""
    import oracle

    from ternary_weight_linear_forward_amd import synth, workloads
    from ternary_weight_linear_forward_amd import bitlinear as bl

    act = synth.activations_student_t_bf16 if wl.act_dist == "student_t" else synth.activations_bf16
    pairs = [(M, li) for M in batches for li in range(len(wl.layers))]
    tern = {}
    done_bytes = 0
    done_ops = 0
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
        m = M if rows is None else min(M, rows)
        x = act(M, layer.K, seed=workloads.seed_for(wl, li, 1) + M)[:m]
        t0 = time.perf_counter()
        oracle.forward(t, g, x)
        t_total += time.perf_counter() - t0
        done_bytes += bl.bitlinear_packed_bytes(layer.N, layer.K, layout)
        done_ops += 2 * m * layer.N * layer.K
        done.append(f"{layer.name}@M{m}")
        i += 1
    sample = (f"{len(done)} BitLinear forwards ({', '.join(done[:8])}{', ...' if len(done) > 8 else ''}) "
              f"in {t_total:.1f} s")
    base = {"cores": oracle.threads_used(), "cpu_model": cpu_model(), "kind": "oracle", "sample": sample}
    if rows is None:
        return {"value": round(done_bytes / t_total / 1e9, 4), "unit": "GB/s", **base}
    return {"value": round(done_ops / t_total / 1e12, 5), "unit": "TOPS", **base,
            "note": f"first {rows} tokens of each forward"}


if __name__ == "__main__":
    main()
