"""Benchmark of the W4A16 decode path on one MI355X.

A step is one decode weight sweep of a LLaMA-3-8B-shaped model at M = 1:
32 layers x (q 4096x4096, k 4096x1024, v 4096x1024, o 4096x4096,
gate 4096x14336, up 4096x14336, down 14336x4096) = 224 launches of
w4a16_gemv (shapes written K x N), every layer reading its own weights from
HBM.  The sweep's launches are captured once in a HIP graph and replayed.

Prints one JSON line: effective HBM GB/s of the sweep (algorithmic bytes
N*K/2 + N*K/64 + 2K + 2N per GEMV over the measured time), us per sweep,
the roofline of the GEMV kernel, and the CPU oracle timed on a sample of the
same sweep.

    python bench.py [--steps 20] [--warmup 5] [--workload llama3-8b-sweep]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, 8 TB/s
MFMA_F16_PEAK_TFLOPS = 2516.6   # MI355X dense fp16 MFMA

WORKLOADS = {
    # name: (layer shapes as (name, K, N), layers)
    "llama3-8b-sweep": ("LLAMA3_8B", "LLAMA3_8B_LAYERS"),
    "qwen2.5-7b-sweep": ("QWEN25_7B", "QWEN25_7B_LAYERS"),
}


def gemv_bytes(N: int, K: int, M: int = 1) -> int:
    """Algorithmic bytes of one launch: codes + scales + activations + outputs."""
    return N * K // 2 + N * (K // 128) * 2 + 2 * M * K + 2 * M * N


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="llama3-8b-sweep", choices=sorted(WORKLOADS))
    p.add_argument("--mode", default="graph", choices=["graph", "eager"],
                   help="replay a captured HIP graph (default) or launch from Python")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-layers", type=int, default=16,
                   help="layers of the sweep the CPU oracle is timed on")
    p.add_argument("--no-check", action="store_true", help="skip the parity check of layer 0")
    p.add_argument("--no-shapes", action="store_true", help="skip per-shape timing")
    return p.parse_args()


def main() -> int:
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU: the W4A16 layer is built and measured on a "
              "single MI355X (no sharding or collectives); use --gpus 1", file=sys.stderr)
        return 2

    import torch
    from weight_only_int4_gemv_amd import inputs, w4a16

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    w4a16.library()  # the built HIP library; an error if absent
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    shape_attr, layers_attr = WORKLOADS[args.workload]
    shapes = getattr(inputs, shape_attr)
    nlayers = getattr(inputs, layers_attr)

    # ---- weights: layer 0 drawn on the host, quantized on the GPU; layers
    # 1.. are device copies (each launch reads its own HBM; GEMV time does
    # not depend on the values).
    t0 = time.time()
    host_w = {}
    layer0 = []
    for mid, (name, K, N) in enumerate(shapes):
        W = inputs.weight(N, K, seed=inputs.matrix_seed(2, 0, mid))
        host_w[name] = W
        packed, scales = w4a16.quantize(torch.from_numpy(W).to(dev))
        layer0.append((name, K, N, packed, scales))
    torch.cuda.synchronize()
    weights = [layer0] + [[(n, K, N, p.clone(), s.clone()) for (n, K, N, p, s) in layer0]
                          for _ in range(nlayers - 1)]
    torch.cuda.synchronize()
    xs = {K: torch.from_numpy(inputs.activation(1, K, seed=[1000, 2, K])[0]).to(dev)
          for _, K, _ in shapes}
    ys = {name: torch.empty((N,), dtype=torch.float16, device=dev) for name, _, N in shapes}
    setup_s = time.time() - t0

    launches = [(xs[K], p, s, ys[n]) for layer in weights for (n, K, N, p, s) in layer]
    step_bytes = sum(gemv_bytes(N, K) for layer in weights for (_, K, N, _, _) in layer)
    weight_bytes = sum(p.numel() * 4 + s.numel() * 2 for layer in weights
                       for (_, _, _, p, s) in layer)

    def step():
        for x, p, s, y in launches:
            w4a16.gemv(x, p, s, y=y)

    stream = torch.cuda.current_stream()
    step()  # first call: device checks outside any capture
    torch.cuda.synchronize()
    run = step
    if args.mode == "graph":
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        run = graph.replay

    # ---- parity of layer 0 at the benchmark's launch configuration
    parity = None
    if not args.no_check:
        import oracle
        orc = oracle.get()
        run()
        torch.cuda.synchronize()
        worst = 0.0
        for (name, K, N, p, s) in layer0:
            po, so = orc.quantize(host_w[name])
            assert np.array_equal(p.cpu().numpy().view(np.uint32), po), name
            assert np.array_equal(s.cpu().numpy().view(np.uint16), so), name
            x = xs[K].cpu().numpy()[None]
            yref, yabs = orc.matmul(x, po, so)
            y = ys[name].cpu().numpy().astype(np.float64)[None]
            tol = oracle.tolerance(yref, yabs)
            ratio = float((np.abs(y - yref) / tol).max())
            assert ratio <= 1.0, "%s out of tolerance (%.3f)" % (name, ratio)
            worst = max(worst, ratio)
        parity = {"layer0": "ok", "max_err_over_tol": round(worst, 4)}

    # ---- timed region
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        run()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = start.elapsed_time(end) / args.steps
    gbs = step_bytes / (ms * 1e-3) / 1e9
    n_launch = len(launches)
    avg_launch_us = ms * 1e3 / n_launch

    # ---- per-shape launch durations (graph of every layer's copy of one matrix)
    per_shape = None
    if not args.no_shapes:
        per_shape = {}
        for mid, (name, K, N) in enumerate(shapes):
            seq = [(xs[K], layer[mid][3], layer[mid][4], ys[name]) for layer in weights]
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for x, p, s, y in seq:
                    w4a16.gemv(x, p, s, y=y)
            for _ in range(3):
                g.replay()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 10
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / (reps * len(seq))
            per_shape[name] = {"K": K, "N": N, "us": round(us, 3),
                               "GB/s": round(gemv_bytes(N, K) / (us * 1e-6) / 1e9, 1)}

    # ---- CPU oracle on a bounded sample of the same sweep
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        orc = oracle.get()
        host = []
        for name, K, N in shapes:
            po, so = orc.quantize(host_w[name])
            host.append((K, N, po, so, xs[K].cpu().numpy()[None]))
        nl = max(1, min(args.cpu_layers, nlayers))
        c0 = time.perf_counter()
        cbytes = 0
        for _ in range(nl):
            for K, N, po, so, x in host:
                orc.matmul(x, po, so)
                cbytes += gemv_bytes(N, K)
        csec = time.perf_counter() - c0
        cpu = {"value": round(cbytes / csec / 1e9, 3), "unit": "GB/s", "cores": orc.num_threads(),
               "kind": "oracle",
               "sample": "%d of %d layers (%d GEMVs, same shapes), fp64 oracle, %.1f s; "
                         "us per full sweep extrapolated: %.0f"
                         % (nl, nlayers, nl * len(shapes), csec, csec / nl * nlayers * 1e6)}

    out = {
        "metric": "W4A16 GEMV effective HBM GB/s (% of peak) + us per 8B-shaped decode weight sweep",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "us_per_sweep": round(ms * 1e3, 2),
        "sweeps_per_s": round(1e3 / ms, 1),
        "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic: N(0,0.02) weights with 0.1% N(0,0.5) outliers, N(0,1) activations; "
                "layer 0 drawn and quantized, layers 1.. device copies",
        "config": {"workload": "%s decode weight sweep, M=1, %d layers x %d GEMVs (%s)"
                               % (args.workload.split("-sweep")[0], nlayers, len(shapes),
                                  ", ".join("%s %dx%d" % s for s in shapes)),
                   "M": 1, "launches_per_step": n_launch, "bytes_per_step": step_bytes,
                   "weight_bytes_resident": weight_bytes, "mode": args.mode,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(step_bytes / n_launch / (avg_launch_us * 1e-6)
                                                      / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(step_bytes / n_launch / (avg_launch_us * 1e-6) / 1e9
                                   / HBM_PEAK_GBS, 4),
                     "traffic": None,
                     "kernel": "gemv_kernel (w4a16_gemv)",
                     "avg_launch_us": round(avg_launch_us, 3),
                     "bytes_per_launch_avg": step_bytes // n_launch},
        "cpu_baseline": cpu,
        "per_shape": per_shape,
        "parity": parity,
        "wall_s_timed": round(wall, 4),
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
