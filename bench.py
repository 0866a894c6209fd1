"""Benchmark of the W4A16 decode path on one MI355X.

A step is one decode weight sweep of a LLaMA-3-8B-shaped model at M = 1:
32 layers x (q 4096x4096, k 4096x1024, v 4096x1024, o 4096x4096,
gate 4096x14336, up 4096x14336, down 14336x4096) (shapes written K x N),
every layer reading its own weights from HBM.  As serving engines store
them, q/k/v and gate/up are concatenated along N (they share their input),
so a layer is 4 launches of w4a16_gemv (qkv 4096x6144, o, gate_up
4096x28672, down): 128 launches per sweep, the same bytes as 224 separate
ones (also reported).  The sweep's launches are captured once in a HIP graph
and replayed.

Prints one JSON line: effective HBM GB/s of the sweep (algorithmic bytes
N*K/2 + N*K/64 + 2K + 2N per GEMV over the measured time), us per sweep,
the roofline of the launch with the largest share of the sweep (gate_up), and
the CPU oracle timed on a sample of the same sweep.

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
    p.add_argument("--layout", default="fused", choices=["fused", "separate"],
                   help="qkv and gate_up concatenated (default) or 7 launches per layer")
    p.add_argument("--launch", default="gemv", choices=["gemv", "chain"],
                   help="one w4a16_gemv launch per matrix, or w4a16_gemv_chain: the "
                        "sweep's matrices as dependent stages, 64 per launch")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="CPU oracle baseline: layers are timed until this many seconds "
                        "have passed (at least one layer, at most --cpu-layers)")
    p.add_argument("--cpu-layers", type=int, default=128,
                   help="layers of the sweep the CPU oracle is timed on")
    p.add_argument("--no-check", action="store_true", help="skip the parity check of layer 0")
    p.add_argument("--no-shapes", action="store_true", help="skip per-shape timing")
    p.add_argument("--no-secondary", action="store_true",
                   help="skip the quantizer, batched-decode and prefill measurements")
    p.add_argument("--secondary-only", default="",
                   help="comma list of secondary rows (%s) to run alone, without the "
                        "sweep (for profiling them); prints their JSON"
                        % ",".join(SECONDARY_ROWS))
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="run one plain device copy of this many MiB first (calibrates "
                        "the FETCH_SIZE / WRITE_SIZE counters against known bytes)")
    return p.parse_args()


def fused_groups(names):
    """Launch groups of a layer: matrices that share an input are stored
    concatenated along N (q/k/v and gate/up)."""
    if names == ["q", "k", "v", "o", "gate", "up", "down"]:
        return [["q", "k", "v"], ["o"], ["gate", "up"], ["down"]]
    return [[n] for n in names]


def sweep_row(torch, w4a16, inputs, dev, workload, case_id):
    """Another model's decode weight sweep (fused layout, graph replays):
    us per sweep, GB/s and the dominant launch, for the secondary rows."""
    shape_attr, layers_attr = WORKLOADS[workload]
    shapes = getattr(inputs, shape_attr)
    nlayers = getattr(inputs, layers_attr)
    names = [n for n, _, _ in shapes]
    dims = {n: (K, N) for n, K, N in shapes}
    layer0 = []
    for group in fused_groups(names):
        K = dims[group[0]][0]
        ps, ss = [], []
        for name in group:
            W = inputs.weight(dims[name][1], K, seed=inputs.matrix_seed(case_id, 0,
                                                                      names.index(name)))
            p, s_ = w4a16.quantize(torch.from_numpy(W).to(dev))
            ps.append(p)
            ss.append(s_)
        layer0.append(("_".join(group), K, torch.cat(ps), torch.cat(ss)))
    layers = [layer0] + [[(g, K, p.clone(), s_.clone()) for (g, K, p, s_) in layer0]
                         for _ in range(nlayers - 1)]
    xs = {K: torch.from_numpy(inputs.activation(1, K, seed=[1000, case_id, K])[0]).to(dev)
          for _, K, _ in shapes}
    ys = {g: torch.empty((p.shape[0],), dtype=torch.float16, device=dev)
          for (g, K, p, _) in layer0}
    seq = [(xs[K], p, s_, ys[g]) for layer in layers for (g, K, p, s_) in layer]
    nbytes = sum(gemv_bytes(p.shape[0], K) for layer in layers for (_, K, p, _) in layer)

    def timed(sub, reps=10):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for x, p, s_, y in sub:
                w4a16.gemv(x, p, s_, y=y)
        for _ in range(3):
            g.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    us = timed(seq)
    per_group = {}
    for (g, K, p, _) in layer0:
        sub = [t for t in seq if t[3] is ys[g]]
        gus = timed(sub) / len(sub)
        per_group[g] = {"K": K, "N": int(p.shape[0]), "us": round(gus, 3),
                        "GB/s": round(gemv_bytes(p.shape[0], K) / (gus * 1e-6) / 1e9, 1)}
    dom = max(per_group, key=lambda g: per_group[g]["us"] * nlayers)
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"workload": workload, "layers": nlayers, "launches_per_sweep": len(seq),
            "bytes_per_sweep": nbytes, "us_per_sweep": round(us, 2), "GB/s": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "per_launch": per_group,
            "dominant_launch": dom,
            "dominant_frac_of_hbm_peak": round(per_group[dom]["GB/s"] / HBM_PEAK_GBS, 4)}


def weight_copies(p0, s0, min_bytes=600 << 20, extra=()):
    """Copies of one quantized matrix (the original first) whose packed
    weights and scales add up to at least min_bytes (more than twice the
    256 MB Infinity Cache), so that every timed launch reads from HBM."""
    one = p0.numel() * 4 + s0.numel() * 2 + sum(t.numel() * t.element_size() for t in extra)
    n = max(2, -(-min_bytes // one))
    return [(p0, s0, *extra)] + [(p0.clone(), s0.clone(), *[t.clone() for t in extra])
                                 for _ in range(n - 1)]


SECONDARY_ROWS = ["quantize", "batched", "prefill", "groups", "act_order", "asym", "q4_0",
                  "sweep"]


def secondary(torch, w4a16, inputs, dev, stream, main_workload="llama3-8b-sweep", rows=None):
    """Other rows of the path on their workload shapes: the quantizer (70B FFN
    matrix, larger than the Infinity Cache), batched decode M = 1..32 on the
    8B FFN shapes with both kernel families (locates the VALU/MFMA
    crossover), 512-token prefill, the decode GEMV and quantizer at group
    sizes 32..256, the decode GEMV with an act-order activation gather, the
    asymmetric-INT4 decode GEMV and quantizer, and the Q4_0 block layout
    against the split layout at group 32.  Each figure is the mean of
    graph replays over enough weight copies to stream from HBM."""
    out = {}

    def want(name):
        return rows is None or name in rows

    # Bring the clocks to their loaded state first: the first rows timed on
    # an idle GPU read up to 15 % slow (prefill, 8192 x 28672: 307 against
    # 262 us).
    a = torch.randn(8192, 8192, device=dev, dtype=torch.float16)
    t_end = time.perf_counter() + 0.5
    while time.perf_counter() < t_end:
        for _ in range(10):
            a @ a
        torch.cuda.synchronize()
    del a

    def timed(seq_fn, reps=5, warm_s=0.1):
        """us per replay of a graph of seq_fn, after replaying it for about
        warm_s seconds: the clocks drop while the host prepares the next
        row's weights, and a row timed right away reads slow."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            seq_fn()
        t0 = time.perf_counter()
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        per = (time.perf_counter() - t0) / 2
        for _ in range(min(500, int(warm_s / max(per, 1e-6)))):
            g.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps     # us per replay

    quantized = {}
    if want("quantize"):
        # quantizer: 28672 x 8192 fp16 (470 MB in, 121 MB out)
        K, N = 8192, 28672
        W = torch.from_numpy(inputs.weight(N, K, seed=[5, 1, 0])).to(dev)
        pq = torch.empty((N, K // 8), dtype=torch.int32, device=dev)
        sq = torch.empty((N, K // 128), dtype=torch.float16, device=dev)
        w4a16.quantize(W, pq, sq)
        us = timed(lambda: w4a16.quantize(W, pq, sq))
        qbytes = N * K * 2 + N * K // 2 + N * (K // 128) * 2
        out["quantize"] = {"K": K, "N": N, "us": round(us, 2),
                           "GB/s": round(qbytes / (us * 1e-6) / 1e9, 1),
                           "frac_of_hbm_peak": round(qbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        del W
        quantized[(K, N)] = (pq, sq)

    def weights_for(K, N):
        if (K, N) not in quantized:
            Wd = torch.from_numpy(inputs.weight(N, K, seed=[5, K, N])).to(dev)
            quantized[(K, N)] = w4a16.quantize(Wd)
            del Wd
        return quantized[(K, N)]

    if want("batched"):
        # batched decode on the 8B FFN shapes
        batched = {}
        for (K, N) in [(4096, 14336), (14336, 4096)]:
            p0, s0 = weights_for(K, N)
            copies = weight_copies(p0, s0)                              # >= 600 MB of weights
            for M in [1, 2, 3, 4, 8, 16, 32]:
                X = torch.from_numpy(inputs.activation(M, K, seed=[6, M, K])).to(dev)
                Y = torch.empty((M, N), dtype=torch.float16, device=dev)
                row = {}
                for algo in ["valu", "mfma"]:
                    us = timed(lambda: [w4a16.gemm(X, p, s_, algo=algo, Y=Y) for p, s_ in copies]) \
                        / len(copies)
                    b = gemv_bytes(N, K, M)
                    row[algo] = {"us": round(us, 3), "GB/s": round(b / (us * 1e-6) / 1e9, 1),
                                 "TFLOP/s": round(2 * M * N * K / (us * 1e-6) / 1e12, 2)}
                row["auto_picks"] = "valu" if M <= w4a16.valu_max_m() else "mfma"
                # K split over blocks through a workspace (w4a16_gemm_ws), where
                # the library splits the shape
                if w4a16.library().w4a16_gemm_workspace_bytes(M, N, K) > 0:
                    ws = w4a16.gemm_workspace(M, N, K, device=dev)
                    us = timed(lambda: [w4a16.gemm_ws(X, p, s_, ws, Y=Y) for p, s_ in copies]) \
                        / len(copies)
                    b = gemv_bytes(N, K, M)
                    row["mfma_split_k"] = {"us": round(us, 3), "GB/s": round(b / (us * 1e-6) / 1e9, 1),
                                           "TFLOP/s": round(2 * M * N * K / (us * 1e-6) / 1e12, 2),
                                           "workspace_bytes": int(ws.numel())}
                batched["%dx%d M=%d" % (K, N, M)] = row
            del copies
        out["batched_decode"] = batched

    if want("prefill"):
        # prefill, M = 512
        prefill = {}
        for (K, N) in [(4096, 14336), (14336, 4096), (8192, 28672)]:
            p0, s0 = weights_for(K, N)
            copies = weight_copies(p0, s0)                              # >= 600 MB of weights
            for M in (512, 256, 128):
                X = torch.from_numpy(inputs.activation(M, K, seed=[7, K])).to(dev)
                Y = torch.empty((M, N), dtype=torch.float16, device=dev)
                # w4a16_gemm_ws: long-K shapes split K over blocks through the
                # workspace (w4a16_gemm does the same eagerly with pool memory;
                # a captured w4a16_gemm keeps the unsplit kernel)
                ws = w4a16.gemm_workspace(M, N, K, device=dev)
                us = timed(lambda: [w4a16.gemm_ws(X, p, s_, ws, Y=Y) for p, s_ in copies]) \
                    / len(copies)
                tf = 2 * M * N * K / (us * 1e-6) / 1e12
                prefill["%dx%d M=%d" % (K, N, M)] = {"us": round(us, 2), "TFLOP/s": round(tf, 1),
                                                     "frac_of_mfma_f16_peak":
                                                         round(tf / MFMA_F16_PEAK_TFLOPS, 4)}
            del copies
        out["prefill"] = prefill

    if want("groups"):
        # group size as a parameter: decode GEMV (M = 1) on the 8B gate shape and
        # the quantizer, per group size (scale bytes N*K*2/group)
        groups = {}
        K, N = 4096, 14336
        Wg = torch.from_numpy(inputs.weight(N, K, seed=[8, K, N])).to(dev)
        x = torch.from_numpy(inputs.activation(1, K, seed=[8, 1])).to(dev)[0]
        y = torch.empty((N,), dtype=torch.float16, device=dev)
        for group in (32, 64, 128, 256, w4a16.PER_CHANNEL):
            pg, sg = w4a16.quantize(Wg, group=group)
            qus = timed(lambda: w4a16.quantize(Wg, pg, sg, group=group))
            copies = weight_copies(pg, sg)
            us = timed(lambda: [w4a16.gemv(x, p, s_, y=y) for p, s_ in copies]) / len(copies)
            ng = w4a16.scales_per_row(K, group)
            b = N * K // 2 + N * ng * 2 + 2 * K + 2 * N
            qb = N * K * 2 + N * K // 2 + N * ng * 2
            label = "per channel" if group == w4a16.PER_CHANNEL else "group %d" % group
            groups[label] = {
                "gemv_us": round(us, 3), "gemv_GB/s": round(b / (us * 1e-6) / 1e9, 1),
                "gemv_frac_of_hbm_peak": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "quantize_us": round(qus, 2), "quantize_GB/s": round(qb / (qus * 1e-6) / 1e9, 1)}
            # batched decode and prefill at this group (the automatic choice:
            # matrix cores above two rows)
            for M in (16, 512):
                X = torch.from_numpy(inputs.activation(M, K, seed=[8, M])).to(dev)
                Y = torch.empty((M, N), dtype=torch.float16, device=dev)
                mus = timed(lambda: [w4a16.gemm(X, p, s_, Y=Y) for p, s_ in copies]) / len(copies)
                groups[label]["M=%d_us" % M] = round(mus, 2)
                groups[label]["M=%d_TFLOP/s" % M] = round(2 * M * N * K / (mus * 1e-6) / 1e12, 1)
            del copies
        out["group_sizes_%dx%d" % (K, N)] = groups
        del Wg

    if want("act_order"):
        # act order: M = 1 GEMV with the activation gather, against the plain GEMV
        act = {}
        for (K, N) in [(4096, 14336), (14336, 4096)]:
            p0, s0 = weights_for(K, N)
            copies = weight_copies(p0, s0)
            x = torch.from_numpy(inputs.activation(1, K, seed=[9, K])).to(dev)[0]
            y = torch.empty((N,), dtype=torch.float16, device=dev)
            perm = torch.randperm(K, generator=torch.Generator().manual_seed(K)).to(
                device=dev, dtype=torch.int32)
            plain = timed(lambda: [w4a16.gemv(x, p, s_, y=y) for p, s_ in copies]) / len(copies)
            gather = timed(lambda: [w4a16.gemv(x, p, s_, y=y, perm=perm) for p, s_ in copies]) \
                / len(copies)
            b = gemv_bytes(N, K) + 4 * K
            act["%dx%d" % (K, N)] = {"plain_us": round(plain, 3), "perm_us": round(gather, 3),
                                     "perm_GB/s": round(b / (gather * 1e-6) / 1e9, 1)}
            # batched decode and prefill: X gathered in the order perm into a
            # workspace, then the matrix-core GEMM (w4a16_linear; graph-captured)
            for M in (16, 512):
                X = torch.from_numpy(inputs.activation(M, K, seed=[9, M, K])).to(dev)
                Y = torch.empty((M, N), dtype=torch.float16, device=dev)
                ws = w4a16.linear_workspace(M, K, device=dev)
                pus = timed(lambda: [w4a16.linear(X, p, s_, perm=perm, Y=Y, workspace=ws)
                                     for p, s_ in copies]) / len(copies)
                qus = timed(lambda: [w4a16.gemm(X, p, s_, Y=Y) for p, s_ in copies]) / len(copies)
                act["%dx%d" % (K, N)]["M=%d_perm_us" % M] = round(pus, 2)
                act["%dx%d" % (K, N)]["M=%d_plain_us" % M] = round(qus, 2)
            del copies
        out["act_order"] = act

    if want("asym"):
        # asymmetric INT4: M = 1 GEMV (zero points streamed beside the scales)
        # and the quantizer, against the symmetric GEMV on the same shape
        asym = {}
        for (K, N) in [(14336, 4096), (4096, 14336)]:
            Wd = torch.from_numpy(inputs.weight_skewed(N, K, seed=[10, K, N])).to(dev)
            pa, sa, za = w4a16.quantize_asym(Wd)
            qus = timed(lambda: w4a16.quantize_asym(Wd, pa, sa, za))
            copies = weight_copies(pa, sa, extra=(za,))
            x = torch.from_numpy(inputs.activation(1, K, seed=[10, K])).to(dev)[0]
            y = torch.empty((N,), dtype=torch.float16, device=dev)
            us = timed(lambda: [w4a16.gemv_asym(x, p, s_, z, y=y) for p, s_, z in copies]) \
                / len(copies)
            p0, s0 = weights_for(K, N)
            sym = weight_copies(p0, s0)
            plain = timed(lambda: [w4a16.gemv(x, p, s_, y=y) for p, s_ in sym]) / len(sym)
            b = gemv_bytes(N, K) + N * (K // 128) * 2
            qb = N * K * 2 + N * K // 2 + 2 * N * (K // 128) * 2
            row = {
                "gemv_us": round(us, 3), "gemv_GB/s": round(b / (us * 1e-6) / 1e9, 1),
                "gemv_frac_of_hbm_peak": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "symmetric_gemv_us": round(plain, 3),
                "quantize_us": round(qus, 2), "quantize_GB/s": round(qb / (qus * 1e-6) / 1e9, 1)}
            # batched decode and prefill with asymmetric weights (matrix cores)
            for M in (16, 512):
                X = torch.from_numpy(inputs.activation(M, K, seed=[10, M, K])).to(dev)
                Y = torch.empty((M, N), dtype=torch.float16, device=dev)
                few = copies
                a_us = timed(lambda: [w4a16.gemm_asym(X, p, s_, z, Y=Y) for p, s_, z in few]) \
                    / len(few)
                fews = sym
                s_us = timed(lambda: [w4a16.gemm(X, p, s_, Y=Y) for p, s_ in fews]) / len(fews)
                row["M=%d_us" % M] = round(a_us, 2)
                row["M=%d_symmetric_us" % M] = round(s_us, 2)
                row["M=%d_TFLOP/s" % M] = round(2 * M * N * K / (a_us * 1e-6) / 1e12, 1)
            # a 128-token prompt, with K split over blocks where the library
            # splits the shape (w4a16_gemm_asym_ws; it runs as gemm_asym elsewhere)
            M = 128
            X = torch.from_numpy(inputs.activation(M, K, seed=[10, M, K])).to(dev)
            Y = torch.empty((M, N), dtype=torch.float16, device=dev)
            ws = w4a16.gemm_asym_workspace(M, N, K, device=dev)
            few = copies
            w_us = timed(lambda: [w4a16.gemm_asym_ws(X, p, s_, z, ws, Y=Y) for p, s_, z in few]) \
                / len(few)
            row["M=128_ws_us"] = round(w_us, 2)
            row["M=128_ws_split"] = ws.numel() > 1
            row["M=128_ws_TFLOP/s"] = round(2 * M * N * K / (w_us * 1e-6) / 1e12, 1)
            asym["%dx%d" % (K, N)] = row
            del copies, sym, Wd
        out["asymmetric"] = asym

    if want("q4_0"):
        # Q4_0 blocks (scale in front of each 32-element block) against the split
        # layout at the same information content (group 32): M = 1 GEMV and the
        # quantizer
        q40 = {}
        for (K, N) in [(4096, 14336), (14336, 4096)]:
            Wd = torch.from_numpy(inputs.weight(N, K, seed=[11, K, N])).to(dev)
            bq = w4a16.quantize_q4_0(Wd)
            qus = timed(lambda: w4a16.quantize_q4_0(Wd, bq))
            copies = [bq]
            for _ in range(max(1, -(-(600 << 20) // bq.numel()) - 1)):
                c = w4a16.q4_0_blocks(N, K, device=dev)
                c.copy_(bq)
                copies.append(c)
            x = torch.from_numpy(inputs.activation(1, K, seed=[11, K])).to(dev)[0]
            y = torch.empty((N,), dtype=torch.float16, device=dev)
            us = timed(lambda: [w4a16.gemv_q4_0(x, b_, y=y) for b_ in copies]) / len(copies)
            pg, sg = w4a16.quantize(Wd, group=32)
            split = weight_copies(pg, sg)
            sus = timed(lambda: [w4a16.gemv(x, p, s_, y=y) for p, s_ in split]) / len(split)
            b = N * (K // 32) * 18 + 2 * K + 2 * N
            qb = N * K * 2 + N * (K // 32) * 18
            q40["%dx%d" % (K, N)] = {
                "gemv_us": round(us, 3), "gemv_GB/s": round(b / (us * 1e-6) / 1e9, 1),
                "gemv_frac_of_hbm_peak": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "split_group32_gemv_us": round(sus, 3),
                "quantize_us": round(qus, 2), "quantize_GB/s": round(qb / (qus * 1e-6) / 1e9, 1)}
            del copies, split, Wd
        out["q4_0_m1"] = q40
        quantized.clear()

    if want("sweep"):
        # the other model's decode weight sweep (Qwen-2.5-7B beside LLaMA-3-8B)
        other = "qwen2.5-7b-sweep" if main_workload == "llama3-8b-sweep" else "llama3-8b-sweep"
        out["sweep_" + other] = sweep_row(torch, w4a16, inputs, dev, other,
                                          3 if other.startswith("qwen") else 2)
    return out


PMC_TRAFFIC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                           "gemv_pmc_traffic.json")
GEMV_SOURCES = [os.path.join("weight_only_int4_gemv_amd", "csrc", f)
                for f in ("gemv.hip", "w4a16_device.h")]


def gemv_sources_sha256() -> str:
    """Hash of the GEMV kernel sources the stored counter figures were taken on."""
    import hashlib
    h = hashlib.sha256()
    root = os.path.dirname(os.path.abspath(__file__))
    for rel in GEMV_SOURCES:
        with open(os.path.join(root, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_traffic(shape: str):
    """HBM bytes per launch of `shape` from the committed rocprofv3 counter runs
    (FETCH_SIZE scaled by the copy-kernel calibration, plus WRITE_SIZE), or
    None when the kernel sources changed since they were taken."""
    try:
        with open(PMC_TRAFFIC) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("sources_sha256") != gemv_sources_sha256():
        return None
    ent = rec.get("per_launch", {}).get(shape)
    return None if ent is None else int(ent["traffic_bytes"])


def host_cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), for the CPU baseline."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def dominant_roofline(per_shape, layer0, step_bytes, n_launch, avg_launch_us):
    """Roofline of the launch with the largest share of the sweep's time,
    timed live (HIP events around graph replays of that launch on the
    bench stream); without per-shape timings, the sweep's average launch."""
    if per_shape:
        groups = [g for (g, _, _, _, _, _) in layer0]
        name = max(groups, key=lambda g: per_shape[g]["us"])
        K, N, us = per_shape[name]["K"], per_shape[name]["N"], per_shape[name]["us"]
        nbytes = gemv_bytes(N, K)
        achieved = nbytes / (us * 1e-6) / 1e9
        shape = "%dx%d" % (K, N)
        return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": stored_traffic(shape),
                "kernel": "w4a16::gemv_persistent_kernel (w4a16_gemv), %s launch K=%d N=%d"
                          % (name, K, N),
                "bytes_per_launch": nbytes, "avg_launch_us": us}
    achieved = step_bytes / n_launch / (avg_launch_us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
            "kernel": "w4a16_gemv launches of the sweep (average)",
            "bytes_per_launch": step_bytes // n_launch, "avg_launch_us": round(avg_launch_us, 3)}


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

    if args.copy_probe_mib > 0:
        src = torch.ones(args.copy_probe_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print("[copy-probe] one copy of %d bytes (read) + %d bytes (write)"
              % (src.numel() * 4, dst.numel() * 4), file=sys.stderr, flush=True)
        del src, dst

    if args.secondary_only:
        rows = [r for r in args.secondary_only.split(",") if r]
        unknown = sorted(set(rows) - set(SECONDARY_ROWS))
        if unknown:
            print("unknown secondary rows: %s (choose from %s)" % (unknown, SECONDARY_ROWS),
                  file=sys.stderr)
            return 2
        sec = secondary(torch, w4a16, inputs, dev, torch.cuda.current_stream(), args.workload,
                        rows=rows)
        print(json.dumps({"secondary_only": rows, "secondary": sec}), flush=True)
        return 0

    shape_attr, layers_attr = WORKLOADS[args.workload]
    shapes = getattr(inputs, shape_attr)
    nlayers = getattr(inputs, layers_attr)

    # ---- weights: layer 0 drawn on the host, quantized on the GPU; layers
    # 1.. are device copies (each launch reads its own HBM; GEMV time does
    # not depend on the values).  Matrices sharing an input are stored
    # concatenated along N.
    t0 = time.time()
    names = [n for n, _, _ in shapes]
    dims = {n: (K, N) for n, K, N in shapes}
    fuse = fused_groups(names)
    host_w = {}
    layer0 = []   # (group name, K, N, packed, scales, [(member, row0, rows)])
    for gi, group in enumerate(fuse):
        K = dims[group[0]][0]
        parts_p, parts_s, members, row0 = [], [], [], 0
        for name in group:
            mid = names.index(name)
            N = dims[name][1]
            W = inputs.weight(N, K, seed=inputs.matrix_seed(2, 0, mid))
            host_w[name] = W
            p, s_ = w4a16.quantize(torch.from_numpy(W).to(dev))
            parts_p.append(p)
            parts_s.append(s_)
            members.append((name, row0, N))
            row0 += N
        layer0.append(("_".join(group), K, row0, torch.cat(parts_p), torch.cat(parts_s), members))
        del parts_p, parts_s
    torch.cuda.synchronize()
    weights = [layer0] + [[(g, K, N, p.clone(), s_.clone(), mem) for (g, K, N, p, s_, mem) in layer0]
                          for _ in range(nlayers - 1)]
    torch.cuda.synchronize()
    xs = {K: torch.from_numpy(inputs.activation(1, K, seed=[1000, 2, K])[0]).to(dev)
          for _, K, _ in shapes}
    ys = {g: torch.empty((N,), dtype=torch.float16, device=dev) for (g, K, N, _, _, _) in layer0}
    setup_s = time.time() - t0

    fused_launches = [(xs[K], p, s_, ys[g]) for layer in weights for (g, K, N, p, s_, _) in layer]
    separate_launches = [(xs[K], p[r0:r0 + n], s_[r0:r0 + n], ys[g][r0:r0 + n])
                         for layer in weights for (g, K, N, p, s_, mem) in layer
                         for (_, r0, n) in mem]
    launches = fused_launches if args.layout == "fused" else separate_launches
    step_bytes = sum(gemv_bytes(N, K) for layer in weights for (_, K, N, _, _, _) in layer) \
        if args.layout == "fused" else \
        sum(gemv_bytes(n, K) for layer in weights for (_, K, _, _, _, mem) in layer
            for (_, _, n) in mem)
    weight_bytes = sum(p.numel() * 4 + s_.numel() * 2 for layer in weights
                       for (_, _, _, p, s_, _) in layer)

    def make_step(seq):
        def step():
            for x, p, s_, y in seq:
                w4a16.gemv(x, p, s_, y=y)
        return step

    sync = w4a16.chain_sync_buffer(dev)

    def make_chain_step(seq):
        parts = [seq[i:i + w4a16.CHAIN_MAX] for i in range(0, len(seq), w4a16.CHAIN_MAX)]

        def step():
            for part in parts:
                w4a16.gemv_chain(part, sync)
        return step

    step = make_step(launches) if args.launch == "gemv" else make_chain_step(launches)
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
        for (g, K, N, p, s_, mem) in layer0:
            po = np.concatenate([orc.quantize(host_w[name])[0] for name, _, _ in mem])
            so = np.concatenate([orc.quantize(host_w[name])[1] for name, _, _ in mem])
            assert np.array_equal(p.cpu().numpy().view(np.uint32), po), g
            assert np.array_equal(s_.cpu().numpy().view(np.uint16), so), g
            x = xs[K].cpu().numpy()[None]
            yref, yabs = orc.matmul(x, po, so)
            y = ys[g].cpu().numpy().astype(np.float64)[None]
            tol = oracle.tolerance(yref, yabs)
            ratio = float((np.abs(y - yref) / tol).max())
            assert ratio <= 1.0, "%s out of tolerance (%.3f)" % (g, ratio)
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

    # ---- spread: 20 single-step samples after the timed region (each step
    # bracketed by its own events)
    samples = []
    for _ in range(20):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        run()
        b.record(stream)
        samples.append((a, b))
    torch.cuda.synchronize()
    sample_us = np.sort(np.array([a.elapsed_time(b) * 1e3 for a, b in samples]))
    step_spread = {"n": len(sample_us), "p10_us": round(float(np.percentile(sample_us, 10)), 2),
                   "p50_us": round(float(np.percentile(sample_us, 50)), 2),
                   "p90_us": round(float(np.percentile(sample_us, 90)), 2)}

    # ---- the same sweep launched the other way (eager launches from the
    # host against graph replays), outside the timed region
    if args.mode == "graph":
        other_run, other_name = step, "eager"
    else:
        og = torch.cuda.CUDAGraph()
        with torch.cuda.graph(og):
            step()
        other_run, other_name = og.replay, "graph"
    for _ in range(3):
        other_run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(10):
        other_run()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / 10
    other_mode = {"mode": other_name, "us_per_sweep": round(us, 2),
                  "GB/s": round(step_bytes / (us * 1e-6) / 1e9, 1)}

    # ---- the other layout, and per-shape launch durations (graph of every
    # layer's copy of one matrix)
    def time_graph(seq, reps=10):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            make_step(seq)()
        for _ in range(3):
            g.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps      # us per replay

    other = None
    per_shape = None
    other_launch = None
    if not args.no_shapes:
        g2 = torch.cuda.CUDAGraph()
        alt = make_chain_step(launches) if args.launch == "gemv" else make_step(launches)
        alt()
        torch.cuda.synchronize()
        with torch.cuda.graph(g2):
            alt()
        for _ in range(3):
            g2.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            g2.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / 10
        other_launch = {"launch": "chain" if args.launch == "gemv" else "gemv",
                        "us_per_sweep": round(us, 2),
                        "GB/s": round(step_bytes / (us * 1e-6) / 1e9, 1),
                        "sync_words_nonzero": int((sync != 0).sum().item())}
        del g2
        other_seq = separate_launches if args.layout == "fused" else fused_launches
        other_bytes = sum(gemv_bytes(int(p.shape[0]), int(p.shape[1]) * 8) for _, p, _, _ in other_seq)
        us = time_graph(other_seq)
        other = {"layout": "separate" if args.layout == "fused" else "fused",
                 "launches_per_step": len(other_seq), "us_per_sweep": round(us, 2),
                 "GB/s": round(other_bytes / (us * 1e-6) / 1e9, 1)}
        per_shape = {}
        for gi, (g, K, N, _, _, mem) in enumerate(layer0):
            seqs = {g: [(xs[K], layer[gi][3], layer[gi][4], ys[g]) for layer in weights]}
            if len(mem) > 1:
                for (name, r0, n) in mem:
                    seqs[name] = [(xs[K], layer[gi][3][r0:r0 + n], layer[gi][4][r0:r0 + n],
                                   ys[g][r0:r0 + n]) for layer in weights]
            for name, seq in seqs.items():
                n_rows = int(seq[0][1].shape[0])
                us = time_graph(seq) / len(seq)
                per_shape[name] = {"K": K, "N": n_rows, "us": round(us, 3),
                                   "GB/s": round(gemv_bytes(n_rows, K) / (us * 1e-6) / 1e9, 1)}

    # ---- CPU oracle on a bounded sample of the same sweep
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        orc = oracle.get()
        host = []
        for name, K, N in shapes:
            po, so = orc.quantize(host_w[name])
            host.append((K, N, po, so, xs[K].cpu().numpy()[None]))
        # same bytes as one layer of the sweep in either layout; whole layers
        # until --cpu-seconds have passed
        c0 = time.perf_counter()
        cbytes = 0
        nl = 0
        while nl < max(1, args.cpu_layers) and (nl == 0 or
                                                 time.perf_counter() - c0 < args.cpu_seconds):
            for K, N, po, so, x in host:
                orc.matmul(x, po, so)
                cbytes += gemv_bytes(N, K)
            nl += 1
        csec = time.perf_counter() - c0
        cpu = {"value": round(cbytes / csec / 1e9, 3), "unit": "GB/s", "cores": orc.num_threads(),
               "cpu_model": host_cpu_model(), "kind": "oracle",
               "sample": "%d layers of the sweep's shapes (%d GEMVs; the sweep has %d layers), "
                         "fp64 oracle, %.1f s; us per full sweep extrapolated: %.0f"
                         % (nl, nl * len(shapes), nlayers, csec, csec / nl * nlayers * 1e6)}

    sec = None
    if not args.no_secondary:
        sec = secondary(torch, w4a16, inputs, dev, stream, args.workload)

    roofline = dominant_roofline(per_shape, layer0, step_bytes, n_launch, avg_launch_us)

    # ---- the box's streaming bandwidth as a second denominator: a 1 GiB
    # device copy (1 GiB read + 1 GiB written), best of 5
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    best = None
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        dst.copy_(src)
        b.record(stream)
        torch.cuda.synchronize()
        t = a.elapsed_time(b) * 1e-3
        best = t if best is None else min(best, t)
    copy_gbs = 2 * src.numel() * 4 / best / 1e9
    del src, dst
    stream_copy = {"bytes": 2 << 30, "GB/s": round(copy_gbs, 1),
                   "dominant_launch_frac_of_it": (round(roofline["achieved"] / copy_gbs, 4)
                                                  if roofline else None)}

    # ---- the GPU's floor per dependent launch on one stream: as many
    # launches of a one-element kernel as the sweep has, captured in a graph
    # (the gap from one kernel's end to the next one's start is part of every
    # launch of the sweep, whatever the kernel)
    tiny = torch.zeros(1, dtype=torch.float32, device=dev)
    fg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(fg):
        for _ in range(n_launch):
            tiny.add_(1.0)
    for _ in range(3):
        fg.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(10):
        fg.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    floor_us = e0.elapsed_time(e1) * 1e3 / 10
    del fg, tiny
    sweep_us = ms * 1e3
    # (under a profiler every dispatch is slowed alike and the floor can
    # reach the sweep's own time: no rate above it is given then)
    above = sweep_us - floor_us
    launch_floor = {"kernel": "one-element add, graph of %d dependent launches" % n_launch,
                    "us_per_launch": round(floor_us / n_launch, 3),
                    "us_per_sweep": round(floor_us, 2),
                    "sweep_us_above_floor": round(above, 2),
                    "GB/s_above_floor": (round(step_bytes / (above * 1e-6) / 1e9, 1)
                                         if above > 0.5 * sweep_us else None)}

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
        "config": {"workload": "%s decode weight sweep, M=1, %d layers x %d matrices (%s)"
                               % (args.workload.split("-sweep")[0], nlayers, len(shapes),
                                  ", ".join("%s %dx%d" % s for s in shapes)),
                   "M": 1, "layout": args.layout,
                   "launch_groups": ["+".join(x[-1][i][0] for i in range(len(x[-1])))
                                     for x in layer0],
                   "launch": args.launch,
                   "launches_per_step": n_launch if args.launch == "gemv" else
                   (n_launch + w4a16.CHAIN_MAX - 1) // w4a16.CHAIN_MAX,
                   "gemvs_per_step": n_launch, "bytes_per_step": step_bytes,
                   "weight_bytes_resident": weight_bytes, "mode": args.mode,
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "other_layout": other,
        "other_launch": other_launch,
        "other_mode": other_mode,
        "step_samples": step_spread,
        "stream_copy": stream_copy,
        "launch_floor": launch_floor,
        "per_shape": per_shape,
        "parity": parity,
        "secondary": sec,
        "wall_s_timed": round(wall, 4),
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
