#!/usr/bin/env python3
"""Benchmark of the speculative verification step on one MI355X.

Workload (8B-class layer shapes at T = K+1 = 5): one step streams one decoder
layer's MX-FP4 weights through mxfp4_verify_gemm — q and o 4096x4096, k and v
1024x4096, gate and up 14336x4096, down 4096x14336 (218,103,808 weights,
115,867,648 bytes of codes + scales) — each against its own bf16 activations
[5, K], then runs spec_accept on one sequence (K = 4 drafts, vocab 128256,
fp32 logits N(0, 3), target = draft + N(0, 1)).

Cold weights: the layers of a pool larger than the 256 MB Infinity Cache
(default 1.5 GB, 13 layers) are visited in turn, so every step reads its
weights from HBM. Inputs are resident in HBM before the timed region. Weights
are N(0, 0.02) fp32 drawn on the GPU and quantized by mxfp4_quantize (not
timed). The logits and uniforms come from the shared seeded generator.

Each step is captured once per pool layer as a HIP graph and the timed region
replays K graphs back to back. Prints one JSON line. `value` is verify-GEMM
algorithmic bytes per step (codes + scales + X + Y) times steps, over the
wall time of all steps (spec_accept and the gaps between kernels included).
`roofline` is the verify-GEMM kernel alone, from HIP events around each launch
in a separate eager pass on the launch stream.
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
T = 5
KD = 4
V = 128256
# (name, n, k) of one 8B-class decoder layer
LAYER = [("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
         ("gate", 14336, 4096), ("up", 14336, 4096), ("down", 4096, 14336)]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "verify_gemm_8b_layer_t5_traffic.json")
GEMM_SRC = os.path.join(ROOT, "mx_fp4_weight_amd", "csrc", "gemm.hip")


def mx_bytes(n, k):
    return n * k // 2 + n * k // 32


def gemm_alg_bytes(n, k, m):
    """Algorithmic bytes of one verify GEMM: codes + scales + X (bf16) + Y (fp32)."""
    return mx_bytes(n, k) + m * k * 2 + m * n * 4


def source_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic():
    """HBM bytes per launch from committed rocprofv3 counters, if taken on the current kernel."""
    try:
        with open(TRAFFIC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("gemm_source_sha") != source_sha(GEMM_SRC):
        return None
    return d.get("traffic_bytes_per_launch")


def cpu_baseline(seconds_budget=15.0):
    """The oracle (fp64 NumPy) on the host cores, on a bounded sample of the same workload.

    Sample: rows [0, 512) of each of the 7 layer matrices (oracle-quantized from
    the shared generator), verify GEMM at T = 5, repeated; plus the oracle
    acceptance loop on sequences of the same spec_accept configuration.
    """
    import numpy as np
    import synth
    from oracle import accept as oacc
    from oracle import gemm as ogemm
    from oracle import mx as omx
    try:
        import threadpoolctl
    except ImportError:
        threadpoolctl = None

    rows = 512
    mats = []
    for i, (name, n, k) in enumerate(LAYER):
        w = synth.weights(2, 1000 + i, n, k, row_start=0, row_stop=rows)
        c, s, _ = omx.quantize(w)
        x = synth.activations(2, 1000 + i, T, k)
        mats.append((c, s, rows, k, x))
    ogemm.verify_gemm(*mats[0])  # warm BLAS
    byts = sum(gemm_alg_bytes(rows, k, T) for (_, _, _, k, _) in mats)
    t0 = time.perf_counter()
    reps = 0
    while True:
        for m in mats:
            ogemm.verify_gemm(*m)
        reps += 1
        if time.perf_counter() - t0 > seconds_budget * 0.6:
            break
    t_gemm = time.perf_counter() - t0
    tgt, dft, tok, u = synth.accept_batch(2, 4, KD, V, 3.0, 1.0, seq0=500)
    t0 = time.perf_counter()
    seqs = 0
    while True:
        for b in range(4):
            oacc.step(tgt[b], dft[b], tok[b], u[b])
        seqs += 4
        if time.perf_counter() - t0 > seconds_budget * 0.4:
            break
    t_acc = time.perf_counter() - t0
    threads = None
    if threadpoolctl is not None:
        info = threadpoolctl.threadpool_info()
        if info:
            threads = max(int(i.get("num_threads", 1)) for i in info)
    return {
        "value": byts * reps / t_gemm / 1e9,
        "unit": "GB/s",
        "cores": threads or os.cpu_count(),
        "kind": "oracle",
        "sample": f"verify GEMM at T=5 on rows [0,{rows}) of each of the 7 layer matrices, "
                  f"{reps} passes in {t_gemm:.1f} s (fp64 NumPy BLAS); acceptance loop on "
                  f"{seqs} sequences (K=4, V=128256) in {t_acc:.1f} s",
        "spec_accept_positions_per_s": seqs * (KD + 1) / t_acc,
        "host_cpus": os.cpu_count(),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--pool-gb", type=float, default=1.5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--seed", type=int, default=2)
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the verification step is benchmarked on a single "
              "MI355X (multi-GPU sharding is a design note, not a measured path). Use --gpus 1.",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import mx_fp4_weight_amd as mxs
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    layer_bytes = sum(mx_bytes(n, k) for _, n, k in LAYER)
    n_layers = max(1, math.ceil(args.pool_gb * 1e9 / layer_bytes))
    print(f"# building pool: {n_layers} layers x {layer_bytes / 1e6:.1f} MB", file=sys.stderr, flush=True)
    pool = []
    gen = torch.Generator(device=dev)
    for li in range(n_layers):
        mats = []
        for j, (name, n, k) in enumerate(LAYER):
            gen.manual_seed(args.seed * 1_000_003 + li * 101 + j)
            w = torch.randn((n, k), generator=gen, device=dev, dtype=torch.float32) * 0.02
            codes, scales = mxs.mxfp4_quantize(w)
            del w
            x = (torch.randn((T, k), generator=gen, device=dev, dtype=torch.float32)).to(torch.bfloat16)
            mats.append((codes, scales, x))
        pool.append(mats)
    ys = [torch.empty((T, n), dtype=torch.float32, device=dev) for _, n, _ in LAYER]

    tgt, dft, tok, u = synth.accept_batch(2, 1, KD, V, 3.0, 1.0, seq0=0)
    d_tgt, d_dft = torch.from_numpy(tgt).to(dev), torch.from_numpy(dft).to(dev)
    d_tok, d_u = torch.from_numpy(tok).to(dev), torch.from_numpy(u).to(dev)
    out_tok = torch.empty((1, KD + 1), dtype=torch.int32, device=dev)
    out_n = torch.empty((1,), dtype=torch.int32, device=dev)
    ws = torch.empty((mxs.spec_accept_workspace_bytes(1, KD, V),), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(s, ev=None):
        st = torch.cuda.current_stream()
        mats = pool[s % n_layers]
        for j, (codes, scales, x) in enumerate(mats):
            if ev is not None:
                ev[j][0].record(st)
            mxs.mxfp4_verify_gemm(codes, scales, x, y=ys[j], stream=st)
            if ev is not None:
                ev[j][1].record(st)
        if ev is not None:
            ev[-1][0].record(st)
        mxs.spec_accept(d_tgt, d_dft, d_tok, d_u, out_tokens=out_tok, out_num=out_n, workspace=ws,
                        stream=st)
        if ev is not None:
            ev[-1][1].record(st)

    # eager warmup, then one HIP graph per pool layer (a graph replays one whole step)
    for s in range(max(args.warmup, n_layers)):
        step(s)
    torch.cuda.synchronize()
    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for li in range(n_layers):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            step(li)
        graphs.append(g)
    torch.cuda.synchronize()
    for s in range(args.warmup):
        graphs[s % n_layers].replay()
    torch.cuda.synchronize()

    # timed region: K graph replays (one step each)
    t0 = time.perf_counter()
    for s in range(args.steps):
        graphs[(args.warmup + s) % n_layers].replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # kernel durations: an eager pass with one event pair around every launch
    mk = lambda: torch.cuda.Event(enable_timing=True)
    events = [[(mk(), mk()) for _ in range(len(LAYER) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        step(args.warmup + s, events[s])
    torch.cuda.synchronize()

    gemm_ms = np.array([[events[s][j][0].elapsed_time(events[s][j][1]) for j in range(len(LAYER))]
                        for s in range(args.steps)])
    acc_ms = np.array([events[s][-1][0].elapsed_time(events[s][-1][1]) for s in range(args.steps)])
    step_gemm_bytes = sum(gemm_alg_bytes(n, k, T) for _, n, k in LAYER)
    value = step_gemm_bytes * args.steps / wall / 1e9
    launches = gemm_ms.size
    avg_launch_ms = gemm_ms.mean()
    avg_launch_bytes = step_gemm_bytes / len(LAYER)
    achieved = avg_launch_bytes / (avg_launch_ms * 1e-3) / 1e9
    per_shape = {name: round(gemm_alg_bytes(n, k, T) / (gemm_ms[:, j].mean() * 1e-3) / 1e9, 1)
                 for j, (name, n, k) in enumerate(LAYER)}
    traffic = load_traffic()
    result = {
        "metric": "MX-FP4 verify-GEMM HBM GB/s (% of peak) at T=5; spec_accept positions/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "8B-class layer shapes at T=5: q,o 4096x4096; k,v 1024x4096; gate,up 14336x4096; "
                        "down 4096x14336 (MX-FP4 weights, bf16 activations, fp32 out) + spec_accept "
                        "B=1 K=4 V=128256",
            "T": T, "K_draft": KD, "vocab": V,
            "pool_layers": n_layers, "pool_bytes": layer_bytes * n_layers,
            "gemm_bytes_per_step": step_gemm_bytes,
            "parallelism": "single GPU",
        },
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "gemm_kernel_GBps_by_shape": per_shape,
        "spec_accept_positions_per_s": round((KD + 1) / (acc_ms.mean() * 1e-3), 1),
        "spec_accept_us": round(acc_ms.mean() * 1e3, 2),
        "numerics": "E2M1 weights decoded exactly to bf16, bf16 x bf16 products summed in fp32 (MFMA); "
                    "spec_accept probabilities in fp64",
        "roofline": {
            "kernel": "gemm_skinny_kernel (mxfp4_verify_gemm)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "avg_launch_us": round(avg_launch_ms * 1e3, 3),
            "avg_launch_alg_bytes": avg_launch_bytes,
            "launches_timed": int(launches),
        },
    }
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline()
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
