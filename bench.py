#!/usr/bin/env python3
"""Benchmark of the speculative verification step on one MI355X.

Workload (8B-class layer shapes at T = K+1 = 5): one step streams one decoder
layer's MX-FP4 weights — q and o 4096x4096, k and v 1024x4096, gate and up
14336x4096, down 4096x14336 (218,103,808 weights, 115,867,648 bytes of codes +
scales), each against its own bf16 activations [5, K] — in dependency order:
mxfp4_verify_gemm_grouped over q | k | v, mxfp4_verify_gemm for o,
mxfp4_verify_gemm_grouped over gate | up, mxfp4_verify_gemm for down. Then it
runs spec_accept on one sequence (K = 4 drafts, vocab 128256, fp32 logits
N(0, 3), target = draft + N(0, 1)).

Cold weights: the layers of a pool (default 4.6 GB, 40 layers) are visited in
turn, so every step reads its weights from HBM; even one launch type alone
(e.g. o over all 40 layers, 356 MB) streams more than the 256 MB Infinity
Cache holds. Inputs are resident in HBM before the timed region. Weights
are N(0, 0.02) fp32 drawn on the GPU and quantized by mxfp4_quantize (not
timed). The logits and uniforms come from the shared seeded generator.

Each step is captured once per pool layer as a HIP graph on one stream; the
timed region replays K graphs back to back. Prints one JSON line. `value` is verify-GEMM
algorithmic bytes per step (codes + scales + X + Y) times steps, over the
wall time of all steps (spec_accept and the gaps between kernels included).
`roofline` is the verify-GEMM kernel alone: for each launch type a graph runs
it on every pool layer back to back between two HIP events on the replay
stream, giving the average launch duration without host gaps.

The same line carries the secondary workloads (skipped with --no-extra):
`t_sweep_8b` (the four launch types at T = 1..8), `shapes_70b_t5` (70B-class
shapes with 1% outlier input channels x20, lm_head 128256x8192, and the
70B tokens/s-equivalent), `batched_64x5` (dense verify GEMM 320x8192x28672 with
its MFMA utilisation, spec_accept for 64 sequences) and `full_8b_step` (32
layers + lm_head 128256x4096, then spec_accept on the lm_head output with draft
rows tuned to acceptance 0.6 / 0.8 / 0.9: step time, tokens/s-equivalent and the
GPU-measured tokens per step against the closed form), `sampled_accept`
(spec_accept_sampled at B = 1 and 64 under temperature only, temperature + top-k +
top-p + a 90% grammar mask, and top-p alone, next to plain spec_accept),
`tree_accept` (spec_accept_tree on three tree shapes at B = 1 and 64), `kv_append`
(mxfp4_kv_append of 5 and 4096 tokens into an 8-head MX-FP4 KV cache) and `kv_attention`
(mxfp4_kv_attention of a T = 5 pass over 4096- and 32768-entry MX-FP4 caches).
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
# launches of a layer in dependency order; projections that read the same input share one
LAUNCHES = [("qkv", (0, 1, 2)), ("o", (3,)), ("gate_up", (4, 5)), ("down", (6,))]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "verify_gemm_8b_layer_t5_traffic.json")
STEPS_PER_GRAPH = 8  # headline steps captured in one HIP graph (the pool's layer count is a multiple)
CALIB_MB = 512
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


def summarize_pmc(fetch_dir, write_dir, out_path=TRAFFIC_FILE):
    """HBM bytes per verify-GEMM launch from two rocprofv3 --pmc runs of this script.

    Each run must use --calib-copy-mb: the counters of that plain elementwise kernel
    of a known size give the bytes-per-count factor (counter KiB x 1024 / true bytes).
    FETCH_SIZE and WRITE_SIZE are read in KiB per dispatch.
    """
    import csv
    import glob

    def rows(d, counter):
        out = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r.get("Counter_Name") == counter:
                    out.append((r["Kernel_Name"], float(r["Counter_Value"])))
        return out

    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rr = rows(d, counter)
        copy = [v for name, v in rr if "neg_kernel" in name]
        gemm = [v for name, v in rr if "gemm_skinny_kernel" in name or "gemm_xglobal_kernel" in name]
        if not copy or not gemm:
            raise SystemExit(f"no copy/gemm dispatches with {counter} in {d}")
        calib_bytes = CALIB_MB * 1024 * 1024
        factor = max(copy) * 1024 / calib_bytes
        res[counter] = {"gemm_kib_mean": sum(gemm) / len(gemm), "dispatches": len(gemm),
                        "copy_kib": max(copy), "factor": factor,
                        "bytes_per_launch": sum(gemm) / len(gemm) * 1024 / factor}
    summary = {
        "kernel": "gemm_skinny_kernel on tiled weights (mxfp4_verify_gemm_tiled / _grouped_tiled), "
                  "8B-class layer shapes at T=5",
        "gemm_source_sha": source_sha(GEMM_SRC),
        "traffic_bytes_per_launch": res["FETCH_SIZE"]["bytes_per_launch"] + res["WRITE_SIZE"]["bytes_per_launch"],
        "alg_bytes_per_launch": sum(gemm_alg_bytes(n, k, T) for _, n, k in LAYER) / len(LAUNCHES),
        "counters": res,
        "calibration": f"torch.neg over {CALIB_MB} MiB of fp32 (reads and writes {CALIB_MB} MiB)",
        "commands": [
            f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {fetch_dir} -o pmc -- "
            f"python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --only headline "
            f"--calib-copy-mb {CALIB_MB}",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {write_dir} -o pmc -- "
            f"python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --only headline "
            f"--calib-copy-mb {CALIB_MB}",
            f"python3 bench.py --summarize-pmc {fetch_dir} {write_dir}",
        ],
    }
    with open(out_path, "w") as f:
        json.dump(summary, f, indent=1)
    print(json.dumps(summary, indent=1))


def _short_kernel_name(name):
    return name.replace("void ", "").replace("mxs::(anonymous namespace)::", "").split("(")[0]


def _label(name, wgs, lds, grid_y):
    """What a library dispatch of the headline workload is, from its kernel, workgroup count and LDS
    (tiled 8B-class layer at T = 5: q|k|v 384 workgroups, o and down 256 with o's smaller activation
    tile, gate|up 512)."""
    if "quantize_act" in name:
        return "MX quantization of activations (W4A8 / W4A4) or of KV entries (kv_append)"
    if "attn_combine" in name:
        return "verification attention: merge of the entry ranges"
    if "attn_kernel" in name:
        return "verification attention"
    if "tree_" in name:
        return "spec_accept_tree"
    if "tile_codes" in name or "tile_scales" in name or "quantize" in name:
        return "weight prep (one-off, untimed)"
    if "stream_read" in name:
        return "read-stream ceiling"
    if "sel_" in name:
        return "top-k / top-p thresholds (spec_accept_sampled)"
    if any(a in name for a in ("stats_kernel", "decide_kernel", "sample_kernel")):
        return "spec_accept"
    if "gemm_skinny" in name:
        return {384: "q|k|v grouped", 512: "gate|up grouped",
                256: "o and down (256 workgroups each)"}.get(wgs, f"{wgs} workgroups")
    if "gemm_dense" in name:
        return "bf16 dense product" + (" (tiled weights)" if ", true>" in name else " (row layout)")
    if "gemm_act" in name:
        fmt = "W4A8" if "<5, 0," in name else "W4A4"
        return fmt + (" (tiled weights)" if ", true>" in name else " (row layout)")
    return ""


def summarize_trace(trace_dir, out_path, title, command):
    """Markdown summary of a rocprofv3 --kernel-trace --stats run: per library kernel and launch
    shape (workgroups, LDS bytes), dispatches and mean / median / min duration, then the --stats
    table of the library kernels."""
    import csv
    import glob
    import statistics as st
    tr = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not tr:
        raise SystemExit(f"no kernel trace under {trace_dir}")
    groups = {}
    for r in csv.DictReader(open(tr[0])):
        if "mxs::" not in r["Kernel_Name"]:
            continue
        n = _short_kernel_name(r["Kernel_Name"])
        wgs = int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))
        key = (n, wgs, int(r["Grid_Size_Y"]), int(r["LDS_Block_Size"]))
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    lines = [f"# Kernel trace: {title}", "", "Command (from /tmp, TMPDIR=/tmp):", "", "```", command, "```", "",
             "Durations from the kernel trace (start to end of each dispatch, µs).", "",
             "| kernel | workgroups x grid y | LDS bytes | what | dispatches | mean µs | median µs | min µs |",
             "|---|---|---|---|---|---|---|---|"]
    for (n, wgs, gy, lds), v in sorted(groups.items()):
        lines.append(f"| `{n}` | {wgs} x {gy} | {lds} | {_label(n, wgs, lds, gy)} | {len(v)} | {st.mean(v):.2f} | "
                     f"{st.median(v):.2f} | {min(v):.2f} |")
    ks = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if ks:
        lines += ["", "rocprofv3 --stats summary (library kernels):", "",
                  "| Name | Calls | AverageNs | MinNs | MaxNs |", "|---|---|---|---|---|"]
        for r in csv.DictReader(open(ks[0])):
            if "mxs::" in r["Name"]:
                lines.append(f"| `{_short_kernel_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                             f"{float(r['MinNs']):.0f} | {float(r['MaxNs']):.0f} |")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_busy(pmc_dir, out_path, title, command):
    """Markdown summary of a rocprofv3 --pmc run of VALUBusy / MfmaUtil (and any other counters in
    it): the mean per dispatch of each counter, per library kernel and launch shape."""
    import csv
    import glob
    import statistics as st
    files = glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter collection under {pmc_dir}")
    vals, counters = {}, set()
    for r in csv.DictReader(open(files[0])):
        if "mxs::" not in r["Kernel_Name"]:
            continue
        n = _short_kernel_name(r["Kernel_Name"])
        wgs = int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"]))
        key = (n, wgs, int(r["LDS_Block_Size"]))
        counters.add(r["Counter_Name"])
        vals.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    cs = sorted(counters)
    lines = [f"# Counters: {title}", "", "Command (from /tmp, TMPDIR=/tmp):", "", "```", command, "```", "",
             "Mean per dispatch. VALUBusy = 100 x SQ_ACTIVE_INST_VALU / CU_NUM / GRBM_GUI_ACTIVE (share of "
             "the kernel's GPU-active time the vector ALUs issue); MfmaUtil = 100 x SQ_VALU_MFMA_BUSY_CYCLES / "
             "(GRBM_GUI_ACTIVE x SIMD_NUM) (share of SIMD cycles the matrix cores are busy).", "",
             "| kernel | workgroups | LDS bytes | what | dispatches | " + " | ".join(cs) + " |",
             "|---|---|---|---|---|" + "---|" * len(cs)]
    for (n, wgs, lds), d in sorted(vals.items()):
        cnt = max(len(v) for v in d.values())
        cells = " | ".join(f"{st.mean(d[c]):.2f}" if c in d else "" for c in cs)
        lines.append(f"| `{n}` | {wgs} | {lds} | {_label(n, wgs, lds, 1)} | {cnt} | {cells} |")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cpu_model():
    """The host CPU's model name (as lscpu reports it), from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(seconds_budget=20.0):
    """The oracle (fp64 NumPy) on the host cores, on a bounded sample of the same workload.

    Sample: rows [0, 512) of each of the 7 layer matrices (oracle-quantized from
    the shared generator), verify GEMM at T = 5, repeated with the BLAS on all
    host threads and on one; the oracle quantizer (one thread) on the same
    rows; plus the oracle acceptance loop (one thread) on sequences of the
    same spec_accept configuration.
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
    mats, wts = [], []
    for i, (name, n, k) in enumerate(LAYER):
        w = synth.weights(2, 1000 + i, n, k, row_start=0, row_stop=rows)
        c, s, _ = omx.quantize(w)
        x = synth.activations(2, 1000 + i, T, k)
        mats.append((c, s, rows, k, x))
        wts.append(w)
    ogemm.verify_gemm(*mats[0])  # warm BLAS
    byts = sum(gemm_alg_bytes(rows, k, T) for (_, _, _, k, _) in mats)

    def timed(fn, budget):
        t0 = time.perf_counter()
        reps = 0
        while True:
            fn()
            reps += 1
            if time.perf_counter() - t0 > budget:
                return reps, time.perf_counter() - t0

    def gemm_pass():
        for m in mats:
            ogemm.verify_gemm(*m)

    reps, t_gemm = timed(gemm_pass, seconds_budget * 0.35)
    threads = None
    if threadpoolctl is not None:
        info = threadpoolctl.threadpool_info()
        if info:
            threads = max(int(i.get("num_threads", 1)) for i in info)
        with threadpoolctl.threadpool_limits(1):
            reps1, t_gemm1 = timed(gemm_pass, seconds_budget * 0.2)
            qreps, t_q = timed(lambda: [omx.quantize(w) for w in wts], seconds_budget * 0.15)
    else:
        reps1, t_gemm1 = reps, t_gemm
        qreps, t_q = timed(lambda: [omx.quantize(w) for w in wts], seconds_budget * 0.15)
    q_bytes = sum(w.nbytes for w in wts)
    tgt, dft, tok, u = synth.accept_batch(2, 4, KD, V, 3.0, 1.0, seq0=500)
    t0 = time.perf_counter()
    seqs = 0
    while True:
        for b in range(4):
            oacc.step(tgt[b], dft[b], tok[b], u[b])
        seqs += 4
        if time.perf_counter() - t0 > seconds_budget * 0.3:
            break
    t_acc = time.perf_counter() - t0
    return {
        "value": byts * reps / t_gemm / 1e9,
        "unit": "GB/s",
        "cores": threads or os.cpu_count(),
        "kind": "oracle",
        "sample": f"verify GEMM at T=5 on rows [0,{rows}) of each of the 7 layer matrices, "
                  f"{reps} passes in {t_gemm:.1f} s (fp64 NumPy BLAS, all threads); the same at 1 thread "
                  f"({reps1} passes in {t_gemm1:.1f} s); oracle quantizer on those rows' fp32 weights "
                  f"(1 thread, {qreps} passes in {t_q:.1f} s); acceptance loop on {seqs} sequences "
                  f"(K=4, V=128256, 1 thread) in {t_acc:.1f} s",
        "gemm_GBps_1_thread": byts * reps1 / t_gemm1 / 1e9,
        "quantize_MBps_fp32_in_1_thread": q_bytes * qreps / t_q / 1e6,
        "spec_accept_positions_per_s": seqs * (KD + 1) / t_acc,
        "host_cpus": os.cpu_count(),
        "cpu_model": cpu_model(),
    }


def gpu_clocks():
    """Current shader (sclk), memory (mclk) and fabric (fclk) clock levels of the GPU, as the
    amdgpu driver reports them (recorded, not locked). From sysfs; rocm-smi otherwise."""
    import glob
    out = {}
    for card in sorted(glob.glob("/sys/class/drm/card*/device")):
        for name in ("pp_dpm_sclk", "pp_dpm_mclk", "pp_dpm_fclk"):
            try:
                with open(os.path.join(card, name)) as f:
                    cur = [ln.split(":", 1)[1].strip().rstrip("*").strip() for ln in f if ln.rstrip().endswith("*")]
            except OSError:
                continue
            if cur:
                out[name[-4:]] = cur[0]
        if out:
            out["source"] = card + "/pp_dpm_*"
            return out
    try:
        import subprocess
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=30)
        d = json.loads(r.stdout)
        card = next(iter(d.values()))
        out = {k: v for k, v in card.items() if "clock" in k.lower()}
        out["source"] = "rocm-smi --showclocks"
        return out
    except Exception as e:  # clocks are context only: never fail the bench for them
        return {"source": None, "error": repr(e)[:200]}


STREAM_BYTES = 4 << 30  # read-ceiling buffer: 16x the 256 MB Infinity Cache, so the reads come from HBM


def stream_ceiling(torch, mxs, reps=20):
    """The measured read ceiling: mxs_stream_read over a 4 GiB buffer (cold: far larger than the
    caches), each call between its own HIP events on the current stream; GB/s median, p10, p90."""
    buf = torch.ones((STREAM_BYTES // 4,), dtype=torch.int32, device="cuda")
    sink = torch.zeros((1,), dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()
    for _ in range(3):
        mxs.stream_read(buf, sink, stream=st)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(st)
    for r in range(reps):
        mxs.stream_read(buf, sink, stream=st)
        ev[r + 1].record(st)
    torch.cuda.synchronize()
    gbps = [STREAM_BYTES / (ev[r].elapsed_time(ev[r + 1]) * 1e-3) / 1e9 for r in range(reps)]
    del buf
    q = pctl(gbps)
    return {"GBps_median": round(q["median"], 1), "GBps_p10": round(q["p10"], 1), "GBps_p90": round(q["p90"], 1),
            "frac_of_hbm_peak": round(q["median"] / HBM_PEAK_GBPS, 4), "bytes_per_call": STREAM_BYTES,
            "calls": reps, "kernel": "stream_read_kernel (mxs_stream_read: 16-byte non-temporal loads, 8 per lane "
                                     "in flight, two 256-thread workgroups per CU)"}


def pctl(vals):
    """median, p10 and p90 of a list (nearest-rank)."""
    v = sorted(vals)
    pick = lambda q: v[min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))]
    return {"median": pick(0.5), "p10": pick(0.1), "p90": pick(0.9), "n": len(v)}


# ---------------------------------------------------------------------------
# Secondary workloads, reported in the same JSON line (not part of `value`).

def _gpu_mx(torch, mxs, gen, n, k, sigma=0.02, outlier_cols=None):
    """MX-FP4 codes/scales of an N(0, sigma) fp32 matrix drawn on the GPU (optionally
    with outlier input columns scaled x20)."""
    w = torch.randn((n, k), generator=gen, device="cuda", dtype=torch.float32) * sigma
    if outlier_cols is not None and len(outlier_cols):
        idx = torch.as_tensor(outlier_cols, device="cuda")
        w[:, idx] *= 20.0
    c, s = mxs.mxfp4_quantize(w)
    del w
    return c, s


CALLS_PER_GRAPH = 8  # a single-call workload runs this many times in one graph (per-call time reported)


def _graph_call_ms(torch, call, reps, copies=CALLS_PER_GRAPH):
    """Average ms per call of a HIP graph that runs call() `copies` times: the graph launch and
    the gap between graph replays are shared by the copies, as by the kernels of a decoding step."""
    def body():
        for _ in range(copies):
            call()
    return _graph_ms(torch, body, reps) / copies


def _graph_ms(torch, body, reps):
    """Average ms per replay of a HIP graph that runs body() once (one warm replay first)."""
    body()  # eager call: one-time library set-up outside the capture
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        body()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        g.replay()
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del g
    return ms


def _rand_bf16(torch, gen, m, k):
    return torch.randn((m, k), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)


def _tile(mxs, c, s, x):
    """(codes, scales, x) -> (tiled codes, tiled scales, n, x): the one-off weight-prep permutation."""
    return (mxs.mxfp4_tile_codes(c), mxs.mxfp4_tile_scales(s), c.shape[0], x)


def _gemm(mxs, items, ys, stream=None):
    """The verify GEMM of items [(tiled codes, tiled scales, n, x)] into ys: one product or a group."""
    if len(items) == 1:
        tc, ts, n, x = items[0]
        mxs.mxfp4_verify_gemm_tiled(tc, ts, n, x.shape[1], x, y=ys[0], stream=stream)
    else:
        mxs.mxfp4_verify_gemm_grouped_tiled(items, ys=ys, stream=stream)


def t_sweep(torch, mxs, pool, gen, reps=3):
    """8B-class shapes at T = 1..8 over the cold pool (tiled weights): per launch type, µs and GB/s."""
    n_layers = len(pool)
    out = {}
    for t in range(1, 9):
        xs = [[_rand_bf16(torch, gen, t, k) for (_, _, k) in LAYER] for _ in range(n_layers)]
        ys = [torch.empty((t, n), dtype=torch.float32, device="cuda") for (_, n, _) in LAYER]
        row = {}
        for name, idx in LAUNCHES:
            def body(idx=idx):
                for li in range(n_layers):
                    _gemm(mxs, [(*pool[li][i][:3], xs[li][i]) for i in idx], [ys[i] for i in idx])
            us = _graph_ms(torch, body, reps) * 1e3 / n_layers
            byts = sum(gemm_alg_bytes(LAYER[i][1], LAYER[i][2], t) for i in idx)
            row[name] = {"us": round(us, 2), "GBps": round(byts / (us * 1e-6) / 1e9, 1)}
        tot_b = sum(gemm_alg_bytes(n, k, t) for _, n, k in LAYER)
        tot_us = sum(v["us"] for v in row.values())
        row["layer_GBps"] = round(tot_b / (tot_us * 1e-6) / 1e9, 1)
        row["layer_pct_of_hbm_peak"] = round(100 * tot_b / (tot_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 2)
        out[f"T{t}"] = row
        del xs, ys
    return out


L70 = [("q", 8192, 8192), ("k", 1024, 8192), ("v", 1024, 8192), ("o", 8192, 8192),
       ("gate", 28672, 8192), ("up", 28672, 8192), ("down", 8192, 28672)]
LM70 = (128256, 8192)
MODEL70_BYTES = 80 * sum(mx_bytes(n, k) for _, n, k in L70) + mx_bytes(*LM70)


def shapes_70b(torch, mxs, synth, gen, reps=3):
    """70B-class shapes at T=5 with 1% outlier input channels x20, tiled weights: per launch µs and GB/s.

    Copies per shape are chosen so each timed graph streams > 256 MB (cold weights).
    """
    import numpy as np
    copies = {"attn": 8, "mlp": 3, "lm": 2}
    outl = {k: synth.outlier_columns(3, j, k, 0.01) for j, k in ((0, 8192), (1, 28672))}
    attn, mlp, lm = [], [], []
    for c in range(copies["attn"]):
        attn.append([(*_gpu_mx(torch, mxs, gen, n, k, outlier_cols=outl[k]), _rand_bf16(torch, gen, T, k))
                     for (_, n, k) in L70[:4]])
    for c in range(copies["mlp"]):
        mlp.append([(*_gpu_mx(torch, mxs, gen, n, k, outlier_cols=outl[k]),
                     _rand_bf16(torch, gen, T, k)) for (_, n, k) in L70[4:]])
    for c in range(copies["lm"]):
        lm.append((*_gpu_mx(torch, mxs, gen, *LM70, outlier_cols=outl[8192]), _rand_bf16(torch, gen, T, LM70[1])))
    # tiled weights (the row-layout copies are dropped)
    attn = [[_tile(mxs, *t) for t in st] for st in attn]
    mlp = [[_tile(mxs, *t) for t in st] for st in mlp]
    lm = [_tile(mxs, *t) for t in lm]
    y_attn = [torch.empty((T, n), dtype=torch.float32, device="cuda") for (_, n, _) in L70[:4]]
    y_mlp = [torch.empty((T, n), dtype=torch.float32, device="cuda") for (_, n, _) in L70[4:]]
    y_lm = torch.empty((T, LM70[0]), dtype=torch.float32, device="cuda")
    plans = [("qkv", attn, (0, 1, 2), y_attn), ("o", attn, (3,), y_attn), ("gate_up", mlp, (0, 1), y_mlp),
             ("down", mlp, (2,), y_mlp), ("lm_head", None, None, None)]
    out = {}
    layer_b = layer_us = 0.0
    for name, sets, idx, ybuf in plans:
        if name == "lm_head":
            def body():
                for t in lm:
                    _gemm(mxs, [t], [y_lm])
            us = _graph_ms(torch, body, reps) * 1e3 / len(lm)
            byts = gemm_alg_bytes(LM70[0], LM70[1], T)
        else:
            def body(sets=sets, idx=idx, ybuf=ybuf):
                for st in sets:
                    _gemm(mxs, [st[i] for i in idx], [ybuf[i] for i in idx])
            us = _graph_ms(torch, body, reps) * 1e3 / len(sets)
            byts = sum(gemm_alg_bytes(sets[0][i][2], sets[0][i][3].shape[1], T) for i in idx)
            layer_b += byts
            layer_us += us
        out[name] = {"us": round(us, 2), "GBps": round(byts / (us * 1e-6) / 1e9, 1)}
    layer_bps = layer_b / (layer_us * 1e-6)
    out["layer_GBps"] = round(layer_bps / 1e9, 1)
    out["layer_pct_of_hbm_peak"] = round(100 * layer_bps / 1e9 / HBM_PEAK_GBPS, 2)
    out["tokens_per_s_equivalent"] = round(layer_bps / MODEL70_BYTES, 1)
    out["note"] = ("tokens/s-equivalent = achieved layer bytes/s / 70B-class model MX bytes "
                   f"({MODEL70_BYTES} B: 80 layers + lm_head), one verification step per token")
    del attn, mlp, lm
    return out


def batched(torch, mxs, gen, reps=5):
    """64 sequences x 5 positions: dense verify GEMM (320 x 8192 x 28672) and spec_accept B=64."""
    n, k, m = 8192, 28672, 320
    copies = [(*_gpu_mx(torch, mxs, gen, n, k), _rand_bf16(torch, gen, m, k)) for _ in range(3)]
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")

    # weight codes and scales in the tiled layouts (a one-off permutation at weight-prep time)
    tiled = [(mxs.mxfp4_tile_codes(c), mxs.mxfp4_tile_scales(s)) for (c, s, _) in copies]

    def body_row():
        for (c, s, x) in copies:
            mxs.mxfp4_verify_gemm(c, s, x, y=y)

    def body():
        for (tc, ts), (_, _, x) in zip(tiled, copies):
            mxs.mxfp4_verify_gemm_tiled(tc, ts, n, k, x, y=y)
    us_row = _graph_ms(torch, body_row, reps) * 1e3 / len(copies)
    us = _graph_ms(torch, body, reps) * 1e3 / len(copies)
    flops = 2.0 * m * n * k
    byts = gemm_alg_bytes(n, k, m)
    out = {"gemm": {"us": round(us, 1), "TFLOPs": round(flops / (us * 1e-6) / 1e12, 1),
                    "mfma_util_vs_bf16_dense_peak": round(flops / (us * 1e-6) / 2.5e15, 4),
                    "GBps": round(byts / (us * 1e-6) / 1e9, 1),
                    "row_layout_us": round(us_row, 1),
                    "kernel": "gemm_dense_kernel (v_mfma_f32_16x16x32_bf16; peak 2.5 PFLOP/s dense bf16); weight "
                              "codes and scales tiled by mxfp4_tile_codes / mxfp4_tile_scales (row_layout_us: "
                              "mxfp4_verify_gemm on the row layout)"}}
    # the same product with MX-quantized activations (W4A8 / W4A4) on the block-scaled MFMA
    for fmt, name, peak in ((mxs.ACT_FP8, "gemm_w4a8", 5.0e15), (mxs.ACT_FP4, "gemm_w4a4", 10.1e15)):
        acts = [mxs.mx_quantize_act(x, fmt) for (_, _, x) in copies]

        def body_q(fmt=fmt):
            for (_, _, x), (ac, asc) in zip(copies, acts):
                mxs.mx_quantize_act(x, fmt, codes=ac, scales=asc)

        def body_g(fmt=fmt, acts=acts):
            for (c, s, _), (ac, asc) in zip(copies, acts):
                mxs.mx_verify_gemm_act(c, s, ac, asc, fmt, y=y)
        def body_t(fmt=fmt, acts=acts, tiled=tiled):
            for (tc, ts), (ac, asc) in zip(tiled, acts):
                mxs.mx_verify_gemm_act_tiled(tc, ts, n, k, ac, asc, fmt, y=y)
        us_g = _graph_ms(torch, body_g, reps) * 1e3 / len(copies)
        us_t = _graph_ms(torch, body_t, reps) * 1e3 / len(copies)
        us_q = _graph_ms(torch, body_q, reps * 4) * 1e3 / len(copies)
        abytes = acts[0][0].numel() + acts[0][1].numel()
        out[name] = {"us": round(us_t, 1), "quantize_act_us": round(us_q, 1),
                     "TFLOPs": round(flops / (us_t * 1e-6) / 1e12, 1),
                     "mfma_util_vs_dense_peak": round(flops / (us_t * 1e-6) / peak, 4),
                     "GBps": round((mx_bytes(n, k) + abytes + m * n * 4) / (us_t * 1e-6) / 1e9, 1),
                     "row_layout_us": round(us_g, 1),
                     "kernel": "gemm_act_kernel (v_mfma_scale_f32_16x16x128_f8f6f4, "
                               f"MX-FP4 x {'MX-FP8' if fmt == mxs.ACT_FP8 else 'MX-FP4'}; "
                               f"dense peak {peak / 1e15:.1f} PFLOP/s); weight codes and scales tiled by "
                               "mxfp4_tile_codes / mxfp4_tile_scales (row_layout_us: the same product on "
                               "the row layout)"}
        del acts
    del copies, tiled
    b = 64
    base = torch.randn((b, KD + 1, V), generator=gen, device="cuda", dtype=torch.float32) * 3.0
    tgt = base + torch.randn((b, KD + 1, V), generator=gen, device="cuda", dtype=torch.float32)
    dft = base[:, :KD].contiguous()
    del base
    tok = torch.multinomial(torch.softmax(dft.double(), -1).reshape(b * KD, V), 1, generator=gen)
    tok = tok.reshape(b, KD).to(torch.int32)
    u = torch.rand((b, KD + 1), generator=gen, device="cuda", dtype=torch.float32)
    ws = torch.empty((mxs.spec_accept_workspace_bytes(b, KD, V),), dtype=torch.uint8, device="cuda")
    ot = torch.empty((b, KD + 1), dtype=torch.int32, device="cuda")
    on = torch.empty((b,), dtype=torch.int32, device="cuda")

    def acc():
        mxs.spec_accept(tgt, dft, tok, u, out_tokens=ot, out_num=on, workspace=ws)
    us_a = _graph_call_ms(torch, acc, reps * 4) * 1e3
    read_b = b * (2 * KD + 1) * V * 4
    out["spec_accept"] = {"B": b, "us": round(us_a, 1),
                          "positions_per_s": round(b * (KD + 1) / (us_a * 1e-6), 1),
                          "logit_read_GBps": round(read_b / (us_a * 1e-6) / 1e9, 1),
                          "mean_accepted": round(float(on.float().mean()), 3)}
    del tgt, dft, ws
    return out


def _pack_mask_gpu(torch, allowed):
    """bool [..., V] -> int32 [..., ceil(V/32)] words in the library's mask layout (bit t % 32 of
    word t // 32), built with torch ops on the GPU (input preparation)."""
    v = allowed.shape[-1]
    w = (v + 31) // 32
    pad = torch.zeros(allowed.shape[:-1] + (w * 32,), dtype=torch.int64, device=allowed.device)
    pad[..., :v] = allowed.to(torch.int64)
    bits = pad.view(allowed.shape[:-1] + (w, 32)) << torch.arange(32, device=allowed.device, dtype=torch.int64)
    words = bits.sum(-1)
    return torch.where(words >= 2 ** 31, words - 2 ** 32, words).to(torch.int32).contiguous()


SAMPLED_SETTINGS = [  # (name, temperature, top_k, top_p, mask keep fraction)
    ("tau0.8", 0.8, 0, 1.0, None),
    ("tau0.8_k50_p0.9_mask0.9", 0.8, 50, 0.9, 0.9),
    ("p0.95", 1.0, 0, 0.95, None),
]


def sampled_accept(torch, mxs, gen, reps=20):
    """spec_accept_sampled at K=4, V=128256 for B = 1 and 64 under three transform settings,
    next to plain spec_accept on the same inputs. Draft tokens are the most probable allowed
    token of each draft row (always inside the transformed support)."""
    out = {}
    for b in (1, 64):
        base = torch.randn((b, KD + 1, V), generator=gen, device="cuda", dtype=torch.float32) * 3.0
        tgt = base + torch.randn((b, KD + 1, V), generator=gen, device="cuda", dtype=torch.float32)
        dft = base[:, :KD].contiguous()
        del base
        u = torch.rand((b, KD + 1), generator=gen, device="cuda", dtype=torch.float32)
        ot = torch.empty((b, KD + 1), dtype=torch.int32, device="cuda")
        on = torch.empty((b,), dtype=torch.int32, device="cuda")
        ws = torch.empty((mxs.spec_accept_sampled_workspace_bytes(b, KD, V),), dtype=torch.uint8,
                         device="cuda")
        tok_plain = dft.argmax(-1).to(torch.int32).contiguous()

        def plain():
            mxs.spec_accept(tgt, dft, tok_plain, u, out_tokens=ot, out_num=on, workspace=ws)
        row = {"plain_us": round(_graph_call_ms(torch, plain, reps) * 1e3, 1)}
        for name, tau, k, p, keep in SAMPLED_SETTINGS:
            mask = None
            tok = tok_plain
            if keep is not None:
                allowed = torch.rand((b, KD + 1, V), generator=gen, device="cuda") < keep
                mask = _pack_mask_gpu(torch, allowed)
                tok = dft.masked_fill(~allowed[:, :KD], float("-inf")).argmax(-1).to(torch.int32).contiguous()
                del allowed

            def call(tau=tau, k=k, p=p, mask=mask, tok=tok):
                mxs.spec_accept_sampled(tgt, dft, tok, u, tau, k, p, mask, out_tokens=ot, out_num=on,
                                        workspace=ws)
            us = _graph_call_ms(torch, call, reps) * 1e3
            row[name] = {"us": round(us, 1), "positions_per_s": round(b * (KD + 1) / (us * 1e-6), 1),
                         "mean_accepted": round(float(on.float().mean()), 3)}
        out[f"B{b}"] = row
        del tgt, dft, ws
    return out


TREE_SHAPES = {  # parent lists: a chain of 4, a 3-way root with 2 children each, a binary tree of depth 3
    "chain4": [-1, 0, 1, 2],
    "3x2": [-1, -1, -1, 0, 0, 1, 1, 2, 2],
    "binary3": [-1, -1, 0, 0, 1, 1, 2, 2, 3, 3, 4, 4, 5, 5],
}


def tree_accept(torch, mxs, gen, reps=20):
    """spec_accept_tree over V = 128256 for B = 1 and 64 on three tree shapes (fp32 logits N(0, 3),
    target = draft + N(0, 1), every node's token drawn from its parent's draft row), next to
    plain spec_accept on the chain's inputs."""
    out = {}
    for b in (1, 64):
        row = {}
        for name, parent in TREE_SHAPES.items():
            nn = len(parent)
            base = torch.randn((b, nn + 1, V), generator=gen, device="cuda", dtype=torch.float32) * 3.0
            tgt = base + torch.randn((b, nn + 1, V), generator=gen, device="cuda", dtype=torch.float32)
            dft = base
            del base
            rows = torch.tensor([p + 1 for p in parent], device="cuda")
            law = torch.softmax(dft[:, rows].double(), -1).reshape(b * nn, V)
            tok = torch.multinomial(law, 1, generator=gen).reshape(b, nn).to(torch.int32)
            del law
            u = torch.rand((b, nn + 1), generator=gen, device="cuda", dtype=torch.float32)
            d = mxs.tree_depth(parent)
            ot = torch.empty((b, d + 1), dtype=torch.int32, device="cuda")
            on = torch.empty((b, d), dtype=torch.int32, device="cuda")
            onum = torch.empty((b,), dtype=torch.int32, device="cuda")
            ws = torch.empty((mxs.spec_accept_tree_workspace_bytes(parent, b, V),), dtype=torch.uint8, device="cuda")

            def call(parent=parent, tgt=tgt, dft=dft, tok=tok, u=u, ot=ot, on=on, onum=onum, ws=ws):
                mxs.spec_accept_tree(parent, tgt, dft, tok, u, out_tokens=ot, out_nodes=on, out_num=onum,
                                     workspace=ws)
            us = _graph_call_ms(torch, call, reps) * 1e3
            entry = {"nodes": nn, "depth": d, "us": round(us, 1),
                     "positions_per_s": round(b * (nn + 1) / (us * 1e-6), 1),
                     "mean_accepted": round(float(onum.float().mean()), 3),
                     "kernels": 2 + (max([parent.count(p) for p in set(parent)] + [0]) + 1)}
            if name == "chain4":
                ot2 = torch.empty((b, nn + 1), dtype=torch.int32, device="cuda")
                on2 = torch.empty((b,), dtype=torch.int32, device="cuda")
                ws2 = torch.empty((mxs.spec_accept_workspace_bytes(b, nn, V),), dtype=torch.uint8, device="cuda")
                tc, dc = tgt.contiguous(), dft[:, :nn].contiguous()

                def lin(tc=tc, dc=dc, tok=tok, u=u, ot2=ot2, on2=on2, ws2=ws2):
                    mxs.spec_accept(tc, dc, tok, u, out_tokens=ot2, out_num=on2, workspace=ws2)
                entry["linear_spec_accept_us"] = round(_graph_call_ms(torch, lin, reps) * 1e3, 1)
                del tc, dc, ws2
            row[name] = entry
            del tgt, dft, ws
        out[f"B{b}"] = row
    return out


def kv_append(torch, mxs, gen, reps=20):
    """mxfp4_kv_append for the 8B-class cache (8 KV heads of 128): a verification step's 5 new
    tokens and a 4096-token prefill, into a 32768-entry cache; GB/s of bf16 read + codes and
    scales written."""
    heads, d, cap = 8, 128, 32768
    codes = torch.zeros((cap, heads, d // 2), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((cap, heads, d // 32), dtype=torch.uint8, device="cuda")
    out = {"cache_entries": cap, "heads": heads, "d": d,
           "footprint_vs_bf16": round((d // 2 + d // 32) / (2 * d), 6)}
    for t in (5, 4096):
        kv = torch.randn((t, heads, d), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
        slots = torch.arange(1000, 1000 + t, dtype=torch.int32, device="cuda")

        def call(kv=kv, slots=slots):
            mxs.mxfp4_kv_append(kv, slots, codes, scales)
        us = _graph_call_ms(torch, call, reps) * 1e3
        byts = t * heads * (2 * d + d // 2 + d // 32)
        out[f"t{t}"] = {"us": round(us, 2), "GBps": round(byts / (us * 1e-6) / 1e9, 1)}
    return out


def kv_attention(torch, mxs, gen, reps=10):
    """mxfp4_kv_attention of the 8B-class verification pass (32 query heads on 8 KV heads of 128,
    T = 5 positions with the chain mask) over MX-FP4 caches of 4096 and 32768 committed entries,
    one sequence and 16; a pool of layers (> 512 MB of cache) is visited in turn so the caches come
    from HBM. GB/s = cache bytes read (codes + scales of K and V over ctx + T entries) + q + out."""
    hq, hkv, d, t = 32, 8, 128, 5
    out = {}
    for b, ctx in ((1, 4096), (1, 32768), (16, 4096)):
        cap = ctx + t
        layer_b = 2 * b * cap * hkv * (d // 2 + d // 32)
        n_layers = max(2, math.ceil(512e6 / layer_b))
        pool = []
        for _ in range(n_layers):
            kc = torch.randint(0, 256, (b, cap, hkv, d // 2), generator=gen, device="cuda", dtype=torch.uint8)
            vc = torch.randint(0, 256, (b, cap, hkv, d // 2), generator=gen, device="cuda", dtype=torch.uint8)
            ks = torch.randint(122, 128, (b, cap, hkv, d // 32), generator=gen, device="cuda", dtype=torch.uint8)
            vs = torch.randint(122, 128, (b, cap, hkv, d // 32), generator=gen, device="cuda", dtype=torch.uint8)
            pool.append((kc, ks, vc, vs))
        q = torch.randn((b, t, hq, d), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
        ctx_len = torch.full((b,), ctx, dtype=torch.int32, device="cuda")
        o = torch.empty((b, t, hq, d), dtype=torch.float32, device="cuda")
        ws = torch.empty((mxs.mxfp4_kv_attention_workspace_bytes(b, t, hq, hkv, cap),), dtype=torch.uint8,
                         device="cuda")
        masks = mxs.chain_masks(t)

        def body(pool=pool, q=q, ctx_len=ctx_len, o=o, ws=ws):
            for (kc, ks, vc, vs) in pool:
                mxs.mxfp4_kv_attention(q, kc, ks, vc, vs, ctx_len, masks, out=o, workspace=ws)
        us = _graph_ms(torch, body, reps) * 1e3 / n_layers
        byts = layer_b + b * t * hq * d * (2 + 4)
        out[f"B{b}_ctx{ctx}"] = {"us": round(us, 2), "GBps": round(byts / (us * 1e-6) / 1e9, 1),
                                 "pct_of_hbm_peak": round(100 * byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 2),
                                 "cache_bytes": layer_b, "pool_layers": n_layers}
        del pool
    out["note"] = "T = 5 chain masks, 32 query heads on 8 KV heads of 128 (one layer's attention per call)"
    return out


def nv_bytes(n, k):
    """NVFP4 weight bytes: 4-bit codes + one E4M3 byte per 16 values (the fp32 tensor scale aside)."""
    return n * k // 2 + n * k // 16


def nvfp4_8b(torch, mxs, gen, pool_gb=2.4, reps=3):
    """NVFP4 weights through the same skinny kernel: the 8B-class layer at T = 1, 5, 8 in the four
    launches of the MX-FP4 headline (q|k|v and gate|up grouped), over a cold pool of > 2 GB."""
    layer_b = sum(nv_bytes(n, k) for _, n, k in LAYER)
    n_layers = max(1, math.ceil(pool_gb * 1e9 / layer_b))
    pool = []
    for _ in range(n_layers):
        mats = []
        for _, n, k in LAYER:
            w = torch.randn((n, k), generator=gen, device="cuda", dtype=torch.float32) * 0.02
            c, sc, g = mxs.nvfp4_quantize(w)
            del w
            # codes tiled once (weight prep); the E4M3 scales stay in the row layout
            mats.append((mxs.mxfp4_tile_codes(c), sc, g, n))
            del c
        pool.append(mats)
    out = {"pool_layers": n_layers, "pool_bytes": layer_b * n_layers,
           "launches": "q|k|v and gate|up grouped, o and down single (nvfp4_verify_gemm_grouped_tiled: "
                       "codes tiled by mxfp4_tile_codes, scales in the row layout)"}
    for t in (1, 5, 8):
        xs = [_rand_bf16(torch, gen, t, k) for (_, _, k) in LAYER]
        ys = [torch.empty((t, n), dtype=torch.float32, device="cuda") for (_, n, _) in LAYER]
        row = {}
        for name, idx in LAUNCHES:
            def body(idx=idx):
                for li in range(n_layers):
                    mxs.nvfp4_verify_gemm_grouped_tiled([(*pool[li][i], xs[i]) for i in idx],
                                                        ys=[ys[i] for i in idx])
            us = _graph_ms(torch, body, reps) * 1e3 / n_layers
            byts = sum(nv_bytes(LAYER[i][1], LAYER[i][2]) + t * LAYER[i][2] * 2 + t * LAYER[i][1] * 4 for i in idx)
            row[name] = {"us": round(us, 2), "GBps": round(byts / (us * 1e-6) / 1e9, 1)}
        tot_b = sum(nv_bytes(n, k) + t * k * 2 + t * n * 4 for _, n, k in LAYER)
        tot_us = sum(v["us"] for v in row.values())
        row["layer_us"] = round(tot_us, 2)
        row["layer_GBps"] = round(tot_b / (tot_us * 1e-6) / 1e9, 1)
        row["layer_pct_of_hbm_peak"] = round(100 * tot_b / (tot_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 2)
        out[f"T{t}"] = row
        del xs, ys
    del pool
    return out


def _overlap(torch, p_logits, q_logits):
    p = torch.softmax(p_logits.double(), -1)
    q = torch.softmax(q_logits.double(), -1)
    return float(torch.minimum(p, q).sum())


def full_8b_step(torch, mxs, gen, steps=10, trials=4096):
    """32 decoder layers + lm_head 128256x4096 at T=5 (tiled weights), then spec_accept on the lm_head output.

    Draft rows i < 4 are target row i + lam_i * N(0,1), with lam_i bisected (fp64, torch,
    outside the timed region) so the per-position acceptance alpha = sum_x min(p, q)
    hits each of 0.6 / 0.8 / 0.9; the GPU acceptance over `trials` cycles gives the
    measured tokens per step, compared with the closed form (1 - a^(K+1)) / (1 - a).
    """
    layers = []
    for li in range(32):
        layers.append([_tile(mxs, *_gpu_mx(torch, mxs, gen, n, k), _rand_bf16(torch, gen, T, k))
                       for (_, n, k) in LAYER])
    lm = _tile(mxs, *_gpu_mx(torch, mxs, gen, V, 4096), _rand_bf16(torch, gen, T, 4096))
    ys = [torch.empty((T, n), dtype=torch.float32, device="cuda") for (_, n, _) in LAYER]
    y_lm = torch.empty((1, T, V), dtype=torch.float32, device="cuda")
    model_bytes = 32 * sum(mx_bytes(n, k) for _, n, k in LAYER) + mx_bytes(V, 4096)
    step_bytes = 32 * sum(gemm_alg_bytes(n, k, T) for _, n, k in LAYER) + gemm_alg_bytes(V, 4096, T)

    def gemms():
        for mats in layers:
            for _, idx in LAUNCHES:
                _gemm(mxs, [mats[i] for i in idx], [ys[i] for i in idx])
        _gemm(mxs, [lm], [y_lm.view(T, V)])
    gemms()
    torch.cuda.synchronize()
    # The lm_head output [1, T, V] is the target law of spec_accept (its rows are the
    # T = K+1 positions); the graph recomputes it each step from the same inputs.
    tgt = y_lm
    tgt_rows = y_lm[0].clone()
    noise = torch.randn((KD, V), generator=gen, device="cuda", dtype=torch.float32)
    result = {"per_alpha": {}}
    ws = torch.empty((mxs.spec_accept_workspace_bytes(1, KD, V),), dtype=torch.uint8, device="cuda")
    ot = torch.empty((1, KD + 1), dtype=torch.int32, device="cuda")
    on = torch.empty((1,), dtype=torch.int32, device="cuda")
    for alpha in (0.6, 0.8, 0.9):
        lams = []
        for i in range(KD):
            lo, hi = 0.0, 64.0
            for _ in range(60):
                mid = 0.5 * (lo + hi)
                if _overlap(torch, tgt_rows[i], tgt_rows[i] + mid * noise[i]) > alpha:
                    lo = mid
                else:
                    hi = mid
            lams.append(0.5 * (lo + hi))
        dft = torch.stack([tgt_rows[i] + lams[i] * noise[i] for i in range(KD)]).unsqueeze(0).contiguous()
        alphas = [_overlap(torch, tgt_rows[i], dft[0, i]) for i in range(KD)]
        # the timed step: all GEMMs, then spec_accept reading the lm_head output buffer
        tok = torch.multinomial(torch.softmax(dft[0].double(), -1), 1, generator=gen).reshape(1, KD).to(torch.int32)
        u = torch.rand((1, KD + 1), generator=gen, device="cuda", dtype=torch.float32)

        def step():
            gemms()
            mxs.spec_accept(tgt, dft, tok, u, out_tokens=ot, out_num=on, workspace=ws)
        ms = _graph_ms(torch, step, steps)
        # acceptance statistics over many cycles (batched, fresh draft tokens and uniforms)
        bt = 512
        tgt_b = tgt_rows.unsqueeze(0).expand(bt, KD + 1, V).contiguous()
        dft_b = dft.expand(bt, KD, V).contiguous()
        wsb = torch.empty((mxs.spec_accept_workspace_bytes(bt, KD, V),), dtype=torch.uint8, device="cuda")
        qd = torch.softmax(dft[0].double(), -1)
        emitted = []
        for _ in range(trials // bt):
            tk = torch.multinomial(qd, bt, replacement=True, generator=gen).t().contiguous().to(torch.int32)
            ub = torch.rand((bt, KD + 1), generator=gen, device="cuda", dtype=torch.float32)
            _, nb = mxs.spec_accept(tgt_b, dft_b, tk, ub, workspace=wsb)
            emitted.append((nb + 1).double())
        em = torch.cat(emitted)
        e_closed = (1 - alpha ** (KD + 1)) / (1 - alpha)
        e_meas = float(em.mean())
        se = float(em.std()) / math.sqrt(em.numel())
        steps_per_s = 1e3 / ms
        result["per_alpha"][str(alpha)] = {
            "alpha_rows": [round(a, 5) for a in alphas],
            "E_closed_form": round(e_closed, 4), "E_measured_gpu": round(e_meas, 4),
            "E_z": round((e_meas - e_closed) / se, 2), "trials": int(em.numel()),
            "step_us": round(ms * 1e3, 1), "steps_per_s": round(steps_per_s, 1),
            "tokens_per_s_equivalent": round(e_closed * steps_per_s, 1)}
        del tgt_b, dft_b, wsb
    ms0 = min(v["step_us"] for v in result["per_alpha"].values()) * 1e-3
    result.update({"model_bytes": model_bytes, "gemm_launches_per_step": 32 * len(LAUNCHES) + 1,
                   "step_GBps": round(step_bytes / (ms0 * 1e-3) / 1e9, 1),
                   "step_pct_of_hbm_peak": round(100 * step_bytes / (ms0 * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2)})
    del layers
    return result


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--pool-gb", type=float, default=4.6)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the secondary workloads (T sweep, 70B shapes, batched, full 8B step)")
    ap.add_argument("--only", choices=["headline", "t_sweep_8b", "shapes_70b_t5", "batched_64x5", "sampled_accept",
                                       "nvfp4_8b", "tree_accept", "kv_append", "kv_attention", "full_8b_step"],
                    help="run one workload alone (profiling); 'headline' = the default line without "
                         "the secondary workloads")
    ap.add_argument("--seed", type=int, default=2)
    ap.add_argument("--layout", choices=["tiled", "row"], default="tiled",
                    help="weight byte order of the headline: tiled (mxfp4_tile_codes / mxfp4_tile_scales, "
                         "done once at weight-prep time) or the mxfp4_quantize row layout")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarize two rocprofv3 --pmc runs into the committed traffic file")
    ap.add_argument("--summarize-busy", nargs=4, metavar=("PMC_DIR", "OUT_MD", "TITLE", "COMMAND"),
                    help="summarize a rocprofv3 --pmc run of VALUBusy / MfmaUtil into a markdown table")
    ap.add_argument("--summarize-trace", nargs=4, metavar=("TRACE_DIR", "OUT_MD", "TITLE", "COMMAND"),
                    help="summarize a rocprofv3 --kernel-trace --stats run into a markdown table")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.summarize_busy:
        summarize_busy(*args.summarize_busy)
        return

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
    # the same weights permuted once into the tiled layouts (for these shapes the same bytes)
    tpool = [[(mxs.mxfp4_tile_codes(c), mxs.mxfp4_tile_scales(s), n, x)
              for (c, s, x), (_, n, _) in zip(mats, LAYER)] for mats in pool]

    def run_launch(li, idx, st, layout):
        """One launch of layer li: the products idx (one, or several sharing the input)."""
        if layout == "tiled":
            tm = tpool[li]
            if len(idx) == 1:
                tc, ts, n, x = tm[idx[0]]
                mxs.mxfp4_verify_gemm_tiled(tc, ts, n, x.shape[1], x, y=ys[idx[0]], stream=st)
            else:
                mxs.mxfp4_verify_gemm_grouped_tiled([tm[i] for i in idx], ys=[ys[i] for i in idx], stream=st)
        else:
            mats = pool[li]
            if len(idx) == 1:
                codes, scales, x = mats[idx[0]]
                mxs.mxfp4_verify_gemm(codes, scales, x, y=ys[idx[0]], stream=st)
            else:
                mxs.mxfp4_verify_gemm_grouped([mats[i] for i in idx], ys=[ys[i] for i in idx], stream=st)

    gen2 = torch.Generator(device=dev)
    gen2.manual_seed(args.seed * 7919 + 17)
    extras = (("t_sweep_8b", lambda: t_sweep(torch, mxs, tpool, gen2)),
              ("shapes_70b_t5", lambda: shapes_70b(torch, mxs, synth, gen2)),
              ("batched_64x5", lambda: batched(torch, mxs, gen2)),
              ("sampled_accept", lambda: sampled_accept(torch, mxs, gen2)),
              ("nvfp4_8b", lambda: nvfp4_8b(torch, mxs, gen2)),
              ("tree_accept", lambda: tree_accept(torch, mxs, gen2)),
              ("kv_append", lambda: kv_append(torch, mxs, gen2)),
              ("kv_attention", lambda: kv_attention(torch, mxs, gen2)),
              ("full_8b_step", lambda: full_8b_step(torch, mxs, gen2)))
    if args.calib_copy_mb:
        # a plain elementwise kernel that reads and writes exactly this many bytes
        src = torch.ones((args.calib_copy_mb << 20) // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    if args.only and args.only != "headline":
        # one secondary workload alone (for per-workload profiles)
        res = dict(extras)[args.only]()
        torch.cuda.synchronize()
        print(json.dumps({"only": args.only, args.only: res}), flush=True)
        return

    tgt, dft, tok, u = synth.accept_batch(2, 1, KD, V, 3.0, 1.0, seq0=0)
    d_tgt, d_dft = torch.from_numpy(tgt).to(dev), torch.from_numpy(dft).to(dev)
    d_tok, d_u = torch.from_numpy(tok).to(dev), torch.from_numpy(u).to(dev)
    out_tok = torch.empty((1, KD + 1), dtype=torch.int32, device=dev)
    out_n = torch.empty((1,), dtype=torch.int32, device=dev)
    ws = torch.empty((mxs.spec_accept_workspace_bytes(1, KD, V),), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(s):
        """One layer: [q | k | v] -> o -> [gate | up] -> down (grouped launches), then spec_accept.

        All launches go on the current stream (cross-stream joins inside a graph
        cost more than the overlap gains on this stack).
        """
        st = torch.cuda.current_stream()
        for _, idx in LAUNCHES:
            run_launch(s % n_layers, idx, st, args.layout)
        mxs.spec_accept(d_tgt, d_dft, d_tok, d_u, out_tokens=out_tok, out_num=out_n, workspace=ws,
                        stream=st)

    # eager warmup, then one HIP graph per pool layer (a graph replays one whole step)
    for s in range(max(args.warmup, n_layers)):
        step(s)
    torch.cuda.synchronize()
    graphs = []
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    for li in range(n_layers):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            step(li)
        graphs.append(g)
    torch.cuda.synchronize()
    # Graphs of STEPS_PER_GRAPH consecutive steps (pool layers i .. i + G - 1, each followed by
    # its spec_accept), as a decoding step replays one graph for the whole forward pass: a graph
    # per single step adds one inter-graph gap per step that a forward pass does not have.
    G = min(STEPS_PER_GRAPH, n_layers)
    group_graphs = []
    for gi in range(0, n_layers - G + 1, G):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for li in range(gi, gi + G):
                step(li)
        group_graphs.append(g)
    torch.cuda.synchronize()
    for s in range(args.warmup):
        graphs[s % n_layers].replay()
    torch.cuda.synchronize()

    def timed_steps(grouped):
        """Wall seconds for exactly args.steps steps after the warmup: whole groups of G steps
        from the grouped graphs, the rest from single-step graphs (grouped=False: all single)."""
        s = args.warmup
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        left = args.steps
        if grouped:
            while left >= G:
                group_graphs[(s // G) % len(group_graphs)].replay()
                s += G
                left -= G
        for _ in range(left):
            graphs[s % n_layers].replay()
            s += 1
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    # timed region: K steps, G per graph replay; then the same K steps one graph per step
    wall = timed_steps(True)
    wall_single = timed_steps(False)

    # Kernel durations: for each launch type one graph that runs it on every pool
    # layer back to back (cold weights, no host gaps between kernels), bracketed by
    # two events on the replay stream; the same for spec_accept alone.
    def launch(j, li, layout=args.layout):
        run_launch(li, LAUNCHES[j][1], torch.cuda.current_stream(), layout)

    def accept_only():
        mxs.spec_accept(d_tgt, d_dft, d_tok, d_u, out_tokens=out_tok, out_num=out_n, workspace=ws,
                        stream=torch.cuda.current_stream())

    type_graphs = []
    for j in range(len(LAUNCHES)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for li in range(n_layers):
                launch(j, li)
        type_graphs.append(g)
    acc_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(acc_graph, stream=cap):
        for _ in range(n_layers):
            accept_only()
    torch.cuda.synchronize()
    reps = max(20, args.steps // n_layers)
    mk = lambda: torch.cuda.Event(enable_timing=True)

    def time_graph(g, dist=None):
        """Mean ms per launch over `reps` replays of g (each runs the launch on every pool layer);
        each replay is bracketed by its own events, so the per-replay means (ms per launch) go to
        `dist` for the median and p10 / p90."""
        g.replay()
        torch.cuda.synchronize()
        st = torch.cuda.current_stream()
        ev = [mk() for _ in range(reps + 1)]
        ev[0].record(st)
        for r in range(reps):
            g.replay()
            ev[r + 1].record(st)
        torch.cuda.synchronize()
        per = [ev[r].elapsed_time(ev[r + 1]) / n_layers for r in range(reps)]
        if dist is not None:
            dist.extend(per)
        return ev[0].elapsed_time(ev[reps]) / (reps * n_layers)  # ms per launch

    clocks_before = gpu_clocks()
    stream = stream_ceiling(torch, mxs)
    launch_dist = [[] for _ in type_graphs]
    launch_ms = [time_graph(g, d) for g, d in zip(type_graphs, launch_dist)]
    acc_ms_mean = time_graph(acc_graph)
    clocks_after = gpu_clocks()
    del type_graphs
    # the other layout's launches for comparison (not in the single-workload runs that
    # profiles and counters are taken from)
    other = "row" if args.layout == "tiled" else "tiled"
    other_ms = None
    if not args.only:
        other_ms = []
        for j in range(len(LAUNCHES)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                for li in range(n_layers):
                    launch(j, li, other)
            torch.cuda.synchronize()
            other_ms.append(time_graph(g))
            del g

    step_gemm_bytes = sum(gemm_alg_bytes(n, k, T) for _, n, k in LAYER)
    value = step_gemm_bytes * args.steps / wall / 1e9
    launches = reps * n_layers * len(LAUNCHES)
    avg_launch_ms = float(np.mean(launch_ms))
    avg_launch_bytes = step_gemm_bytes / len(LAUNCHES)
    achieved = avg_launch_bytes / (avg_launch_ms * 1e-3) / 1e9
    launch_bytes = [sum(gemm_alg_bytes(LAYER[i][1], LAYER[i][2], T) for i in idx) for _, idx in LAUNCHES]
    per_shape = {}
    for j, ((name, _), b) in enumerate(zip(LAUNCHES, launch_bytes)):
        q = pctl(launch_dist[j])
        per_shape[name] = {"GBps": round(b / (launch_ms[j] * 1e-3) / 1e9, 1), "us": round(launch_ms[j] * 1e3, 2),
                           "us_median": round(q["median"] * 1e3, 2), "us_p10": round(q["p10"] * 1e3, 2),
                           "us_p90": round(q["p90"] * 1e3, 2), "replays": q["n"]}
    # the per-replay distribution of the four-launch average (one replay of each launch type)
    avg_dist = [sum(t) / len(t) for t in zip(*launch_dist)]
    avg_q = pctl(avg_dist)
    traffic = load_traffic()
    result = {
        "metric": "MX-FP4 verify-GEMM HBM GB/s (% of peak) at T=5; spec_accept positions/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "steps_per_graph": G,
        "ms_per_step_one_graph_per_step": round(wall_single / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "8B-class layer shapes at T=5: q,o 4096x4096; k,v 1024x4096; gate,up 14336x4096; "
                        "down 4096x14336 (MX-FP4 weights, bf16 activations, fp32 out) + spec_accept "
                        "B=1 K=4 V=128256",
            "T": T, "K_draft": KD, "vocab": V, "weight_layout": args.layout,
            "pool_layers": n_layers, "pool_bytes": layer_bytes * n_layers,
            "gemm_bytes_per_step": step_gemm_bytes,
            "parallelism": "single GPU",
        },
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "gemm_launches": per_shape,
        "weight_layout": args.layout,
        f"gemm_launches_{other}_layout": None if other_ms is None else {
            name: {"us": round(other_ms[j] * 1e3, 2), "GBps": round(b / (other_ms[j] * 1e-3) / 1e9, 1)}
            for j, ((name, _), b) in enumerate(zip(LAUNCHES, launch_bytes))},
        "spec_accept_positions_per_s": round((KD + 1) / (acc_ms_mean * 1e-3), 1),
        "spec_accept_us": round(acc_ms_mean * 1e3, 2),
        "numerics": "E2M1 weights decoded exactly to bf16, bf16 x bf16 products summed in fp32 (MFMA); "
                    "spec_accept probabilities in fp64",
        "roofline": {
            "kernel": ("gemm_skinny_kernel<1, 4, 2, false, false, true, true> (mxfp4_verify_gemm_tiled / "
                       "mxfp4_verify_gemm_grouped_tiled: tiled weight codes and scales)") if args.layout == "tiled"
                      else "gemm_skinny_kernel<1, 4, 2, false, false, false> (mxfp4_verify_gemm / _grouped)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "frac_of_stream_ceiling": round(achieved / stream["GBps_median"], 4),
            "traffic": traffic,
            "avg_launch_us": round(avg_launch_ms * 1e3, 3),
            "avg_launch_us_median": round(avg_q["median"] * 1e3, 3),
            "avg_launch_us_p10": round(avg_q["p10"] * 1e3, 3),
            "avg_launch_us_p90": round(avg_q["p90"] * 1e3, 3),
            "replays_per_launch_type": avg_q["n"],
            "avg_launch_alg_bytes": avg_launch_bytes,
            "launches_timed": int(launches),
            "timing": "HIP events around graph replays that run one launch type on every pool "
                      "layer back to back; average over the four launch types of a layer (mean over "
                      "all replays; median / p10 / p90 over the per-replay averages)",
        },
        "gpu_clocks": {"before": clocks_before, "after": clocks_after},
        "stream_ceiling": stream,
    }
    if not args.no_extra and not args.only:
        for key, fn in extras:
            print(f"# workload {key}", file=sys.stderr, flush=True)
            result[key] = fn()
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline()
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
