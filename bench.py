#!/usr/bin/env python3
"""Throughput of the dequant-fused projection matmul on one MI355X.

A step is one pass of the LFM2.5-350M-shaped 512-token prefill: the four
projection shapes (ffn_gate 4608x1024, ffn_down 1024x4608, conv_in 3072x1024,
attn_out 1024x1024; shapes of cera wgpu_gemm_bench.rs, SHAPES) in each of the
five weight formats (f32, q4_0, q8_0, q4_k, q6_k) = 20 GEMMs with n = 512,
all on the f16 matrix-core path.  `value` is TFLOP/s (2*m*k*n per GEMM) over
the K timed steps, inputs resident in HBM.

The same JSON line also carries the other half of the metric, decode GEMV
HBM GB/s at n = 1 (q4_k and q6_k, 14336x4096 and 4608x1024, weight copies
rotated over >= 1 GiB so every read comes from HBM), the NVFP4 MoE gate/up at
t = 1 and t = 16, the load-only twin's GB/s on the decode shapes, the roofline
of the dominant kernel (HIP events around every launch in the timed region)
and the CPU oracle timed on the host cores.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--quick]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_F16_TFLOPS = 2516.6   # MI355X dense f16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
SHAPES = [("ffn_gate", 4608, 1024), ("ffn_down", 1024, 4608), ("conv_in", 3072, 1024),
          ("attn_out", 1024, 1024)]
QTS = ["f32", "q4_0", "q8_0", "q4_k", "q6_k"]
KERNEL_NAME = {"gemm": "gemm_mfma_kernel", "gemv": "gemv_kernel", "moe": "moe_gateup_kernel"}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gemv_prefill_decode_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel: str):
    """HBM bytes per launch from committed rocprofv3 PMC summaries, only if
    they were taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            tab = json.load(f)
    except (OSError, ValueError):
        return None
    ent = tab.get(kernel)
    if not ent or ent.get("source_hash") != kernel_source_hash():
        return None
    return ent.get("bytes_per_launch")


def gen_weights(qt, m, k, buf_id):
    from synth import gen
    import gemv_prefill_decode_amd as qmm
    if qt == "f32":
        return gen.dense_weights(m * k, True, buf_id)
    if qt == "nvfp4":
        return gen.nvfp4_rows(m, k, gen.SEED_MOE_W + buf_id)
    return gen.dense_weights(m * qmm.row_bytes(qt, k), False, buf_id)


def to_dev(a):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


# ---------------------------------------------------------------- prefill step

def prefill_setup(n):
    from synth import gen
    import torch
    bufs = []
    xs = {}
    outs = {}
    for si, (label, m, k) in enumerate(SHAPES):
        if k not in xs:
            xs[k] = to_dev(gen.unit_f32(n * k, gen.SEED_X + k).reshape(n, k))
        outs[label] = torch.empty((n, m), dtype=torch.float32, device="cuda")
    for qi, qt in enumerate(QTS):
        for si, (label, m, k) in enumerate(SHAPES):
            w = to_dev(gen_weights(qt, m, k, 16 * qi + si))
            bufs.append((qt, label, m, k, w))
    return bufs, xs, outs


def prefill_step(bufs, xs, outs, events=None):
    import gemv_prefill_decode_amd as qmm
    for i, (qt, label, m, k, w) in enumerate(bufs):
        if events is not None:
            events[i][0].record()
        qmm.gemm(w, xs[k], m, qt, out=outs[label], path="mfma")
        if events is not None:
            events[i][1].record()


def run_prefill(args, n):
    import torch
    bufs, xs, outs = prefill_setup(n)
    flops = [2.0 * m * k * n for (_, _, m, k, _) in bufs]
    step_flops = sum(flops)
    for _ in range(args.warmup):
        prefill_step(bufs, xs, outs)
    torch.cuda.synchronize()
    # timed region: K steps, events around every launch on the launch stream
    ev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
           for _ in bufs] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        prefill_step(bufs, xs, outs, ev[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_launch = [[ev[s][i][0].elapsed_time(ev[s][i][1]) * 1e-3 for s in range(args.steps)]
                  for i in range(len(bufs))]
    # per-qtype aggregates
    per_qt = {}
    for i, (qt, label, m, k, _) in enumerate(bufs):
        d = per_qt.setdefault(qt, {"flops": 0.0, "sec": 0.0, "launches": 0, "shapes": {}})
        t = statistics.median(per_launch[i])
        d["flops"] += flops[i]
        d["sec"] += sum(per_launch[i]) / args.steps
        d["launches"] += 1
        d["shapes"][label] = {"us": round(t * 1e6, 2), "TFLOP/s": round(flops[i] / t / 1e12, 1)}
    for qt, d in per_qt.items():
        d["TFLOP/s"] = round(d["flops"] / d["sec"] / 1e12, 1)
        d["frac_mfma_peak"] = round(d["flops"] / d["sec"] / 1e12 / PEAK_F16_TFLOPS, 4)
    dom = max(per_qt, key=lambda q: per_qt[q]["sec"])
    d = per_qt[dom]
    avg_launch = d["sec"] / d["launches"]
    flops_per_launch = d["flops"] / d["launches"]
    ach = flops_per_launch / avg_launch / 1e12
    roofline = {
        "kernel": f"{KERNEL_NAME['gemm']}<{dom}>",
        "bound": "mfma",
        "achieved": round(ach, 2),
        "peak": PEAK_F16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(ach / PEAK_F16_TFLOPS, 4),
        "avg_launch_us": round(avg_launch * 1e6, 3),
        "algorithmic_flops_per_launch": flops_per_launch,
        "traffic": traffic_from_profiles(f"gemm_mfma<{dom}>"),
    }
    for qt in per_qt:
        per_qt[qt].pop("flops"); per_qt[qt].pop("sec"); per_qt[qt].pop("launches")
    return step_flops, wall, per_qt, roofline, bufs, xs


# ---------------------------------------------------------------- decode GEMV

def run_decode(args):
    import torch
    import gemv_prefill_decode_amd as qmm
    from synth import gen
    res = {}
    shapes = [(14336, 4096), (4608, 1024)]
    for qt in ("q4_k", "q6_k"):
        for (m, k) in shapes:
            wbytes = m * qmm.row_bytes(qt, k)
            copies = max(4, -(-(1 << 30) // wbytes))
            if args.quick:
                copies = max(4, copies // 8)
            base = to_dev(gen_weights(qt, m, k, 99))
            ws = []
            for c in range(copies):       # clone-and-perturb one payload byte per copy
                w = base.clone()
                w[5] ^= (c * 16 + 1) & 0xFF
                ws.append(w)
            x = to_dev(gen.unit_f32(k, gen.SEED_X))
            x = x.view(1, k)
            out = torch.empty((1, m), dtype=torch.float32, device="cuda")
            sink = torch.empty(m, dtype=torch.int32, device="cuda")
            reps = args.decode_reps
            for i in range(min(copies, 20)):
                qmm.gemm(ws[i], x, m, qt, out=out, path="gemv")
            torch.cuda.synchronize()

            def timed(fn):
                evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                       for _ in range(reps)]
                for r in range(reps):
                    evs[r][0].record()
                    fn(ws[r % copies])
                    evs[r][1].record()
                torch.cuda.synchronize()
                return statistics.median(a.elapsed_time(b) * 1e-3 for a, b in evs)
            t = timed(lambda w: qmm.gemm(w, x, m, qt, out=out, path="gemv"))
            tl = timed(lambda w: qmm.stream_loadonly(w, m, k, qt, sink=sink))
            alg = wbytes + 4 * k + 4 * m
            res[f"{qt}_{m}x{k}"] = {
                "us": round(t * 1e6, 2),
                "GB/s": round(alg / t / 1e9, 1),
                "frac_hbm_peak": round(alg / t / 1e9 / PEAK_HBM_GBS, 4),
                "weight_GB/s": round(wbytes / t / 1e9, 1),
                "loadonly_us": round(tl * 1e6, 2),
                "loadonly_GB/s": round(wbytes / tl / 1e9, 1),
                "copies": copies,
                "footprint_MiB": round(copies * wbytes / 2**20),
            }
            del ws, base
            torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------- MoE gate/up

def run_moe(args):
    import numpy as np
    import torch
    import gemv_prefill_decode_amd as qmm
    from synth import gen
    n_expert, in_f, n_ff, n_used = 64, 4096, 2048, 8
    rb = qmm.row_bytes("nvfp4", in_f)
    per_e = n_ff * rb
    planes = []
    for plane in range(2):
        host = np.empty(n_expert * per_e, dtype=np.uint8)
        for e in range(n_expert):
            host[e * per_e:(e + 1) * per_e] = gen.nvfp4_rows(n_ff, in_f, gen.SEED_MOE_W + 2 * e + plane)
        planes.append(to_dev(host))
    copies = 2 if args.quick else 4
    sets = []
    for c in range(copies):
        g = planes[0].clone(); u = planes[1].clone()
        for e in range(n_expert):           # perturb one payload byte of every expert slab
            g[e * per_e + 5] ^= (c * 16 + 1) & 0xFF
            u[e * per_e + 5] ^= (c * 16 + 2) & 0xFF
        sets.append((g, u))
    del planes
    res = {}
    for t in (1, 16):
        n_pairs = t * n_used
        draws = [to_dev(gen.expert_ids(t, n_used, n_expert, gen.SEED_EXPERTS + d)) for d in range(8)]
        sc = to_dev(gen.pair_scales(2 * n_pairs))
        x = to_dev(gen.xorshift_f32(t * in_f, gen.SEED_MOE_X).reshape(t, in_f))
        go = torch.empty((n_pairs, n_ff), dtype=torch.float32, device="cuda")
        uo = torch.empty((n_pairs, n_ff), dtype=torch.float32, device="cuda")
        uniq = [len(np.unique(gen.expert_ids(t, n_used, n_expert, gen.SEED_EXPERTS + d))) for d in range(8)]
        for i in range(10):
            qmm.moe_gateup(sets[i % copies][0], sets[i % copies][1], draws[i % 8], sc, x, n_expert,
                           n_ff, gate_out=go, up_out=uo)
        torch.cuda.synchronize()
        reps = args.moe_reps
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for r in range(reps):
            evs[r][0].record()
            qmm.moe_gateup(sets[r % copies][0], sets[r % copies][1], draws[r % 8], sc, x, n_expert, n_ff,
                           gate_out=go, up_out=uo)
            evs[r][1].record()
        torch.cuda.synchronize()
        times = [a.elapsed_time(b) * 1e-3 for a, b in evs]
        byts = [2 * uniq[r % 8] * per_e + 4 * t * in_f + 2 * 4 * n_pairs * n_ff for r in range(reps)]
        gbs = statistics.median(b / s / 1e9 for b, s in zip(byts, times))
        res[f"t{t}"] = {
            "us": round(statistics.median(times) * 1e6, 2),
            "GB/s": round(gbs, 1),
            "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "unique_experts_mean": round(sum(uniq) / len(uniq), 2),
        }
    return res


# ---------------------------------------------------------------- CPU oracle

def run_cpu_baseline(args, n):
    import numpy as np
    from oracle import ref
    from synth import gen
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        cores = os.cpu_count() or 1
    import gemv_prefill_decode_amd as qmm
    work = []
    for qi, qt in enumerate(QTS):
        for si, (label, m, k) in enumerate(SHAPES):
            w = gen_weights(qt, m, k, 16 * qi + si)
            x = gen.unit_f32(n * k, gen.SEED_X + k).reshape(n, k)
            work.append((qt, m, k, w, x))
    flops = sum(2.0 * m * k * n for (_, m, k, _, _) in work)

    def once():
        t0 = time.perf_counter()
        for (qt, m, k, w, x) in work:
            ref.gemm_value(qt, w, x, m, k, n)
        return time.perf_counter() - t0
    once()
    ts = [once() for _ in range(3)]
    t = statistics.median(ts)
    return {
        "value": round(flops / t / 1e12, 5),
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"the full 20-GEMM prefill step (4 shapes x 5 formats, n={n}): numpy decode to "
                  f"f64 + f64 matmul (OpenBLAS); median of 3 after 1 warm-up, {t:.2f} s per step",
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--n", type=int, default=512, help="prefill tokens (default 512)")
    ap.add_argument("--decode-reps", type=int, default=200)
    ap.add_argument("--moe-reps", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the decode and MoE measurements")
    ap.add_argument("--quick", action="store_true", help="fewer rotation copies")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import gemv_prefill_decode_amd as qmm
    qmm.load()
    n = args.n
    log(f"prefill step: {len(SHAPES)} shapes x {len(QTS)} formats, n={n}, warmup={args.warmup} steps={args.steps}")
    step_flops, wall, per_qt, roofline, _, _ = run_prefill(args, n)
    value = step_flops * args.steps / wall / 1e12
    log(f"prefill: {value:.1f} TFLOP/s, {wall / args.steps * 1e3:.3f} ms/step")
    extras = {}
    if not args.no_extras:
        log("decode GEMV n=1 with rotation")
        extras["decode_n1"] = run_decode(args)
        log("MoE gate/up NVFP4")
        extras["moe_gateup"] = run_moe(args)
    cpu = None
    if not args.no_cpu_baseline:
        log("CPU oracle baseline")
        cpu = run_cpu_baseline(args, n)
    line = {
        "metric": "TFLOP/s (prefill n=512) and HBM GB/s (decode n=1) per qtype, % of roofline",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16-mfma/f32-acc",
        "data": "synthetic (seeded LCG packed weights and uniform[-1,1) activations)",
        "config": {"workload": "LFM2.5-350M-shaped prefill n=512: ffn_gate 4608x1024, ffn_down 1024x4608, "
                               "conv_in 3072x1024, attn_out 1024x1024 in f32/q4_0/q8_0/q4_k/q6_k",
                   "n": n, "gemms_per_step": len(SHAPES) * len(QTS)},
        "per_qtype": per_qt,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    line.update(extras)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
