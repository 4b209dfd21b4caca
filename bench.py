#!/usr/bin/env python3
"""Throughput of the dequant-fused projection matmul on one MI355X.

A step is one pass of the LFM2.5-350M-shaped 512-token prefill: the four
projection shapes (ffn_gate 4608x1024, ffn_down 1024x4608, conv_in 3072x1024,
attn_out 1024x1024; the SHAPES of cera wgpu_gemm_bench.rs) in each of the
five weight formats (f32, q4_0, q8_0, q4_k, q6_k) = 20 GEMMs with n = 512,
all on the f16 matrix-core path.  Each format's four calls (with their f16
pre-pass and k-split sum, where the plan has them) are captured once in a HIP
graph; a timed step replays the five graphs back to back on one stream, with
HIP events between them.  `value` is TFLOP/s (2*m*k*n per GEMM) over the K
timed steps, inputs resident in HBM.

The same JSON line also carries the other half of the metric:
  decode   the GEMV sweep n in {1,4,8,16,32}, q4_k and q6_k at 14336x4096 and
           4608x1024, weight copies rotated over >= 1 GiB so that every read
           comes from HBM; GB/s of algorithmic bytes (packed W + x + dst) and
           TFLOP/s, each against its roof; the load-only twin at n = 1.
  moe      the NVFP4 gate/up rows at t = 1 and t = 16 (64 experts, 8 used,
           in_f 4096, n_ff 2048), rotated over 4 weight copies x 8 id draws,
           and the down projection after it (4096 rows over 2048 inputs per
           expert, per-pair activations, slots summed per token); each also
           on the same values in NVFP4 V2 rows (outputs checked bit-identical
           to V1 before timing); the gate/up also on Q8_1 activations
           (quantization included in the timed launches).
  roofline the dominant format's prefill calls (the largest time per step):
           algorithmic flops per call over the average call time from the
           events of the timed region, with the GEMM kernel instance and grid
           each call runs, and their HBM bytes from the counter profiles.
  cpu_baseline  the CPU oracle over the whole prefill step on the host cores.
Decode and MoE launches are graph-replayed too (32+ launches per graph).

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extras] [--quick]
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
# MI355X f32 vector FMA: 157.3 TFLOP/s needs packed FMA (v_pk_fma_f32), which
# this build disables; the roof of the code built is the unpacked rate
PEAK_F32_TFLOPS = 78.6
PEAK_F32_PACKED_TFLOPS = 157.3
# MI355X f32 matrix cores (v_mfma_f32_*): the roof of the GEMV's matrix-core stream
PEAK_F32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
SHAPES = [("ffn_gate", 4608, 1024), ("ffn_down", 1024, 4608), ("conv_in", 3072, 1024),
          ("attn_out", 1024, 1024)]
QTS = ["f32", "q4_0", "q8_0", "q4_k", "q6_k"]
DECODE_SHAPES = [(14336, 4096), (4608, 1024)]
DECODE_NS = [1, 4, 8, 16, 32]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


CSRC = os.path.join(ROOT, "gemv_prefill_decode_amd", "csrc")


def tu_source_hashes() -> dict:
    """Per kernel translation unit (csrc/*.hip), a hash of its source and of
    every local header it includes, directly or not: the measured traffic of a
    kernel is used only while its own translation unit hashes the same."""
    def includes(path):
        out = []
        for ln in open(path):
            ln = ln.strip()
            if ln.startswith("#include \""):
                out.append(ln.split("\"")[1])
        return out

    hashes = {}
    for tu in sorted(f for f in os.listdir(CSRC) if f.endswith(".hip")):
        seen, todo = set(), [tu]
        while todo:
            f = todo.pop()
            if f in seen or not os.path.exists(os.path.join(CSRC, f)):
                continue
            seen.add(f)
            todo.extend(includes(os.path.join(CSRC, f)))
        h = hashlib.sha256()
        for f in sorted(seen):
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(f.encode() + fh.read())
        hashes[tu] = h.hexdigest()[:16]
    return hashes


def kernel_tu(kernel: str):
    """The translation unit that defines a kernel (by its unqualified name)."""
    base = kernel.replace("qmm::", "").split("<")[0].split("@")[0].strip()
    for tu in sorted(f for f in os.listdir(CSRC) if f.endswith(".hip")):
        src = open(os.path.join(CSRC, tu)).read()
        if f" {base}(" in src and "__global__" in src:
            return tu
    return None


def traffic_from_profiles(kernel: str):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel
    calibration) from profiles/traffic.json, or None if absent or if the
    kernel's translation unit has changed since it was measured."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            tab = json.load(f)
    except (OSError, ValueError):
        return None
    ent = tab.get("kernels", {}).get(kernel)
    if not ent or ent.get("tu") is None:
        return None
    if tab.get("tu_hashes", {}).get(ent["tu"]) != tu_source_hashes().get(ent["tu"]):
        return None
    return ent.get("bytes_per_launch")


def plan_grid_size(plan, m, n):
    """Work-items of the GEMM kernel a qmm_gemm_plan() result launches (the
    Grid_Size the profiler records for that dispatch)."""
    x16, rows, kg, split = plan["x16"], plan["tile_rows"], plan["k_groups"], plan["n_split"]
    cols = 256 if x16 in (3, 7) else 64 if x16 in (5, 6) else 128
    threads = 512 if x16 == 7 else 256 * kg
    groups = -(-m // rows) * -(-n // cols) * split
    return groups * threads


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


def capture(fns):
    """Capture the calls in fns (in order) into one HIP graph."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):          # first calls outside capture (library load, lazy state)
        for f in fns[:2]:
            f()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for f in fns:
            f()
    torch.cuda.synchronize()
    return g


def time_graph(g, launches, rounds):
    """Median seconds per launch over `rounds` replays of g (events on the
    replay stream)."""
    import torch
    g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(rounds):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b) * 1e-3 / launches)
    return statistics.median(ts)


# ---------------------------------------------------------------- prefill step

def run_prefill(args, n):
    import torch
    import gemv_prefill_decode_amd as qmm
    from synth import gen
    xs, outs, bufs = {}, {}, []
    for label, m, k in SHAPES:
        if k not in xs:
            xs[k] = to_dev(gen.unit_f32(n * k, gen.SEED_X + k).reshape(n, k))
        outs[label] = torch.empty((n, m), dtype=torch.float32, device="cuda")
    for qi, qt in enumerate(QTS):
        for si, (label, m, k) in enumerate(SHAPES):
            bufs.append((qt, label, m, k, to_dev(gen_weights(qt, m, k, 16 * qi + si))))

    def call(b):
        qt, label, m, k, w = b
        return lambda: qmm.gemm(w, xs[k], m, qt, out=outs[label], path="mfma")

    graphs = {qt: capture([call(b) for b in bufs if b[0] == qt]) for qt in QTS}
    flops = {qt: sum(2.0 * m * k * n for (q, _, m, k, _) in bufs if q == qt) for qt in QTS}
    step_flops = sum(flops.values())
    for _ in range(args.warmup):
        for qt in QTS:
            graphs[qt].replay()
    torch.cuda.synchronize()
    # per-format times (before the timed region): each format's graph between
    # two events, as many rounds as timed steps
    per_qt = {}
    for qt in QTS:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for s in range(args.steps):
            ev[s][0].record()
            graphs[qt].replay()
            ev[s][1].record()
        torch.cuda.synchronize()
        sec = [a.elapsed_time(b) * 1e-3 for (a, b) in ev]
        mean = sum(sec) / len(sec)
        per_qt[qt] = {"us_per_step": round(mean * 1e6, 2),
                      "TFLOP/s": round(flops[qt] / mean / 1e12, 1),
                      "frac_mfma_peak": round(flops[qt] / mean / 1e12 / PEAK_F16_TFLOPS, 4)}
    # the dominant format (the largest time per step); its four calls, each a
    # GEMM kernel (plus the f16 pre-pass and the k-split sum where planned)
    dom = max(QTS, key=lambda q: per_qt[q]["us_per_step"])
    # A timed step: the other formats' 16 calls as one graph, then the
    # dominant format's graph between two events (its time per call for the
    # roofline).  Every event recorded between graphs costs the stream a few
    # microseconds, so the step records only these two.
    rest = capture([call(b) for b in bufs if b[0] != dom])
    for _ in range(args.warmup):
        rest.replay()
        graphs[dom].replay()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        rest.replay()
        ev[s][0].record()
        graphs[dom].replay()
        ev[s][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dom_sec = sum(a.elapsed_time(b) * 1e-3 for (a, b) in ev) / args.steps
    del rest
    # per-shape times (outside the timed region): each launch graph-replayed alone
    kern = {}
    for (qt, label, m, k, w) in bufs:
        g = capture([call((qt, label, m, k, w))] * 8)
        t = time_graph(g, 8, 5)
        plan = qmm.gemm_plan(m, k, n, qt, "mfma")
        kern[(qt, label)] = (qmm.plan_kernel_name(plan, qt), plan_grid_size(plan, m, n))
        per_qt[qt].setdefault("shapes", {})[label] = {
            "us": round(t * 1e6, 2), "TFLOP/s": round(2.0 * m * k * n / t / 1e12, 1),
            "kernel": kern[(qt, label)][0], "grid": kern[(qt, label)][1], "k_split": plan["n_split"]}
        del g
    calls = [b for b in bufs if b[0] == dom]
    launches = len(calls)
    avg_launch = dom_sec / launches
    fpl = flops[dom] / launches
    ach = fpl / avg_launch / 1e12
    names = [kern[(dom, label)] for (_, label, _, _, _) in calls]
    traffic = [traffic_from_profiles(f"{kn}@{grid}") for (kn, grid) in names]
    roofline = {
        "kernel": " + ".join(f"qmm::{kn} (grid {grid})" for (kn, grid) in names) +
                  f" ({dom} weights, the four LFM2 shapes; per qmm_gemm_ws call)",
        "bound": "mfma",
        "achieved": round(ach, 2),
        "peak": PEAK_F16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(ach / PEAK_F16_TFLOPS, 4),
        # HBM bytes of the GEMM kernels, averaged over the four calls
        "traffic": round(sum(traffic) / launches) if all(t is not None for t in traffic) else None,
        "avg_launch_us": round(avg_launch * 1e6, 3),
        "launches_per_step": launches,
        "algorithmic_flops_per_launch": fpl,
        "algorithmic_bytes_per_launch": sum(
            (m * qmm.row_bytes(q, k) + 4 * n * k + 4 * n * m) for (q, _, m, k, _) in calls) / launches,
    }
    return step_flops, wall, per_qt, roofline


# ---------------------------------------------------------------- decode GEMV

def rotated_copies(base, copies):
    """copies of base, each with one payload byte perturbed (distinct buffers)."""
    ws = []
    for c in range(copies):
        w = base.clone()
        w[5] ^= (c * 16 + 1) & 0xFF
        ws.append(w)
    return ws


def run_decode(args):
    import torch
    import gemv_prefill_decode_amd as qmm
    from synth import gen
    res = {}
    for qt in ("q4_k", "q6_k"):
        for (m, k) in DECODE_SHAPES:
            wbytes = m * qmm.row_bytes(qt, k)
            copies = max(4, -(-(1 << 30) // wbytes))
            if args.quick:
                copies = max(4, copies // 8)
            ws = rotated_copies(to_dev(gen_weights(qt, m, k, 99)), copies)
            L = max(copies, 32)
            ent = {"copies": copies, "footprint_MiB": round(copies * wbytes / 2**20),
                   "weight_bytes": wbytes}
            for n in DECODE_NS:
                x = to_dev(gen.unit_f32(n * k, gen.SEED_X).reshape(n, k))
                out = torch.empty((n, m), dtype=torch.float32, device="cuda")
                g = capture([(lambda w=ws[i % copies]: qmm.gemm(w, x, m, qt, out=out, path="gemv"))
                             for i in range(L)])
                t = time_graph(g, L, 5)
                del g
                alg = wbytes + 4 * n * k + 4 * n * m
                stream = qmm.gemm_plan(m, k, n, qt, "gemv")["stream"]
                roof = PEAK_F32_MFMA_TFLOPS if stream == "matrix" else PEAK_F32_TFLOPS
                ent[f"n{n}"] = {"us": round(t * 1e6, 2),
                                "GB/s": round(alg / t / 1e9, 1),
                                "frac_hbm_peak": round(alg / t / 1e9 / PEAK_HBM_GBS, 4),
                                "TFLOP/s": round(2.0 * m * k * n / t / 1e12, 2),
                                "stream": stream,
                                # f32 products: unpacked FMA (78.6) or f32 matrix cores (157.3)
                                "f32_roof_TFLOP/s": roof,
                                "frac_f32_roof": round(2.0 * m * k * n / t / 1e12 / roof, 4)}
            sink = torch.empty(m, dtype=torch.int32, device="cuda")
            g = capture([(lambda w=ws[i % copies]: qmm.stream_loadonly(w, m, k, qt, sink=sink))
                         for i in range(L)])
            tl = time_graph(g, L, 5)
            del g
            ent["loadonly_us"] = round(tl * 1e6, 2)
            ent["loadonly_GB/s"] = round(wbytes / tl / 1e9, 1)
            res[f"{qt}_{m}x{k}"] = ent
            log(f"decode {qt} {m}x{k}: n=1 {ent['n1']['us']} us {ent['n1']['GB/s']} GB/s; "
                f"load-only {ent['loadonly_us']} us")
            del ws
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
        g = planes[0].clone()
        u = planes[1].clone()
        for e in range(n_expert):           # perturb one payload byte of every expert slab
            g[e * per_e + 5] ^= (c * 16 + 1) & 0xFF
            u[e * per_e + 5] ^= (c * 16 + 2) & 0xFF
        sets.append((g, u))
    del planes
    rows = n_expert * n_ff
    sets_v2 = [(qmm.repack_nvfp4_v2(g, rows, in_f), qmm.repack_nvfp4_v2(u, rows, in_f)) for g, u in sets]
    res = {}
    L = 32
    for t in (1, 16):
        n_pairs = t * n_used
        draws_h = [gen.expert_ids(t, n_used, n_expert, gen.SEED_EXPERTS + d) for d in range(8)]
        draws = [to_dev(d) for d in draws_h]
        uniq = [len(np.unique(d)) for d in draws_h]
        sc = to_dev(gen.pair_scales(2 * n_pairs))
        x = to_dev(gen.xorshift_f32(t * in_f, gen.SEED_MOE_X).reshape(t, in_f))
        go = torch.empty((n_pairs, n_ff), dtype=torch.float32, device="cuda")
        uo = torch.empty((n_pairs, n_ff), dtype=torch.float32, device="cuda")
        g = capture([(lambda c=sets[i % copies], d=draws[i % 8]:
                      qmm.moe_gateup(c[0], c[1], d, sc, x, n_expert, n_ff, gate_out=go, up_out=uo))
                     for i in range(L)])
        tt = time_graph(g, L, 5)
        del g
        byts = statistics.mean(2 * uniq[i % 8] * per_e + 4 * t * in_f + 2 * 4 * n_pairs * n_ff
                               for i in range(L))
        # the same values in NVFP4 V2 rows: bit-identical outputs, then timed
        ref_g, ref_u = qmm.moe_gateup(sets[0][0], sets[0][1], draws[0], sc, x, n_expert, n_ff)
        ref_g, ref_u = ref_g.clone(), ref_u.clone()
        v2_g, v2_u = qmm.moe_gateup(sets_v2[0][0], sets_v2[0][1], draws[0], sc, x, n_expert, n_ff,
                                    "nvfp4_v2")
        if not (torch.equal(ref_g, v2_g) and torch.equal(ref_u, v2_u)):
            raise SystemExit("MoE gate/up: NVFP4 V2 differs from V1")
        g = capture([(lambda c=sets_v2[i % copies], d=draws[i % 8]:
                      qmm.moe_gateup(c[0], c[1], d, sc, x, n_expert, n_ff, "nvfp4_v2", gate_out=go,
                                     up_out=uo))
                     for i in range(L)])
        tv2 = time_graph(g, L, 5)
        del g
        # Q8_1 activations: the quantization once per call, then the gate/up
        xq, xd = qmm.quantize_q8_1(x)
        g = capture([(lambda c=sets[i % copies], d=draws[i % 8]:
                      (qmm.quantize_q8_1(x, q=xq, d=xd),
                       qmm.moe_gateup_q8(c[0], c[1], d, sc, xq, xd, n_expert, n_ff, gate_out=go,
                                         up_out=uo)))
                     for i in range(L)])
        tq8 = time_graph(g, L, 5)
        del g
        # the gate/up fused with the SwiGLU/clamp activation (limit 7.0):
        # the same weight bytes, the act rows written instead of gate and up
        act = torch.empty((n_pairs, n_ff), dtype=torch.float32, device="cuda")
        g = capture([(lambda c=sets[i % copies], d=draws[i % 8]:
                      qmm.moe_gateup_act(c[0], c[1], d, sc, x, n_expert, n_ff, "nvfp4", 7.0, act=act))
                     for i in range(L)])
        tact = time_graph(g, L, 5)
        del g
        byts_act = statistics.mean(2 * uniq[i % 8] * per_e + 4 * t * in_f + 4 * n_pairs * n_ff for i in range(L))
        # the measurement twins of the gate/up kernel (the memra page's
        # ceiling-probe arms): load-only and math-only on the same grid
        twins = {}
        for arm in ("loadonly", "mathonly"):
            g = capture([(lambda c=sets[i % copies], d=draws[i % 8], a=arm:
                          qmm.moe_gateup_probe(a, c[0], c[1], d, sc, x, n_expert, n_ff, gate_out=go, up_out=uo))
                         for i in range(L)])
            tw = time_graph(g, L, 5)
            del g
            twins[arm] = {"us": round(tw * 1e6, 2), "GB/s": round(byts / tw / 1e9, 1)}
        res[f"t{t}"] = {"us": round(tt * 1e6, 2),
                        "GB/s": round(byts / tt / 1e9, 1),
                        "frac_hbm_peak": round(byts / tt / 1e9 / PEAK_HBM_GBS, 4),
                        "unique_experts_mean": round(statistics.mean(uniq), 2),
                        "algorithmic_bytes_mean": round(byts),
                        "v2": {"us": round(tv2 * 1e6, 2), "GB/s": round(byts / tv2 / 1e9, 1),
                               "bit_identical_to_v1": True},
                        "q8_1": {"us": round(tq8 * 1e6, 2), "GB/s": round(byts / tq8 / 1e9, 1),
                                 "includes": "quantize_q8_1 + gate/up"},
                        "swiglu_clamp_fused": {"us": round(tact * 1e6, 2), "GB/s": round(byts_act / tact / 1e9, 1),
                                               "frac_hbm_peak": round(byts_act / tact / 1e9 / PEAK_HBM_GBS, 4),
                                               "limit": 7.0},
                        "loadonly_twin": twins["loadonly"], "mathonly_twin": twins["mathonly"]}
        log(f"moe t={t}: {res[f't{t}']['us']} us {res[f't{t}']['GB/s']} GB/s; "
            f"V2 {res[f't{t}']['v2']['us']} us; Q8_1 {res[f't{t}']['q8_1']['us']} us; "
            f"+SwiGLU {res[f't{t}']['swiglu_clamp_fused']['us']} us; load-only {twins['loadonly']['us']} us, "
            f"math-only {twins['mathonly']['us']} us")
    return res


# ---------------------------------------------------------------- MoE down

def run_moe_down(args):
    """The down projection after the gate/up: 64 experts of d_model = 4096
    rows over n_ff = 2048 inputs, 8 per token, t in {1, 16}; per-pair
    activation rows; rotated over weight copies x 8 id draws.  Algorithmic
    bytes: the unique experts' rows + the activations + y (the per-pair terms
    the first kernel writes and the slot sum reads back are reported apart)."""
    import numpy as np
    import torch
    import gemv_prefill_decode_amd as qmm
    from synth import gen
    n_expert, n_ff, d_model, n_used = 64, 2048, 4096, 8
    rb = qmm.row_bytes("nvfp4", n_ff)
    per_e = d_model * rb
    host = np.empty(n_expert * per_e, dtype=np.uint8)
    for e in range(n_expert):
        host[e * per_e:(e + 1) * per_e] = gen.nvfp4_rows(d_model, n_ff, gen.SEED_MOE_DOWN_W + e)
    base = to_dev(host)
    del host
    copies = 2 if args.quick else 4
    sets = []
    for c in range(copies):
        w = base.clone()
        for e in range(n_expert):
            w[e * per_e + 7] ^= (c * 16 + 3) & 0xFF
        sets.append(w)
    del base
    sets_v2 = [qmm.repack_nvfp4_v2(w, n_expert * d_model, n_ff) for w in sets]
    res = {}
    L = 32
    for t in (1, 16):
        n_pairs = t * n_used
        draws_h = [gen.expert_ids(t, n_used, n_expert, gen.SEED_EXPERTS + d) for d in range(8)]
        draws = [to_dev(d) for d in draws_h]
        uniq = [len(np.unique(d)) for d in draws_h]
        sc = to_dev(gen.pair_scales(3 * n_pairs)[2 * n_pairs:])
        act = to_dev(gen.xorshift_f32(n_pairs * n_ff, gen.SEED_MOE_ACT).reshape(n_pairs, n_ff))
        y = torch.empty((t, d_model), dtype=torch.float32, device="cuda")
        po = torch.empty((n_pairs, d_model), dtype=torch.float32, device="cuda")
        g = capture([(lambda w=sets[i % copies], d=draws[i % 8]:
                      qmm.moe_down(w, d, sc, act, n_expert, d_model, y=y, pair_out=po))
                     for i in range(L)])
        tt = time_graph(g, L, 5)
        del g
        byts = statistics.mean(uniq[i % 8] * per_e + 4 * n_pairs * n_ff + 4 * t * d_model
                               for i in range(L))
        y1, _ = qmm.moe_down(sets[0], draws[0], sc, act, n_expert, d_model)
        y1 = y1.clone()
        y2, _ = qmm.moe_down(sets_v2[0], draws[0], sc, act, n_expert, d_model, "nvfp4_v2")
        if not torch.equal(y1, y2):
            raise SystemExit("MoE down: NVFP4 V2 differs from V1")
        g = capture([(lambda w=sets_v2[i % copies], d=draws[i % 8]:
                      qmm.moe_down(w, d, sc, act, n_expert, d_model, "nvfp4_v2", y=y, pair_out=po))
                     for i in range(L)])
        tv2 = time_graph(g, L, 5)
        del g
        # the down arm of the page on Q8_1 pair activations (quantization of
        # the activation rows included in the timed launches)
        aq, ad = qmm.quantize_q8_1(act)
        g = capture([(lambda w=sets_v2[i % copies], d=draws[i % 8]:
                      (qmm.quantize_q8_1(act, q=aq, d=ad),
                       qmm.moe_down_q8(w, d, sc, aq, ad, n_expert, d_model, "nvfp4_v2", y=y, pair_out=po)))
                     for i in range(L)])
        tq8 = time_graph(g, L, 5)
        del g
        res[f"t{t}"] = {"us": round(tt * 1e6, 2),
                        "GB/s": round(byts / tt / 1e9, 1),
                        "frac_hbm_peak": round(byts / tt / 1e9 / PEAK_HBM_GBS, 4),
                        "unique_experts_mean": round(statistics.mean(uniq), 2),
                        "algorithmic_bytes_mean": round(byts),
                        "pair_terms_bytes": 2 * 4 * n_pairs * d_model,
                        "v2": {"us": round(tv2 * 1e6, 2), "GB/s": round(byts / tv2 / 1e9, 1),
                               "bit_identical_to_v1": True},
                        "q8_1_v2": {"us": round(tq8 * 1e6, 2), "GB/s": round(byts / tq8 / 1e9, 1),
                                    "includes": "quantize_q8_1 of the pair rows + down on V2 rows"}}
        log(f"moe down t={t}: {res[f't{t}']['us']} us {res[f't{t}']['GB/s']} GB/s; "
            f"V2 {res[f't{t}']['v2']['us']} us; Q8_1 on V2 {res[f't{t}']['q8_1_v2']['us']} us")
    del sets, sets_v2
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------- MoE block

def run_moe_block(args):
    """The MoE block on the device: gate/up fused with the SwiGLU/clamp
    activation (limit 7.0), then the down projection with its slot sum, for
    t in {1, 16}; 64 experts, 8 used, d_model 4096, n_ff 2048; 2 copies of
    all three planes (1.8 GB) x 8 id draws rotated.  Algorithmic bytes: the
    unique experts' gate, up and down rows, x, the activation rows (written
    and read back) and y."""
    import numpy as np
    import torch
    import gemv_prefill_decode_amd as qmm
    from synth import gen
    n_expert, d_model, n_ff, n_used = 64, 4096, 2048, 8
    rb_gu, rb_d = qmm.row_bytes("nvfp4", d_model), qmm.row_bytes("nvfp4", n_ff)
    per_gu, per_d = n_ff * rb_gu, d_model * rb_d
    copies = 2
    sets = []
    for c in range(copies):
        planes = []
        for plane, (per, rows, cols, seed) in enumerate(((per_gu, n_ff, d_model, gen.SEED_MOE_W),
                                                         (per_gu, n_ff, d_model, gen.SEED_MOE_W),
                                                         (per_d, d_model, n_ff, gen.SEED_MOE_DOWN_W))):
            host = np.empty(n_expert * per, dtype=np.uint8)
            for e in range(n_expert):
                sd = seed + (2 * e + plane if plane < 2 else e)
                host[e * per:(e + 1) * per] = gen.nvfp4_rows(rows, cols, sd)
                host[e * per + 5] ^= (c * 16 + plane + 1) & 0xFF
            planes.append(to_dev(host))
            del host
        sets.append(planes)
    res = {}
    L = 32
    for t in (1, 16):
        n_pairs = t * n_used
        draws_h = [gen.expert_ids(t, n_used, n_expert, gen.SEED_EXPERTS + d) for d in range(8)]
        draws = [to_dev(d) for d in draws_h]
        uniq = [len(np.unique(d)) for d in draws_h]
        sc = to_dev(gen.pair_scales(3 * n_pairs))
        sc_gu, sc_d = sc[:2 * n_pairs], sc[2 * n_pairs:]
        x = to_dev(gen.xorshift_f32(t * d_model, gen.SEED_MOE_X).reshape(t, d_model))
        act = torch.empty((n_pairs, n_ff), dtype=torch.float32, device="cuda")
        y = torch.empty((t, d_model), dtype=torch.float32, device="cuda")
        po = torch.empty((n_pairs, d_model), dtype=torch.float32, device="cuda")

        def block(c, d):
            qmm.moe_gateup_act(c[0], c[1], d, sc_gu, x, n_expert, n_ff, "nvfp4", 7.0, act=act)
            qmm.moe_down(c[2], d, sc_d, act, n_expert, d_model, y=y, pair_out=po)
        g = capture([(lambda c=sets[i % copies], d=draws[i % 8]: block(c, d)) for i in range(L)])
        tt = time_graph(g, L, 5)
        del g
        byts = statistics.mean(uniq[i % 8] * (2 * per_gu + per_d) + 4 * t * d_model + 2 * 4 * n_pairs * n_ff +
                               4 * t * d_model for i in range(L))
        res[f"t{t}"] = {"us": round(tt * 1e6, 2), "GB/s": round(byts / tt / 1e9, 1),
                        "frac_hbm_peak": round(byts / tt / 1e9 / PEAK_HBM_GBS, 4),
                        "algorithmic_bytes_mean": round(byts),
                        "launches": "gate/up+SwiGLU/clamp, down, slot sum"}
        log(f"moe block t={t}: {res[f't{t}']['us']} us {res[f't{t}']['GB/s']} GB/s")
    del sets
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------- other prefill configs

PREFILL_CONFIGS = [("q4_0_1024x1024_n64", "q4_0", 1024, 1024, 64),
                   ("8b_q4_k_14336x4096_n2048", "q4_k", 14336, 4096, 2048),
                   ("8b_q4_k_4096x14336_n2048", "q4_k", 4096, 14336, 2048),
                   ("8b_q6_k_14336x4096_n2048", "q6_k", 14336, 4096, 2048),
                   ("8b_q6_k_4096x14336_n2048", "q6_k", 4096, 14336, 2048)]


def run_prefill_configs(args):
    """The Q4_0 1024x1024 n=64 GEMM (qmm_gemm's AUTO dispatch, the matrix
    cores) and the 8B-class n=2048 GEMMs (qmm_gemm_ws), each graph-replayed
    8 times, median of 5; TFLOP/s against the f16 MFMA peak."""
    import torch
    import gemv_prefill_decode_amd as qmm
    from synth import gen
    res = {}
    for tag, qt, m, k, n in PREFILL_CONFIGS:
        w = to_dev(gen_weights(qt, m, k, 7))
        x = to_dev(gen.unit_f32(n * k, gen.SEED_X + k).reshape(n, k))
        out = torch.empty((n, m), dtype=torch.float32, device="cuda")
        path = "auto" if n <= 64 else "mfma"
        g = capture([lambda: qmm.gemm(w, x, m, qt, out=out, path=path)] * 8)
        for _ in range(2):
            g.replay()
        t = time_graph(g, 8, 5)
        del g
        plan = qmm.gemm_plan(m, k, n, qt, path)
        fl = 2.0 * m * k * n
        res[tag] = {"us": round(t * 1e6, 2), "TFLOP/s": round(fl / t / 1e12, 1),
                    "frac_mfma_peak": round(fl / t / 1e12 / PEAK_F16_TFLOPS, 4),
                    "kernel": qmm.plan_kernel_name(plan, qt), "k_split": plan.get("n_split", 1)}
        log(f"{tag}: {res[tag]['us']} us {res[tag]['TFLOP/s']} TFLOP/s ({res[tag]['kernel']})")
        del w, x, out
        torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------- HBM traffic

COPY_PROBE_BYTES = 1 << 30
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def run_crossover():
    """GEMV against the matrix-core path over n (the measurement behind the
    AUTO dispatch): both paths graph-replayed over weight copies rotated
    through >= 1 GiB; prints one JSON object {shape: {n: [gemv_us, mfma_us]}}."""
    import torch
    import gemv_prefill_decode_amd as qmm
    from synth import gen
    res = {}
    for qt, m, k in (("q4_k", 4608, 1024), ("q6_k", 4608, 1024), ("q4_k", 14336, 4096),
                     ("q4_0", 1024, 4608), ("f32", 3072, 1024)):
        wbytes = m * qmm.row_bytes(qt, k)
        copies = max(4, -(-(1 << 30) // wbytes))
        base = to_dev(gen_weights(qt, m, k, 5))
        ws = rotated_copies(base if base.dtype == torch.uint8 else base.view(torch.uint8), copies)
        L = max(copies, 32)
        ent = {}
        for n in (4, 8, 12, 16, 24, 32, 48, 64):
            x = to_dev(gen.unit_f32(n * k, gen.SEED_X).reshape(n, k))
            out = torch.empty((n, m), dtype=torch.float32, device="cuda")
            t = []
            for path in ("gemv", "mfma"):
                g = capture([(lambda w=ws[i % copies], p=path: qmm.gemm(w, x, m, qt, out=out, path=p))
                             for i in range(L)])
                t.append(round(time_graph(g, L, 5) * 1e6, 2))
                del g
            ent[n] = t
        res[f"{qt} {m}x{k}"] = ent
        log(f"crossover {qt} {m}x{k}: {ent}")
        del ws
        torch.cuda.empty_cache()
    print(json.dumps({"crossover_us_gemv_mfma": res}))


PLAN_SHAPES = [("ffn_gate", 4608, 1024, 512), ("ffn_down", 1024, 4608, 512), ("conv_in", 3072, 1024, 512),
               ("attn_out", 1024, 1024, 512), ("8b_up", 14336, 4096, 2048), ("8b_down", 4096, 14336, 2048),
               ("q4_0_1024_n64", 1024, 1024, 64)]
# forced prefill plans compared with the planned one (QMM_MFMA_PLAN codes)
PLAN_FAMILIES = ["0,2,1,2", "2,2,1", "2,2,1,2", "3,2,1", "3,2,1,2", "4,2,1,2", "2,1,1", "2,1,1,2", "4,1,1,2",
                 "4,1,4,2", "5,1,1", "5,1,1,2", "6,1,1,2", "6,1,2,2"]


def run_prefill_plans(families=None, shapes=None):
    """The planned prefill kernel against forced kernel families, unsplit, per
    LFM2 and 8B-class shape and format (graph of 8 calls, median of 5).
    families / shapes: restrict to these QMM_MFMA_PLAN codes / shape labels."""
    import torch
    import gemv_prefill_decode_amd as qmm
    from synth import gen
    rows = []
    for label, m, k, n in PLAN_SHAPES:
        if shapes and label not in shapes:
            continue
        qts = ["q4_k", "q6_k"] if label.startswith("8b") else (["q4_0"] if label.startswith("q4_0") else QTS)
        x = to_dev(gen.unit_f32(n * k, gen.SEED_X + k).reshape(n, k))
        for qi, qt in enumerate(qts):
            w = to_dev(gen_weights(qt, m, k, 16 * qi))
            out = torch.empty((n, m), dtype=torch.float32, device="cuda")
            # the planned kernel last: the row's first graphs also warm the
            # clocks and bring the fresh weights in
            for force in (families or PLAN_FAMILIES) + [None]:
                if force is None:
                    os.environ.pop("QMM_MFMA_PLAN", None)
                else:
                    os.environ["QMM_MFMA_PLAN"] = force
                plan = qmm.gemm_plan(m, k, n, qt, "mfma")
                if force is not None and (plan["x16"], plan["k_groups"], plan["n_split"]) != (
                        int(force.split(",")[0]), int(force.split(",")[3]) if force.count(",") == 3 else 1,
                        int(force.split(",")[2])):
                    continue  # a family this format does not run
                ws = torch.empty(max(qmm.workspace_bytes(m, k, n, qt, "mfma"), 256), dtype=torch.uint8,
                                 device="cuda")
                g = capture([lambda: qmm.gemm(w, x, m, qt, out=out, path="mfma", workspace=ws)] * 8)
                for _ in range(3):
                    g.replay()
                t = time_graph(g, 8, 5)
                rows.append({"shape": f"{label} {m}x{k} n={n}", "qtype": qt, "plan": force or "auto",
                             "kernel": qmm.plan_kernel_name(plan, qt), "k_split": plan["n_split"],
                             "us": round(t * 1e6, 2), "TFLOP/s": round(2.0 * m * k * n / t / 1e12, 1)})
                log(f"{label} {qt} {force or 'auto':8s} {t * 1e6:8.2f} us {rows[-1]['kernel']} split {plan['n_split']}")
                del g, ws
            os.environ.pop("QMM_MFMA_PLAN", None)
            del w, out
            torch.cuda.empty_cache()
    print(json.dumps({"prefill_plans": rows}), flush=True)


COUNTER_SETS = [
    # (rocprofv3 --pmc set, one run each: at most 8 SQ counters per run)
    "SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES "
    "SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_WAIT_INST_ANY",
    "SQ_WAVE_CYCLES SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_VMEM SQ_ACTIVE_INST_MISC "
    "SQ_INSTS_SALU SQ_VALU_MFMA_COEXEC_CYCLES SQ_WAIT_ANY",
]
COUNTER_SHAPES = [("q4_0_1024_n64", "q4_0", 1024, 1024, 64)] + \
    [(f"lfm2_{label}_{qt}", qt, m, k, 512) for qt in QTS for (label, m, k) in SHAPES] + \
    [(f"8b_{m}x{k}_{qt}", qt, m, k, 2048) for qt in ("q4_k", "q6_k") for (m, k) in ((14336, 4096), (4096, 14336))]


def run_counter_workload():
    """The prefill calls of every headline configuration, three times each
    (synchronized), for rocprofv3 --pmc runs: the Q4_0 1024x1024 n=64 GEMM,
    the 20 LFM2 n=512 GEMMs and the four 8B-class n=2048 GEMMs, each with
    the workspace bench.py uses."""
    import torch
    import gemv_prefill_decode_amd as qmm
    from synth import gen
    for tag, qt, m, k, n in COUNTER_SHAPES:
        w = to_dev(gen_weights(qt, m, k, 3))
        x = to_dev(gen.unit_f32(n * k, gen.SEED_X + k).reshape(n, k))
        out = torch.empty((n, m), dtype=torch.float32, device="cuda")
        for _ in range(3):
            qmm.gemm(w, x, m, qt, out=out, path="mfma")
        torch.cuda.synchronize()
        plan = qmm.gemm_plan(m, k, n, qt, "mfma")
        print(json.dumps({"tag": tag, "qt": qt, "m": m, "k": k, "n": n,
                          "kernel": qmm.plan_kernel_name(plan, qt),
                          "grid": plan_grid_size(plan, m, n)}), flush=True)
        del w, x, out
        torch.cuda.empty_cache()


STREAM_COUNTER_SET = ("SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_SALU SQ_BUSY_CYCLES SQ_WAVE_CYCLES "
                      "SQ_WAIT_INST_ANY SQ_ACTIVE_INST_VALU")


def run_stream_counter_workload():
    """The streaming kernels three times each (synchronized, eager), for a
    rocprofv3 --pmc run: the n=1 GEMV and its load-only twin on 14336x4096
    Q4_K and Q6_K; the n=4 and n=16 Q4_K GEMV on its FMA and matrix-core
    streams; the NVFP4 MoE gate/up at t=1 and t=16 with its load-only and
    math-only twins.  Each tag line lists its arms in call order."""
    import numpy as np
    import torch
    import gemv_prefill_decode_amd as qmm
    from synth import gen
    m, k = 14336, 4096
    for qt in ("q4_k", "q6_k"):
        w = to_dev(gen_weights(qt, m, k, 99))
        x = to_dev(gen.unit_f32(k, gen.SEED_X).reshape(1, k))
        out = torch.empty((1, m), dtype=torch.float32, device="cuda")
        sink = torch.empty(m, dtype=torch.int32, device="cuda")
        for _ in range(3):
            qmm.gemm(w, x, m, qt, out=out, path="gemv")
            torch.cuda.synchronize()
            qmm.stream_loadonly(w, m, k, qt, sink)
            torch.cuda.synchronize()
        print(json.dumps({"tag": f"gemv_n1_{qt}_{m}x{k}", "weights": m * k,
                          "arms": ["served", "load-only twin"]}), flush=True)
        del w, x, out, sink
    w = to_dev(gen_weights("q4_k", m, k, 99))
    for n in (4, 16):
        x = to_dev(gen.unit_f32(n * k, gen.SEED_X).reshape(n, k))
        out = torch.empty((n, m), dtype=torch.float32, device="cuda")
        for _ in range(3):
            for path in ("gemv_fma", "gemv_matrix"):
                qmm.gemm(w, x, m, "q4_k", out=out, path=path)
                torch.cuda.synchronize()
        print(json.dumps({"tag": f"gemv_n{n}_q4_k_{m}x{k}", "weights": m * k,
                          "arms": ["FMA stream", "matrix-core stream"]}), flush=True)
        del x, out
    del w
    n_expert, in_f, n_ff, n_used = 64, 4096, 2048, 8
    wg = to_dev(np.concatenate([gen.nvfp4_rows(n_ff, in_f, gen.SEED_MOE_W + 2 * e) for e in range(n_expert)]))
    wu = to_dev(np.concatenate([gen.nvfp4_rows(n_ff, in_f, gen.SEED_MOE_W + 2 * e + 1) for e in range(n_expert)]))
    for t in (1, 16):
        ids_h = gen.expert_ids(t, n_used, n_expert, gen.SEED_EXPERTS)
        ids = to_dev(ids_h)
        sc = to_dev(gen.pair_scales(2 * t * n_used))
        x = to_dev(gen.xorshift_f32(t * in_f, gen.SEED_MOE_X).reshape(t, in_f))
        for _ in range(3):
            qmm.moe_gateup(wg, wu, ids, sc, x, n_expert, n_ff)
            torch.cuda.synchronize()
            qmm.moe_gateup_probe("loadonly", wg, wu, ids, sc, x, n_expert, n_ff)
            torch.cuda.synchronize()
            qmm.moe_gateup_probe("mathonly", wg, wu, ids, sc, x, n_expert, n_ff)
            torch.cuda.synchronize()
        print(json.dumps({"tag": f"moe_gateup_t{t}", "weights": 2 * len(np.unique(ids_h)) * n_ff * in_f,
                          "arms": ["served", "load-only twin", "math-only twin"]}), flush=True)


def stream_counter_summary(tags_path, csv_path, out_path):
    """profiles/stream_counters.md from --stream-counter-workload's tags and
    its --pmc counter_collection.csv: per streaming kernel and grid, wave
    instructions per weight (VALU, LDS, SALU), VALU issue time per SIMD at 4
    cycles per wave64 instruction, and the share of wave cycles spent waiting
    or issuing VALU."""
    import csv
    import collections
    tags = [json.loads(ln) for ln in open(tags_path) if ln.startswith("{")]
    order = []
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(csv_path)):
        name = r["Kernel_Name"].split("(")[0].replace("void ", "").replace("qmm::", "").strip()
        if not name.startswith(("gemv_kernel", "gemv_mfma_kernel", "loadonly_kernel", "moe_kernel")):
            continue
        key = (name, int(r["Grid_Size"]))
        if key not in vals:
            order.append(key)
        vals[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
    # distinct (kernel, grid) pairs in first-call order match the tags' arms in call order
    labels = [(t, arm) for t in tags for arm in t["arms"]]
    with open(out_path, "w") as f:
        f.write("# Streaming-kernel counters: the GEMV (n=1 with its load-only twin; n=4, 16 on both streams) "
                "and the NVFP4 MoE gate/up with its twins\n\n"
                "Commands (on one MI355X, from the repository root):\n\n"
                "```\ncd /tmp && export TMPDIR=/tmp && cd -\n"
                f"rocprofv3 --pmc {STREAM_COUNTER_SET} --output-format csv -d {os.path.dirname(csv_path)} -o run -- "
                f"python3 bench.py --stream-counter-workload > {tags_path}\n"
                f"python3 bench.py --stream-summary {tags_path} {csv_path} {out_path}\n```\n\n"
                "Wave instructions per weight of the matrix (x 64 lanes / weights; the MoE's weights are those of "
                "its distinct experts, the n = 16 GEMV streams its weights twice, once per token group of 8); VALU counts the matrix-core instructions, MFMA lists them apart; VALU "
                "issue per SIMD = SQ_INSTS_VALU x 4 cycles / 1024 SIMDs at 2.4 GHz (the VALU time if nothing "
                "else ran); the last two columns as shares of SQ_WAVE_CYCLES.\n\n")
        f.write("| config | arm | kernel | grid | VALU / weight | MFMA / weight | LDS / weight | SALU / weight | "
                "VALU issue per SIMD (us) | VALU-active / wave cycles | wait-inst / wave cycles |\n"
                "|---|---|---|---:|---:|---:|---:|---:|---:|---:|---:|\n")
        for (t, arm), key in zip(labels, order):
            c = {k: statistics.mean(v) for k, v in vals[key].items()}
            wgt = t["weights"]
            valu = c.get("SQ_INSTS_VALU", float("nan"))
            f.write(f"| {t['tag']} | {arm} | `{key[0]}` | {key[1]} | "
                    f"{64 * valu / wgt:.2f} | {64 * c.get('SQ_INSTS_MFMA', 0) / wgt:.3f} | "
                    f"{64 * c.get('SQ_INSTS_LDS', 0) / wgt:.3f} | "
                    f"{64 * c.get('SQ_INSTS_SALU', 0) / wgt:.3f} | {valu * 4 / 1024 / 2.4e3:.2f} | "
                    f"{c.get('SQ_ACTIVE_INST_VALU', 0) / c.get('SQ_WAVE_CYCLES', 1):.3f} | "
                    f"{c.get('SQ_WAIT_INST_ANY', 0) / c.get('SQ_WAVE_CYCLES', 1):.3f} |\n")
    print(open(out_path).read())


def mfma_counter_summary(tags_path, csv_paths, out_path):
    """profiles/mfma_counters_prefill.md from --counter-workload's printed
    tags and the counter_collection.csv of each --pmc run: per GEMM kernel
    dispatch (kernel name and grid size), MFMA flops from
    SQ_INSTS_VALU_MFMA_MOPS_F16 (x 512) against 2mkn, matrix cores busy =
    SQ_VALU_MFMA_BUSY_CYCLES / (SQ_BUSY_CYCLES x 32 SIMDs per shader
    engine), VALU and LDS instructions per MFMA, waits."""
    import csv
    import collections
    tags = [json.loads(ln) for ln in open(tags_path) if ln.startswith("{")]
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in csv_paths:
        for r in csv.DictReader(open(path)):
            name = r["Kernel_Name"].split("(")[0].replace("void ", "").replace("qmm::", "").strip()
            vals[(name, int(r["Grid_Size"]))][r["Counter_Name"]].append(float(r["Counter_Value"]))
    rows = []
    for t in tags:
        key = (t["kernel"], t["grid"])
        c = {k: statistics.mean(v) for k, v in vals.get(key, {}).items()}
        if not c:
            continue
        flops = 2.0 * t["m"] * t["k"] * t["n"]
        mops = c.get("SQ_INSTS_VALU_MFMA_MOPS_F16", float("nan")) * 512
        mfma = c.get("SQ_INSTS_MFMA", float("nan"))
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan")) / (c.get("SQ_BUSY_CYCLES", float("nan")) * 32)
        rows.append((t["tag"], t["kernel"], t["grid"], mops / flops, busy,
                     c.get("SQ_INSTS_VALU", float("nan")) / mfma, c.get("SQ_INSTS_LDS", float("nan")) / mfma,
                     c.get("SQ_LDS_BANK_CONFLICT", float("nan")),
                     c.get("SQ_WAIT_INST_ANY", float("nan")) / c.get("SQ_WAVE_CYCLES", float("nan")),
                     c.get("SQ_ACTIVE_INST_VALU", float("nan")) / c.get("SQ_WAVE_CYCLES", float("nan")),
                     c.get("SQ_VALU_MFMA_COEXEC_CYCLES", float("nan")) /
                     c.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan"))))
    with open(out_path, "w") as f:
        f.write("# Matrix-core counters of the prefill GEMM kernels (current sources)\n\n"
                "Commands (on one MI355X, from the repository root; two counter passes, then the table):\n\n"
                "```\ncd /tmp && export TMPDIR=/tmp && cd -\n" +
                "".join(f"rocprofv3 --pmc {cs} --output-format csv -d {os.path.dirname(cp)} -o run -- "
                        f"python3 bench.py --counter-workload > {tags_path if i == 0 else os.devnull}\n"
                        for i, (cs, cp) in enumerate(zip(COUNTER_SETS, csv_paths))) +
                f"python3 bench.py --mfma-summary {tags_path} {out_path} {' '.join(csv_paths)}\n```\n\n"
                "Per GEMM call of each headline configuration (the planned kernel at its grid, mean of 3 "
                "dispatches): MFMA flops from SQ_INSTS_VALU_MFMA_MOPS_F16 x 512 against 2mkn; matrix cores busy = "
                "SQ_VALU_MFMA_BUSY_CYCLES / (SQ_BUSY_CYCLES x 32); VALU / MFMA counts the matrix-core "
                "instructions among the VALU ones (SQ_INSTS_VALU includes them), other VALU / MFMA does not.\n\n")
        f.write("| config | kernel | grid | MFMA flops / 2mkn | matrix cores busy | VALU / MFMA | "
                "other VALU / MFMA | LDS / MFMA | LDS bank conflicts | wait-inst / wave cycles | "
                "VALU-active / wave cycles | VALU co-issued / MFMA busy |\n"
                "|---|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|\n")
        for r in rows:
            f.write(f"| {r[0]} | `{r[1]}` | {r[2]} | {r[3]:.3f} | {100 * r[4]:.1f}% | {r[5]:.2f} | {r[5] - 1:.2f} | "
                    f"{r[6]:.2f} | {r[7]:.0f} | {r[8]:.3f} | {r[9]:.3f} | {r[10]:.3f} |\n")
    print(open(out_path).read())


def copy_probe():
    """Three device-to-device copies of 1 GiB (the runtime's copy kernel): the
    calibration for the FETCH_SIZE / WRITE_SIZE counters.  The largest copies
    in the run, so the summary can find them."""
    import torch
    a = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b
    torch.cuda.empty_cache()


def pmc_summary(fetch_csv, write_csv, out_path):
    """profiles/traffic.json from two rocprofv3 --pmc counter_collection.csv
    files (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch).  Each counter is
    scaled by what it reads for the copy probe (COPY_PROBE_BYTES read and
    written per copy)."""
    import csv
    import collections

    def read(path, counter):
        # per kernel name, and per kernel name @ grid size (one launch shape)
        per = collections.defaultdict(list)
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"].split("(")[0].replace("void ", "").strip()
            v = float(r["Counter_Value"]) * 1024.0
            per[name].append(v)
            if r.get("Grid_Size"):
                per[f"{name}@{r['Grid_Size']}"].append(v)
        return per

    fetch, write = read(fetch_csv, "FETCH_SIZE"), read(write_csv, "WRITE_SIZE")
    fac = {}
    for lab, per in (("fetch", fetch), ("write", write)):
        vals = per.get(COPY_KERNEL, [])
        if not vals:
            raise SystemExit(f"no {COPY_KERNEL} dispatches in the {lab} counters")
        top = max(vals)
        probe = [v for v in vals if v >= 0.5 * top]
        fac[lab] = COPY_PROBE_BYTES / statistics.mean(probe)
    kernels = {}
    for name in sorted(set(fetch) & set(write)):
        if not name.startswith("qmm::"):
            continue
        f = statistics.mean(fetch[name]) * fac["fetch"]
        w = statistics.mean(write[name]) * fac["write"]
        short = name.replace("qmm::", "")
        kernels[short] = {"fetch_bytes": round(f), "write_bytes": round(w),
                          "bytes_per_launch": round(f + w), "dispatches": len(fetch[name]),
                          "tu": kernel_tu(short)}
    tab = {"tu_hashes": tu_source_hashes(),
           "calibration": {"copy_bytes": COPY_PROBE_BYTES, "fetch_scale": round(fac["fetch"], 4),
                           "write_scale": round(fac["write"], 4)},
           "kernels": kernels}
    with open(out_path, "w") as f:
        json.dump(tab, f, indent=1)
    print(json.dumps(tab["calibration"]))
    for k, v in kernels.items():
        print(f"{k:70s} {v['bytes_per_launch'] / 1e6:10.3f} MB/launch  (n={v['dispatches']})")


# ---------------------------------------------------------------- CPU oracle

def host_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def run_cpu_baseline(args, n):
    """The oracle (numpy decode to f64, then f64 BLAS matmul) on the host
    cores, median of 3 after 1 warm-up, decode and contraction timed apart.
    The headline entry is the whole LFM2 step; the other configurations are
    bounded samples scaled to their whole job (said per entry)."""
    import numpy as np
    from oracle import formats, ref
    from synth import gen
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        threads = os.cpu_count() or 1

    def timed(decode_jobs, contract):
        """(decode s, contraction s): decode_jobs() -> decoded matrices,
        contract(mats) -> None; median of 3 after a warm-up."""
        def once():
            t0 = time.perf_counter()
            mats = decode_jobs()
            t1 = time.perf_counter()
            contract(mats)
            return t1 - t0, time.perf_counter() - t1
        once()
        runs = [once() for _ in range(3)]
        return statistics.median(r[0] for r in runs), statistics.median(r[1] for r in runs)

    out = {}
    # the LFM2 step: 20 GEMMs at n = 512
    work = []
    for qi, qt in enumerate(QTS):
        for si, (label, m, k) in enumerate(SHAPES):
            work.append((qt, m, k, gen_weights(qt, m, k, 16 * qi + si), gen.unit_f32(n * k, gen.SEED_X + k).reshape(n, k)))
    flops = sum(2.0 * m * k * n for (_, m, k, _, _) in work)
    xs = [x.astype(np.float64) for (_, _, _, _, x) in work]
    td, tc = timed(lambda: [formats.decode(qt, w, m, k) for (qt, m, k, w, _) in work],
                   lambda mats: [x @ W.T for x, W in zip(xs, mats)])
    out["lfm2_prefill_n512"] = {"TFLOP/s": round(flops / (td + tc) / 1e12, 5), "decode_s": round(td, 4),
                                "contraction_s": round(tc, 4), "sample": "the whole 20-GEMM step"}
    # Q4_0 1024x1024 n=64
    w = gen_weights("q4_0", 1024, 1024, 0)
    x = gen.unit_f32(64 * 1024, gen.SEED_X).reshape(64, 1024).astype(np.float64)
    td1, tc1 = timed(lambda: formats.decode("q4_0", w, 1024, 1024), lambda W: x @ W.T)
    out["q4_0_1024x1024_n64"] = {"TFLOP/s": round(2.0 * 1024 ** 2 * 64 / (td1 + tc1) / 1e12, 5),
                                 "decode_s": round(td1, 4), "contraction_s": round(tc1, 4), "sample": "whole"}
    # decode GEMV n = 1, q4_k 14336x4096
    w = gen_weights("q4_k", 14336, 4096, 99)
    x1 = gen.unit_f32(4096, gen.SEED_X).astype(np.float64)
    td2, tc2 = timed(lambda: formats.decode("q4_k", w, 14336, 4096), lambda W: W @ x1)
    out["decode_q4_k_14336x4096_n1"] = {"GB/s": round(w.size / (td2 + tc2) / 1e9, 4), "decode_s": round(td2, 4),
                                        "contraction_s": round(tc2, 4), "sample": "whole"}
    # MoE gate/up t = 1: 8 experts x 2 planes of 2048 x 4096 NVFP4 rows
    rows = [gen.nvfp4_rows(2048, 4096, gen.SEED_MOE_W + i) for i in range(16)]
    xm = gen.xorshift_f32(4096, gen.SEED_MOE_X).astype(np.float64)
    td3, tc3 = timed(lambda: [formats.decode("nvfp4", r, 2048, 4096) for r in rows],
                     lambda mats: [W @ xm for W in mats])
    out["moe_gateup_t1"] = {"GB/s": round(sum(r.size for r in rows) / (td3 + tc3) / 1e9, 4),
                            "decode_s": round(td3, 4), "contraction_s": round(tc3, 4), "sample": "whole"}
    # 8B-class q4_k 14336x4096 n = 2048: one 2048-row block of W, scaled by 7
    m_s = 2048
    w = gen_weights("q4_k", m_s, 4096, 7)
    x8 = gen.unit_f32(2048 * 4096, gen.SEED_X + 4096).reshape(2048, 4096).astype(np.float64)
    td4, tc4 = timed(lambda: formats.decode("q4_k", w, m_s, 4096), lambda W: x8 @ W.T)
    out["8b_q4_k_14336x4096_n2048"] = {"TFLOP/s": round(2.0 * m_s * 4096 * 2048 / (td4 + tc4) / 1e12, 5),
                                       "decode_s": round(td4 * 7, 4), "contraction_s": round(tc4 * 7, 4),
                                       "sample": "rows 0..2047 of 14336 (1/7), times scaled by 7"}
    main = out["lfm2_prefill_n512"]
    return {
        "value": main["TFLOP/s"],
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"the whole 20-GEMM prefill step (4 shapes x 5 formats, n={n}): numpy decode to f64 "
                  f"({main['decode_s']:.3f} s) + f64 matmul ({main['contraction_s']:.3f} s, BLAS); "
                  f"median of 3 after 1 warm-up",
        "host_cpus": os.cpu_count(),
        "host_model": host_model(),
        "configs": out,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--n", type=int, default=512, help="prefill tokens (default 512)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the decode and MoE measurements")
    ap.add_argument("--quick", action="store_true", help="fewer rotation copies")
    ap.add_argument("--crossover", action="store_true",
                    help="only measure GEMV vs matrix-core time over n (prints its own JSON)")
    ap.add_argument("--prefill-plans", action="store_true",
                    help="only time the planned prefill kernel against forced kernel families (own JSON)")
    ap.add_argument("--plans", default=None,
                    help="with --prefill-plans: forced QMM_MFMA_PLAN codes separated by ';'")
    ap.add_argument("--plan-shapes", default=None,
                    help="with --prefill-plans: shape labels separated by ',' (ffn_gate, 8b_up, ...)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="first run the 1 GiB copy that calibrates the HBM byte counters")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--counter-workload", action="store_true",
                    help="only run every headline prefill GEMM three times (for rocprofv3 --pmc runs)")
    ap.add_argument("--mfma-summary", nargs="+", metavar="FILE",
                    help="TAGS OUT_MD CSV...: the MFMA counter table from --counter-workload runs")
    ap.add_argument("--stream-counter-workload", action="store_true",
                    help="only run the n=1 GEMV and MoE gate/up kernels and twins (for a rocprofv3 --pmc run)")
    ap.add_argument("--stream-summary", nargs=3, metavar=("TAGS", "CSV", "OUT_MD"),
                    help="the streaming counter table from a --stream-counter-workload run")
    args = ap.parse_args()
    if args.stream_summary:
        stream_counter_summary(args.stream_summary[0], args.stream_summary[1], args.stream_summary[2])
        return
    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], os.path.join(ROOT, "profiles", "traffic.json"))
        return
    if args.mfma_summary:
        mfma_counter_summary(args.mfma_summary[0], args.mfma_summary[2:], args.mfma_summary[1])
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; there is no multi-GPU path (asked for --gpus {args.gpus})",
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
    if args.crossover:
        run_crossover()
        return
    if args.prefill_plans:
        run_prefill_plans(args.plans.split(";") if args.plans else None,
                          args.plan_shapes.split(",") if args.plan_shapes else None)
        return
    if args.counter_workload:
        run_counter_workload()
        return
    if args.stream_counter_workload:
        run_stream_counter_workload()
        return
    if args.copy_probe:
        log("copy probe: 3 x 1 GiB device copies")
        copy_probe()
    n = args.n
    log(f"prefill step: {len(SHAPES)} shapes x {len(QTS)} formats, n={n}, warmup={args.warmup} steps={args.steps}")
    step_flops, wall, per_qt, roofline = run_prefill(args, n)
    value = step_flops * args.steps / wall / 1e12
    log(f"prefill: {value:.1f} TFLOP/s, {wall / args.steps * 1e3:.3f} ms/step")
    extras = {}
    if not args.no_extras:
        log("decode GEMV sweep with rotation")
        extras["decode"] = run_decode(args)
        log("MoE gate/up NVFP4")
        extras["moe_gateup"] = run_moe(args)
        torch.cuda.empty_cache()
        log("MoE down NVFP4")
        extras["moe_down"] = run_moe_down(args)
        torch.cuda.empty_cache()
        log("MoE block: gate/up + SwiGLU/clamp + down")
        extras["moe_block"] = run_moe_block(args)
        log("prefill configs: Q4_0 1024^2 n=64, 8B-class n=2048")
        extras["prefill_configs"] = run_prefill_configs(args)
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
        "dtype": "f16",
        "data": "synthetic (seeded LCG packed weights, uniform[-1,1) activations)",
        "config": {"workload": "LFM2.5-350M-shaped prefill, n=512: ffn_gate 4608x1024, ffn_down 1024x4608, "
                               "conv_in 3072x1024, attn_out 1024x1024, each in f32/q4_0/q8_0/q4_k/q6_k "
                               "(f16 MFMA operands, f32 accumulation)",
                   "n": n, "gemms_per_step": len(SHAPES) * len(QTS)},
        "per_qtype": per_qt,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    line.update(extras)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
