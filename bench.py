#!/usr/bin/env python3
"""Benchmark of the PARO W4A8 linear hot path on one MI355X.

A step is one pass of the whole path over one batch: the rotate-quant prologue followed by
the W4A8 group GEMM, on the gate_up prefill workload (M=2048 tokens, K=5120, N=17408,
synthetic seeded inputs, DRAM-fed: each step uses the next of `--copies` copies of the
activations and weights so nothing stays resident in the 256 MB last-level cache).

Prints ONE JSON line: whole-step TFLOP/s (2*M*N*K per step), the GEMM's roofline against
the dense fp8 matrix peak (kernel time from HIP events on the launch stream), the decode
M=1 / M=8 GEMM's HBM bandwidth against the 8 TB/s peak, and the oracle's CPU throughput on a
bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A8 GEMM µs + TFLOP/s (gate_up M=2048), decode M=1 HBM GB/s vs peak"
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 matrix peak
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
PAGES_GEMM_TFLOPS = 125.5     # the pages' GEMM alone (per-group fold v2, 2910 us) on gfx1201: context
COPY_CALIBRATION_BYTES = 64 << 20


PROBES_SRC = os.path.join(ROOT, "bench_probes.hip")
PROBES_LIB = os.path.join(ROOT, "bench_probes.so")
SETTLE_MS = 300.0             # untimed steps before the timed region (the clock's ramp)


def build_probes():
    """Compiles the ceiling probes (bench_probes.hip) for gfx950 into bench_probes.so."""
    import subprocess
    tmp = PROBES_LIB + ".tmp"
    subprocess.run(["/opt/rocm/bin/hipcc", "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", PROBES_SRC, "-o", tmp], check=True)
    os.replace(tmp, PROBES_LIB)
    return PROBES_LIB


def measure_ceilings(torch, np):
    """Measured HBM read and fp8 matrix-core ceilings on this GPU (bench_probes.hip), best median
    of 20 HIP-event-timed launches over a few launch widths, after ~100 ms of untimed launches."""
    import ctypes
    if not os.path.exists(PROBES_LIB):
        raise RuntimeError(f"{PROBES_LIB} is missing: run `python __graft_entry__.py build`")
    L = ctypes.CDLL(PROBES_LIB)
    L.probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    L.probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def timed(launch, reps=20):
        settle_clock(torch, lambda i: launch(), 8, ms=100.0)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record()
            launch()
            b.record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) * 1e-3 for a, b in ev]))

    nbytes = 2 << 30                                   # 2 GiB: 8x the last-level cache
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    out = torch.empty(1 << 20, dtype=torch.int32, device="cuda")
    read = {}
    for blocks in (1024, 2048, 4096, 8192):
        def launch(b=blocks):
            if L.probe_read(ctypes.c_void_p(buf.data_ptr()), nbytes, b, ctypes.c_void_p(out.data_ptr()), stream) != 0:
                raise RuntimeError("probe_read failed")
        read[blocks] = nbytes / timed(launch) / 1e9
    del buf
    mfma = {}
    iters = 2000
    outf = torch.empty(8192 * 256, dtype=torch.float32, device="cuda")
    for blocks in (512, 1024, 2048):                  # 2, 4, 8 waves per SIMD on 256 CUs
        def launch(b=blocks):
            if L.probe_mfma(b, iters, ctypes.c_void_p(outf.data_ptr()), stream) != 0:
                raise RuntimeError("probe_mfma failed")
        mfma[blocks] = blocks * 4 * 8 * iters * 65536.0 / timed(launch) / 1e12
    torch.cuda.empty_cache()
    best_r = max(read, key=read.get)
    best_m = max(mfma, key=mfma.get)
    return {"hbm_read_GBs": round(read[best_r], 1), "hbm_read_blocks": best_r,
            "fp8_mfma_TFLOPs": round(mfma[best_m], 1), "fp8_mfma_blocks": best_m,
            "read_sweep_GBs": {str(k): round(v, 1) for k, v in read.items()},
            "mfma_sweep_TFLOPs": {str(k): round(v, 1) for k, v in mfma.items()},
            "probes": "bench_probes.hip: 2 GiB nontemporal 16-byte reads; 8 independent fp8 16x16x128 products per wave step"}


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "gemm_prefill_gate_up_m2048_traffic.json")
GEMM_SOURCE = os.path.join(ROOT, "rotated_w4a8_group_amd", "csrc", "pq_gemm.hip")


def measured_traffic():
    """HBM bytes per GEMM launch from the committed rocprofv3 counter record (FETCH_SIZE and
    WRITE_SIZE scaled by the copy-kernel calibration), or None if the record is missing or was
    taken on a different version of the GEMM source."""
    import hashlib
    try:
        rec = json.load(open(TRAFFIC_RECORD))
        src = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != src:
        return None
    return rec.get("bytes_per_launch")


def gemm_bytes(M, K, N, P=1, w5=False):
    """Algorithmic GEMM bytes: packed codes (4 bits per weight, 5 for int5), SZ words,
    activation codes, scales and row-sums, bf16 output."""
    G = K // 128
    return K * N // 2 + (K * N // 8 if w5 else 0) + G * N * 4 + P * M * K + 2 * P * M * G * 4 + M * N * 2


def prologue_bytes(M, K, P=1):
    G = K // 128
    return M * K * 2 + P * K * 2 + P * 8 * (K // 2) * 8 + P * M * K + 2 * P * M * G * 4


# timed repetitions of the per-configuration measurements: eager calls (M > 16), and replays of a
# HIP graph of one launch per weight copy (M <= 16, 12 copies: 120 launches)
REPS_LONG = 50
REPS_SHORT = 10


def spread(ts):
    """(median, p10, p90) of a list of seconds."""
    import numpy as np
    return float(np.median(ts)), float(np.percentile(ts, 10)), float(np.percentile(ts, 90))


def settle_clock(torch, fn, n, ms=30.0):
    """Untimed calls fn(0), fn(1), ... for about `ms` of wall time (synchronising every n calls),
    so that the timed calls after it run at the GPU's settled clock rather than during its ramp
    after the host-side set-up of a measurement."""
    t0 = time.perf_counter()
    i = 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        fn(i % n)
        i += 1
        if i % n == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 200 steps after 50 warm-up steps (about 60 ms of GPU work): the GPU's clock settles over the
    # first few ms of a process, and 20 steps after 5 read the GEMM 15% slower than steady state
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--copies", type=int, default=12)
    ap.add_argument("--decode-reps", type=int, default=60)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-config measurements (merged QKV M=4 P=3, M=8192 gate_up and down)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 64 MiB device copy 5 times (HBM counter calibration)")
    ap.add_argument("--ceilings-only", action="store_true",
                    help="only measure the HBM read and fp8 matrix-core ceilings and print them")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the measured ceilings")
    ap.add_argument("--prologue-only", metavar="WORKLOAD",
                    help="only run one synthetic workload's prologues, 5 calls each of the per-group, "
                         "per-token and GEMM-workspace-filling forms (for counter passes)")
    ap.add_argument("--gemm-only", metavar="WORKLOAD",
                    help="only run one synthetic workload (synth.WORKLOADS name): its prologue once, then "
                         "5 GEMM calls (for counter passes that must see one shape)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this build measures one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}); the multi-GPU path is design-only.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        # a plain device-to-device copy of known size: under rocprofv3 --pmc FETCH_SIZE /
        # WRITE_SIZE its counter values give the scale from counter units to HBM bytes
        src = torch.ones(COPY_CALIBRATION_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": COPY_CALIBRATION_BYTES, "launches": 5}), flush=True)
        return

    if args.ceilings_only:
        print(json.dumps({"ceilings": measure_ceilings(torch, np)}), flush=True)
        return

    if args.gemm_only:
        gemm_only(args.gemm_only, torch, np)
        return
    if args.prologue_only:
        prologue_only(args.prologue_only, torch, np)
        return
    ceilings = None if args.no_ceilings else measure_ceilings(torch, np)

    import rotated_w4a8_group_amd as pq
    import synth

    dev = torch.device("cuda:0")
    wl = synth.WORKLOADS["prefill"]
    M, K, N, G, P = wl.M, wl.K, wl.N, wl.G, wl.P
    C = max(1, args.copies)

    # ---- inputs: C copies of activations and packed weights (DRAM-fed timing)
    x0 = synth.activations(wl)
    pl, tl, cl = synth.rotations(wl)
    w = synth.weights(wl)
    rec = torch.from_numpy(np.stack([pq.build_records(p, t) for p, t in zip(pl, tl)])).to(dev)
    cs = torch.from_numpy(np.stack(cl)).to(dev)
    xs = [torch.from_numpy(x0).to(dev)]
    wq = [pq.pack_weights(torch.from_numpy(w.qweight).to(dev), torch.from_numpy(w.qzeros).to(dev),
                          torch.from_numpy(w.scales).to(dev))]
    for _ in range(C - 1):
        xs.append(xs[0].clone())
        wq.append((wq[0][0].clone(), wq[0][1].clone()))
    A = torch.empty((P, M, K), dtype=torch.uint8, device=dev)
    S = torch.empty((P, M, G), dtype=torch.float32, device=dev)
    R = torch.empty((P, M, G), dtype=torch.float32, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    ws = torch.empty(max(1, pq.gemm_workspace_bytes(M, N, K)), dtype=torch.uint8, device=dev)

    # the step: the prologue writes the GEMM's prefill operands into its workspace
    # (pq_rotate_quant_for_gemm), the GEMM reads them there (pq_gemm_prepared): two launches
    def step(i, ev=None):
        c = i % C
        if ev is not None:
            ev[0].record()
        pq.rotate_quant_for_gemm(xs[c], rec, cs, ws, out=(A, S, R))
        if ev is not None:
            ev[1].record()
        pq.gemm_prepared(A, S, R, wq[c][0], wq[c][1], N, *wl.bounds, out=y, workspace=ws)
        if ev is not None:
            ev[2].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # untimed steps for a fixed wall time whatever --warmup is: the clock ramps over the first
    # tens of ms of work, and a short timed region would otherwise land on the ramp
    settle_clock(torch, lambda i: step(i), C, ms=SETTLE_MS)
    # per-phase breakdown: eager launches with events between the two calls
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step_eager = (t1 - t0) * 1e3 / args.steps
    pro_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    gemm_all = [e[1].elapsed_time(e[2]) for e in evs]
    gemm_ms = float(np.mean(gemm_all))
    # the timed steps: the K steps (cycling the weight copies) captured once in a HIP graph and
    # replayed, which removes the host launch gaps between the step's kernels
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        for i in range(args.steps):
            step(i)
    graph.replay()                      # untimed: first replay
    torch.cuda.synchronize()
    settle_clock(torch, lambda i: graph.replay(), 1, ms=SETTLE_MS / 3)
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    # the replayed graph must reproduce the eager result of its last step bit for bit
    y_graph = y.clone()
    step(args.steps - 1)
    torch.cuda.synchronize()
    if not torch.equal(y_graph.view(torch.int16), y.view(torch.int16)):
        raise RuntimeError("bench: graph replay differs from the eager step")
    del graph
    # the same steps through the two plain calls (pq_rotate_quant, then pq_gemm, which derives
    # its prefill operands in a pass of its own), for comparison in the same run
    ws2 = torch.empty_like(ws)

    def step_two_calls(i):
        c = i % C
        pq.rotate_quant(xs[c], rec, cs, out=(A, S, R))
        pq.gemm(A, S, R, wq[c][0], wq[c][1], N, *wl.bounds, out=y, workspace=ws2)

    graph2 = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph2):
        for i in range(args.steps):
            step_two_calls(i)
    graph2.replay()
    torch.cuda.synchronize()
    settle_clock(torch, lambda i: graph2.replay(), 1, ms=SETTLE_MS / 3)
    t0 = time.perf_counter()
    graph2.replay()
    torch.cuda.synchronize()
    ms_per_step_two_calls = (time.perf_counter() - t0) * 1e3 / args.steps
    if not torch.equal(y_graph.view(torch.int16), y.view(torch.int16)):
        raise RuntimeError("bench: the two-call step differs from the shared-workspace step")
    del graph2
    flops = 2.0 * M * N * K
    value = flops / (ms_per_step * 1e-3) / 1e12
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "timing": "HIP graph of the K steps, replayed once after an untimed replay; wall clock between synchronizations",
        "ms_per_step_eager": round(ms_per_step_eager, 4),
        "ms_per_step_two_calls": round(ms_per_step_two_calls, 4),
        "step": "pq_rotate_quant_for_gemm + pq_gemm_prepared (ms_per_step_two_calls: pq_rotate_quant + pq_gemm)",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 x u4 (fp32 accumulate)",
        "data": "synthetic (seeded; shapes and distributions of the gate_up prefill workload)",
        "config": {"workload": "gate_up prefill: rotate-quant prologue + W4A8 GEMM",
                   "M": M, "K": K, "N": N, "partitions": P, "dram_fed_copies": C},
        "gemm_us": round(gemm_ms * 1e3, 2),
        "gemm_us_p10_p90": [round(float(np.percentile(gemm_all, q)) * 1e3, 2) for q in (10, 90)],
        "prologue_us": round(pro_ms * 1e3, 2),
        "gemm_tflops": round(gemm_tflops, 2),
        "gemm_vs_pages_gfx1201": round(gemm_tflops / PAGES_GEMM_TFLOPS, 3),
        "prologue_gbs": round(prologue_bytes(M, K, P) / (pro_ms * 1e-3) / 1e9, 1),
        "roofline": {"bound": "mfma", "kernel": "pq_gemm_prepared (the prefill kernel; its zero-point operands come from the prologue)",
                     "achieved": round(gemm_tflops, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gemm_tflops / PEAK_FP8_TFLOPS, 4), "traffic": measured_traffic()},
        "settle_ms": SETTLE_MS,
    }
    if ceilings is not None:
        out["ceilings"] = ceilings
        out["roofline"]["peak_measured"] = ceilings["fp8_mfma_TFLOPs"]
        out["roofline"]["frac_measured"] = round(gemm_tflops / ceilings["fp8_mfma_TFLOPs"], 4)

    # ---- decode GEMM bandwidth (M = 1 and 8), DRAM-fed over the same weight copies. The C
    # launches (one per weight copy) are captured in one HIP graph and replayed, so the
    # per-launch time is the GPU's, not Python's launch overhead.
    if not args.no_decode:
        dec = {}
        for Md in (1, 8):
            Ad, Sd, Rd = A[:, :Md].contiguous(), S[:, :Md].contiguous(), R[:, :Md].contiguous()
            yd = torch.empty((Md, N), dtype=torch.bfloat16, device=dev)
            for i in range(C):
                pq.gemm(Ad, Sd, Rd, wq[i][0], wq[i][1], N, out=yd)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for i in range(C):
                    pq.gemm(Ad, Sd, Rd, wq[i][0], wq[i][1], N, out=yd)
            graph.replay()
            torch.cuda.synchronize()
            settle_clock(torch, lambda i: graph.replay(), 1)
            reps = max(3, args.decode_reps // C)
            e = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
            for i in range(reps):
                e[i][0].record()
                graph.replay()
                e[i][1].record()
            torch.cuda.synchronize()
            t = np.array([a.elapsed_time(b) for a, b in e]) * 1e-3 / C
            gbs = gemm_bytes(Md, K, N) / np.median(t) / 1e9
            dec[f"M{Md}"] = {"us_median": round(float(np.median(t)) * 1e6, 2),
                             "us_p10": round(float(np.percentile(t, 10)) * 1e6, 2),
                             "us_p90": round(float(np.percentile(t, 90)) * 1e6, 2),
                             "bytes": gemm_bytes(Md, K, N), "GBs": round(float(gbs), 1),
                             "frac_hbm": round(float(gbs) / PEAK_HBM_GBS, 4),
                             "frac_hbm_measured": (round(float(gbs) / ceilings["hbm_read_GBs"], 4)
                                                   if ceilings else None),
                             "timing": f"HIP graph of {C} launches over {C} weight copies, per-launch average after ~30 ms of untimed replays"}
        out["decode"] = dec

    # ---- every other configuration: prologue and GEMM timed separately
    if not args.no_configs:
        out["configs"] = {"c3_gate_up_m2048": {
            "prologue_us": out["prologue_us"], "prologue_GBs": out["prologue_gbs"],
            "gemm_us": out["gemm_us"], "gemm_us_p10_p90": out["gemm_us_p10_p90"], "gemm_TFLOPs": out["gemm_tflops"],
            "gemm_GBs": round(gemm_bytes(M, K, N) / (gemm_ms * 1e-3) / 1e9, 1),
            "roofline": {"bound": "mfma", "frac": out["roofline"]["frac"]},
            "timing": f"HIP events around each call of the {args.steps} eager steps (mean), DRAM-fed over {C} copies"}}
        for name, key in (("c2_qkv_m4_p3", "qkv"), ("c3_gate_up_m2048_pq_gemm", "prefill"),
                          ("c4_gate_up_m8192", "full_gate_up"), ("c4_down_m8192", "full_down")):
            out["configs"][name] = config_measurement(synth.WORKLOADS[key], pq, torch, np, dev, C)
        # the per-token activation-scale path on the same prefill workloads
        out["per_token"] = {}
        for name, key in (("c3_gate_up_m2048", "prefill"), ("c4_gate_up_m8192", "full_gate_up"),
                          ("c4_down_m8192", "full_down")):
            out["per_token"][name] = config_measurement(synth.WORKLOADS[key], pq, torch, np, dev, C, tok=True)
        # the per-group int8 activation mode
        out["int8_per_group"] = {}
        for name, key in (("c1_decode_m1", "decode_m1"), ("c3_gate_up_m2048", "prefill"),
                          ("c4_down_m8192", "full_down")):
            out["int8_per_group"][name] = config_measurement(synth.WORKLOADS[key], pq, torch, np, dev, C, i8=True)
        # the fused residual add + RMSNorm + rotate-quant producer against the unfused chain
        out["fused_producer"] = {}
        for name, key in (("c1_decode_m1", "decode_m1"), ("c1_decode_m8", "decode_m8"), ("c3_gate_up_m2048", "prefill")):
            out["fused_producer"][name] = producer_measurement(synth.WORKLOADS[key], pq, torch, np, dev, C)
        # int5 bit-plane weights (the e4m3 per-group activations)
        out["int5_weights"] = {}
        for name, key in (("c1_decode_m1", "decode_m1"), ("c3_gate_up_m2048", "prefill")):
            out["int5_weights"][name] = config_measurement(synth.WORKLOADS[key], pq, torch, np, dev, C, w5=True)
        if not args.no_cpu_baseline:
            for name, key in (("c2_qkv_m4_p3", "qkv"), ("c4_gate_up_m8192", "full_gate_up"),
                              ("c4_down_m8192", "full_down")):
                cfg = out["configs"][name]
                orc = oracle_config_time(synth.WORKLOADS[key], rows=min(synth.WORKLOADS[key].M, 384))
                gpu_s = (cfg["prologue_us"] + cfg["gemm_us"]) * 1e-6
                orc["gpu_over_oracle"] = round(orc["full_s_estimate"] / gpu_s, 1)
                cfg["oracle"] = orc

    # ---- the oracle on the host, bounded sample of the same workload
    if not args.no_cpu_baseline:
        out["cpu_baseline"], wall = cpu_baseline(x0, pl, tl, cl, w, wl)
        if "configs" in out:
            c3 = out["configs"]["c3_gate_up_m2048"]
            c3["oracle"] = {"rows": wl.M, "full_s": round(wall, 2),
                            "gpu_over_oracle": round(wall / ((c3["prologue_us"] + c3["gemm_us"]) * 1e-6), 1)}

    print(json.dumps(out), flush=True)


def producer_measurement(wl, pq, torch, np, dev, copies):
    """pq_add_rms_rotate_quant against the unfused chain (torch add, torch rms_norm in float32 with
    the Gemma 1 + w weight, pq_rotate_quant): per-launch averages of HIP graphs over `copies` input
    copies when M <= 16, else HIP events around eager calls alternating two copies."""
    import synth
    M, K, G, P = wl.M, wl.K, wl.G, wl.P
    short = M <= 16
    C = copies if short else 2
    pl, tl, cl = synth.rotations(wl)
    rec = torch.from_numpy(np.stack([pq.build_records(p, t) for p, t in zip(pl, tl)])).to(dev)
    cs = torch.from_numpy(np.stack(cl)).to(dev)
    xs = [torch.from_numpy(synth.activations(wl)).to(dev) for _ in range(C)]
    rs = [torch.from_numpy(synth.residual(wl)).to(dev) for _ in range(C)]
    w = torch.from_numpy(synth.norm_weight(wl)).to(dev)
    w1 = (1.0 + w.float())
    ro = torch.empty((M, K), dtype=torch.float16, device=dev)
    hs = torch.empty((M, K), dtype=torch.float16, device=dev)
    A = torch.empty((P, M, K), dtype=torch.uint8, device=dev)
    S = torch.empty((P, M, G), dtype=torch.float32, device=dev)
    R = torch.empty((P, M, G), dtype=torch.float32, device=dev)
    fused = lambda i: pq.add_rms_rotate_quant(xs[i % C], rs[i % C], w, 1e-6, rec, cs, residual_out=ro, out=(hs, A, S, R))

    def chain(i):
        h = xs[i % C].float().add_(rs[i % C].float()).half()
        hn = torch.nn.functional.rms_norm(h.float(), (K,), weight=w1, eps=1e-6).half()
        pq.rotate_quant(hn, rec, cs, out=(A, S, R))

    def timed(fn, reps):
        for i in range(C):
            fn(i)
        torch.cuda.synchronize()
        if short:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for i in range(C):
                    fn(i)
            graph.replay()
            torch.cuda.synchronize()
            settle_clock(torch, lambda i: graph.replay(), 1)
            e = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
            for a, b in e:
                a.record()
                graph.replay()
                b.record()
            torch.cuda.synchronize()
            return spread([a.elapsed_time(b) * 1e-3 / C for a, b in e])
        settle_clock(torch, fn, C)
        e = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for i, (a, b) in enumerate(e):
            a.record()
            fn(i)
            b.record()
        torch.cuda.synchronize()
        return spread([a.elapsed_time(b) * 1e-3 for a, b in e])

    reps = REPS_SHORT if short else REPS_LONG
    t_f, f10, f90 = timed(fused, reps)
    t_c, _, _ = timed(chain, reps)
    nbytes = 2 * M * K * 2 + K * 2 + P * K * 2 + P * 8 * (K // 2) * 8 + 2 * M * K * 2 + P * M * K + 2 * P * M * G * 4
    return {"M": M, "K": K, "partitions": P, "fused_us": round(t_f * 1e6, 2),
            "fused_us_p10_p90": [round(f10 * 1e6, 2), round(f90 * 1e6, 2)], "chain_us": round(t_c * 1e6, 2),
            "bytes": nbytes, "fused_GBs": round(nbytes / t_f / 1e9, 1),
            "chain": "torch add + torch rms_norm (float32) + pq_rotate_quant",
            "timing": (f"HIP graph of {C} launches over {C} copies, per-launch median (p10, p90) of {REPS_SHORT} replays after ~30 ms of untimed replays" if short
                       else f"HIP events around each eager call, median (p10, p90) of {REPS_LONG} after ~30 ms of untimed calls, two alternating copies")}


def gemm_only(name, torch, np, calls=5):
    """One workload's prologue, then `calls` GEMM calls on its codes, nothing else (so that a
    rocprofv3 counter pass sees the dispatches of one shape only)."""
    import rotated_w4a8_group_amd as pq
    import synth
    wl = synth.WORKLOADS[name]
    dev = torch.device("cuda:0")
    M, K, N, G, P = wl.M, wl.K, wl.N, wl.G, wl.P
    pl, tl, cl = synth.rotations(wl)
    rec = torch.from_numpy(np.stack([pq.build_records(p, t) for p, t in zip(pl, tl)])).to(dev)
    cs = torch.from_numpy(np.stack(cl)).to(dev)
    x = torch.from_numpy(synth.activations(wl)).to(dev)
    w = synth.weights(wl)
    wpk, sz = pq.pack_weights(torch.from_numpy(w.qweight).to(dev), torch.from_numpy(w.qzeros).to(dev),
                              torch.from_numpy(w.scales).to(dev))
    A, S, R = pq.rotate_quant(x, rec, cs)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(1, pq.gemm_workspace_bytes(M, N, K)), dtype=torch.uint8, device=dev)
    for _ in range(calls):
        pq.gemm(A, S, R, wpk, sz, N, *wl.bounds, out=y, workspace=ws)
    torch.cuda.synchronize()
    print(json.dumps({"gemm_only": name, "M": M, "K": K, "N": N, "partitions": P, "calls": calls,
                      "algorithmic_bytes": gemm_bytes(M, K, N, P)}), flush=True)


def prologue_only(name, torch, np, calls=5):
    """One workload's prologues, `calls` launches each of pq_rotate_quant, pq_rotate_quant_tok and
    pq_rotate_quant_for_gemm, nothing else (for rocprofv3 counter passes over the prologue kernels)."""
    import rotated_w4a8_group_amd as pq
    import synth
    wl = synth.WORKLOADS[name]
    dev = torch.device("cuda:0")
    M, K, N = wl.M, wl.K, wl.N
    pl, tl, cl = synth.rotations(wl)
    rec = torch.from_numpy(np.stack([pq.build_records(p, t) for p, t in zip(pl, tl)])).to(dev)
    cs = torch.from_numpy(np.stack(cl)).to(dev)
    x = torch.from_numpy(synth.activations(wl)).to(dev)
    out = pq.rotate_quant(x, rec, cs)
    out_tok = pq.rotate_quant_tok(x, rec, cs)
    ws = torch.empty(max(1, pq.gemm_workspace_bytes(M, N, K)), dtype=torch.uint8, device=dev)
    for _ in range(calls):
        pq.rotate_quant(x, rec, cs, out=out)
    for _ in range(calls):
        pq.rotate_quant_tok(x, rec, cs, out=out_tok)
    for _ in range(calls):
        pq.rotate_quant_for_gemm(x, rec, cs, ws, out=out)
    torch.cuda.synchronize()
    print(json.dumps({"prologue_only": name, "M": M, "K": K, "partitions": wl.P, "calls": calls,
                      "algorithmic_bytes": prologue_bytes(M, K, wl.P)}), flush=True)


def config_measurement(wl, pq, torch, np, dev, copies, tok=False, i8=False, w5=False):
    """Prologue and GEMM of one workload timed separately: per-launch averages of HIP graphs that
    cycle through weight and activation copies when the call is short (M <= 16), else HIP events
    around eager calls alternating two copies (one such call streams far more than the 256 MB
    last-level cache)."""
    import synth
    M, K, N, G, P = wl.M, wl.K, wl.N, wl.G, wl.P
    short = M <= 16
    C = copies if short else 2
    x0 = synth.activations(wl)
    pl, tl, cl = synth.rotations(wl)
    rec = torch.from_numpy(np.stack([pq.build_records(p, t) for p, t in zip(pl, tl)])).to(dev)
    cs = torch.from_numpy(np.stack(cl)).to(dev)
    xs = [torch.from_numpy(x0).to(dev) for _ in range(C)]
    if w5:
        w = synth.weights5(wl)
        wq0 = pq.pack_weights5(*[torch.from_numpy(t).to(dev) for t in (w.qweight, w.qweight_hi, w.qzeros,
                                                                         w.qzeros_hi, w.scales)])
    else:
        w = synth.weights(wl)
        wq0 = pq.pack_weights(torch.from_numpy(w.qweight).to(dev), torch.from_numpy(w.qzeros).to(dev),
                              torch.from_numpy(w.scales).to(dev))
    wq = [wq0] + [(wq0[0].clone(), wq0[1].clone()) for _ in range(C - 1)]
    A = torch.empty((P, M, K), dtype=torch.int8 if i8 else torch.uint8, device=dev)
    S = torch.empty((P, M) if tok else (P, M, G), dtype=torch.float32, device=dev)
    R = torch.empty((P, M, G), dtype=torch.float32, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    if tok:
        ws = torch.empty(max(1, pq.gemm_tok_workspace_bytes(M, N, K)), dtype=torch.uint8, device=dev)
        pro = lambda i: pq.rotate_quant_tok(xs[i % C], rec, cs, out=(A, S, R))
        gem = lambda i: pq.gemm_tok(A, S, R, wq[i % C][0], wq[i % C][1], N, *wl.bounds, out=y, workspace=ws)
    elif i8:
        ws = torch.empty(max(1, pq.gemm_workspace_bytes(M, N, K)), dtype=torch.uint8, device=dev)
        pro = lambda i: pq.rotate_quant_i8(xs[i % C], rec, cs, out=(A, S, R))
        gem = lambda i: pq.gemm_i8(A, S, R, wq[i % C][0], wq[i % C][1], N, *wl.bounds, out=y, workspace=ws)
    elif w5:
        ws = torch.empty(max(1, pq.gemm_workspace_bytes(M, N, K)), dtype=torch.uint8, device=dev)
        pro = lambda i: pq.rotate_quant(xs[i % C], rec, cs, out=(A, S, R))
        gem = lambda i: pq.gemm5(A, S, R, wq[i % C][0], wq[i % C][1], N, *wl.bounds, out=y, workspace=ws)
    else:
        ws = torch.empty(max(1, pq.gemm_workspace_bytes(M, N, K)), dtype=torch.uint8, device=dev)
        pro = lambda i: pq.rotate_quant(xs[i % C], rec, cs, out=(A, S, R))
        gem = lambda i: pq.gemm(A, S, R, wq[i % C][0], wq[i % C][1], N, *wl.bounds, out=y, workspace=ws)

    def timed(fn, reps):
        for i in range(C):
            fn(i)
        torch.cuda.synchronize()
        if short:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for i in range(C):
                    fn(i)
            graph.replay()
            torch.cuda.synchronize()
            settle_clock(torch, lambda i: graph.replay(), 1)
            e = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
            for a, b in e:
                a.record()
                graph.replay()
                b.record()
            torch.cuda.synchronize()
            return spread([a.elapsed_time(b) * 1e-3 / C for a, b in e])
        settle_clock(torch, fn, C)
        e = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for i, (a, b) in enumerate(e):
            a.record()
            fn(i)
            b.record()
        torch.cuda.synchronize()
        return spread([a.elapsed_time(b) * 1e-3 for a, b in e])

    t_pro, p10, p90 = timed(pro, REPS_SHORT if short else REPS_LONG)
    t_gem, g10, g90 = timed(gem, REPS_SHORT if short else REPS_LONG)
    flops = 2.0 * M * N * K
    gb = gemm_bytes(M, K, N, P, w5=w5)
    res = {"M": M, "K": K, "N": N, "partitions": P,
           "prologue_us": round(t_pro * 1e6, 2), "prologue_us_p10_p90": [round(p10 * 1e6, 2), round(p90 * 1e6, 2)],
           "prologue_GBs": round(prologue_bytes(M, K, P) / t_pro / 1e9, 1),
           "gemm_us": round(t_gem * 1e6, 2), "gemm_us_p10_p90": [round(g10 * 1e6, 2), round(g90 * 1e6, 2)],
           "gemm_TFLOPs": round(flops / t_gem / 1e12, 2), "gemm_bytes": gb, "gemm_GBs": round(gb / t_gem / 1e9, 1)}
    if short:
        res["roofline"] = {"bound": "hbm", "frac": round(gb / t_gem / 1e9 / PEAK_HBM_GBS, 4)}
        res["timing"] = f"HIP graph of {C} launches over {C} copies, per-launch median (p10, p90) of {REPS_SHORT} replays after ~30 ms of untimed replays"
    else:
        res["roofline"] = {"bound": "mfma", "frac": round(flops / t_gem / 1e12 / PEAK_FP8_TFLOPS, 4)}
        res["timing"] = f"HIP events around each eager call, median (p10, p90) of {REPS_LONG} after ~30 ms of untimed calls, two alternating copies"
    del xs, wq, A, S, R, y, ws
    torch.cuda.empty_cache()
    return res


def oracle_config_time(wl, rows):
    """Wall seconds of the oracle (prologue float32 emulation, then the fp64 GEMM) on the first
    `rows` token rows of a workload, and that time scaled to all M rows (both parts are linear in
    the rows)."""
    import numpy as np
    import synth
    from oracle import gemm as ogemm
    from oracle import prologue as opro
    x = synth.activations(wl)[:rows]
    pl, tl, cl = synth.rotations(wl)
    w = synth.weights(wl)
    t0 = time.perf_counter()
    A, S, _ = opro.rotate_quant(x, pl, tl, cl)
    t1 = time.perf_counter()
    ogemm.gemm_ref(A, S, w.qweight, w.qzeros, w.scales, *wl.bounds)
    t2 = time.perf_counter()
    scale = wl.M / rows
    return {"rows": rows, "prologue_s": round(t1 - t0, 3), "gemm_s": round(t2 - t1, 3),
            "full_s_estimate": round((t2 - t0) * scale, 2)}


def cpu_baseline(x0, pl, tl, cl, w, wl):
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import gemm as ogemm
    from oracle import prologue as opro

    rows = np.arange(wl.M)
    t0 = time.perf_counter()
    A, S, _ = opro.rotate_quant(x0[rows], pl, tl, cl)
    ogemm.gemm_ref(A, S, w.qweight, w.qzeros, w.scales, *wl.bounds)
    dt = time.perf_counter() - t0
    flops = 2.0 * len(rows) * wl.N * wl.K
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "cpu_model": model, "affinity_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{len(rows)} of {wl.M} token rows, all {wl.N} columns, prologue + GEMM "
                      f"({dt:.1f} s wall; BLAS threads for the per-group fp64 products)"}, dt


if __name__ == "__main__":
    main()
