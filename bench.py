#!/usr/bin/env python3
"""Benchmark of the Q2_K weight path on one MI355X.

Timed step: one q2k_matmul call on the decode GEMV workload (M = 1, N = K =
4096, Q2_K weights, f32 activations), the workload the headline metric is
quoted on. Each step reads a different one of R byte-identical weight replicas
(R * 5.5 MB >= 512 MiB, twice the 256 MiB Infinity Cache), so every step
streams its weights from HBM. The other rows of the path (dequantize, gather,
M = 8 GEMV, M = 512 matrix-core GEMM) are timed after the headline region and
reported under "rows". The CPU oracle is timed on the host cores on a bounded
sample and reported as "cpu_baseline".

Prints one JSON line on stdout; progress goes to stderr.
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
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, 8 TB/s
BF16_PEAK_TFLOPS = 2516.6       # MI355X dense bf16 matrix (no sparsity)
FP32_PEAK_TFLOPS = 157.3        # MI355X fp32 vector
METRIC = "Q2_K matmul: GEMV HBM GB/s (M=1) and TFLOP/s at M=512, % of roofline"
COLD_BYTES = 512 << 20          # rotate replicas over at least this many bytes
KERNEL_SRC = os.path.join(ROOT, "ggml_q2_dequant_amd", "csrc", "q2k_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg: str) -> None:
    print("[bench] " + msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(kernel: str):
    """HBM bytes per launch recorded from rocprofv3 counters for the current kernel source, else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(kernel)
    if not ent or ent.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return ent.get("hbm_bytes_per_launch")


def time_launches(torch, launch, n: int, warmup: int):
    """Average device time per launch over n back-to-back launches (events on the launch stream)."""
    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(n):
        launch(i)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / n * 1e-3  # seconds per launch


def cpu_baseline(inp, budget_s: float):
    """Time the oracle on the whole decode-GEMV workload, repeated to fill ~budget_s."""
    import oracle
    c = inp.config
    threads = oracle.host_threads()
    oracle.matmul(inp.x, inp.blocks, c.M, c.N, c.K, nthreads=threads)  # warm (build, page-in)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.matmul(inp.x, inp.blocks, c.M, c.N, c.K, nthreads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 10000:
            break
    return el / reps, threads, reps


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-rows", action="store_true", help="skip the per-row measurements")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import ggml_q2_dequant_amd as q2k
    import synth

    q2k.load_library()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream().cuda_stream

    # ---------------------------------------------------------------- headline: decode GEMV
    log("generating decode GEMV inputs")
    inp1 = synth.make_inputs(1)
    c1 = inp1.config
    w_bytes = inp1.blocks.size
    algo_bytes = w_bytes + c1.M * c1.K * 4 + c1.M * c1.N * 4
    reps = max(1, math.ceil(COLD_BYTES / w_bytes))
    w_host = torch.from_numpy(inp1.blocks)
    replicas = [w_host.to(dev) for _ in range(reps)]
    x1 = torch.from_numpy(inp1.x).to(dev)
    y1 = torch.empty((c1.M, c1.N), dtype=torch.float32, device=dev)
    lib = q2k.load_library()

    def gemv_step(i):
        rc = lib.q2k_matmul(x1.data_ptr(), replicas[i % reps].data_ptr(), y1.data_ptr(), c1.M, c1.N, c1.K, stream)
        if rc:
            raise RuntimeError(lib.q2k_last_error_message().decode())

    log("timing %d GEMV steps (%d warmup) over %d weight replicas" % (args.steps, args.warmup, reps))
    for i in range(args.warmup):
        gemv_step(i)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record()
    for i in range(args.steps):
        gemv_step(i)
    t_end.record()
    torch.cuda.synchronize()
    sec_per_step = t_start.elapsed_time(t_end) * 1e-3 / args.steps
    gbs = algo_bytes / sec_per_step / 1e9
    log("GEMV M=1: %.3f us/step, %.1f GB/s" % (sec_per_step * 1e6, gbs))

    rows = {}
    if not args.no_rows:
        # ------------------------------------------------------------ dequantize (write-bound stream)
        out_dq = torch.empty(w_bytes // 84 * 256, dtype=torch.float32, device=dev)
        dq_bytes = w_bytes + out_dq.numel() * 4
        t = time_launches(torch, lambda i: q2k.q2k_dequantize(replicas[i % reps], out_dq, stream=stream), 200, 20)
        rows["dequantize"] = {"workload": "%d blocks (the decode GEMV weights)" % (w_bytes // 84),
                              "us": t * 1e6, "GB/s": dq_bytes / t / 1e9,
                              "frac_hbm": dq_bytes / t / 1e9 / HBM_PEAK_GBS}
        log("dequantize: %.2f us, %.1f GB/s" % (t * 1e6, dq_bytes / t / 1e9))
        del out_dq

        # ------------------------------------------------------------ gather
        log("generating gather inputs")
        inp2 = synth.make_inputs(2)
        c2 = inp2.config
        table = torch.from_numpy(inp2.blocks).to(dev)
        rng = np.random.Generator(np.random.PCG64(2000))
        id_sets = [torch.from_numpy(rng.integers(0, c2.vocab, c2.n_tokens).astype(np.int32)).to(dev)
                   for _ in range(64)]
        outs = [torch.empty((c2.n_tokens, c2.embed_dim), dtype=torch.float32, device=dev) for _ in range(8)]
        g_bytes = c2.n_tokens * (c2.embed_dim // 256) * 84 + c2.n_tokens * c2.embed_dim * 4 + c2.n_tokens * 4
        t = time_launches(torch, lambda i: q2k.q2k_embedding_gather(table, id_sets[i % 64], outs[i % 8], c2.vocab,
                                                                    c2.embed_dim, c2.n_tokens, stream=stream),
                          200, 20)
        rows["gather"] = {"workload": "512 ids into a 262144 x 4096 table (64 rotating id sets)",
                          "us_per_call_incl_sync": t * 1e6, "GB/s": g_bytes / t / 1e9,
                          "frac_hbm": g_bytes / t / 1e9 / HBM_PEAK_GBS}
        log("gather: %.2f us/call (synchronous), %.1f GB/s" % (t * 1e6, g_bytes / t / 1e9))
        del table, outs, id_sets, inp2

        # ------------------------------------------------------------ M = 8 GEMV
        log("generating M=8 GEMV inputs")
        inp3 = synth.make_inputs(3)
        c3 = inp3.config
        w3 = torch.from_numpy(inp3.blocks)
        reps3 = max(1, math.ceil(COLD_BYTES / inp3.blocks.size))
        w3r = [w3.to(dev) for _ in range(reps3)]
        x3 = torch.from_numpy(inp3.x).to(dev)
        y3 = torch.empty((c3.M, c3.N), dtype=torch.float32, device=dev)
        t = time_launches(torch, lambda i: q2k.q2k_matmul(x3, w3r[i % reps3], y3, c3.M, c3.N, c3.K, stream=stream),
                          300, 30)
        b3 = inp3.blocks.size + c3.M * c3.K * 4 + c3.M * c3.N * 4
        f3 = 2.0 * c3.M * c3.N * c3.K
        rows["gemv_m8"] = {"workload": "M=8 N=14336 K=4096 (%d weight replicas)" % reps3, "us": t * 1e6,
                           "GB/s": b3 / t / 1e9, "TFLOP/s": f3 / t / 1e12,
                           "frac_hbm": b3 / t / 1e9 / HBM_PEAK_GBS, "frac_fp32": f3 / t / 1e12 / FP32_PEAK_TFLOPS}
        log("GEMV M=8: %.2f us, %.1f GB/s, %.2f TFLOP/s" % (t * 1e6, b3 / t / 1e9, f3 / t / 1e12))
        del w3r

        # ------------------------------------------------------------ M = 512 matrix-core path
        log("generating M=512 inputs")
        inp4 = synth.make_inputs(4)
        c4 = inp4.config
        w4 = torch.from_numpy(inp4.blocks).to(dev)
        x4 = torch.from_numpy(inp4.x).to(dev)
        y4 = torch.empty((c4.M, c4.N), dtype=torch.float32, device=dev)
        t = time_launches(torch, lambda i: q2k.q2k_matmul(x4, w4, y4, c4.M, c4.N, c4.K, stream=stream), 50, 5)
        f4 = 2.0 * c4.M * c4.N * c4.K
        rows["mfma_m512"] = {"workload": "M=512 N=14336 K=4096", "us": t * 1e6, "TFLOP/s": f4 / t / 1e12,
                             "frac_bf16_mfma": f4 / t / 1e12 / BF16_PEAK_TFLOPS}
        log("MFMA M=512: %.2f us, %.1f TFLOP/s" % (t * 1e6, f4 / t / 1e12))
        del w4, x4, y4

    # ---------------------------------------------------------------- CPU oracle baseline
    log("timing the CPU oracle (~%.0f s)" % args.cpu_seconds)
    sec_cpu, threads, cpu_reps = cpu_baseline(inp1, args.cpu_seconds)
    cpu_gbs = algo_bytes / sec_cpu / 1e9

    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": sec_per_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": c1.name + " (Q2_K weights, f32 activations, cold weights)",
                   "M": c1.M, "N": c1.N, "K": c1.K, "weight_replicas": reps,
                   "algorithmic_bytes_per_step": algo_bytes, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": measured_traffic("k_gemv_m1")},
        "cpu_baseline": {"value": round(cpu_gbs, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
                         "sample": "the whole decode GEMV workload (M=1, N=K=4096), %d calls of the f64 "
                                   "oracle matmul, %.3f s per call" % (cpu_reps, sec_cpu)},
        "rows": rows,
        "input_sha256": inp1.hashes,
    }
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
