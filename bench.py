#!/usr/bin/env python3
"""Benchmark of the Q2_K weight path on one MI355X.

Timed step: one q2k_matmul call on the decode GEMV workload (M = 1, N = K =
4096, Q2_K weights, f32 activations), the workload the headline metric is
quoted on. Each step reads a different one of R byte-identical weight replicas
(R * 5.5 MB >= 512 MiB, twice the 256 MiB Infinity Cache), so every step
streams its weights from HBM. Before the K timed steps a 768 MiB read of other
memory leaves nothing they read in a cache; they are then issued back to back
behind a GPU spin long enough for the host to queue them all, and timed with
events on the launch stream, so the figure is the GPU's and not the host's
launch rate. A HIP-graph replay of the same steps and host-paced launches are
reported beside it. The other rows of the path (dequantize, gather,
M = 8 GEMV, M = 512 matrix-core GEMM, batched mat-vec, argmax + candidates, expert-routed decode and
prefill) are timed after the headline region and
reported under "rows", each against the roofline that bounds it, timed the
same way (the synchronous gather, which waits on the host in every call,
without the spin). The CPU
oracle is timed on the host cores on a bounded sample and reported as
"cpu_baseline".

Other modes (used to collect rocprofv3 counters; they print one short JSON line):
  --only ROW         run only one row's timed loop, launches issued eagerly (gemv1, dequant, gather,
                     gemv1_wide, gemv8, mfma, mfma_context, batched, sample, moe_decode, moe_prefill)
  --copy-probe       also run a device-to-device copy of COPY_BYTES (counter calibration)
  --no-context       skip the M=512 context timings (used when profiling every kernel, so the
                     GEMM's statistics hold only the row's own calls)
  --sweep            M=1 GEMV over N = 4096 .. 131072 (K = 4096, cold) beside the plain-read ceiling
  --derive-traffic FETCH_CSV WRITE_CSV KEY
                     turn two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) of
                     `--only ROW --copy-probe` into HBM bytes per launch of that row's kernel,
                     recorded in profiles/traffic.json under KEY (k_gemv_m1, k_dequantize,
                     k_gather, k_gemv_m8): each counter scaled by known bytes / what it reads
                     for the copy.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import ctypes
import csv
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
COPY_BYTES = 256 << 20          # size of the calibration copy
KERNEL_SRC = os.path.join(ROOT, "ggml_q2_dequant_amd", "csrc", "q2k_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
PROBE_LIB = os.path.join(ROOT, "ggml_q2_dequant_amd", "libq2k_probe.so")
PROBE_GRIDS = (256, 512, 1024, 2048, 4096, 8192, 16384)
PROBE_UNROLLS = (1, 2, 4, 8, 16)
COPY_KERNEL = "__amd_rocclr_copyBuffer"
# Rows whose HBM bytes come from counters: key -> (--only row, kernel name fragment in rocprofv3 output,
# algorithmic bytes per launch).
TRAFFIC_ROWS = {
    "k_gemv_m1": ("gemv1", "k_gemv_seg<1", 5537792),
    "k_dequantize": ("dequant", "k_dequantize", 65536 * 84 + 65536 * 1024),
    "k_gather": ("gather", "k_gather(", 9078784),  # not k_gather_done
    "k_gemv_m8": ("gemv8", "k_gemv_mfma", 19857408),
}
ROWS = ("gemv1", "dequant", "gather", "gemv1_wide", "gemv8", "mfma", "mfma_context", "batched", "sample",
        "moe_decode", "moe_prefill")


def log(msg: str) -> None:
    print("[bench] " + msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_row(key: str):
    """{hbm_bytes_per_launch, over_algorithmic} from the counters recorded for the current kernel source, else None."""
    hbm = measured_traffic(key)
    if hbm is None:
        return None
    return {"hbm_bytes_per_launch": hbm, "over_algorithmic": round(hbm / TRAFFIC_ROWS[key][2], 4)}


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


_probe = None


def load_probe():
    """libq2k_probe.so: the plain-read kernel timed beside the path (a measurement aid, not the C ABI)."""
    global _probe
    if _probe is None:
        if not os.path.exists(PROBE_LIB):
            raise RuntimeError("libq2k_probe.so is not built; run `python -m ggml_q2_dequant_amd.build`")
        lib = ctypes.CDLL(PROBE_LIB)
        P, U32, SZ = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_size_t
        lib.q2k_probe_read.argtypes = [P, SZ, P, SZ, U32, U32, P]
        lib.q2k_probe_read.restype = ctypes.c_int
        lib.q2k_probe_default_grid.argtypes = [SZ, U32]
        lib.q2k_probe_default_grid.restype = U32
        _probe = lib
    return _probe


FLUSH_BYTES = 768 << 20         # read before each timed region: more than the Infinity Cache and the L2s hold
_flush = {}
EAGER_ONLY = [False]            # --only: launch eagerly (profiler runs count kernels, they need no graphs)


def flush_caches(torch):
    """Read FLUSH_BYTES of other memory on the current stream, so nothing a timed region reads next is still in
    the Infinity Cache or an L2 (its inputs are then cold unless the region itself reuses them)."""
    if "buf" not in _flush:
        _flush["buf"] = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda:0")
        _flush["sink"] = torch.empty(16384, dtype=torch.int32, device="cuda:0")
    b, sink = _flush["buf"], _flush["sink"]
    rc = load_probe().q2k_probe_read(b.data_ptr(), b.numel(), sink.data_ptr(), sink.numel(), 0, 4,
                                     torch.cuda.current_stream().cuda_stream)
    if rc:
        raise RuntimeError("flush read rejected (%d)" % rc)


_spin = {}


def gpu_spin(torch, us: float = 2000.0):
    """Keep the GPU busy for about `us` microseconds (a spin kernel on the current stream) while the host submits
    the timed work, so the timer starts with that work already queued and host launch cost does not show in it.
    The spin's cycles per microsecond are measured once with events."""
    sleep = getattr(torch.cuda, "_sleep", None)
    if sleep is None:
        return
    if "cyc_per_us" not in _spin:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        sleep(1_000_000)
        torch.cuda.synchronize()
        a.record()
        sleep(4_000_000)
        b.record()
        torch.cuda.synchronize()
        _spin["cyc_per_us"] = 4_000_000 / max(a.elapsed_time(b) * 1e3, 1.0)
    sleep(int(min(us, 200_000.0) * _spin["cyc_per_us"]))


def time_launches(torch, launch, n: int, warmup: int, graph: bool = False, spin: bool = True):
    """Average time per launch over n back-to-back launches on the current stream, from events on that stream.

    The caches are flushed first (the launches' inputs are cold unless they reuse them among themselves). By
    default the n launches are issued eagerly behind a GPU spin long enough for the host to queue them all, so
    the figure is the GPU's time for the n calls and not the host's rate of issuing them. graph=True captures the
    n launches in a HIP graph instead and times one replay (after an untimed one). Calls that wait on the host
    (the synchronous gather) cannot be queued ahead: EAGER_ONLY or a host wait inside a call makes the spin moot,
    and the figure then includes the host's part."""
    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if EAGER_ONLY[0]:
        start.record(s)
        for i in range(n):
            launch(i)
        end.record(s)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / n * 1e-3
    g = None
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for i in range(n):
                launch(i)
        g.replay()
        torch.cuda.synchronize()
    flush_caches(torch)
    if spin:
        gpu_spin(torch, 500.0 + 40.0 * n)
    start.record(s)
    if g is not None:
        g.replay()
    else:
        for i in range(n):
            launch(i)
    end.record(s)
    torch.cuda.synchronize()
    del g
    return start.elapsed_time(end) / n * 1e-3  # seconds per launch


def time_blocks(torch, launch, blocks: int = 50, per: int = 20, warmup: int = 20):
    """Spread of the per-call time: `blocks` runs of `per` back-to-back calls, one event between runs (an event
    before every call would stall the queue on each one); p10, p50, p90 and mean of the run averages, seconds."""
    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(blocks + 1)]
    ev[0].record()
    for j in range(blocks):
        for i in range(per):
            launch(j * per + i)
        ev[j + 1].record()
    torch.cuda.synchronize()
    per_call = sorted(ev[j].elapsed_time(ev[j + 1]) * 1e-3 / per for j in range(blocks))
    pick = lambda q: per_call[min(blocks - 1, int(q * blocks))]
    return {"mean": ev[0].elapsed_time(ev[blocks]) * 1e-3 / (blocks * per), "p10": pick(0.10), "p50": pick(0.50),
            "p90": pick(0.90)}


def dist_us(d):
    return {k: round(v * 1e6, 3) for k, v in d.items()}


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


# --------------------------------------------------------------------------- rocprofv3 counters

def _per_dispatch(path: str, counter: str):
    """{kernel name: [per-dispatch value]} for one counter of a rocprofv3 counter_collection.csv."""
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def _pick(vals: dict, prefix: str):
    got = [v for name, v in vals.items() if prefix in name]
    if not got:
        raise SystemExit("no dispatches of %r in the counter file" % prefix)
    return [x for lst in got for x in lst]


def derive_traffic(fetch_csv: str, write_csv: str, key: str) -> int:
    """HBM bytes per launch of one row's kernel from a FETCH_SIZE and a WRITE_SIZE counter run of
    `bench.py --only ROW --copy-probe`, each scaled by the known size of the calibration copy over what the same
    counter reads for it; recorded in profiles/traffic.json under `key` with the kernel source's hash."""
    if key not in TRAFFIC_ROWS:
        raise SystemExit("unknown traffic key %r (one of %s)" % (key, ", ".join(TRAFFIC_ROWS)))
    row, kernel, algo = TRAFFIC_ROWS[key]
    fetch = _per_dispatch(fetch_csv, "FETCH_SIZE")
    write = _per_dispatch(write_csv, "WRITE_SIZE")
    copy_f = max(_pick(fetch, COPY_KERNEL))   # the calibration copy is the largest copy dispatch
    copy_w = max(_pick(write, COPY_KERNEL))
    known_kib = COPY_BYTES / 1024.0
    rs, ws = known_kib / copy_f, known_kib / copy_w
    gf, gw = _pick(fetch, kernel), _pick(write, kernel)
    f_kib, w_kib = sum(gf) / len(gf), sum(gw) / len(gw)
    hbm = (f_kib * rs + w_kib * ws) * 1024.0
    rec = {}
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        pass
    rec[key] = {
        "kernel_source_sha256": kernel_source_hash(),
        "hbm_bytes_per_launch": round(hbm), "algorithmic_bytes_per_launch": algo,
        "traffic_over_algorithmic": hbm / algo,
        "fetch_kib_per_launch": f_kib, "write_kib_per_launch": w_kib,
        "copy_bytes": COPY_BYTES, "copy_fetch_kib": copy_f, "copy_write_kib": copy_w,
        "read_scale": rs, "write_scale": ws, "launches": len(gf),
        "how": "rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE of `bench.py --only %s --copy-probe`; each counter "
               "scaled by known bytes / its reading for a %d-byte device copy" % (row, COPY_BYTES),
    }
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps({key: rec[key]}))
    return 0


# --------------------------------------------------------------------------- workloads

class Bench:
    def __init__(self, torch, q2k, synth, np):
        self.torch, self.q2k, self.synth, self.np = torch, q2k, synth, np
        self.dev = torch.device("cuda:0")
        # Every call runs on this stream (made current by main): HIP graphs cannot capture the null stream.
        self.stream = torch.cuda.current_stream().cuda_stream
        if self.stream == 0:
            raise RuntimeError("run the benchmark on a side stream")

    def gemv1_setup(self):
        inp = self.synth.make_inputs(1)
        c = inp.config
        reps = max(1, math.ceil(COLD_BYTES / inp.blocks.size))
        w_host = self.torch.from_numpy(inp.blocks)
        self.g1 = dict(inp=inp, reps=reps, replicas=[w_host.to(self.dev) for _ in range(reps)],
                       x=self.torch.from_numpy(inp.x).to(self.dev),
                       y=self.torch.empty((c.M, c.N), dtype=self.torch.float32, device=self.dev),
                       bytes=inp.blocks.size + c.M * c.K * 4 + c.M * c.N * 4)
        lib = self.q2k.load_library()
        g = self.g1

        def make_step(st):
            def step(i):
                rc = lib.q2k_matmul(g["x"].data_ptr(), g["replicas"][i % reps].data_ptr(), g["y"].data_ptr(),
                                    c.M, c.N, c.K, st)
                if rc:
                    raise RuntimeError(lib.q2k_last_error_message().decode())
            return step
        g["make_step"] = make_step
        return make_step(self.stream)

    def read_ceiling(self, replicas, n=200, sweep=False):
        """Plain streaming read of the same cold replicas (libq2k_probe): the bandwidth a transfer of this size
        can reach at all. The default shape is the GEMV's (a few hundred 256-thread workgroups, four 16-byte
        loads per thread); with sweep=True every workgroup count x loads-per-thread pair that covers the bytes
        is timed, and a device-to-device copy of the same bytes (it also writes them) is timed beside it; the
        fastest read shape is the ceiling reported."""
        torch = self.torch
        probe = load_probe()
        sink = torch.empty(max(PROBE_GRIDS), dtype=torch.int32, device=self.dev)
        views = [r[: r.numel() // 16 * 16] for r in replicas]
        b = views[0].numel()
        st = self.stream

        def timed(grid, unroll):
            def launch(i):
                rc = probe.q2k_probe_read(views[i % len(views)].data_ptr(), b, sink.data_ptr(), sink.numel(), grid,
                                          unroll, st)
                if rc:
                    raise RuntimeError("q2k_probe_read rejected its arguments (%d)" % rc)
            return time_launches(torch, launch, n, 20)

        t = timed(0, 4)
        out = {"bytes": b, "us": t * 1e6, "GB/s": b / t / 1e9,
               "shape": {"grid": int(probe.q2k_probe_default_grid(b, 4)), "loads_per_thread": 4}}
        if not sweep or EAGER_ONLY[0]:
            return out
        shapes = []
        for grid in PROBE_GRIDS:
            for unroll in PROBE_UNROLLS:
                if grid * 256 * unroll * 16 > 4 * b and unroll > 1:
                    continue  # more loads in flight than the buffer holds: same as a smaller unroll
                ts = timed(grid, unroll)
                shapes.append({"grid": grid, "loads_per_thread": unroll, "us": round(ts * 1e6, 3),
                               "GB/s": round(b / ts / 1e9, 1)})
        best = min(shapes, key=lambda e: e["us"])
        dst = torch.empty_like(views[0])
        tc = time_launches(torch, lambda i: dst.copy_(views[i % len(views)]), n, 20)
        out.update(sweep=shapes, best={"grid": best["grid"], "loads_per_thread": best["loads_per_thread"],
                                       "us": best["us"], "GB/s": best["GB/s"]},
                   d2d_copy={"us": round(tc * 1e6, 3), "read_GB/s": round(b / tc / 1e9, 1),
                             "note": "hipMemcpyAsync device to device of the same bytes (reads and writes them)"})
        return out

    def write_ceiling(self, outs, n=200):
        """torch's own fill kernel over the same output buffers: the bandwidth a plain write of this size reaches."""
        torch = self.torch  # fills run on torch's current stream, the stream the library calls use
        t = time_launches(torch, lambda i: outs[i % len(outs)].zero_(), n, 20)
        b = outs[0].numel() * outs[0].element_size()
        return {"bytes": b, "us": t * 1e6, "GB/s": b / t / 1e9}

    def dequant(self, n=200):
        g = self.g1
        w_bytes = g["inp"].blocks.size
        out = self.torch.empty(w_bytes // 84 * 256, dtype=self.torch.float32, device=self.dev)
        b = w_bytes + out.numel() * 4
        t = time_launches(self.torch, lambda i: self.q2k.q2k_dequantize(g["replicas"][i % g["reps"]], out,
                                                                        stream=self.stream), n, 20)
        gbs = b / t / 1e9
        log("dequantize: %.2f us, %.1f GB/s" % (t * 1e6, gbs))
        return {"workload": "%d blocks (the decode GEMV weights), cold replicas" % (w_bytes // 84),
                "us": t * 1e6, "algorithmic_bytes": b, "GB/s": gbs, "bound": "hbm",
                "frac_hbm": gbs / HBM_PEAK_GBS, "write_ceiling": self.write_ceiling([out]),
                "traffic": traffic_row("k_dequantize")}

    def gather(self, n=200):
        np, torch = self.np, self.torch
        log("generating gather inputs")
        inp = self.synth.make_inputs(2)
        c = inp.config
        table = torch.from_numpy(inp.blocks).to(self.dev)
        rng = np.random.Generator(np.random.PCG64(2000))
        id_sets = [torch.from_numpy(rng.integers(0, c.vocab, c.n_tokens).astype(np.int32)).to(self.dev)
                   for _ in range(64)]
        outs = [torch.empty((c.n_tokens, c.embed_dim), dtype=torch.float32, device=self.dev) for _ in range(8)]
        b = c.n_tokens * (c.embed_dim // 256) * 84 + c.n_tokens * c.embed_dim * 4 + c.n_tokens * 4
        t = time_launches(torch, lambda i: self.q2k.q2k_embedding_gather(table, id_sets[i % 64], outs[i % 8],
                                                                         c.vocab, c.embed_dim, c.n_tokens,
                                                                         stream=self.stream), n, 20, spin=False)
        gbs = b / t / 1e9
        log("gather: %.2f us/call (synchronous), %.1f GB/s" % (t * 1e6, gbs))
        # The asynchronous entry point on the same calls: back-to-back launches, one status word checked
        # once after the timed region.
        status = torch.zeros(1, dtype=torch.int32, device=self.dev)
        ta = time_launches(torch, lambda i: self.q2k.q2k_embedding_gather_async(
            table, id_sets[i % 64], outs[i % 8], c.vocab, c.embed_dim, c.n_tokens, status, stream=self.stream), n, 20)
        if int(status.item()) != 0:
            raise RuntimeError("gather: a valid id set raised the status word")
        log("gather: %.2f us/call (asynchronous), %.1f GB/s" % (ta * 1e6, b / ta / 1e9))
        return {"workload": "512 ids into a 262144 x 4096 table (64 rotating id sets); the call waits for "
                            "its id check", "us_per_call_incl_sync": t * 1e6, "algorithmic_bytes": b,
                "GB/s": gbs, "bound": "hbm", "frac_hbm": gbs / HBM_PEAK_GBS,
                "async": {"us_per_call": ta * 1e6, "GB/s": b / ta / 1e9, "frac_hbm": b / ta / 1e9 / HBM_PEAK_GBS},
                "write_ceiling": self.write_ceiling(outs), "traffic": traffic_row("k_gather")}

    def gemv1_wide(self, n=100):
        """M=1 GEMV at N=65536, K=4096 (352 MB of weights per call, two cold replicas): the large-N decode shape
        (an LM-head-sized or expert-sized matrix), where the GEMV is limited by instruction issue, not HBM."""
        torch, np = self.torch, self.np
        N, K = 65536, 4096
        rng = np.random.Generator(np.random.PCG64(5000 + N))
        blocks = self.synth.random_blocks(rng, N * K // 256)
        reps = max(2, math.ceil(COLD_BYTES / blocks.size))
        wh = torch.from_numpy(blocks)
        wr = [wh.to(self.dev) for _ in range(reps)]
        x = torch.from_numpy(rng.standard_normal((1, K), dtype=np.float32)).to(self.dev)
        y = torch.empty((1, N), dtype=torch.float32, device=self.dev)
        t = time_launches(torch, lambda i: self.q2k.q2k_matmul(x, wr[i % reps], y, 1, N, K, stream=self.stream), n,
                          10)
        b = blocks.size + 4 * K + 4 * N
        log("GEMV M=1 N=65536: %.2f us, %.1f GB/s" % (t * 1e6, b / t / 1e9))
        return {"workload": "M=1 N=65536 K=4096 (%d cold weight replicas)" % reps, "us": t * 1e6,
                "algorithmic_bytes": b, "GB/s": b / t / 1e9, "bound": "hbm", "frac_hbm": b / t / 1e9 / HBM_PEAK_GBS,
                "read_ceiling": self.read_ceiling(wr, 50, sweep=True)}

    def gemv8(self, n=300):
        torch = self.torch
        log("generating M=8 GEMV inputs")
        inp = self.synth.make_inputs(3)
        c = inp.config
        w3 = torch.from_numpy(inp.blocks)
        reps = max(1, math.ceil(COLD_BYTES / inp.blocks.size))
        wr = [w3.to(self.dev) for _ in range(reps)]
        x = torch.from_numpy(inp.x).to(self.dev)
        y = torch.empty((c.M, c.N), dtype=torch.float32, device=self.dev)
        t = time_launches(torch, lambda i: self.q2k.q2k_matmul(x, wr[i % reps], y, c.M, c.N, c.K,
                                                               stream=self.stream), n, 30)
        b = inp.blocks.size + c.M * c.K * 4 + c.M * c.N * 4
        f = 2.0 * c.M * c.N * c.K
        log("GEMV M=8: %.2f us, %.1f GB/s, %.2f TFLOP/s" % (t * 1e6, b / t / 1e9, f / t / 1e12))
        return {"workload": "M=8 N=14336 K=4096 (%d cold weight replicas)" % reps, "us": t * 1e6,
                "algorithmic_bytes": b, "flop": f, "GB/s": b / t / 1e9, "TFLOP/s": f / t / 1e12,
                "bound": "hbm", "frac_hbm": b / t / 1e9 / HBM_PEAK_GBS,
                "frac_fp32": f / t / 1e12 / FP32_PEAK_TFLOPS, "read_ceiling": self.read_ceiling(wr, 100, sweep=True),
                "traffic": traffic_row("k_gemv_m8")}

    def mfma(self, n=400):
        torch = self.torch
        log("generating M=512 inputs")
        inp = self.synth.make_inputs(4)
        c = inp.config
        w = torch.from_numpy(inp.blocks).to(self.dev)
        x = torch.from_numpy(inp.x).to(self.dev)
        y = torch.empty((c.M, c.N), dtype=torch.float32, device=self.dev)
        # Enough calls (about 30 ms) that the clock has settled; a short run reads 10 % slow.
        call = lambda i: self.q2k.q2k_matmul(x, w, y, c.M, c.N, c.K, stream=self.stream)
        t = time_launches(torch, call, n, n // 10)
        torch.cuda.synchronize()
        want = y.clone()
        y.fill_(float("nan"))
        tg = time_launches(torch, call, n, n // 10, graph=True)
        torch.cuda.synchronize()
        if not torch.equal(y.view(torch.int32), want.view(torch.int32)):
            raise RuntimeError("M=512: graph replay differs from the eager result")
        f = 2.0 * c.M * c.N * c.K
        log("MFMA M=512: %.2f us, %.1f TFLOP/s (graph replay: %.2f us)" % (t * 1e6, f / t / 1e12, tg * 1e6))
        return {"workload": "M=512 N=14336 K=4096 (one call: bf16(x) pre-pass + GEMM)", "us": t * 1e6,
                "flop": f, "TFLOP/s": f / t / 1e12, "bound": "mfma",
                "frac_bf16_mfma": f / t / 1e12 / BF16_PEAK_TFLOPS,
                "graph_replay": {"us": tg * 1e6, "TFLOP/s": f / tg / 1e12,
                                 "frac_bf16_mfma": f / tg / 1e12 / BF16_PEAK_TFLOPS}}

    def mfma_context(self, n=400):
        """Context for the M=512 row, not part of the path: the same call with all-zero activations (the
        part's clock is power-managed and matrix-core power depends on the operand bits), and torch's own
        bf16 linear layer on the same shape with both operands already bf16 in memory (no decode, no
        conversion)."""
        torch = self.torch
        inp = self.synth.make_inputs(4)
        c = inp.config
        w = torch.from_numpy(inp.blocks).to(self.dev)
        x0 = torch.zeros((c.M, c.K), dtype=torch.float32, device=self.dev)
        y = torch.empty((c.M, c.N), dtype=torch.float32, device=self.dev)
        t0 = time_launches(torch, lambda i: self.q2k.q2k_matmul(x0, w, y, c.M, c.N, c.K, stream=self.stream), n,
                           n // 10)
        x16 = torch.from_numpy(inp.x).to(self.dev).to(torch.bfloat16)
        w16 = torch.randn((c.N, c.K), dtype=torch.float32, device=self.dev).to(torch.bfloat16)
        tv = time_launches(torch, lambda i: torch.nn.functional.linear(x16, w16), n, n // 10)
        f = 2.0 * c.M * c.N * c.K
        log("M=512 context: same call on zero activations %.2f us; torch bf16 linear, same shape %.2f us" % (
            t0 * 1e6, tv * 1e6))
        return {"zero_activations_us": t0 * 1e6,
                "torch_bf16_linear_same_shape": {"us": tv * 1e6, "TFLOP/s": f / tv / 1e12,
                                                 "frac_bf16_mfma": f / tv / 1e12 / BF16_PEAK_TFLOPS}}

    def batched(self, n=200):
        """Batched mat-vec: 8 independent decode GEMVs (M=1, N=K=4096) in one call, cold weights."""
        torch, np = self.torch, self.np
        bt, M, N, K = 8, 1, 4096, 4096
        rng = np.random.Generator(np.random.PCG64(3000))
        blocks = self.synth.random_blocks(rng, bt * N * K // 256)
        x = torch.from_numpy(rng.standard_normal((bt, M, K), dtype=np.float32)).to(self.dev)
        reps = max(1, math.ceil(COLD_BYTES / blocks.size))
        wh = torch.from_numpy(blocks)
        wr = [wh.to(self.dev) for _ in range(reps)]
        y = torch.empty((bt, M, N), dtype=torch.float32, device=self.dev)
        t = time_launches(torch, lambda i: self.q2k.q2k_matmul_batched(x, wr[i % reps], y, bt, M, N, K,
                                                                       stream=self.stream), n, 20)
        b = blocks.size + bt * M * K * 4 + bt * M * N * 4
        log("batched mat-vec 8 x (M=1, N=K=4096): %.2f us, %.1f GB/s" % (t * 1e6, b / t / 1e9))
        return {"workload": "8 matrices x (M=1, N=K=4096) in one call, %d cold weight replicas" % reps,
                "us": t * 1e6, "algorithmic_bytes": b, "GB/s": b / t / 1e9, "bound": "hbm",
                "frac_hbm": b / t / 1e9 / HBM_PEAK_GBS, "read_ceiling": self.read_ceiling(wr, 100, sweep=True)}

    def sample(self, n=200):
        """First-max argmax + threshold candidates over 8 slots x 262144 logits (cap 64)."""
        torch, np = self.torch, self.np
        ns, vocab, cap = 8, 262144, 64
        rng = np.random.Generator(np.random.PCG64(4000))
        sets = [torch.from_numpy(rng.standard_normal((ns, vocab), dtype=np.float32)).to(self.dev) for _ in range(64)]
        d = self.dev
        idx = torch.empty(ns, dtype=torch.int32, device=d)
        val = torch.empty(ns, dtype=torch.float32, device=d)
        cnt = torch.empty(ns, dtype=torch.int32, device=d)
        ovf = torch.empty(ns, dtype=torch.int32, device=d)
        ids = torch.empty((ns, cap), dtype=torch.int32, device=d)
        t = time_launches(torch, lambda i: self.q2k.q2k_argmax_candidates(sets[i % 64], ns, vocab, cap, idx, val, cnt,
                                                                          ovf, ids, stream=self.stream), n, 20)
        b = ns * vocab * 4 + ns * 16 + ns * cap * 4
        log("argmax + candidates 8 x 262144: %.2f us, %.1f GB/s" % (t * 1e6, b / t / 1e9))
        return {"workload": "8 slots x 262144 logits, cap 64 (64 rotating logit sets, 512 MiB)", "us": t * 1e6,
                "algorithmic_bytes": b, "GB/s": b / t / 1e9, "bound": "hbm", "frac_hbm": b / t / 1e9 / HBM_PEAK_GBS}

    def _moe(self, ci):
        torch, np = self.torch, self.np
        inp = self.synth.make_moe_inputs(ci)
        c = inp.config
        p = self.q2k.MatmulIdParams(n_tokens=c.tokens, top_k=c.top_k, n=c.n, k=c.K, n_experts=c.experts,
                                    reserved=0, expert_stride=c.n * (c.K // 256) * 84)
        x = torch.from_numpy(inp.x).to(self.dev)
        ids = torch.from_numpy(inp.ids.astype(np.int32)).to(self.dev)
        y = torch.empty((c.routes, c.n), dtype=torch.float32, device=self.dev)
        return inp, c, p, x, ids, y

    def moe_decode(self, n=200):
        """Expert-routed decode: 1 token, top_k 6 of 8 experts (fp32 per-route schedule), cold weights."""
        torch = self.torch
        log("generating expert-routed decode inputs")
        inp, c, p, x, ids, y = self._moe(0)
        wh = torch.from_numpy(inp.blocks)
        reps = max(1, math.ceil(COLD_BYTES / inp.blocks.size))
        wr = [wh.to(self.dev) for _ in range(reps)]
        t = time_launches(torch, lambda i: self.q2k.q2k_matmul_id(x, wr[i % reps], ids, y, p, stream=self.stream),
                          n, 20)
        experts_read = len(set(inp.ids.tolist()))
        b = experts_read * c.n * (c.K // 256) * 84 + c.tokens * c.K * 4 + c.routes * 4 + c.routes * c.n * 4
        log("expert-routed decode: %.2f us, %.1f GB/s" % (t * 1e6, b / t / 1e9))
        return {"workload": c.name + " (%d experts read, %d cold weight replicas)" % (experts_read, reps),
                "us": t * 1e6, "algorithmic_bytes": b, "GB/s": b / t / 1e9, "bound": "hbm",
                "frac_hbm": b / t / 1e9 / HBM_PEAK_GBS}

    def moe_prefill(self, n=60):
        """Expert-routed prefill: 512 tokens, top_k 6 of 8 experts (matrix-core schedule, one call)."""
        torch = self.torch
        log("generating expert-routed prefill inputs")
        inp, c, p, x, ids, y = self._moe(1)
        w = torch.from_numpy(inp.blocks).to(self.dev)
        t = time_launches(torch, lambda i: self.q2k.q2k_matmul_id(x, w, ids, y, p, stream=self.stream), n, 6)
        f = 2.0 * c.routes * c.n * c.K
        log("expert-routed prefill: %.2f us, %.1f TFLOP/s" % (t * 1e6, f / t / 1e12))
        return {"workload": c.name + " (one call: routing + bf16 row gather + GEMM)", "us": t * 1e6, "flop": f,
                "TFLOP/s": f / t / 1e12, "bound": "mfma", "frac_bf16_mfma": f / t / 1e12 / BF16_PEAK_TFLOPS}

    def copy_probe(self):
        torch = self.torch
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=self.dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy probe: %d bytes" % COPY_BYTES)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-rows", action="store_true", help="skip the per-row measurements")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the M=512 context timings (zero activations, torch bf16 linear)")
    ap.add_argument("--only", choices=ROWS, help="run only this row's timed loop")
    ap.add_argument("--copy-probe", action="store_true", help="also run the calibration copy")
    ap.add_argument("--derive-traffic", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "KEY"),
                    help="record HBM bytes per launch of one row's kernel (KEY: %s)" % ", ".join(TRAFFIC_ROWS))
    ap.add_argument("--sweep", action="store_true",
                    help="M=1, K=4096 GEMV and read ceiling over N = 4096 .. 131072 (cold), one JSON line per N")
    args = ap.parse_args()

    if args.derive_traffic:
        return derive_traffic(*args.derive_traffic)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import ggml_q2_dequant_amd as q2k
    import synth

    q2k.load_library()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        return run(args, torch, q2k, synth, np)


def run(args, torch, q2k, synth, np) -> int:
    b = Bench(torch, q2k, synth, np)

    if args.sweep:
        lib = q2k.load_library()
        for N in (4096, 8192, 16384, 32768, 65536, 131072):
            K = 4096
            rng = np.random.Generator(np.random.PCG64(5000 + N))
            blocks = synth.random_blocks(rng, N * K // 256)
            reps = max(1, math.ceil(COLD_BYTES / blocks.size))
            wh = torch.from_numpy(blocks)
            wr = [wh.to(b.dev) for _ in range(reps)]
            x = torch.from_numpy(rng.standard_normal((1, K), dtype=np.float32)).to(b.dev)
            y = torch.empty((1, N), dtype=torch.float32, device=b.dev)
            st = b.stream

            def step(i):
                rc = lib.q2k_matmul(x.data_ptr(), wr[i % reps].data_ptr(), y.data_ptr(), 1, N, K, st)
                if rc:
                    raise RuntimeError(lib.q2k_last_error_message().decode())
            t = time_launches(torch, step, 200, 20)
            byt = blocks.size + 4 * K + 4 * N
            rc = b.read_ceiling(wr, 100, sweep=True)
            print(json.dumps({"sweep": "gemv_m1", "N": N, "K": K, "weight_replicas": reps, "bytes": byt,
                              "us": t * 1e6, "GB/s": byt / t / 1e9, "of_best_read": rc["best"]["us"] / (t * 1e6),
                              "read_ceiling": rc}), flush=True)
            del wr
        return 0

    if args.only:
        EAGER_ONLY[0] = True
        out = {"only": args.only}
        if args.copy_probe:
            b.copy_probe()
        if args.only in ("gemv1", "dequant"):
            step = b.gemv1_setup()
            if args.only == "gemv1":
                t = time_launches(torch, step, args.steps, args.warmup)
                out.update(us=t * 1e6, GBs=b.g1["bytes"] / t / 1e9)
            else:
                out.update(b.dequant(args.steps))
        else:
            out.update(getattr(b, args.only)(args.steps))
        print(json.dumps(out), flush=True)
        return 0

    # ------------------------------------------------------------------- headline: decode GEMV
    log("generating decode GEMV inputs")
    step = b.gemv1_setup()
    g = b.g1
    c1 = g["inp"].config
    log("timing %d GEMV steps (%d warmup) over %d weight replicas" % (args.steps, args.warmup, g["reps"]))
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    want = g["y"].clone()
    g["y"].fill_(float("nan"))
    # The K timed steps: after a read of other memory that leaves every replica cold, issued back to back behind a
    # GPU spin that lets the host queue them all before the first starts; events on the launch stream.
    sec_per_step = time_launches(torch, step, args.steps, 0)
    if not torch.equal(g["y"].view(torch.int32), want.view(torch.int32)):
        raise RuntimeError("decode GEMV: the timed steps' result differs from the warm-up result")
    gbs = g["bytes"] / sec_per_step / 1e9
    log("GEMV M=1: %.3f us/step, %.1f GB/s" % (sec_per_step * 1e6, gbs))
    # Context after the timed region: the same steps from a HIP graph replay, the steps issued by the host one by
    # one with nothing queued ahead (runs of 20: the host's launch rate shows in these), and the plain-read
    # ceiling for the same cold bytes.
    graph_s = time_launches(torch, step, max(args.steps, 200), 0, graph=True)
    dist = time_blocks(torch, step, 50, 20)
    ceiling = b.read_ceiling(g["replicas"], sweep=True)
    log("GEMV M=1 graph replay %.2f us/call; host-paced runs of 20: p10/p50/p90 %.2f/%.2f/%.2f us; read ceiling "
        "%.2f us (%.0f GB/s), best read shape %s: %.2f us; d2d copy %.2f us" % (
            graph_s * 1e6, dist["p10"] * 1e6, dist["p50"] * 1e6, dist["p90"] * 1e6, ceiling["us"], ceiling["GB/s"],
            (ceiling["best"]["grid"], ceiling["best"]["loads_per_thread"]), ceiling["best"]["us"],
            ceiling["d2d_copy"]["us"]))

    rows = {}
    if not args.no_rows:
        rows["dequantize"] = b.dequant()
        rows["gather"] = b.gather()
        rows["gemv_m1_n65536"] = b.gemv1_wide()
        rows["gemv_m8"] = b.gemv8()
        rows["mfma_m512"] = b.mfma()
        if not args.no_context:
            rows["mfma_m512"]["context"] = b.mfma_context()
        rows["batched_mv"] = b.batched()
        rows["argmax_candidates"] = b.sample()
        rows["moe_decode"] = b.moe_decode()
        rows["moe_prefill"] = b.moe_prefill()

    # ------------------------------------------------------------------- CPU oracle baseline
    log("timing the CPU oracle (~%.0f s)" % args.cpu_seconds)
    sec_cpu, threads, cpu_reps = cpu_baseline(g["inp"], args.cpu_seconds)
    cpu_gbs = g["bytes"] / sec_cpu / 1e9

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
                   "M": c1.M, "N": c1.N, "K": c1.K, "weight_replicas": g["reps"],
                   "algorithmic_bytes_per_step": g["bytes"], "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": measured_traffic("k_gemv_m1")},
        "timing": "the %d steps issued back to back behind a GPU spin (queued before the first starts), cold "
                  "weights, events on the launch stream" % args.steps,
        "step_us": {"graph_replay": round(graph_s * 1e6, 3), "host_paced_runs_of_20": dist_us(dist)},
        "read_ceiling": ceiling,
        "cpu_baseline": {"value": round(cpu_gbs, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
                         "sample": "the whole decode GEMV workload (M=1, N=K=4096), %d calls of the f64 "
                                   "oracle matmul, %.4f s per call" % (cpu_reps, sec_cpu)},
        "rows": rows,
        "input_sha256": g["inp"].hashes,
    }
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
