"""Benchmark of the SSD chunked-scan forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one full forward (ssd_forward: one launch of the scan kernel) over
the workload's batch, with inputs and outputs already resident in HBM.
Prints one JSON line: tokens/s over K timed steps, the roofline of the scan
kernel from one pair of HIP events around the K back-to-back launches on their
stream (warm: part of the inputs may still sit in the last-level cache), beside
it the median of singly bracketed launches and a cold pass (each call timed
alone after an untimed 1 GiB scrub write: median, p10, p90), the bandwidth of a
1 GiB device copy and the fraction of it reached, the HBM traffic and pipe
counters from the committed rocprofv3 summaries (while the kernel sources match
the hash they were taken on), and the CPU oracle timed on the same workload.
The line also carries a "backward" object:
the time of one ssd_backward call (every gradient) on the same workload and its
fraction of the HBM roofline (skipped with --no-backward); a "step" object: the
single-token decoding step (ssd_step) at the workload's batch and heads, bound by
one read and one write of the fp32 state (eager and replayed from a HIP graph of
16 steps); and a "fused_step_size" object: the same forward fed the raw step
size and a per-head bias with the softplus map and the Euler input scaling done
in the kernel (skipped with --no-extra-legs).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
COPY_BYTES = 1 << 30           # size of the calibration copy (read and written once each)
SCRUB_BYTES = 1 << 30          # written before each cold timed call: more than L2 and the 256 MB MALL
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense


def algorithmic_bytes(w, init_nonzero: bool) -> int:
    """Bytes the method itself must move: x, B, C, dt, A_log, D read once; y and final states written once."""
    sx = 2 if w.dtype == "bf16" else 4
    b, T, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    nseqs = w.nseqs_packed * b if w.nseqs_packed else b
    total = sx * (b * T * H * P + 2 * b * T * G * N) + 4 * b * T * H + 8 * H + 4 * b * T * H * P
    total += 4 * nseqs * H * P * N
    if init_nonzero:
        total += 4 * nseqs * H * P * N
    if w.nseqs_packed:
        total += 4 * b * T      # seq_idx
    return total


HEADLINE_METRIC = "SSD fwd tokens/sec (2.7B-layer shape, T=4096) and % of MFMA/HBM roofline"


def metric_name(w) -> str:
    """The headline metric for the 2.7B-layer workload; the same measure named for its own shape elsewhere."""
    if w.name == "m2p7_bf16":
        return HEADLINE_METRIC
    return "SSD fwd tokens/sec (%s: b=%d, T=%d, H=%d, P=%d, N=%d, %s) and %% of MFMA/HBM roofline" % (
        w.name, w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.dtype)


def algorithmic_flops(w) -> int:
    b, T, H, P, N, G, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk_len
    nc = -(-T // Q)
    return 2 * (b * H * nc * (Q * (Q + 1) // 2 * P + 2 * Q * N * P) + b * G * nc * Q * (Q + 1) // 2 * N)


def backward_algorithmic_bytes(w, init_nonzero: bool) -> int:
    """Bytes the gradients must move: the forward's inputs, dy and dfinal read once;
    dx, ddt, dB, dC, dinit and the per-head gradients written once."""
    sx = 2 if w.dtype == "bf16" else 4
    b, T, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    ns = w.nseqs_packed * b if w.nseqs_packed else b
    reads = sx * (b * T * H * P + 2 * b * T * G * N) + 4 * b * T * H + 8 * H + 4 * b * T * H * P + 4 * ns * H * P * N
    if init_nonzero:
        reads += 4 * ns * H * P * N
    if w.nseqs_packed:
        reads += 4 * b * T      # seq_idx
    writes = 4 * b * T * H * P + 4 * b * T * H + 2 * 4 * b * T * G * N + 4 * ns * H * P * N + 12 * H
    return reads + writes


def backward_leg(w, prob, d, steps: int, warmup: int):
    """Time ssd_backward (every gradient of <dy, y> + <dfinal, final>) on the workload."""
    import numpy as np
    import torch

    import mamba_ssd_scan_chunked_amd as ssd
    dev = d["x"].device
    rng = np.random.default_rng(1234)
    b, T, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    ns = prob["nseqs"]
    dy = torch.from_numpy(rng.standard_normal((b, T, H, P), dtype=np.float32)).to(dev)
    dfinal = torch.from_numpy(rng.standard_normal((ns, H, P, N), dtype=np.float32)).to(dev)
    dtype = ssd.DTYPE_BF16 if w.dtype == "bf16" else ssd.DTYPE_F32
    p = ssd.problem(b, T, H, P, N, G, w.chunk_len, ns, dtype, 0)
    f32 = dict(dtype=torch.float32, device=dev)
    out = {"dx": torch.empty((b, T, H, P), **f32), "ddt": torch.empty((b, T, H), **f32),
           "dA_log": torch.empty((H,), **f32), "dB": torch.empty((b, T, G, N), **f32),
           "dC": torch.empty((b, T, G, N), **f32), "dD": torch.empty((H,), **f32),
           "dinit": torch.empty((ns, H, P, N), **f32), "ddt_bias": torch.empty((H,), **f32)}
    ws = torch.empty(max(1, ssd.backward_workspace_size(p)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def run():
        ssd.backward_into(p, d["x"], d["dt"], None, d["A_log"], d["B"], d["C"], d["D"], d["init"], dy, dfinal, out,
                          ws, stream=stream, seq_idx=d["seq_idx"])

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in evs:
        e[0].record(stream)
        run()
        e[1].record(stream)
    torch.cuda.synchronize()
    ms = sorted(e[0].elapsed_time(e[1]) for e in evs)
    mean = sum(ms) / len(ms)
    balg = backward_algorithmic_bytes(w, prob["init"] is not None)
    return {"what": "ssd_backward: dx, ddt, dA_log, dB, dC, dD, dinit, ddt_bias of <dy, y> + <dfinal, final>",
            "ms_per_step": round(mean, 5), "ms_median": round(ms[len(ms) // 2], 5),
            "tokens_per_s": round(b * T / (mean / 1000.0), 1),
            "roofline": {"bound": "hbm", "achieved": round(balg / (mean / 1000.0) / 1e9, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(balg / (mean / 1000.0) / 1e9 / HBM_PEAK_GBS, 4),
                         "traffic": committed_backward_traffic(w.name),
                         "alg_bytes_per_step": balg, "kernels": "all launches of one ssd_backward call"}}


def step_leg(w, prob, d, steps: int, warmup: int):
    """Time ssd_step (one token per (row, head) on the fp32 state, in place) at the
    workload's batch and heads, on the workload's first token."""
    import torch

    import mamba_ssd_scan_chunked_amd as ssd
    if d["seq_idx"] is not None:
        return None
    dev = d["x"].device
    b, H, P, N, G = w.batch, w.nheads, w.headdim, w.dstate, w.ngroups
    sx = 2 if w.dtype == "bf16" else 4
    x1, dt1, B1, C1 = (d[k][:, :1].contiguous() for k in ("x", "dt", "B", "C"))
    state = torch.zeros((b, H, P, N), dtype=torch.float32, device=dev)
    y1 = torch.empty((b, 1, H, P), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def run():
        # on torch's current stream: the bench stream here, the capture stream below
        ssd.step(x1, dt1, d["A_log"], B1, C1, d["D"], state, y=y1)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    t0 = time.perf_counter()
    for e in evs:
        e[0].record(stream)
        run()
        e[1].record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    ms = sorted(e[0].elapsed_time(e[1]) for e in evs)
    kms = sum(ms) / len(ms)
    # a decoding loop of 16 steps captured once and replayed
    K, R = 16, max(2, steps // 16)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(K):
            run()
    g.replay()
    torch.cuda.synchronize()
    ge = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    t0 = time.perf_counter()
    ge[0].record(stream)
    for _ in range(R):
        g.replay()
    ge[1].record(stream)
    torch.cuda.synchronize()
    gwall = (time.perf_counter() - t0) * 1000.0 / (R * K)
    gms = ge[0].elapsed_time(ge[1]) / (R * K)
    balg = 2 * 4 * b * H * P * N + sx * (b * H * P + 2 * b * G * N) + 4 * b * H + 4 * b * H * P
    # A launch takes a few microseconds, about what an event pair around it adds, so
    # the roofline uses the back-to-back launches of the graph (HIP events around
    # all replays on the stream; the gaps between launches are included).
    return {"what": "ssd_step: one token per (row, head), fp32 state read and written in place",
            "batch": b, "graph_ms_per_token": round(gms, 5), "graph_wall_ms_per_token": round(gwall, 5),
            "tokens_per_s": round(b / (gms / 1000.0), 1),
            "eager_ms_per_token": round(wall * 1000.0, 5), "eager_event_ms_per_launch": round(kms, 5),
            "roofline": {"bound": "hbm", "achieved": round(balg / (gms / 1000.0) / 1e9, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(balg / (gms / 1000.0) / 1e9 / HBM_PEAK_GBS, 4),
                         "alg_bytes_per_launch": balg, "kernel": "ssd_step_kernel",
                         "timing": "16 launches per graph replay, HIP events around the replays"}}


def fused_step_size_leg(w, prob, d, steps: int, warmup: int):
    """Time the forward fed the raw step size and a per-head bias (softplus(dt + bias)
    and the Euler input scaling computed in the scan kernel's per-token preparation)
    against the plain forward, the two launches alternating so that both see the
    same clock state."""
    import torch

    import ssd_inputs as si
    import mamba_ssd_scan_chunked_amd as ssd
    dev = d["x"].device
    b, T, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    raw = si.raw_step_sizes(b, T, H, seed=w.seed + 100, lo=w.dt_range[0], hi=w.dt_range[1])
    dt_raw, bias = raw["dt"].to(dev), raw["dt_bias"].to(dev)
    dtype = ssd.DTYPE_BF16 if w.dtype == "bf16" else ssd.DTYPE_F32
    pf = ssd.problem(b, T, H, P, N, G, w.chunk_len, prob["nseqs"], dtype, ssd.FLAG_DT_SOFTPLUS | ssd.FLAG_DT_SCALES_X)
    pp = ssd.problem(b, T, H, P, N, G, w.chunk_len, prob["nseqs"], dtype, 0)
    y = torch.empty((b, T, H, P), dtype=torch.float32, device=dev)
    fin = torch.empty((prob["nseqs"], H, P, N), dtype=torch.float32, device=dev)
    wsb = max(ssd.workspace_size(pf), ssd.workspace_size(pp))
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb > 0 else None
    stream = torch.cuda.current_stream(dev)

    def fused():
        ssd.forward_into(pf, d["x"], dt_raw, d["A_log"], d["B"], d["C"], d["D"], d["init"], d["seq_idx"], y, fin,
                         ws, stream=stream, dt_bias=bias)

    def plain():
        ssd.forward_into(pp, d["x"], d["dt"], d["A_log"], d["B"], d["C"], d["D"], d["init"], d["seq_idx"], y, fin,
                         ws, stream=stream)

    for _ in range(warmup):
        fused()
        plain()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for e in evs:
        e[0].record(stream)
        fused()
        e[1].record(stream)
        e[2].record(stream)
        plain()
        e[3].record(stream)
    torch.cuda.synchronize()
    mf = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    mp = sum(e[2].elapsed_time(e[3]) for e in evs) / steps
    balg = algorithmic_bytes(w, prob["init"] is not None) + 4 * H
    return {"what": "ssd_forward with the step-size map softplus(dt + dt_bias) and the Euler input scaling "
                    "fused into the scan kernel, launches alternating with the plain forward",
            "kernel_ms": round(mf, 5), "plain_kernel_ms": round(mp, 5), "ratio_to_plain": round(mf / mp, 4),
            "roofline": {"bound": "hbm", "achieved": round(balg / (mf / 1000.0) / 1e9, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(balg / (mf / 1000.0) / 1e9 / HBM_PEAK_GBS, 4),
                         "alg_bytes_per_launch": balg}}


def kernel_source_hash() -> str:
    """Hash of the sources of the forward path (kernels, instantiations, host
    launch code); the backward's files, the instance generator and the header
    that only declares the launchers are left out."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mamba_ssd_scan_chunked_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.startswith("ssd_bwd") or name in ("gen_instances.py", "ssd_launch.hpp"):
            continue
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def all_source_hash() -> str:
    """Hash of every kernel and launch source (the backward runs the forward's local
    pass and combine too)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mamba_ssd_scan_chunked_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name == "gen_instances.py":
            continue
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def committed_backward_traffic(workload: str):
    """HBM bytes moved by one ssd_backward call (FETCH_SIZE and WRITE_SIZE of every
    launch, scaled by the copy calibration) from profiles/bwd_traffic_<workload>.json,
    if they were taken on the current sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", "bwd_traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha") != all_source_hash():
        return None
    return rec.get("traffic_bytes_per_call")


def committed_counters(workload: str, what: str = "traffic"):
    """A figure from the committed rocprofv3 counter summaries of the scan kernel
    (profiles/scan_<what>_<workload>.json), if they were taken on the current kernel
    sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", "scan_%s_%s.json" % (what, workload))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != kernel_source_hash():
        return None
    return rec


def committed_traffic(workload: str):
    """HBM traffic per scan launch from the committed rocprofv3 counter runs, if
    they were taken on the current kernel sources; otherwise None."""
    rec = committed_counters(workload, "traffic")
    return rec.get("traffic_bytes_per_launch") if rec else None


def copy_bandwidth(dev, reps: int = 10):
    """Achieved HBM bandwidth of a plain device copy of COPY_BYTES (read + write
    bytes per second), timed with HIP events: the practical ceiling beside the
    8 TB/s peak."""
    import torch
    n = COPY_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(reps):
        dst.copy_(src)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    del src, dst
    return 2.0 * COPY_BYTES / (ms / 1000.0) / 1e9


def gemm_tflops(dev, n: int = 8192, reps: int = 10):
    """Dense bf16 MFMA throughput a large library GEMM (torch.mm of contiguous
    n x n operands) reaches on this device, in TFLOP/s: the practical ceiling beside
    the 2.5 PFLOP/s peak."""
    import torch
    a = torch.randn((n, n), dtype=torch.bfloat16, device=dev)
    b = torch.randn((n, n), dtype=torch.bfloat16, device=dev)
    c = torch.mm(a, b)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(reps):
        c = torch.mm(a, b)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    del a, b, c
    return 2.0 * n ** 3 / (ms / 1000.0) / 1e12


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(prob, w):
    """Time the fp64 oracle on every row of the workload (all heads, full length) on all host cores."""
    import numpy as np

    import oracle
    sub = {k: prob[k] for k in ("x", "dt", "B", "C")}
    rows = w.batch
    sub = {k: np.ascontiguousarray(v[:rows].to(dtype=__import__("torch").float64).numpy()) for k, v in sub.items()}
    A_log = prob["A_log"].double().numpy()
    D = prob["D"].double().numpy() if prob["D"] is not None else None
    init = prob["init"][:rows].double().numpy() if (prob["init"] is not None and prob["seq_idx"] is None) else None
    seq = None
    nseqs = None
    if prob["seq_idx"] is not None:
        seq = prob["seq_idx"][:rows].numpy()
        nseqs = int(seq.max()) + 1
        init = prob["init"][:nseqs].double().numpy() if prob["init"] is not None else None
    threads = oracle.max_threads()
    times = []
    while True:                 # the median of three runs, or one run if it takes over 10 s
        t0 = time.perf_counter()
        oracle.recurrence(sub["x"], sub["dt"], A_log, sub["B"], sub["C"], D, init, seq, nseqs, nthreads=threads)
        times.append(time.perf_counter() - t0)
        if times[0] > 10.0 or len(times) == 3:
            break
    dt = sorted(times)[len(times) // 2]
    tokens = rows * w.seqlen    # full rows of the workload, every head
    return {"value": tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "host_cpus": os.cpu_count(),
            "sample": "%d of %d rows (all %d heads, %d tokens each), fp64 recurrence, median of %d runs, %.2f s wall"
                      % (rows, w.batch, w.nheads, w.seqlen, len(times), dt)}


def cpu_single_thread():
    """The oracle on one thread: the tiny workload whole and one row of the 130M-layer
    workload (all heads, full length), in tokens/s."""
    import numpy as np

    import oracle
    import ssd_inputs as si
    out = {}
    for name, rows in (("tiny_f32", None), ("m130_bf16", 1)):
        w = si.WORKLOADS[name]
        prob = si.make_workload(w)
        r = w.batch if rows is None else rows
        f64 = lambda t: np.ascontiguousarray(t[:r].double().numpy())
        D = prob["D"].double().numpy() if prob["D"] is not None else None
        t0 = time.perf_counter()
        oracle.recurrence(f64(prob["x"]), f64(prob["dt"]), prob["A_log"].double().numpy(), f64(prob["B"]),
                          f64(prob["C"]), D, None, None, None, nthreads=1)
        dt = time.perf_counter() - t0
        out[name] = {"tokens_per_s": round(r * w.seqlen / dt, 1), "sample": "%d of %d rows, %.2f s" % (r, w.batch, dt)}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="m2p7_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward-pass leg")
    ap.add_argument("--no-extra-legs", action="store_true", help="skip the decoding-step and fused step-size legs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain device copy of known size (reference for the HBM traffic counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the SSD forward here has no multi-GPU path "
              "(sharding over heads or sequence is a design note, not built); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import mamba_ssd_scan_chunked_amd as ssd
    import ssd_inputs as si

    if args.copy_calibration:
        # A plain copy of COPY_BYTES: FETCH_SIZE / WRITE_SIZE of this dispatch give
        # the counters' scale (bytes of HBM traffic per counted KiB).
        n = COPY_BYTES // 4
        src = torch.arange(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": COPY_BYTES}), flush=True)
        return

    w = si.WORKLOADS[args.workload]
    prob = si.make_workload(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in prob.items()}
    dtype = ssd.DTYPE_BF16 if w.dtype == "bf16" else ssd.DTYPE_F32
    nseqs = prob["nseqs"]
    p = ssd.problem(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk_len, nseqs, dtype, 0)
    y = torch.empty((w.batch, w.seqlen, w.nheads, w.headdim), dtype=torch.float32, device=dev)
    fin = torch.empty((nseqs, w.nheads, w.headdim, w.dstate), dtype=torch.float32, device=dev)
    wsb = ssd.workspace_size(p)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb > 0 else None
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        ssd.forward_into(p, d["x"], d["dt"], d["A_log"], d["B"], d["C"], d["D"], d["init"], d["seq_idx"], y, fin,
                         ws, stream=stream)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # The timed region: K back-to-back forwards between one pair of HIP events on
    # their stream (an event pair around every launch would add its own few
    # microseconds to each).
    region = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    region[0].record(stream)
    for _ in range(args.steps):
        step()
    region[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    scan_ms = region[0].elapsed_time(region[1]) / args.steps

    # The spread of single launches, each between its own events (not timed above).
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    kms = sorted(e[0].elapsed_time(e[1]) for e in evs)
    median_ms = kms[len(kms) // 2]
    ms_per_step = wall * 1000.0 / args.steps

    # Cold calls: before each, an untimed write of SCRUB_BYTES evicts the inputs
    # from L2 and the MALL; each call is timed alone between its own events.
    scrub = torch.empty(SCRUB_BYTES // 4, dtype=torch.float32, device=dev)
    cold = []
    for i in range(args.steps):
        scrub.fill_(float(i))
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        step(e)
        cold.append(e)
    torch.cuda.synchronize()
    cms = sorted(e[0].elapsed_time(e[1]) for e in cold)
    del scrub
    pct = lambda v, q: v[min(len(v) - 1, int(round(q * (len(v) - 1))))]
    cold_med, cold_p10, cold_p90 = pct(cms, 0.5), pct(cms, 0.1), pct(cms, 0.9)
    copy_gbs = copy_bandwidth(dev)
    gemm = gemm_tflops(dev)
    tokens = w.batch * w.seqlen
    value = tokens / (ms_per_step / 1000.0)

    balg = algorithmic_bytes(w, prob["init"] is not None)
    falg = algorithmic_flops(w)
    achieved = balg / (scan_ms / 1000.0) / 1e9
    pipe = committed_counters(w.name, "pipe")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": committed_traffic(w.name),
                "kernel": "ssd_scan_kernel", "kernel_ms": round(scan_ms, 5),
                "timing": "HIP events around the timed region's back-to-back launches (warm)",
                "single_launch_ms_median": round(median_ms, 5),
                "cold": {"what": "each call after an untimed %d MiB scrub write, timed alone" % (SCRUB_BYTES >> 20),
                         "calls": len(cms), "ms_median": round(cold_med, 5), "ms_p10": round(cold_p10, 5),
                         "ms_p90": round(cold_p90, 5),
                         "frac_median": round(balg / (cold_med / 1000.0) / 1e9 / HBM_PEAK_GBS, 4)},
                "copy_gbs": round(copy_gbs, 1), "frac_of_copy": round(achieved / copy_gbs, 4),
                "gemm_tflops": round(gemm, 1),
                "flops_frac_of_gemm": round(falg / (scan_ms / 1000.0) / 1e12 / gemm, 4),
                "mfma_busy": pipe.get("mfma_busy") if pipe else None,
                "lds_active": pipe.get("lds_active") if pipe else None,
                "alg_bytes_per_launch": balg, "alg_flops_per_step": falg,
                "step_frac_of_hbm_roofline": round(balg / (ms_per_step / 1000.0) / 1e9 / HBM_PEAK_GBS, 4)}

    bwd = None
    if not args.no_backward:
        bwd = backward_leg(w, prob, d, steps=max(5, min(args.steps, 20)), warmup=2)

    step = fused = None
    if not args.no_extra_legs:
        step = step_leg(w, prob, d, steps=max(20, args.steps), warmup=3)
        fused = fused_step_size_leg(w, prob, d, steps=max(5, min(args.steps, 20)), warmup=2)

    base = None
    if not args.no_cpu_baseline:
        base = cpu_baseline(prob, w)
        base["single_thread"] = cpu_single_thread()

    out = {"metric": metric_name(w),
           "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": w.dtype, "data": "synthetic (seeded; random inputs of the layer's shapes)",
           "config": {"workload": w.name, "batch": w.batch, "seq_len": w.seqlen, "nheads": w.nheads,
                      "headdim": w.headdim, "dstate": w.dstate, "ngroups": w.ngroups, "chunk_len": w.chunk_len,
                      "kernel_block": 64 if w.chunk_len >= 64 else 32, "outputs": "y fp32 + final fp32",
                      "parallelism": "single GPU"},
           "roofline": roofline, "cpu_baseline": base, "backward": bwd, "step": step,
           "fused_step_size": fused}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
