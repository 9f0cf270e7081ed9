"""Throughput of the chunked gated delta-rule prefill on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload I] [--io bf16|f16|f32]
                    [--path auto|pipe|split|seg] [--chunk 32|64|128] [--segments K]
                    [--head-shard G] [--kda] [--prologue] [--eager] [--no-cpu-baseline]

A step is one prefill call over the whole workload (all heads, all chunks) with inputs
resident in HBM.  --path auto (the default) calls gdn_prefill_auto, the library's own
choice among the one-launch kernel (gdn_prefill), the two-launch path (gdn_prefill_split:
a chunk-parallel map kernel, then the chain kernel) and the segmented one
(gdn_prefill_seg); --path pipe|split|seg calls that entry point instead.  Workspaces are
allocated once outside the timed region.  --chunk sets the two-launch paths' chunk length
(64 by default; the one-launch and KDA paths run 64).  The default workload is the
headline one: one sequence of T=4096 tokens, 16 heads, d=128, bf16 q/k/v/o, fp32
g/beta/state, chunk 64.  Input sets are rotated across steps (more bytes than the 256 MB
Infinity Cache) so that every step streams from HBM.  The W warm-up and K timed steps
run as launches from Python (HIP events between them give the eager mean, median and
minimum); the K steps are then captured in one HIP graph and replayed, and that replay
is what ms_per_step and value time (--eager: the eager loop instead).  Prints ONE JSON
line.

roofline.achieved = algorithmic bytes of one launch / mean launch time, where the
mean launch time comes from HIP events recorded on the launch stream around the
timed steps (one call per step; for the two-launch paths the step's two kernels together).
Algorithmic bytes per launch:
    T*(Hk*2*Dk*s + Hv*(2*Dv*s + 8)) + N*Hv*Dv*Dk*4*(2 if an initial state else 1)
with s = 2 (bf16, fp16) or 4 (fp32): q, k read once per key head, v read and o written once
per value head, g and beta (fp32) read, the fp32 state read (if given) and written.
Algorithmic FLOPs per full chunk and value head: 6*C*Dk*Dv (three state products)
+ 2*C^2*Dv (intra-chunk output) + 2*C^2*Dk (the K K^T gram) ... see `algorithmic_flops`.

roofline.traffic: HBM bytes per launch measured by rocprofv3 (FETCH_SIZE and WRITE_SIZE,
each scaled by what the counter reads for a device copy of known size), read from
profiles/hbm_traffic.json; null when no record matches this kernel's current sources.
To refresh it, profile bench.py under `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE`
(files fetch_* / write_*) and `bench.py --calibrate-copy 256` likewise (copyfetch_* /
copywrite_*), then run `bench.py --summarize-pmc DIR`.

decode (workloads with decode steps): microseconds per gdn_decode_step, launched eagerly
and replayed from a HIP graph (see `decode_bench`).  measured_peaks: copy bandwidth and
a bf16 GEMM measured on this GPU, beside the published peaks used for the fractions.

cpu_baseline: the fp64 CPU oracle (test infrastructure, untuned) timed on the host
cores over the same workload.

--prologue: the same workload's draws before the input prologue (q, k unnormalised,
beta and g logits), run with all three prologue steps applied in the kernels
(gdn_prefill_auto with the prologue flags); the oracle applies the same steps for the
parity block.

--kda: the same workload with one decay per key channel (gdn_kda_prefill: a
chunk-parallel map kernel, then the chain kernel, over a workspace allocated once
outside the timed region).  The step is the whole call (both kernels); g adds
T*Hv*Dk*4 bytes and the grams are per value head (see `algorithmic_bytes`,
`algorithmic_flops`).
"""
from __future__ import annotations

import argparse
import gc
import csv
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN prefill tokens/sec (H=16, d=128, T=4096) + % of MFMA/HBM roofline"
KDA_METRIC = "KDA prefill tokens/sec (H={H}, d=128, T={T}) + % of HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense
FP32_MFMA_PEAK_TFLOPS = 157.3
MALL_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
CSRC = os.path.join(ROOT, "linear_attention_chunked_gdn_amd", "csrc")
IO_CODE = {"f32": 0, "bf16": 1, "f16": 2}   # gdn_dtype
# sources each kernel is compiled from: the HBM counters recorded for a kernel are
# reported only while these are unchanged
KERNEL_SOURCES = {
    "gdn_prefill_pipe_kernel": ["gdn_prefill_pipe.hip", "gdn_device.h", "gdn_launch.h"],
    "gdn_prefill_kernel": ["gdn_prefill.hip", "gdn_device.h", "gdn_launch.h"],
    "gdn_prefill_pipe_kernel(prologue)": ["gdn_prefill_pipe.hip", "gdn_device.h", "gdn_launch.h"],
    "kda_map_kernel+kda_chain_kernel": ["kda_map.hip", "kda_chain.hip", "gdn_wy.h", "gdn_device.h",
                                        "gdn_launch.h"],
    "gdn_map_kernel+kda_chain_kernel": ["gdn_map.hip", "kda_chain.hip", "gdn_wy.h", "gdn_device.h",
                                        "gdn_launch.h"],
    "gdn_map_kernel+kda_chain_kernel(prologue)": ["gdn_map.hip", "kda_chain.hip", "gdn_wy.h", "gdn_device.h",
                                                  "gdn_launch.h"],
    "gdn_map_kernel+kda_chain_kernel+gdn_seg_join_kernel+gdn_seg_fix_kernel": [
        "gdn_map.hip", "kda_chain.hip", "gdn_seg.hip", "gdn_wy.h", "gdn_device.h", "gdn_launch.h"],
}


def sources_sha256(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, or None when there is
    none for this kernel and workload or the kernel's sources changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(f"{kernel}@{workload}")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("sources_sha256") != sources_sha256(kernel):
        return None
    return rec["fetch_bytes"] + rec["write_bytes"]


def _counter_median(path: str, counter: str, kernel_substr: str) -> float:
    per_dispatch = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter and kernel_substr in r["Kernel_Name"]:
                d = r["Dispatch_Id"]
                per_dispatch[d] = per_dispatch.get(d, 0.0) + float(r["Counter_Value"])
    if not per_dispatch:
        raise RuntimeError(f"no {counter} rows for {kernel_substr!r} in {path}")
    return statistics.median(per_dispatch.values())


def choose_path(x, path: str, prologue: bool, segments: int = 1) -> str:
    """pipe (gdn_prefill / gdn_prefill_fused), split (gdn_prefill_split / _fused) or seg
    (gdn_prefill_seg) for this workload: the rule gdn_prefill_auto_plan applies on a
    256-CU device (the timed run asks the library itself; this copy names the kernels
    of a counter summary on a host without the GPU).  A two-launch path for 16-bit I/O
    when its chain's N * Hv * 4 workgroups (two 16-channel slices each) fit the 256 CUs
    in one round, or for a packed batch of several sequences; among them the segmented
    one when gdn_prefill_seg_choose gave three segments or more (not with the
    prologue)."""
    if path != "auto":
        return path
    if x.io != "f32" and (x.N * x.Hv * chain_workgroups_per_head(64, True) <= 256 or x.N > 1):
        return "seg" if segments >= 3 and not prologue else "split"
    return "pipe"


def chain_workgroups_per_head(chunk: int, wide: bool) -> int:
    """The chain kernel's workgroups per (sequence, head): one per 16 value channels, or
    with two slices per workgroup (chunks of up to 64 tokens) one per 32."""
    return 4 if wide and chunk <= 64 else 8


def summarize_pmc(directory: str, workload: int, calib_mib: int, io=None, kda=False, prologue=False,
                  path: str = "auto", shard: int = 1, segments: int = 1) -> dict:
    """Scale the FETCH_SIZE / WRITE_SIZE counters (KiB per dispatch) of the prefill kernel by
    what the same counters read for a copy of known size; rocprofv3 runs of bench.py wrote
    fetch_, write_, copyfetch_ and copywrite_counter_collection.csv into `directory`.  With
    kda the step's two kernels are added (bytes per step); with prologue the counters are
    those of a `bench.py --prologue` run; `segments` is the count the run's library chose
    (the host has no device to ask)."""
    from linear_attention_chunked_gdn_amd import gdn, inputs
    x = inputs.head_shard(inputs.make_workload(workload, io=io, per_channel=kda, raw=prologue), shard)
    if kda:
        kernel = "kda_map_kernel+kda_chain_kernel"
    elif choose_path(x, path, prologue, segments) == "seg":
        kernel = "gdn_map_kernel+kda_chain_kernel+gdn_seg_join_kernel+gdn_seg_fix_kernel"
    elif choose_path(x, path, prologue, segments) == "split":
        kernel = "gdn_map_kernel+kda_chain_kernel"
    else:
        plan = gdn.prefill_plan(x.N, x.Hv, IO_CODE[x.io])
        kernel = "gdn_prefill_pipe_kernel" if plan["threads_per_workgroup"] == 512 else "gdn_prefill_kernel"
    true_kib = calib_mib * 1024.0
    f = lambda n, c, k: _counter_median(os.path.join(directory, f"{n}_counter_collection.csv"), c, k)  # noqa: E731
    fscale = true_kib / f("copyfetch", "FETCH_SIZE", "")
    wscale = true_kib / f("copywrite", "WRITE_SIZE", "")
    if prologue:
        kernel += "(prologue)"
    parts = [p.split("(")[0] for p in kernel.split("+")]
    fetch = sum(f("fetch", "FETCH_SIZE", k) for k in parts) * fscale * 1024
    write = sum(f("write", "WRITE_SIZE", k) for k in parts) * wscale * 1024
    return {f"{kernel}@{x.name}": {
        "sources_sha256": sources_sha256(kernel), "fetch_bytes": fetch, "write_bytes": write,
        "fetch_scale": fscale, "write_scale": wscale, "algorithmic_bytes": algorithmic_bytes(x)}}


def algorithmic_bytes(x) -> int:
    """q, k once per key head; v, o once per value head; beta and g (fp32; g per key
    channel for KDA); the fp32 state read (if given) and written."""
    s = 4 if x.io == "f32" else 2
    T, Hk, Hv, Dk, Dv, N = x.T_tot, x.Hk, x.Hv, x.Dk, x.Dv, x.N
    state = N * Hv * Dv * Dk * 4 * (2 if x.initial_state is not None else 1)
    gate = 4 * (Dk if x.per_channel else 1)
    return T * (Hk * 2 * Dk * s + Hv * (2 * Dv * s + 4 + gate)) + state


def algorithmic_flops(x, C: int = 64) -> int:
    """Sum over chunks of n_c tokens: Hv*(6*n_c*Dk*Dv + 2*n_c^2*Dv) + Hk*2*n_c^2*Dk
    (the three state products K S^T, Q S^T and v^T K; the intra-chunk P v product;
    the K K^T gram per key head).  This is the method's own work, not the padded
    tile work of any kernel.  With a per-key-channel gate the decays enter the sums over
    key channels, so both grams (K K^T and Q K^T, 4*n_c^2*Dk) are per value head."""
    total = 0
    for L in x.seq_lengths():
        full, tail = divmod(int(L), C)
        for n_c, cnt in ((C, full), (tail, 1 if tail else 0)):
            if x.per_channel:
                total += cnt * x.Hv * (6 * n_c * x.Dk * x.Dv + 2 * n_c * n_c * x.Dv + 4 * n_c * n_c * x.Dk)
            else:
                total += cnt * (x.Hv * (6 * n_c * x.Dk * x.Dv + 2 * n_c * n_c * x.Dv)
                                + x.Hk * 2 * n_c * n_c * x.Dk)
    return total


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(x, min_repeats: int = 3, min_seconds: float = 5.0, prologue: int = 0,
                 single_thread: bool = False) -> dict:
    """Median wall time of whole-workload oracle runs (with the input prologue's steps
    when given): at least min_repeats runs and at least min_seconds of CPU work in total,
    on every OpenMP thread; with single_thread, also one run on one thread."""
    import oracle
    oracle.load_library()
    cores = oracle.max_threads()

    def run(nthreads):
        t0 = time.perf_counter()
        q, k, g, b = oracle.prologue(x.q, x.k, x.g, x.beta, prologue)
        oracle.recurrent(q, k, x.v, g, b, x.initial_state, x.cu_seqlens, nthreads=nthreads)
        return time.perf_counter() - t0

    times = []
    while len(times) < min_repeats or sum(times) < min_seconds:
        times.append(run(cores))
    repeats = len(times)
    dt = float(np.median(times))
    threads_used = min(cores, x.N * x.Hv)   # OpenMP over (sequence, head) pairs
    rec = {"value": x.T_tot / dt, "unit": "tokens/s", "cores": threads_used,
           "kind": "oracle", "cpu_model": cpu_model(), "omp_threads": cores,
           "sample": f"the whole workload ({x.T_tot} tokens x {x.Hv} heads), fp64 token-by-token "
                     f"recurrence, OpenMP over (sequence, head); median of {repeats} runs, "
                     f"{dt:.3f} s each"}
    if single_thread:   # last: the oracle keeps the thread count it was last given
        t1 = run(1)
        rec["single_thread"] = {"value": x.T_tot / t1, "unit": "tokens/s", "cores": 1,
                                "sample": f"the whole workload on one thread, one run of {t1:.3f} s"}
    return rec


def decode_bench(x, dev, state0) -> dict:
    """The workload's single-token decode steps (gdn_decode_step, B = N), started from the
    prefill's final state: mean time per step with the steps launched from Python (each
    launch waits on the host), and with the same steps captured once in a HIP graph and
    replayed (launches back to back, so the figure is the kernels' own time).  Every
    replay is checked bitwise against the eager run."""
    import torch
    from linear_attention_chunked_gdn_amd import gdn
    dec = x.decode
    n = dec["steps"]
    io = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[x.io]
    dq, dk, dv = (torch.from_numpy(np.ascontiguousarray(dec[k])).to(dev, io) for k in ("q", "k", "v"))
    dg, db = (torch.from_numpy(np.ascontiguousarray(dec[k])).to(dev, torch.float32) for k in ("g", "beta"))
    outs = torch.empty((n, x.N, x.Hv, x.Dv), dtype=io, device=dev)
    step_fn = gdn.kda_decode_step if x.per_channel else gdn.decode_step
    state = torch.empty_like(state0)
    B = x.N

    def run():
        for i in range(n):
            sl = slice(i * B, (i + 1) * B)
            step_fn(dq[sl], dk[sl], dv[sl], dg[sl], db[sl], state, out=outs[i])

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    state.copy_(state0)
    run()
    state.copy_(state0)
    torch.cuda.synchronize()
    e0, e1 = ev(), ev()
    e0.record()
    run()
    e1.record()
    torch.cuda.synchronize()
    eager_us = e0.elapsed_time(e1) * 1e3 / n
    ref_o, ref_s = outs.clone(), state.clone()

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        state.copy_(state0)
        run()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(graph):
        run()
    times, exact = [], True
    for _ in range(5):
        state.copy_(state0)
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3 / n)
        exact &= bool(torch.equal(outs, ref_o)) and bool(torch.equal(state, ref_s))
    if not exact:
        raise RuntimeError("decode graph replay differs from the eager decode steps")
    graph_us = float(np.median(times))
    state_bytes = B * x.Hv * x.Dv * x.Dk * 4 * 2
    return {"steps": n, "batch": B, "us_per_step_graph": graph_us, "us_per_step_eager": eager_us,
            "state_bytes_per_step": state_bytes,
            "state_GBps_graph": state_bytes / (graph_us * 1e-6) / 1e9,
            "note": "state read + written once per step; 4 MiB at H=32 stays in the Infinity "
                    "Cache between steps, so this is not an HBM fraction"}


def measured_peaks(dev) -> dict:
    """Peaks measured on this GPU beside the published ones: a 1 GiB device copy (bytes
    read + written per second) and a 8192^3 bf16 GEMM through torch (hipBLASLt)."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty(n, dtype=torch.uint8, device=dev)
    m = 8192
    x = torch.randn((m, m), dtype=torch.bfloat16, device=dev)
    y = torch.randn((m, m), dtype=torch.bfloat16, device=dev)
    res = {}
    for name, fn, work in (("copy_GBps", lambda: b.copy_(a), 2 * n / 1e9),
                           ("bf16_gemm_TFLOPs", lambda: torch.mm(x, y), 2 * m ** 3 / 1e12)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = work / (e0.elapsed_time(e1) / 10 / 1e3)
    del a, b, x, y
    torch.cuda.empty_cache()
    return res


def calibrate_copy(mib: int, steps: int) -> int:
    """Copies of a known number of bytes, for scaling FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = mib << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").random_(0, 255)
    bufs = [torch.empty(n, dtype=torch.uint8, device="cuda:0") for _ in range(2)]
    for i in range(steps):
        bufs[i % 2].copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes_read": n, "calibrate_copy_bytes_written": n,
                      "copies": steps}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=1)
    ap.add_argument("--io", choices=sorted(IO_CODE), default=None,
                    help="storage type of q, k, v, o (default: the workload's own)")
    ap.add_argument("--path", choices=["auto", "pipe", "split", "seg"], default="auto",
                    help="scalar-gate prefill entry point: gdn_prefill (pipe), gdn_prefill_split, "
                         "gdn_prefill_seg, or by shape (auto)")
    ap.add_argument("--chunk", type=int, choices=[32, 64, 128], default=64,
                    help="chunk length of the two-launch paths (gdn_prefill_split, gdn_prefill_seg)")
    ap.add_argument("--segments", type=int, default=0,
                    help="segments per sequence of gdn_prefill_seg (0: gdn_prefill_seg_choose's count)")
    ap.add_argument("--head-shard", type=int, default=1, metavar="G",
                    help="run one GPU's share of the workload's heads when they are split over G GPUs")
    ap.add_argument("--kda", action="store_true",
                    help="one decay per key channel (gdn_kda_prefill) on the same workload")
    ap.add_argument("--prologue", action="store_true",
                    help="raw inputs, the q/k norm, sigmoid and softplus steps applied in the kernels "
                         "(gdn_prefill_auto with all prologue flags; with --path, gdn_prefill_fused or "
                         "gdn_prefill_split_fused)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="time the K steps as launches from Python instead of one HIP graph of the K steps")
    ap.add_argument("--rotate-bytes", type=int, default=2 * MALL_BYTES,
                    help="input copies are rotated until they span at least this many bytes")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run device-to-device copies of MIB MiB "
                         "(the known-size reference for HBM byte counters)")
    ap.add_argument("--summarize-pmc", metavar="DIR",
                    help="instead of the benchmark, scale the FETCH_SIZE/WRITE_SIZE counter runs in "
                         "DIR by the copy calibration (--calibrate-copy MIB) and merge the result "
                         "into profiles/hbm_traffic.json")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only; --gpus must be 1", file=sys.stderr)
        return 2
    if args.summarize_pmc:
        entry = summarize_pmc(args.summarize_pmc, args.workload, args.calibrate_copy or 256, args.io, args.kda,
                              args.prologue, args.path, args.head_shard, args.segments or 1)
        try:
            with open(TRAFFIC_FILE) as f:
                table = json.load(f)
        except (OSError, ValueError):
            table = {}
        table.update(entry)
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(table, f, indent=1, sort_keys=True)
            f.write("\n")
        print(json.dumps(entry))
        return 0
    if args.calibrate_copy:
        return calibrate_copy(args.calibrate_copy, args.steps)

    import torch
    from linear_attention_chunked_gdn_amd import gdn, inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.prologue and args.kda:
        print("bench.py: --prologue applies to the scalar-gate prefill only", file=sys.stderr)
        return 2
    x = inputs.head_shard(inputs.make_workload(args.workload, io=args.io, per_channel=args.kda,
                                               raw=args.prologue), args.head_shard)
    pro = gdn.PROLOGUE_ALL if args.prologue else 0
    io = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[x.io]

    per_copy = algorithmic_bytes(x)
    copies = max(1, -(-args.rotate_bytes // per_copy))
    sets = []
    for _ in range(copies):
        t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)  # noqa: E731
        sets.append(dict(q=t(x.q, io), k=t(x.k, io), v=t(x.v, io), g=t(x.g, torch.float32),
                         beta=t(x.beta, torch.float32),
                         init=None if x.initial_state is None else t(x.initial_state, torch.float32),
                         cu=t(x.cu_seqlens, torch.int32) if x.N > 1 else None,
                         o=torch.empty((x.T_tot, x.Hv, x.Dv), dtype=io, device=dev),
                         fs=torch.empty((x.N, x.Hv, x.Dv, x.Dk), dtype=torch.float32, device=dev)))

    auto = None
    if args.path == "auto" and not args.kda and args.chunk == 64 and not args.segments:
        # the library's own choice (gdn_prefill_auto_plan), run through gdn_prefill_auto
        auto = gdn.prefill_auto_plan(x.N, x.T_tot, x.Hv, IO_CODE[x.io], pro)
        segments = auto["segments"]
        path = {"one_launch": "pipe", "split": "split", "seg": "seg"}[auto["path"]]
    else:
        segments = args.segments or gdn.prefill_seg_choose(x.N, x.T_tot, x.Hv, args.chunk)
        path = "kda" if args.kda else choose_path(x, args.path, args.prologue, segments)
    if path in ("split", "seg") and x.io == "f32":
        print(f"bench.py: --path {path} takes bf16 or fp16 I/O", file=sys.stderr)
        return 2
    if path == "seg" and pro:
        print("bench.py: --path seg runs without the prologue", file=sys.stderr)
        return 2
    chunk = args.chunk if path in ("split", "seg") else 64
    if args.chunk != 64 and path not in ("split", "seg"):
        print("bench.py: --chunk applies to the two-launch paths only", file=sys.stderr)
        return 2
    ws_bytes = {"kda": gdn.kda_workspace_size, "split": gdn.prefill_split_workspace_size,
                "seg": lambda N, T, Hv, C: gdn.prefill_seg_workspace_size(N, T, Hv, C, segments)}
    ws = (torch.empty(ws_bytes[path](x.N, x.T_tot, x.Hv, chunk), dtype=torch.uint8, device=dev)
          if path in ws_bytes else None)
    if auto is not None:
        ws = torch.empty(max(1, auto["workspace_bytes"]), dtype=torch.uint8, device=dev)

    def step(i):
        s = sets[i % copies]
        if auto is not None:
            gdn.prefill_auto(s["q"], s["k"], s["v"], s["g"], s["beta"], s["init"], s["cu"],
                             out=s["o"], final_state=s["fs"], workspace=ws, prologue=pro)
        elif path == "kda":
            gdn.kda_prefill(s["q"], s["k"], s["v"], s["g"], s["beta"], s["init"], s["cu"],
                            out=s["o"], final_state=s["fs"], workspace=ws)
        elif path == "split":
            gdn.prefill_split(s["q"], s["k"], s["v"], s["g"], s["beta"], s["init"], s["cu"], chunk_size=chunk,
                              out=s["o"], final_state=s["fs"], workspace=ws, prologue=pro)
        elif path == "seg":
            gdn.prefill_seg(s["q"], s["k"], s["v"], s["g"], s["beta"], s["init"], s["cu"], chunk_size=chunk,
                            segments=segments, out=s["o"], final_state=s["fs"], workspace=ws)
        else:
            gdn.prefill(s["q"], s["k"], s["v"], s["g"], s["beta"], s["init"], s["cu"],
                        out=s["o"], final_state=s["fs"], prologue=pro)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # no Python garbage collection inside the timed region: a collection pass while the
    # GPU has no queued work (right after the synchronisation) would be timed as GPU time
    gc.collect()
    gc.disable()
    # an event between consecutive steps as well: per-step times for the median and minimum
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps - 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
        if i < args.steps - 1:
            evs[i].record(stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gc.enable()
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = gpu_ms / args.steps
    marks = [ev0] + evs + [ev1]
    per_step = [marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)]
    timing = {"mode": "eager", "eager_ms_per_step": ms_per_step}
    if not args.eager:
        # The same K steps (same inputs, same order) captured once in a HIP graph and
        # replayed: the kernels then run back to back, without the host's launch gaps that
        # the eager loop above leaves between them.  The library makes no allocation, memset
        # or synchronisation inside a call, so a call is capturable as it stands.
        graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            for i in range(args.steps):
                step(i)
        graph.replay()   # untimed first replay
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gc.collect()
        gc.disable()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        g0.record(stream)
        graph.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        gc.enable()
        ms_per_step = g0.elapsed_time(g1) / args.steps
        timing = {"mode": "hip_graph", "eager_ms_per_step": gpu_ms / args.steps}
    tokens = x.T_tot

    # parity of the timed launches' last output against the oracle: every value head up to
    # 2^17 (token, head) pairs, else three value heads at the full length (first, middle,
    # last; the oracle's heads are independent, so a subset is exact)
    import oracle
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gpu_support import TOL_BF16_REL_RMS, TOL_F32_ABS, error_stats
    s = sets[(args.steps - 1) % copies]
    heads = list(range(x.Hv)) if x.T_tot * x.Hv <= (1 << 17) else sorted({0, x.Hv // 2, x.Hv - 1})
    xs = x if len(heads) == x.Hv else inputs.select_heads(x, heads)
    q_, k_, g_, b_ = oracle.prologue(xs.q, xs.k, xs.g, xs.beta, pro)
    ro, rf = oracle.recurrent(q_, k_, xs.v, g_, b_, xs.initial_state, xs.cu_seqlens)
    half = x.io != "f32"
    hsel = torch.tensor(heads, device=dev)
    eo = error_stats(s["o"].index_select(1, hsel).double().cpu().numpy(), ro, storage=x.io if half else None)
    ef = error_stats(s["fs"].index_select(1, hsel).double().cpu().numpy(), rf)
    # 16-bit I/O: kernel error / rms beside the stored outputs' rounding (the tests' bar)
    ok = (max(eo["kernel_rel_rms"], ef["kernel_rel_rms"]) <= TOL_BF16_REL_RMS if half
          else max(eo["max_abs"], ef["max_abs"]) <= TOL_F32_ABS)
    parity = {"value_heads": "all" if len(heads) == x.Hv else heads,
              "o_kernel_err_over_rms": eo["kernel_rel_rms"], "o_max_err_over_rms": eo["rel_rms"],
              "state_err_over_rms": ef["rel_rms"], "o_nmse": eo["nmse"], "state_nmse": ef["nmse"],
              "within_tolerance": ok}

    nbytes = algorithmic_bytes(x)
    flops = algorithmic_flops(x, chunk)
    sec = ms_per_step / 1e3
    if path in ("kda", "split", "seg"):
        kernel = ("kda_map_kernel" if path == "kda" else "gdn_map_kernel") + "+kda_chain_kernel"
        nseg = segments if path == "seg" else 1
        launch = {"path": path, "kernel": kernel, "map_workgroups": (x.T_tot // chunk + x.N) * x.Hv,
                  "chain_workgroups": x.N * x.Hv * (2 * nseg - 1) * chain_workgroups_per_head(
                      chunk, path == "seg" or x.N * x.Hv * 8 > 256),
                  "workspace_bytes": int(ws.numel()),
                  "input_copies_rotated": copies}
        if path == "seg":
            kernel += "+gdn_seg_join_kernel+gdn_seg_fix_kernel"
            launch.update(kernel=kernel, segments=nseg, join_workgroups=x.N * x.Hv * 8,
                          fix_workgroups=(x.T_tot // chunk + x.N) * x.Hv)
        if pro:
            kernel += "(prologue)"
            launch.update(kernel=kernel, prologue_flags=pro)
    else:
        plan = gdn.prefill_plan(x.N, x.Hv, IO_CODE[x.io])
        kernel = "gdn_prefill_pipe_kernel" if plan["threads_per_workgroup"] == 512 else "gdn_prefill_kernel"
        if pro:
            kernel += "(prologue)"
        launch = {"path": path, "kernel": kernel, "prologue_flags": pro,
                  "dv_per_workgroup": plan["dv_per_workgroup"], "workgroups": plan["workgroups"],
                  "lds_bytes": plan["lds_bytes"], "threads": plan["threads_per_workgroup"],
                  "input_copies_rotated": copies}
    launch["entry_point"] = "gdn_prefill_auto" if auto is not None else {
        "kda": "gdn_kda_prefill", "split": "gdn_prefill_split_fused" if pro else "gdn_prefill_split",
        "seg": "gdn_prefill_seg", "pipe": "gdn_prefill_fused" if pro else "gdn_prefill"}[path]
    if auto is not None:
        launch["auto_plan"] = auto
    mfma_peak = FP32_MFMA_PEAK_TFLOPS if x.io == "f32" else BF16_MFMA_PEAK_TFLOPS  # fp16 = bf16 rate
    rec = {
        "metric": KDA_METRIC.format(H=x.Hv, T=x.T_tot) if args.kda else METRIC,
        "value": tokens / sec,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "ms_per_step_median": float(np.median(per_step)),
        "ms_per_step_min": float(min(per_step)),
        "timing": dict(timing, note="ms_per_step and value time the K steps as timing.mode says; "
                                    "the median and minimum are of the eager loop's per-step events"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": x.io,
        "data": "synthetic",
        "config": {"workload": x.name, "head_shard_of_gpus": args.head_shard, "sequences": x.N, "tokens": x.T_tot, "Hk": x.Hk, "Hv": x.Hv,
                   "d": x.Dk, "chunk": chunk, "io": x.io, "state": "fp32",
                   "initial_state": x.initial_state is not None},
        "roofline": {"bound": "hbm", "achieved": nbytes / sec / 1e9, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": nbytes / sec / 1e9 / HBM_PEAK_GBS,
                     "traffic": recorded_traffic(kernel, x.name) if chunk == 64 else None},
        "mfma": {"achieved": flops / sec / 1e12, "peak": mfma_peak, "unit": "TFLOP/s",
                 "frac": flops / sec / 1e12 / mfma_peak, "algorithmic_flops": flops},
        "algorithmic_bytes": nbytes,
        "launch": launch,
        "wall_s_timed": wall,
        "parity": parity,
    }
    if x.decode is not None:
        rec["decode"] = decode_bench(x, dev, sets[(args.steps - 1) % copies]["fs"])
    rec["measured_peaks"] = measured_peaks(dev)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(x, prologue=pro,
                                           single_thread=args.workload in (0, 1) and args.head_shard == 1)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
