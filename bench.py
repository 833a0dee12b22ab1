#!/usr/bin/env python3
"""Decode-step benchmark on one MI355X: the paged KV write followed by paged decode attention.

A step is one pass of the whole path over one batch of synthetic, seeded inputs that are
resident in HBM before timing starts. The default workload is the long-context decode pair:
64 sequences x 8192 tokens, then 2 sequences x 32768 tokens (32 query heads, 8 KV heads,
head_dim 128, block_size 16, bf16, logits of std ~3); each step writes one new token per
sequence and then attends over all cached tokens of every sequence.

Prints ONE JSON line. `value` is the whole step's algorithmic HBM throughput (GB/s):
K and V of every context token (bf16), q (bf16), out (fp32) and the written K/V rows, over
the measured step time. `config.us_per_call` / `pct_of_peak` time each sub-workload's whole
attention call (the fused write, the attention kernel and the split-K merge) with HIP events
around the call; `roofline` reports the main attention kernel alone, timed with HIP events
the library records on its stream around each launch (even timed steps carry those, odd ones
the call events); `cpu_baseline` is the float64 CPU oracle timed on a bounded sample of the
same workload on this host, on all its cores and on one.

    python bench.py [--steps K] [--warmup W] [--workload c5|c5a|c5b|c1..c4]
"""
from __future__ import annotations

import argparse
import dataclasses
import ctypes
import hashlib
import re
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

METRIC = "paged decode attention µs/call and achieved HBM GB/s (% of MI355X peak)"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, vendor figure
TRAFFIC_FILE = os.path.join(HERE, "profiles", "decode_traffic.json")
OUT_TORCH = {"f32": "float32", "bf16": "bfloat16", "f16": "float16"}  # torch dtype names


def warm_up(args, torch, step):
    """The untimed warm-up: args.warmup steps when given; otherwise at least 5 and until
    args.warmup_seconds of them have run. Sets args.warmup to the number done."""
    if args.warmup is not None:
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        return args.warmup
    n = 0
    t0 = time.perf_counter()
    while True:
        for _ in range(5):
            step()
        n += 5
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= args.warmup_seconds:
            break
    args.warmup = n
    return n


def event_steps(steps, per_kind):
    """Indices of the timed steps that carry kernel events and of those that carry call
    events: per_kind of each, spread evenly over the steps (every step, alternating, when
    there are not enough steps for both kinds; a single step times the kernel)."""
    if steps <= 1:
        return [0], []
    if per_kind <= 0 or 2 * per_kind >= steps:
        return list(range(0, steps, 2)), list(range(1, steps, 2))
    kern = [int((j + 0.25) * steps / per_kind) for j in range(per_kind)]
    call = [int((j + 0.75) * steps / per_kind) for j in range(per_kind)]
    return kern, call


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=None,
                   help="untimed warm-up steps (default: at least 5, and as many as run in "
                        "--warmup-seconds; the JSON line reports the number done)")
    p.add_argument("--event-steps", type=int, default=4,
                   help="decode workloads: timed steps that carry the kernel's timing events, "
                        "and as many that carry the whole call's; the other timed steps carry "
                        "none (0, or too few steps for both: every step, alternating)")
    p.add_argument("--warmup-seconds", type=float, default=0.5,
                   help="without --warmup: keep warming up until the GPU has run the step "
                        "this long (its clocks rise over the first tens of milliseconds of "
                        "sustained work: a p1 prefill call measured 473 us after 5 warm-up "
                        "calls and 383 us after 100)")
    p.add_argument("--workload", default="c5")
    p.add_argument("--kernel", default="auto",
                   choices=["auto", "valu", "mfma", "mfma_hw", "mfma_sk"])
    p.add_argument("--partition", type=int, default=0,
                   help="tokens per partition (multi-query workloads: keys per partition of a "
                        "query tile, a multiple of 32): 0 automatic, -1 never split")
    p.add_argument("--in-dtype", default="bf16", choices=["bf16", "f16"],
                   help="format of q and the K/V pools")
    p.add_argument("--out-dtype", default="f32", choices=["f32", "bf16", "f16"],
                   help="attention output format: f32 or the input format")
    p.add_argument("--row-blocks", type=int, default=0, choices=[0, 1, 2, 4],
                   help="multi-query workloads: 16-row query blocks per wave (0 = library's choice)")
    p.add_argument("--separate", action="store_true",
                   help="decode workloads: KV write and attention as two calls instead of the "
                        "fused decode step")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-read-probe", action="store_true",
                   help="skip the plain streaming-read reference after the timed steps")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="wall-time budget of each of the two oracle baseline passes")
    p.add_argument("--json-out", default=None)
    p.add_argument("--jsonl", default=None,
                   help="after the timed steps, also write one JSON row per (decode workload, "
                        "cold / hot) to this file: call and kernel times, GB/s, read probe, "
                        "max |out - oracle|, oracle times, seeds, input hashes, versions")
    p.add_argument("--rope", action="store_true",
                   help="rotate q and the new keys first (positions L-1, Llama 3 base 500000 "
                        "frequencies) and attend with the rotated q: one fused launch, or "
                        "with --separate the rotation + write call, then attention")
    p.add_argument("--graph", action="store_true",
                   help="also capture one step in a graph and time K replays: through torch's "
                        "graph wrapper (graph_ms_per_step) and through the HIP runtime's own "
                        "stream capture (hip_graph_ms_per_step), beside K plain steps with no "
                        "timing events (eager_ms_per_step_no_events)")
    p.add_argument("--graph-steps", type=int, default=1,
                   help="with --graph: decode steps captured in one graph (as a model captures "
                        "all its layers' steps in one graph); the times are per step")
    p.add_argument("--flush-mib", type=int, default=0,
                   help="before every step, read a buffer of this many MiB so no input stays "
                        "in the 256 MB last-level cache (cold-cache timing; the read is inside "
                        "the measured step time, the kernel times exclude it)")
    p.add_argument("--prepared", action="store_true",
                   help="decode workloads: also time the fused step as prepared calls "
                        "(checks and argument conversion done once; prepared_ms_per_step)")
    p.add_argument("--block-size", type=int, default=16,
                   help="decode workloads: tokens per cache block (a multiple of 16); the "
                        "table width and pool shrink by the same factor, so the contexts and "
                        "the bytes read stay those of the workload")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="run one plain device-to-device copy of this many MiB before the "
                        "steps (reference dispatch for hardware byte counters)")
    p.add_argument("--record-traffic", default=None, metavar="DIR",
                   help="no GPU run: read the FETCH_SIZE and WRITE_SIZE counter passes under "
                        "DIR/FETCH_SIZE and DIR/WRITE_SIZE (rocprofv3 csv of this script with "
                        "--copy-calibration-mib 1024), scale them by the copy's readings and "
                        "store the workload's HBM bytes per attention launch in "
                        "profiles/decode_traffic.json")
    args = p.parse_args()
    if args.block_size < 16 or args.block_size % 16:
        p.error(f"--block-size {args.block_size}: a multiple of 16 tokens")
    return args


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch has already loaded. They are created
    timing-only (hipEventDisableSystemFence): recording them performs no system-scope fence,
    so they neither add a cache write-back to the measured interval nor disturb the next
    kernel; the host reads them only after a full device synchronisation."""

    DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence (hip_runtime_api.h)

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                                     ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.events = []

    def create(self):
        ev = ctypes.c_void_p()
        if self.hip.hipEventCreateWithFlags(ctypes.byref(ev), self.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        self.events.append(ev.value)
        return ev.value

    def record(self, ev, stream):
        if self.hip.hipEventRecord(ev, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self):
        for ev in self.events:
            self.hip.hipEventDestroy(ev)
        self.events = []


def hip_graph_replay_ms(args, torch, dev, step):
    """args.graph_steps steps captured with the HIP runtime's own stream capture
    (hipStreamBeginCapture on a side stream the library is called on, no torch graph wrapper)
    into one graph, instantiated and replayed back to back for about args.steps steps;
    milliseconds per step."""
    hip = ctypes.CDLL("libamdhip64.so.7")
    vp = ctypes.c_void_p
    hip.hipStreamBeginCapture.argtypes = [vp, ctypes.c_int]
    hip.hipStreamEndCapture.argtypes = [vp, ctypes.POINTER(vp)]
    hip.hipGraphInstantiate.argtypes = [ctypes.POINTER(vp), vp, vp, vp, ctypes.c_size_t]
    hip.hipGraphLaunch.argtypes = [vp, vp]
    hip.hipGraphExecDestroy.argtypes = [vp]
    hip.hipGraphDestroy.argtypes = [vp]
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        step()  # first call on this stream outside the capture
    torch.cuda.synchronize()
    handle = side.cuda_stream
    graph, exe = vp(), vp()
    with torch.cuda.stream(side):
        if hip.hipStreamBeginCapture(handle, 2):  # hipStreamCaptureModeRelaxed
            raise RuntimeError("hipStreamBeginCapture failed")
        for _ in range(args.graph_steps):
            step()
        if hip.hipStreamEndCapture(handle, ctypes.byref(graph)):
            raise RuntimeError("hipStreamEndCapture failed")
    if hip.hipGraphInstantiate(ctypes.byref(exe), graph, None, None, 0):
        raise RuntimeError("hipGraphInstantiate failed")
    try:
        for _ in range(min(args.warmup, 20)):
            hip.hipGraphLaunch(exe, handle)
        torch.cuda.synchronize()
        reps = max(1, args.steps // args.graph_steps)
        t0 = time.perf_counter()
        for _ in range(reps):
            if hip.hipGraphLaunch(exe, handle):
                raise RuntimeError("hipGraphLaunch failed")
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / (reps * args.graph_steps)
    finally:
        hip.hipGraphExecDestroy(exe)
        hip.hipGraphDestroy(graph)


KERNEL_SOURCES = {"valu": "decode_valu.hip", "mfma": "decode_mfma.hip",
                  "mfma_hw": "decode_mfma.hip", "mfma_sk": "decode_sk.hip"}
KERNEL_SYMBOLS = {"valu": "decode_valu_kernel<", "mfma": "decode_mfma_kernel<",
                  "mfma_hw": "decode_mfma_hw_kernel<", "mfma_sk": "decode_mfma_sk_kernel<"}


def _code_hash(files) -> str:
    """Hash of the code of these csrc files with comments and blank lines removed."""
    csrc = os.path.join(HERE, "paged_kv_decode_write_amd", "csrc")
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            text = re.sub(r"/\*.*?\*/", "", fh.read(), flags=re.S)
        for line in text.splitlines():
            code = line.split("//", 1)[0].rstrip()
            if code.strip():
                h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def kernel_source_hash(kernel: str) -> str:
    """Hash of the code of the sources the decode kernel families `kernel` ("a" or "a+b") are
    built from: a recorded traffic figure stays valid across comment edits only."""
    files = ["device_common.h", "launch.h", "mfma_tiles.h", "decode_step.h"]
    for k in kernel.split("+"):
        if KERNEL_SOURCES[k] not in files:
            files.append(KERNEL_SOURCES[k])
    return _code_hash(files)


def library_source_hash() -> str:
    """Hash of the code of every source the library is built from."""
    csrc = os.path.join(HERE, "paged_kv_decode_write_amd", "csrc")
    return _code_hash(sorted(f for f in os.listdir(csrc) if f.endswith((".h", ".hip", ".cpp"))))


def record_traffic(args):
    """HBM bytes per attention launch from two rocprofv3 counter passes of this script
    (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled so that the plain copy of
    --copy-calibration-mib 1024 run in the same pass reads and writes exactly 1 GiB; the
    figure is stored with the hash of the kernel's sources, and a later run reports it only
    while that hash still matches."""
    import csv
    import statistics
    copy_mib = 1024
    copy_grid = 131072  # work items of the runtime's copyBuffer dispatch for a 1 GiB copy
    per, copy = {}, {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        path = os.path.join(args.record_traffic, counter, "run_counter_collection.csv")
        with open(path, newline="") as f:
            rows = [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]
        # every attention dispatch, in order (the merge kernels are not among these)
        fam = [next((k for k, sym in KERNEL_SYMBOLS.items() if sym in r["Kernel_Name"]), None)
               for r in rows]
        used = [k for k in dict.fromkeys(fam) if k is not None]
        if args.kernel != "auto":
            used = [args.kernel]
        kernel = "+".join(used)
        per[counter] = [float(r["Counter_Value"]) for r, k in zip(rows, fam) if k in used]
        copies = [float(r["Counter_Value"]) for r in rows
                  if "copyBuffer" in r["Kernel_Name"] and int(r["Grid_Size"]) == copy_grid]
        if not per[counter] or not copies:
            raise SystemExit(f"{path}: no {kernel} dispatch or no {copy_mib} MiB copy")
        copy[counter] = copies[0]
    fetch_scale = (copy_mib << 10) / copy["FETCH_SIZE"]
    write_scale = (copy_mib << 10) / copy["WRITE_SIZE"]
    fetch = statistics.fmean(per["FETCH_SIZE"]) * 1024 * fetch_scale
    write = statistics.fmean(per["WRITE_SIZE"]) * 1024 * write_scale
    cmd = ("rocprofv3 --pmc {c} --output-format csv -d {d}/{c} -o run -- python -u bench.py "
           "--workload {w} --steps 3 --warmup 1 --no-cpu-baseline --no-read-probe "
           "--copy-calibration-mib 1024")
    rec = {"kernel": kernel, "kernel_source": kernel_source_hash(kernel),
           "bytes_per_launch": int(round(fetch + write)),
           "fetch_bytes_per_launch": int(round(fetch)), "write_bytes_per_launch": int(round(write)),
           "fetch_scale": round(fetch_scale, 5), "write_scale": round(write_scale, 5),
           "launches": len(per["FETCH_SIZE"]),
           "fetch_kib_per_launch": per["FETCH_SIZE"], "write_kib_per_launch": per["WRITE_SIZE"],
           "copy_fetch_kib": copy["FETCH_SIZE"], "copy_write_kib": copy["WRITE_SIZE"],
           "commands": [cmd.format(c=c, d=args.record_traffic, w=args.workload)
                        for c in ("FETCH_SIZE", "WRITE_SIZE")]}
    table = {}
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            table = json.load(f)
    table[args.workload] = rec
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(table, f, indent=1)
        f.write("\n")
    print(json.dumps({k: rec[k] for k in ("kernel", "bytes_per_launch", "fetch_scale",
                                          "write_scale", "launches")}))


def read_probe(torch, dev, nbytes, reps=5):
    """Achievable streaming-read rate at this byte count: read kernels (libpagedkv_probe.so)
    over a buffer of nbytes, cold (a 1 GiB buffer is read in between so neither L2 nor the MALL
    holds it), timed with events: grid-stride with plain loads, grid-stride with the
    non-temporal hint, and contiguous chunks per workgroup with the hint (four workgroups per
    CU: the fastest simple read measured on this part). Returns the fastest as (median us,
    GB/s), and every rate."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(HERE, "paged_kv_decode_write_amd", "libpagedkv_probe.so"))
    for fn in (lib.pagedkv_read_probe, lib.pagedkv_read_probe_nt,
               lib.pagedkv_read_probe_chunked_nt):
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int32,
                       ctypes.c_void_p]
    grid = 256 * 16
    chunk_grid = 4 * torch.cuda.get_device_properties(dev).multi_processor_count
    nbytes = (nbytes + 15) // 16 * 16
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    flush = torch.ones((1 << 30) // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros(grid, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rates = {}
    for name, fn, g in (("plain", lib.pagedkv_read_probe, grid),
                        ("nontemporal", lib.pagedkv_read_probe_nt, grid),
                        ("chunked_nontemporal", lib.pagedkv_read_probe_chunked_nt, chunk_grid)):
        times = []
        for i in range(reps + 1):
            if lib.pagedkv_read_probe(flush.data_ptr(), flush.numel() * 4, sink.data_ptr(), grid,
                                      stream):
                raise RuntimeError("read probe launch failed")
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            if fn(buf.data_ptr(), nbytes, sink.data_ptr(), g, stream):
                raise RuntimeError("read probe launch failed")
            b.record()
            torch.cuda.synchronize()
            if i:
                times.append(a.elapsed_time(b) * 1e3)
        rates[name] = sorted(times)[len(times) // 2]
    del buf, flush, sink
    us = min(rates.values())
    return us, nbytes / (us * 1e-6) / 1e9, {k: round(nbytes / (v * 1e-6) / 1e9, 1)
                                              for k, v in rates.items()}


def _oracle_pass(subs, seconds):
    """The float64 oracle, as it stands, on the sequences of the step's sub-workloads in order
    (KV write + attention, all heads) until `seconds` of wall time are spent. Returns
    (algorithmic bytes covered, seconds, sample description)."""
    import numpy as np
    import torch

    import oracle
    from paged_kv_decode_write_amd import workloads as wl

    spent, nbytes, parts = 0.0, 0, []
    for d in subs:
        w = d["workload"]
        bs = w.block_size
        tables = d["block_tables"].cpu().numpy()
        lens = d["context_lens"].cpu().numpy()
        q = wl.to_bits(d["q"])
        kn, vn = wl.to_bits(d["k_new"]), wl.to_bits(d["v_new"])
        done = 0
        for b in range(w.batch):
            if spent >= seconds:
                break
            L = int(lens[b])
            n = (L + bs - 1) // bs
            ids = torch.from_numpy(tables[b, :n].astype(np.int64)).to(d["k_cache"].device)
            kc = wl.to_bits(d["k_cache"].index_select(0, ids))
            vc = wl.to_bits(d["v_cache"].index_select(0, ids))
            local = np.arange(n, dtype=np.int32)[None]
            slot = np.array([(n - 1) * bs + (L - 1) % bs], dtype=np.int64)
            t0 = time.perf_counter()
            kc2, vc2 = oracle.kv_write(kn[b:b + 1], vn[b:b + 1], slot, kc, vc)
            oracle.decode_attention(q[b:b + 1], kc2, vc2, local, lens[b:b + 1], d["scale"])
            spent += time.perf_counter() - t0
            ab = wl.algorithmic_bytes(w, [L])
            nbytes += ab["kv"] + (ab["q"] + ab["out"] + ab["write"]) // w.batch
            done += 1
        if done:
            parts.append(f"{w.name}: sequences 0..{done - 1} of {w.batch}")
    return nbytes, spent, "; ".join(parts)


def cpu_baseline(subs, seconds):
    """The oracle timed on this host: once with numpy's BLAS on every core this process may
    run on (its default), once on one thread. Each pass gets `seconds` of wall time at most."""
    import numpy  # noqa: F401  (loads the BLAS whose thread pool is read below)
    from threadpoolctl import threadpool_info, threadpool_limits

    host_cores = len(os.sched_getaffinity(0))
    blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    threads = max((p.get("num_threads", 1) for p in blas), default=1)
    nb_all, t_all, sample_all = _oracle_pass(subs, seconds)
    with threadpool_limits(limits=1):
        nb_one, t_one, sample_one = _oracle_pass(subs, seconds)
    what = " (KV write + attention, all query heads), float64 numpy"
    return {"value": round(nb_all / t_all / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{sample_all}{what}, {threads} BLAS threads on {host_cores} host "
                      f"cores, {t_all:.1f} s",
            "host_cores": host_cores,
            "single_thread": {"value": round(nb_one / t_one / 1e9, 4), "unit": "GB/s",
                              "cores": 1,
                              "sample": f"{sample_one}{what}, one BLAS thread, "
                                        f"{t_one:.1f} s"}}


RECORD_WORKLOADS = ["c1", "c2", "c3", "c4", "c5a", "c5b"]


def _gather_sequences(d):
    """Each sequence's blocks as host bit patterns, local table, slot of its new row."""
    import numpy as np
    import torch
    from paged_kv_decode_write_amd import workloads as wl

    w = d["workload"]
    bs = w.block_size
    tables = d["block_tables"].cpu().numpy()
    lens = d["context_lens"].cpu().numpy()
    seqs = []
    for b in range(w.batch):
        L = int(lens[b])
        n = (L + bs - 1) // bs
        ids = torch.from_numpy(tables[b, :n].astype(np.int64)).to(d["k_cache"].device)
        kc = wl.to_bits(d["k_cache"].index_select(0, ids))
        vc = wl.to_bits(d["v_cache"].index_select(0, ids))
        slot = np.array([(n - 1) * bs + (L - 1) % bs if L else -1], dtype=np.int64)
        seqs.append((kc, vc, np.arange(n, dtype=np.int32)[None], slot, lens[b:b + 1]))
    return seqs


def _oracle_step(d, seqs):
    """The oracle's decode step (write + attention, all heads), sequence by sequence; returns
    (float64 output [B, Hq, D], seconds spent in the oracle)."""
    import numpy as np

    import oracle
    from paged_kv_decode_write_amd import workloads as wl

    q = wl.to_bits(d["q"])
    kn, vn = wl.to_bits(d["k_new"]), wl.to_bits(d["v_new"])
    out = np.zeros(q.shape, dtype=np.float64)
    spent = 0.0
    for b, (kc, vc, local, slot, L) in enumerate(seqs):
        t0 = time.perf_counter()
        kc2, vc2 = oracle.kv_write(kn[b:b + 1], vn[b:b + 1], slot, kc, vc)
        out[b:b + 1] = oracle.decode_attention(q[b:b + 1], kc2, vc2, local, L, d["scale"])
        spent += time.perf_counter() - t0
    return out, spent


def _environment(torch):
    props = torch.cuda.get_device_properties(0)
    rocm = None
    for path in ("/opt/rocm/.info/version", "/opt/rocm/.info/version-dev"):
        if os.path.exists(path):
            with open(path) as f:
                rocm = f.read().strip()
            break
    return {"gpu": props.name, "gcn_arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "rocm": rocm,
            "hip": torch.version.hip, "torch": torch.__version__,
            "host_cores": len(os.sched_getaffinity(0)),
            "library_source": library_source_hash()}


def _input_sha256(d):
    from paged_kv_decode_write_amd import workloads as wl
    h = hashlib.sha256()
    for key in ("q", "k_cache", "v_cache", "k_new", "v_new"):
        h.update(wl.to_bits(d[key]).tobytes())
    for key in ("block_tables", "context_lens", "slot_mapping"):
        h.update(d[key].cpu().numpy().tobytes())
    return h.hexdigest()


def measurement_record(args, torch, pk, wl, path):
    """One JSON row per (workload, cold / hot) for every decode workload, written to `path`:
    the fused decode step (write + attention + merge) timed with HIP events around the call
    on its stream, 3 warm-up calls and the median of 10 samples. Cold: a 512 MiB buffer is
    read before each sample (no input left in L2 or the 256 MB last-level cache); hot: 100
    back-to-back calls per sample, enqueued behind a GPU-side delay so that the host's launch
    rate does not set the pace. Each cold row also carries the attention kernel alone, a
    cold streaming read of the same bytes, the max |out - oracle| over every output row, and
    the float64 oracle's time for the same step on all host cores and on one (median of 3
    for the three smallest workloads, one run otherwise)."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    dev = torch.device("cuda:0")
    env = _environment(torch)
    hip = HipEvents()
    flush = torch.zeros((512 << 20) // 4, dtype=torch.float32, device=dev)
    blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    threads = max((p.get("num_threads", 1) for p in blas), default=1)
    rows = []
    for name in RECORD_WORKLOADS:
        w = wl.WORKLOADS[name]
        big = name.startswith("c5")
        inp = wl.make_inputs(w, device="cuda" if big else "cpu")
        d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
        del inp
        sha = _input_sha256(d)
        out = torch.empty(w.batch, w.num_q_heads, w.head_dim, dtype=torch.float32, device=dev)
        ws = pk.new_workspace(pk.decode_workspace_bytes(w.batch, w.num_q_heads, w.head_dim,
                                                        w.max_blocks, w.block_size, 0), dev)
        plan = pk.decode_plan(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.max_blocks,
                              w.block_size, 0, "auto", with_kernel=True)
        ab = wl.algorithmic_bytes(w, d["context_lens"].cpu().tolist())
        stream = torch.cuda.current_stream(dev).cuda_stream

        def call(events=None):
            pk.paged_decode_step(d["q"], d["k_new"], d["v_new"], d["slot_mapping"],
                                 d["k_cache"], d["v_cache"], d["block_tables"],
                                 d["context_lens"], d["scale"], out, workspace=ws,
                                 events=events)

        def sample(cold, reps=1, kernel_only=False):
            if cold:
                torch.sum(flush)
            else:
                # keep the GPU busy (a bounded spin, no memory traffic) while the host enqueues
                # the burst, so back-to-back calls are timed, not the host's launch rate
                torch.cuda._sleep(4_000_000)
            a, b = hip.create(), hip.create()
            if kernel_only:
                call((a, b))
            else:
                hip.record(a, stream)
                for _ in range(reps):
                    call()
                hip.record(b, stream)
            torch.cuda.synchronize()
            return hip.elapsed_ms(a, b) * 1e3 / reps

        for _ in range(3):
            sample(True)
        cold = sorted(sample(True) for _ in range(10))
        kern = sorted(sample(True, kernel_only=True) for _ in range(10))
        for _ in range(3):
            sample(False)
        hot = sorted(sample(False, reps=100) for _ in range(10))
        probe_us, probe_gbs, _ = read_probe(torch, dev, ab["attention"])
        hip.close()

        seqs = _gather_sequences(d)
        runs = 1 if name in ("c4", "c5a", "c5b") else 3
        ref, t_all = None, []
        for _ in range(runs):
            ref, t = _oracle_step(d, seqs)
            t_all.append(t)
        t_one = []
        with threadpool_limits(limits=1):
            for _ in range(runs):
                t_one.append(_oracle_step(d, seqs)[1])
        del seqs
        err = float(np.abs(out.cpu().double().numpy() - ref).max())
        base = {"workload": name, "description": w.description, "seed": w.seed,
                "input_sha256": sha, "batch": w.batch, "num_q_heads": w.num_q_heads,
                "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                "block_size": w.block_size, "num_blocks": w.num_blocks,
                "kernel": plan[2], "partitions": plan[0], "tokens_per_partition": plan[1],
                "call": "paged_decode_step (write + attention + merge), bf16 in, f32 out",
                "algorithmic_bytes": ab["attention"], "env": env}
        for mode, us in (("cold", cold), ("hot", hot)):
            med = us[len(us) // 2]
            row = dict(base, mode=mode,
                       us={"median": round(med, 2), "min": round(us[0], 2),
                           "max": round(us[-1], 2), "samples": len(us)},
                       GBps=round(ab["attention"] / (med * 1e-6) / 1e9, 1),
                       pct_of_peak=round(100 * ab["attention"] / (med * 1e-6) / 1e9
                                         / PEAK_HBM_GBS, 2),
                       max_abs_err=err)
            if mode == "cold":
                row["attn_kernel_us_median"] = round(kern[len(kern) // 2], 2)
                row["read_probe"] = {"us": round(probe_us, 2), "GBps": round(probe_gbs, 1)}
                row["oracle"] = {"seconds_median": round(sorted(t_all)[len(t_all) // 2], 4),
                                 "blas_threads": threads,
                                 "seconds_one_thread_median": round(
                                     sorted(t_one)[len(t_one) // 2], 4),
                                 "runs": runs}
            rows.append(row)
        print(f"[record] {name}: cold {cold[len(cold) // 2]:.2f} us, hot "
              f"{hot[len(hot) // 2]:.2f} us, max|err| {err:.2e}", file=sys.stderr, flush=True)
        del d, out, ws
        torch.cuda.empty_cache()
    with open(path, "w") as f:
        for row in rows:
            f.write(json.dumps(row) + "\n")
    return rows


PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix throughput, vendor figure


def bench_prefill(args, torch, pk, wl):
    """Multi-query causal workloads: step = write the chunk's K/V + causal attention."""
    dev = torch.device("cuda:0")
    w = wl.PREFILL_WORKLOADS[args.workload]
    d = wl.make_prefill_inputs(w, device="cuda", dtype=args.in_dtype)
    T, Hq, D = d["q"].shape
    out = torch.empty(T, Hq, D, dtype=getattr(torch, OUT_TORCH[args.out_dtype]), device=dev)
    alg = wl.prefill_algorithmic(w)
    write_bytes = T * w.num_kv_heads * w.head_dim * 2 * 2 * 2
    plan = pk.prefill_plan(T, d["max_q_len"], len(w.context_lens), Hq, w.num_kv_heads, D,
                           w.max_blocks, w.block_size, args.row_blocks, args.partition)

    def step(ev=None):
        pk.paged_kv_write(d["k_new"], d["v_new"], d["slot_mapping"], d["k_cache"], d["v_cache"])
        if ev is not None:
            ev[0].record()
        pk.paged_prefill_attention(d["q"], d["cu_seqlens_q"], d["k_cache"], d["v_cache"],
                                   d["block_tables"], d["context_lens"], d["scale"], out,
                                   max_q_len=d["max_q_len"], row_blocks=args.row_blocks,
                                   partition_tokens=args.partition)
        if ev is not None:
            ev[1].record()

    warm_up(args, torch, step)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    durs = sorted(a.elapsed_time(b) for a, b in evs)
    mean = sum(durs) / len(durs)
    tflops = alg["flops"] / (mean * 1e-3) / 1e12
    line = {
        "metric": "paged multi-query causal attention us/call and achieved TFLOP/s",
        "value": round(alg["flops"] / (ms_per_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": args.in_dtype,
        "data": f"synthetic (seeded N(0,1) {args.in_dtype}), resident in HBM",
        "config": {"workload": w.description, "kernel": "prefill_mfma",
                   "row_blocks": plan[0], "key_partitions": plan[1],
                   "keys_per_partition": plan[2],
                   "formats": f"{args.in_dtype} in, {args.out_dtype} out",
                   "us_per_call": round(mean * 1e3, 2),
                   "GBps": round(alg["bytes"] / (mean * 1e-3) / 1e9, 1),
                   "step": "KV write of the chunk + multi-query causal attention"
                           + (" + partition merge" if plan[1] > 1 else "")},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": None},
        "details": {"flops": alg["flops"], "bytes": alg["bytes"], "write_bytes": write_bytes,
                    "attn_us_median": round(durs[len(durs) // 2] * 1e3, 2)},
    }
    return line


def main():
    args = parse_args()
    if args.record_traffic:
        record_traffic(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the path has no "
              "multi-GPU leg to time.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    from paged_kv_decode_write_amd import _binding as pk
    from paged_kv_decode_write_amd import workloads as wl

    pk.load_library()
    dev = torch.device("cuda:0")
    if args.out_dtype not in ("f32", args.in_dtype):
        print(f"output format {args.out_dtype} is not built for {args.in_dtype} inputs "
              "(fp32 or the input format)", file=sys.stderr)
        sys.exit(2)
    if args.rope and args.in_dtype != "bf16":
        print("the rotary embedding takes bf16 inputs only", file=sys.stderr)
        sys.exit(2)
    if args.workload in wl.PREFILL_WORKLOADS:
        line = bench_prefill(args, torch, pk, wl)
        out = json.dumps(line)
        print(out, flush=True)
        if args.json_out:
            with open(args.json_out, "w") as f:
                f.write(out + "\n")
        return
    names = ["c5a", "c5b"] if args.workload == "c5" else [args.workload]
    subs = []
    for name in names:
        w = wl.WORKLOADS[name]
        if args.block_size != w.block_size:
            k = args.block_size // w.block_size
            if k < 1 or args.block_size % w.block_size or w.max_blocks % k or w.num_blocks % k:
                print(f"--block-size {args.block_size} does not divide {name}'s table",
                      file=sys.stderr)
                sys.exit(2)
            w = dataclasses.replace(w, block_size=args.block_size, max_blocks=w.max_blocks // k,
                                    num_blocks=w.num_blocks // k)
        d = wl.make_inputs(w, device="cuda", dtype=args.in_dtype)
        d["out"] = torch.empty(w.batch, w.num_q_heads, w.head_dim,
                               dtype=getattr(torch, OUT_TORCH[args.out_dtype]), device=dev)
        need = pk.decode_workspace_bytes(w.batch, w.num_q_heads, w.head_dim, w.max_blocks,
                                         w.block_size, args.partition)
        d["ws"] = pk.new_workspace(need, dev)
        d["bytes"] = wl.algorithmic_bytes(w, d["context_lens"].cpu().tolist(),
                                          out_bytes=4 if args.out_dtype == "f32" else 2)
        d["plan"] = pk.decode_plan(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                   w.max_blocks, w.block_size, args.partition, args.kernel,
                                   with_kernel=True)
        if args.rope:
            d["pos"] = (d["context_lens"] - 1).to(torch.int32)
            d["inv_freq"] = (500000.0 ** (-torch.arange(0, w.head_dim, 2, device=dev,
                                                          dtype=torch.float64) / w.head_dim)
                             ).to(torch.float32)
            d["q_rot"] = torch.empty_like(d["q"])
            d["bytes"]["write"] += d["q"].numel() * 2  # the rotated q is written out
        subs.append(d)
    torch.cuda.synchronize()

    # Eviction by reading only: a written buffer would leave dirty lines whose write-back
    # would then compete with the measured kernel.
    flush = (torch.zeros((args.flush_mib << 20) // 4, dtype=torch.float32, device=dev)
             if args.flush_mib > 0 else None)

    hip = HipEvents()

    def attend(d, ev):
        """The sub-workload's attention call (the fused step, or with --separate the write
        call and then the attention call); ev = (kernel begin, kernel end) or None."""
        if args.rope and not args.separate:
            # one launch rotates q and the new key, stores the rows and attends
            pk.paged_decode_step_rope(d["q"], d["k_new"], d["v_new"], d["pos"],
                                      d["inv_freq"], d["slot_mapping"], d["q_rot"],
                                      d["k_cache"], d["v_cache"], d["block_tables"],
                                      d["context_lens"], d["scale"], d["out"],
                                      partition_tokens=args.partition, kernel=args.kernel,
                                      workspace=d["ws"], events=ev)
        elif not args.separate:
            # one launch stores the new rows and attends (plus the merge when split)
            pk.paged_decode_step(d["q"], d["k_new"], d["v_new"], d["slot_mapping"],
                                 d["k_cache"], d["v_cache"], d["block_tables"],
                                 d["context_lens"], d["scale"], d["out"],
                                 partition_tokens=args.partition, kernel=args.kernel,
                                 workspace=d["ws"], events=ev)
        else:
            pk.paged_decode_attention(d["q_rot"] if args.rope else d["q"], d["k_cache"],
                                      d["v_cache"], d["block_tables"],
                                      d["context_lens"], d["scale"], d["out"],
                                      partition_tokens=args.partition, kernel=args.kernel,
                                      workspace=d["ws"], events=ev)

    def step(events=None, kernel_events=False):
        """One decode step over every sub-workload. events[i] = (begin, end) of sub-workload
        i. With kernel_events the library records them around the attention kernel alone;
        otherwise they bracket the whole attention call on its stream (the fused write, the
        attention kernel and the partition merge), with no event between its launches."""
        if flush is not None:
            torch.sum(flush)
        stream = torch.cuda.current_stream(dev).cuda_stream
        for i, d in enumerate(subs):
            ev = events[i] if events is not None else None
            if args.separate:
                if args.rope:
                    pk.paged_kv_write_rope(d["q"], d["k_new"], d["v_new"], d["pos"],
                                           d["inv_freq"], d["slot_mapping"], d["k_cache"],
                                           d["v_cache"], q_out=d["q_rot"])
                else:
                    pk.paged_kv_write(d["k_new"], d["v_new"], d["slot_mapping"], d["k_cache"],
                                      d["v_cache"])
            if ev is not None and not kernel_events:
                hip.record(ev[0], stream)
            attend(d, ev if kernel_events else None)
            if ev is not None and not kernel_events:
                hip.record(ev[1], stream)

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    warm_up(args, torch, step)

    # Some timed steps time the attention kernel (events the library records around it),
    # others the whole call (events around the call only), spread over the timed region; the
    # rest carry no events, since each event record costs the GPU about 2 us between kernels
    # (the c5 step measured 370.2 us with none, 377.7 with four per step).
    kern_steps, call_steps = event_steps(args.steps, args.event_steps)
    evs = {i: [(hip.create(), hip.create()) for _ in subs] for i in kern_steps + call_steps}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs.get(i), kernel_events=i in kern_steps)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    per = []
    for j, d in enumerate(subs):
        kern = sorted(hip.elapsed_ms(*evs[i][j]) for i in kern_steps)
        call = sorted(hip.elapsed_ms(*evs[i][j]) for i in call_steps) or kern
        kmean = sum(kern) / len(kern)
        cmean = sum(call) / len(call)
        w = d["workload"]
        ab = d["bytes"]["attention"]
        per.append({
            "workload": w.name, "description": w.description,
            "kernel": d["plan"][2],
            "partitions": d["plan"][0], "tokens_per_partition": d["plan"][1],
            "call_us_mean": round(cmean * 1e3, 2),
            "call_us_median": round(call[len(call) // 2] * 1e3, 2),
            "call_us_min": round(call[0] * 1e3, 2),
            "call_us_max": round(call[-1] * 1e3, 2),
            "attn_bytes": ab,
            "call_GBps": round(ab / (cmean * 1e-3) / 1e9, 1),
            "pct_of_peak": round(100 * ab / (cmean * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
            "attn_kernel_us_mean": round(kmean * 1e3, 2),
            "attn_kernel_us_median": round(kern[len(kern) // 2] * 1e3, 2),
            "attn_kernel_us_min": round(kern[0] * 1e3, 2),
            "attn_kernel_us_max": round(kern[-1] * 1e3, 2),
            "attn_kernel_GBps": round(ab / (kmean * 1e-3) / 1e9, 1),
            "attn_kernel_pct_of_peak": round(100 * ab / (kmean * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                             2),
        })
    hip.close()

    graph_ms = hip_graph_ms = eager_ms = None
    if args.graph:
        # The same steps, plain, with no timing events: the reference for the replays.
        for _ in range(min(args.warmup, 20)):
            step()
        torch.cuda.synchronize()
        e0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        eager_ms = (time.perf_counter() - e0) * 1e3 / args.steps
        hip_graph_ms = hip_graph_replay_ms(args, torch, dev, step)
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(args.graph_steps):
                step()
        for _ in range(min(args.warmup, 20)):
            graph.replay()
        torch.cuda.synchronize()
        reps = max(1, args.steps // args.graph_steps)
        g0 = time.perf_counter()
        for _ in range(reps):
            graph.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - g0) * 1e3 / (reps * args.graph_steps)

    prepared_ms = plain_ms = None
    if args.prepared and not args.rope and not args.separate:
        prepared = [pk.prepare_decode_step(d["q"], d["k_new"], d["v_new"], d["slot_mapping"],
                                           d["k_cache"], d["v_cache"], d["block_tables"],
                                           d["context_lens"], d["scale"], d["out"],
                                           partition_tokens=args.partition, kernel=args.kernel,
                                           workspace=d["ws"])
                    for d in subs]

        def prepared_step():
            if flush is not None:
                torch.sum(flush)
            for call in prepared:
                call()

        def per_step_ms(fn):
            for _ in range(min(args.warmup, 20)):
                fn()
            torch.cuda.synchronize()
            t = time.perf_counter()
            for _ in range(args.steps):
                fn()
            torch.cuda.synchronize()
            return (time.perf_counter() - t) * 1e3 / args.steps

        # the same calls through the plain binding, with no timing events, for comparison
        plain_ms = per_step_ms(step)
        prepared_ms = per_step_ms(prepared_step)

    probe = {}
    if not args.no_read_probe:
        for d in subs:
            us, gbs, both = read_probe(torch, dev, d["bytes"]["attention"])
            probe[d["workload"].name] = {"us": round(us, 2), "GBps": round(gbs, 1),
                                         "GBps_by_load": both}

    step_bytes = sum(d["bytes"]["attention"] + d["bytes"]["write"] for d in subs)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    launch_bytes = sum(d["bytes"]["attention"] for d in subs) / len(subs)
    launch_s = sum(p["attn_kernel_us_mean"] for p in per) / len(per) * 1e-6
    achieved = launch_bytes / launch_s / 1e9
    kernel = "+".join(dict.fromkeys(p["kernel"] for p in per))

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        rec = t.get(args.workload, {})
        if (rec.get("kernel_source") == kernel_source_hash(kernel) and rec.get("kernel") == kernel
                and (args.in_dtype, args.out_dtype) == ("bf16", "f32")):
            traffic = rec.get("bytes_per_launch")

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.in_dtype if kernel.startswith("mfma") else "fp32",
        "event_steps": {"kernel": len(kern_steps), "call": len(call_steps),
                        "none": args.steps - len(kern_steps) - len(call_steps)},
        "data": (f"synthetic (seeded N(0,1) {args.in_dtype} K/V pools, shuffled block tables), "
                 "resident in HBM"),
        "config": {
            "workload": "+".join(d["workload"].description for d in subs),
            "kernel": kernel,
            "partition_tokens": args.partition,
            "block_size": subs[0]["workload"].block_size,
            "formats": f"{args.in_dtype} in, {args.out_dtype} out",
            "us_per_call": {p["workload"]: p["call_us_mean"] for p in per},
            "pct_of_peak": {p["workload"]: p["pct_of_peak"] for p in per},
            "attn_kernel_us": {p["workload"]: p["attn_kernel_us_mean"] for p in per},
            "kernels": {p["workload"]: p["kernel"] for p in per},
            "step": ("RoPE + KV write, then decode attention (two calls)"
                     if args.rope and args.separate else
                     "fused decode step with RoPE: rotation + KV write + decode attention in "
                     "one launch" if args.rope else
                     "KV write, then decode attention (two calls)" if args.separate else
                     "fused decode step: KV write + decode attention in one launch") +
                    " per sub-workload",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
        },
        "details": per,
    }
    if graph_ms is not None:
        line["graph_ms_per_step"] = round(graph_ms, 4)
        line["hip_graph_ms_per_step"] = round(hip_graph_ms, 4)
        line["eager_ms_per_step_no_events"] = round(eager_ms, 4)
    if prepared_ms is not None:
        line["prepared_ms_per_step"] = round(prepared_ms, 4)
        line["plain_ms_per_step_no_events"] = round(plain_ms, 4)
    if probe:
        # plain streaming read (cold) of the attention's algorithmic bytes: the rate HBM
        # delivers to a simple kernel on this part, beside the 8 TB/s vendor peak
        line["read_probe"] = probe
    if not args.no_cpu_baseline and (args.in_dtype, args.out_dtype) == ("bf16", "f32"):
        line["cpu_baseline"] = cpu_baseline(subs, args.cpu_seconds)
    if args.jsonl:
        del subs
        torch.cuda.empty_cache()
        measurement_record(args, torch, pk, wl, args.jsonl)
    out = json.dumps(line)
    print(out, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(out + "\n")


if __name__ == "__main__":
    main()
