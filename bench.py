#!/usr/bin/env python3
"""Throughput of the sparse-delta-memory hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config c2|c1|c3|c4|c0] [--entry steps|step]

The default workload is c2: 4096 streams over a 16 GiB bfloat16 bank, W = R = 64
rows of 256 bytes, a gate per write, 32 tokens per stream.

A step is one decode token for every stream of the workload (one pass of the
decode step), or one sdm_gather launch over every token (--config c3). Inputs
are seeded and synthetic (gen/), generated on the GPU and resident in HBM
before the timed region; the decode runs the workload's token sequence, the
bank changing from token to token as the method intends. By default a decode
launch is one sdm_decode_steps call over the whole sequence, and K defaults to
four passes of it, timed back to back (any K is accepted: whole passes, then
the sequence's first K mod T tokens in one more launch); ``--entry step``
launches sdm_decode_step once per token instead (K defaults to one pass). The timed launches run as one HIP-graph replay (``--launch
eager`` launches from Python instead) bracketed by HIP events on the stream
the kernels run on. Before each timed leg the device is first kept busy with
plain copies for --settle-ms (100 ms by default), so that its clocks are out of
any idle state (the CPU baseline before it leaves the device idle for seconds);
then come the W warm-up steps.

Prints one JSON line: stream-steps/s (tokens/s for the gather), the achieved
bank-row bandwidth against the MI355X's 8 TB/s HBM peak, and the CPU oracle
timed on a bounded sample of the same workload (one thread, and all host
cores). A decode run with the default entry also times the same tokens as one
sdm_decode_step launch each, reported under "single_token". The line also gives
the rate of a plain streaming device copy measured in the same run
(roofline.copy_gbps) and each rate as a fraction of it (copy_frac), and the
host the CPU baseline ran on (cpu_baseline.host).
"""

from __future__ import annotations

import argparse
import glob
import hashlib
import json
import re
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "stream-steps/sec + achieved HBM GB/s (bank row bytes) on one MI355X"
HBM_PEAK_GBPS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
STORAGE_DTYPE = {"torch.bfloat16": "bf16", "torch.float32": "f32"}


# The sources a launch kind's kernels are built from (besides the shared header
# and the C ABI, which sets up every launch).
KIND_SOURCES = {"decode": "sdm_decode.hip", "gather": "sdm_gather.hip"}


def kernel_source_hash(kind: str = None) -> str:
    """Hash of the HIP kernel sources' code (comments and whitespace removed): of the
    shared header, the C ABI and the kind's own kernel file (a decode kind: "step",
    "steps"; a gather kind: "gather..."), or of every source (kind None). Stored
    HBM-traffic figures are valid only for the hash of their kind."""
    h = hashlib.sha256()
    paths = sorted(glob.glob(os.path.join(ROOT, "sparse_delta_rule_amd", "csrc", "*")))
    if kind is not None:
        own = KIND_SOURCES["gather" if kind.startswith("gather") else "decode"]
        paths = [p for p in paths if os.path.basename(p) in (own, "sdm_kernels.h", "sdm_api.hip")]
    for p in paths:
        with open(p, encoding="utf-8") as f:
            text = f.read()
        code = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        code = re.sub(r"//[^\n]*", " ", code)
        h.update(os.path.basename(p).encode())
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def launch_kind(config: str, entry: str, gather: str = "two-ops") -> str:
    """What one timed launch runs: the gather (or one of its other launch shapes), the
    multi-token decode or the single step."""
    if config == "c3":
        return "gather" if gather == "two-ops" else f"gather-{gather}"
    return "steps" if entry == "steps" else "step"


def kernel_pattern(kind: str) -> str:
    return KERNEL_PATTERN["gather" if kind.startswith("gather") else kind]


# Name fragment that selects a launch kind's kernels in a rocprofv3 trace (the
# multi-token decode has two loops and the gather two layouts; the library picks
# one per launch shape).
KERNEL_PATTERN = {"gather": "sdm_gather_", "steps": "sdm_decode_steps", "step": "sdm_decode_kernel"}

# Gather launch shapes: (both operands, stash), as bench.py --gather names them.
GATHER_SHAPES = {"two-ops": (True, True), "one-op": (False, True), "no-stash": (True, False),
                 "one-op-no-stash": (False, False)}


def stored_traffic(config: str, kind: str, tokens_per_launch: int = 1, live_tokens=None):
    """(HBM bytes, kernel name) that rocprofv3 measured for one launch of this shape
    (profiles/traffic.json), or (None, None) when no figure applies.

    A figure applies only while the kernel sources are the ones it was taken on. A
    decode entry holds the bytes of a launch of ``tokens_per_launch`` tokens and is
    scaled to the asked launch's token count (each token of a launch moves the same
    rows); a multi-token figure does not stand for a single-token launch, which runs
    another kernel. A gather entry applies only to a launch with the same live-token
    count."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None, None
    with open(path) as f:
        data = json.load(f)
    entry = data.get(f"{config}/{kind}")
    if not entry or entry.get("kernel_source_hash") != kernel_source_hash(kind):
        return None, None
    stored_tokens = entry.get("tokens_per_launch")
    if not stored_tokens or not entry.get("bytes_per_launch"):
        return None, None
    if kind.startswith("gather"):
        if live_tokens is None or entry.get("live_tokens") != live_tokens:
            return None, None
        return entry["bytes_per_launch"], entry.get("kernel")
    if (stored_tokens == 1) != (tokens_per_launch == 1):
        return None, None
    return entry["bytes_per_launch"] / stored_tokens * tokens_per_launch, entry.get("kernel")


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None, help="timed steps (default: the workload's sequence)")
    p.add_argument("--warmup", type=int, default=8)
    p.add_argument("--settle-ms", type=float, default=100.0,
                   help="before each timed leg, keep the device busy with plain copies for this long (0: none)")
    p.add_argument("--config", default="c2", choices=["c0", "c1", "c2", "c3", "c4"])
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--launch", default="graph", choices=["graph", "eager"])
    p.add_argument("--entry", default="steps", choices=["steps", "step"],
                   help="decode: one sdm_decode_steps launch per token sequence (steps), or one "
                        "sdm_decode_step launch per token (step)")
    p.add_argument("--gather", default="two-ops",
                   choices=["two-ops", "one-op", "no-stash", "one-op-no-stash", "compact"],
                   help="gather launch shape on the c3 tokens: both operands with the stash (the workload), "
                        "operand 0 only (the backward's gather), either without the stash, or both operands "
                        "with a compact stash (sdm_gather_compact, positions from each chunk's sorted slots)")
    p.add_argument("--streams", default=None, metavar="N[,N...]",
                   help="decode: run the workload with N streams instead (each stream keeps its slot range, so "
                        "the bank holds N x slots-per-stream rows); a list runs each in turn, one line each")
    p.add_argument("--ingest-stream-sweep", metavar="TRACE",
                   help="summarise a rocprofv3 kernel trace of a --streams sweep into profiles/ (no GPU): the "
                        "kernel's duration per stream count, and its fit as a fixed cost plus a cost per stream")
    p.add_argument("--ceiling", default=None, metavar="MODE[,MODE...]",
                   help="measure reference access patterns instead of the method (libsdm_ceiling): read, stash, "
                        "rmw, mix (two row reads and one row write per unit, the decode's mix), copy or copy-nt "
                        "(non-temporal); one line per pattern and bank size")
    p.add_argument("--bank-gib", default="16", metavar="G[,G...]", help="with --ceiling: bank sizes in GiB")
    p.add_argument("--row-bytes", type=int, default=256, help="with --ceiling: bytes per row")
    p.add_argument("--ceiling-layout", default="uniform", choices=["uniform", "streams"],
                   help="with --ceiling: rows uniform over the bank, or (rmw, mix) laid out as the decode's c2 "
                        "streams: each run of 64 units draws its rows from its own range of 16384 slots")
    p.add_argument("--host-call-cost", action="store_true",
                   help="host time per call of a small gather (64 tokens, two operands, no stash), launched "
                        "back to back: sdm_gather and a gather plan's launch, from Python and through ctypes")
    p.add_argument("--ingest-ceiling", nargs=5, metavar=("TRACE", "FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                   help="summarise rocprofv3 output of one --ceiling run (one bank size) into profiles/ (no GPU)")
    p.add_argument("--tokens", type=int, default=None,
                   help="gather: launch over this many tokens (a multiple of the chunk) instead of the workload's")
    p.add_argument("--head-dim", type=int, default=None,
                   help="gather: bank rows of this many elements instead of the workload's (same slots and tokens)")
    p.add_argument("--bank-dtype", choices=["bf16", "f32"], default=None,
                   help="gather: bank element type instead of the workload's")
    p.add_argument("--outputs-apart", type=int, default=None, metavar="ROWS",
                   help="gather with two operands: both outputs in one allocation, operand 1's starting ROWS "
                        "output rows after operand 0's last (0: back to back, the two a power of two apart "
                        "when the token count is one); measures how the kernel depends on where the outputs lie")
    p.add_argument("--valid", default="per-chunk",
                   help="gather: per-chunk (the workload's per-chunk counts), all (every token live, no counts) "
                        "or N (one count N for every chunk, passed as the scalar valid)")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of the oracle sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="run only a plain 1 GiB device copy (for scaling rocprofv3 byte counters)")
    p.add_argument("--ingest-profile", nargs=5, metavar=("TRACE", "FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                   help="summarise rocprofv3 output directories of this config into profiles/ (no GPU)")
    p.add_argument("--profile-commands", default="", help="text of the commands that made the directories")
    p.add_argument("--extra-counters", nargs="*", default=[], metavar="DIR",
                   help="with --ingest-profile: rocprofv3 --pmc runs of TCC_HIT_sum/TCC_MISS_sum, VmemLatency, "
                        "TCC_EA0_RDREQ_LEVEL_sum/TCC_EA0_RDREQ_sum, summarised as L2 hit rate and latencies")
    return p.parse_args(argv)


def _timed(torch, stream, fn):
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end)  # ms


def settle_device(torch, ms: float) -> None:
    """Keep the device busy with plain 256 MiB copies for about ``ms`` milliseconds, so
    that its clocks have left any idle state before a measurement (after the CPU
    baseline, for instance, the device has idled for seconds). Outside every timed
    region, and on buffers of its own."""
    if ms <= 0:
        return
    n = (256 << 20) // 4
    a = torch.ones(n, device="cuda")
    b = torch.empty_like(a)
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
    del a, b


def _run_steps(torch, args, launch_one, K):
    """Settle the device, warm up, then time K launches (as one graph replay, or
    eagerly). Returns ms."""
    stream = torch.cuda.current_stream()
    settle_device(torch, args.settle_ms)
    for i in range(args.warmup):
        launch_one(i)
    torch.cuda.synchronize()
    if args.launch == "eager":
        return _timed(torch, stream, lambda: [launch_one(i) for i in range(K)])
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(K):
            launch_one(i)
    graph.replay()  # untimed first replay
    torch.cuda.synchronize()
    return _timed(torch, torch.cuda.current_stream(), graph.replay)


# ------------------------------------------------------------------ CPU baseline
THREAD_CAP = 16
THREAD_CAP_REASON = ("one GPU's share of the host: the GPU box gives a one-GPU job 16 CPUs "
                     "(OMP_NUM_THREADS=16 there), whatever the machine's core count")


def host_threads() -> int:
    """Host threads for the all-cores oracle run: the process's CPUs, at most the
    OMP_NUM_THREADS share when that is set, and at most THREAD_CAP."""
    n = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, min(n, THREAD_CAP))


def cpu_model() -> str:
    """The host CPU's model name as lscpu reports it (else from /proc/cpuinfo)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
        for line in out.splitlines():
            if line.split(":", 1)[0].strip() == "Model name":
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_record() -> dict:
    """What the CPU baseline ran on: core counts, model and the thread cap."""
    return {"nproc": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)), "model": cpu_model(),
            "thread_cap": THREAD_CAP, "thread_cap_reason": THREAD_CAP_REASON,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


class pinned_to_one_cpu:
    """Pin the calling thread (and the threads it starts meanwhile, which inherit its
    mask) to one CPU of the process's set, as ``taskset -c`` would; restore on exit."""

    def __enter__(self):
        self.saved = os.sched_getaffinity(0)
        self.cpu = min(self.saved)
        os.sched_setaffinity(0, {self.cpu})
        return self

    def __exit__(self, *exc):
        os.sched_setaffinity(0, self.saved)
        return False


def _bank_np(torch, t):
    import numpy as np
    t = t.detach().cpu().contiguous()
    return t.view(torch.int16).numpy().view(np.uint16).copy() if t.dtype == torch.bfloat16 else t.float().numpy().copy()


def decode_groups(torch, wl, bank, seq, n, groups):
    """Streams [0, n) of a decode workload as ``groups`` contiguous stream ranges, each
    with the bank rows its sequence touches (its private rows that some step writes or
    reads, in slot order) and its inputs with the slots renumbered into those rows:
    what one oracle thread steps through the whole sequence. Rows no step touches
    cannot change any reading or touched row, so they are left out."""
    bounds = [n * g // groups for g in range(groups + 1)]
    out = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        if a == b:
            continue
        used = torch.unique(torch.cat([inp[k][a:b].reshape(-1).to(torch.int64)
                                       for inp in seq for k in ("k_idx", "q_idx")]))
        steps = []
        for inp in seq:
            d = {}
            for k, v in inp.items():
                v = v[a:b]
                if k in ("k_idx", "q_idx"):
                    d[k] = torch.searchsorted(used, v.to(torch.int64).contiguous()).cpu().numpy()
                else:
                    d[k] = v.detach().cpu().float().numpy()
            steps.append(d)
        out.append((_bank_np(torch, bank[used]), steps))
    return out


def sample_streams(wl, target_streams: int, max_bytes: int = 2 << 30) -> int:
    """Streams in an oracle sample: ``target_streams``, at most every stream, and at most
    as many as keep the sample's touched bank rows within ``max_bytes`` of host memory."""
    es = 2 if "bfloat16" in str(wl.bank_dtype) else 4
    rows_per_stream = min(wl.slots_per_stream, (wl.W + wl.R) * wl.steps)
    cap = max(1, max_bytes // (rows_per_stream * wl.head_dim * es))
    return int(max(1, min(wl.streams, target_streams, cap)))


def run_decode_groups(groups):
    """Step every group through its sequence, one thread per group (the oracle's C
    calls release the GIL). Returns each group's readings per step."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle

    def one(grp):
        b, steps = grp
        return [oracle.decode_step(b, **inp) for inp in steps]

    with ThreadPoolExecutor(max_workers=max(1, len(groups))) as ex:
        return list(ex.map(one, groups))


def cpu_baseline_decode(torch, wl, bank, seq, target_s, cfg_name):
    """Time the oracle on a subset of streams over the whole sequence: one thread pinned
    to one CPU, and one thread per host core (up to THREAD_CAP) over contiguous stream
    groups."""
    # calibrate on 32 streams x 2 steps (enough work that fixed call costs do not
    # dominate), then size the sample for ~target_s of work
    m = min(32, wl.streams)
    (b, steps), = decode_groups(torch, wl, bank, seq[:2], m, 1)
    with pinned_to_one_cpu():
        t0 = time.perf_counter()
        run_decode_groups([(b, steps)])
        per = (time.perf_counter() - t0) / (2 * m)
    n = sample_streams(wl, int(target_s / max(per * len(seq), 1e-9)))
    grp = decode_groups(torch, wl, bank, seq, n, 1)
    with pinned_to_one_cpu() as pin:
        t0 = time.perf_counter()
        run_decode_groups(grp)
        dt = time.perf_counter() - t0
    cores = host_threads()
    n_all = sample_streams(wl, n * cores)
    grp = decode_groups(torch, wl, bank, seq, n_all, cores)
    t0 = time.perf_counter()
    run_decode_groups(grp)
    dt_all = time.perf_counter() - t0
    return {"value": n * len(seq) / dt, "unit": "stream-steps/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} of {wl.streams} streams x all {len(seq)} steps of {cfg_name} "
                      f"(single-threaded C oracle pinned to CPU {pin.cpu}, {dt:.1f} s)",
            "pinned_cpu": pin.cpu, "host": host_record(),
            "all_cores": {"value": n_all * len(seq) / dt_all, "unit": "stream-steps/s", "cores": len(grp),
                          "sample": f"{n_all} of {wl.streams} streams x all {len(seq)} steps, one thread per "
                                    f"group of streams ({dt_all:.1f} s)"}}


def gather_ranges(torch, wl, bank, inp, n, groups):
    """Tokens [0, n) of the gather workload (n a multiple of the chunk) as ``groups``
    chunk-aligned token ranges over one shared sub-bank of the rows they touch."""
    sel = torch.arange(n, device=bank.device)
    i0, i1 = inp["idx0"][sel].long(), inp["idx1"][sel].long()
    uniq, inv = torch.unique(torch.cat([i0.ravel(), i1.ravel()]), return_inverse=True)
    sub = _bank_np(torch, bank[uniq])
    a0 = inv[:i0.numel()].view_as(i0).cpu().numpy()
    a1 = inv[i0.numel():].view_as(i1).cpu().numpy()
    w0 = inp["w0"][sel].float().cpu().numpy()
    w1 = inp["w1"][sel].float().cpu().numpy()
    cv = inp["chunk_valid"][: n // wl.chunk].cpu().numpy()
    chunks = n // wl.chunk
    bounds = [chunks * g // groups * wl.chunk for g in range(groups + 1)]
    return sub, [(a0[a:b], w0[a:b], a1[a:b], w1[a:b], cv[a // wl.chunk:b // wl.chunk])
                 for a, b in zip(bounds[:-1], bounds[1:]) if a < b]


def run_gather_ranges(wl, sub, ranges):
    """The oracle's gather over each token range, one thread per range. Returns each
    range's (out0, stash, out1)."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle

    def one(r):
        a0, w0, a1, w1, cv = r
        return oracle.gather(sub, a0, w0, chunk=wl.chunk, chunk_valid=cv, idx1=a1, w1=w1)

    with ThreadPoolExecutor(max_workers=max(1, len(ranges))) as ex:
        return list(ex.map(one, ranges))


def cpu_baseline_gather(torch, wl, bank, inp, target_s, cfg_name):
    """Time the oracle on the first tokens of the launch: one thread pinned to one CPU,
    and one thread per host core (up to THREAD_CAP) over chunk-aligned token ranges."""
    def timed(n, groups):
        sub, ranges = gather_ranges(torch, wl, bank, inp, n, groups)
        t0 = time.perf_counter()
        run_gather_ranges(wl, sub, ranges)
        return time.perf_counter() - t0, len(ranges)

    with pinned_to_one_cpu():
        per = timed(wl.chunk * 4, 1)[0] / (wl.chunk * 4)
    n = int(max(wl.chunk, min(wl.tokens, target_s / max(per, 1e-9))) // wl.chunk * wl.chunk)
    with pinned_to_one_cpu() as pin:
        dt, _ = timed(n, 1)
    cores = host_threads()
    n_all = int(max(wl.chunk, min(wl.tokens, n * cores)) // wl.chunk * wl.chunk)
    dt_all, used = timed(n_all, cores)
    return {"value": n / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n} of {wl.tokens} tokens of {cfg_name} (single-threaded C oracle pinned to "
                      f"CPU {pin.cpu}, {dt:.1f} s)",
            "pinned_cpu": pin.cpu, "host": host_record(),
            "all_cores": {"value": n_all / dt_all, "unit": "tokens/s", "cores": used,
                          "sample": f"first {n_all} of {wl.tokens} tokens, one thread per chunk-aligned "
                                    f"range ({dt_all:.1f} s)"}}


# ------------------------------------------------------------------ workloads
def bench_decode(torch, args, cfg_name, wl):
    import gen
    from sparse_delta_rule_amd import sdm_decode_step, sdm_decode_steps
    dev = torch.device("cuda", 0)
    es = torch.empty((), dtype=wl.bank_dtype).element_size()
    T = wl.steps
    bank = gen.decode_bank(wl, args.seed, dev)
    seq = [gen.decode_step_inputs(wl, args.seed, t, dev) for t in range(T)]
    torch.cuda.synchronize()
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_decode(torch, wl, bank, seq, args.cpu_seconds, cfg_name)
    # default: four passes of the token sequence (the multi-token entry point), or
    # the sequence once (one launch per token); any K >= 1 is accepted
    K = args.steps if args.steps is not None else (4 * T if args.entry == "steps" else T)
    if K < 1:
        raise SystemExit("bench.py: --steps must be at least 1")
    row_bytes_step = wl.streams * (2 * wl.W + wl.R) * wl.head_dim * es
    if args.entry == "steps":
        stacked = {k: torch.stack([d[k] for d in seq]) for k in seq[0]}
        readings = torch.empty((T, wl.streams, wl.head_dim), dtype=wl.bank_dtype, device=dev)
        # K tokens per stream: whole passes of the sequence, then its first K mod T tokens
        plan = [T] * (K // T) + ([K % T] if K % T else [])
        part = {k: v[:K % T].contiguous() for k, v in stacked.items()} if K % T else None

        def launch_one(i):
            if plan[i % len(plan)] == T:
                sdm_decode_steps(bank, **stacked, readings=readings)
            else:
                sdm_decode_steps(bank, **part, readings=readings[:K % T])

        launches, per_launch = len(plan), plan[0]
    else:
        readings = [torch.empty((wl.streams, wl.head_dim), dtype=wl.bank_dtype, device=dev) for _ in seq]

        def launch_one(i):
            j = i % len(seq)
            sdm_decode_step(bank, **seq[j], readings=readings[j])

        launches, per_launch = K, 1
    ms = _run_steps(torch, args, launch_one, launches)
    ms_step = ms / K
    launch_bytes = row_bytes_step * per_launch
    gbps = row_bytes_step * K / (ms * 1e-3) / 1e9  # = bytes per launch / mean launch time
    name = f"{cfg_name}: {wl.name}"
    if wl.streams != gen.WORKLOADS[cfg_name].streams:
        name += f" [{wl.streams} streams]"
    config = {"workload": name, "streams": wl.streams, "slots": wl.num_slots,
              "head_dim": wl.head_dim, "W": wl.W, "R": wl.R, "G": wl.G,
              "bank_dtype": str(wl.bank_dtype).replace("torch.", ""), "index_dtype":
              str(wl.idx_dtype).replace("torch.", ""), "sequence_steps": T,
              "entry": "sdm_decode_steps" if args.entry == "steps" else "sdm_decode_step",
              "tokens_per_launch": per_launch, "launch": args.launch, "seed": args.seed}
    value = wl.streams * K / (ms * 1e-3)
    single = None
    if args.entry == "steps":
        # the same tokens, one sdm_decode_step launch each (the bank keeps changing)
        del stacked, readings
        outs = [torch.empty((wl.streams, wl.head_dim), dtype=wl.bank_dtype, device=dev) for _ in seq]

        def launch_single(i):
            sdm_decode_step(bank, **seq[i % T], readings=outs[i % T])

        ms1 = _run_steps(torch, args, launch_single, T)
        single = {"entry": "sdm_decode_step", "tokens_per_launch": 1, "steps": T, "ms_per_step": ms1 / T,
                  "value": wl.streams * T / (ms1 * 1e-3), "unit": "stream-steps/s",
                  "achieved": row_bytes_step / (ms1 / T * 1e-3) / 1e9, "frac":
                  row_bytes_step / (ms1 / T * 1e-3) / 1e9 / HBM_PEAK_GBPS}
    return dict(value=value, unit="stream-steps/s", ms_step=ms_step, K=K, config=config, gbps=gbps,
                row_bytes=launch_bytes, cpu=cpu, tokens_per_s=value, single=single, tokens_per_launch=per_launch,
                live_tokens=None)


def bench_gather(torch, args, cfg_name, wl):
    import gen
    from sparse_delta_rule_amd import sdm_gather, sdm_gather_compact
    dev = torch.device("cuda", 0)
    if args.tokens is not None:
        if args.tokens < wl.chunk or args.tokens % wl.chunk:
            raise SystemExit("bench.py: --tokens must be a positive multiple of the chunk")
        wl = wl.replace(tokens=args.tokens)
    if args.head_dim is not None:
        if args.head_dim < 1:
            raise SystemExit("bench.py: --head-dim must be positive")
        wl = wl.replace(head_dim=args.head_dim)
    if args.bank_dtype is not None:
        wl = wl.replace(bank_dtype={"bf16": torch.bfloat16, "f32": torch.float32}[args.bank_dtype])
    es = torch.empty((), dtype=wl.bank_dtype).element_size()
    bank = gen.gather_bank(wl, args.seed, dev)
    inp = gen.gather_inputs(wl, args.seed, dev)
    T = wl.tokens
    # padding: the workload's per-chunk counts, or one scalar count for every chunk
    if args.valid == "per-chunk":
        cv, valid = inp["chunk_valid"], wl.chunk
        live = gen.live_tokens(wl, cv)
    else:
        cv, valid = None, wl.chunk if args.valid == "all" else int(args.valid)
        if not 0 <= valid <= wl.chunk:
            raise SystemExit("bench.py: --valid must be per-chunk, all or a count in [0, chunk]")
        live = T // wl.chunk * valid
    two = args.gather in ("two-ops", "no-stash", "compact")
    with_stash = args.gather in ("two-ops", "one-op")
    compact = args.gather == "compact"
    if args.outputs_apart is not None:
        if not two or args.outputs_apart < 0:
            raise SystemExit("bench.py: --outputs-apart takes a row count >= 0 and a two-operand gather")
        both = torch.empty((2 * T + args.outputs_apart, wl.head_dim), device=dev)
        out0, out1 = both[:T], both[T + args.outputs_apart:]
    else:
        out0 = torch.empty((T, wl.head_dim), device=dev)
        out1 = torch.empty((T, wl.head_dim), device=dev) if two else None
    stash = torch.empty((T, wl.width0, wl.head_dim), dtype=wl.bank_dtype, device=dev) if with_stash else None
    if compact:
        kpos = gen.compact_positions(inp["idx0"], wl.chunk,
                                     cv if cv is not None else torch.full((T // wl.chunk,), valid, device=dev))
        chunk_of = (torch.arange(T, device=dev) // wl.chunk)[:, None].expand_as(kpos)
        stored = kpos >= 0
        # rows the compact stash must hold: distinct (chunk, position) pairs
        compact_rows = int(torch.unique(chunk_of[stored] * (wl.chunk * wl.width0) + kpos[stored].long()).numel())
        stash = torch.empty((T // wl.chunk, wl.chunk * wl.width0, wl.head_dim), dtype=wl.bank_dtype, device=dev)
    torch.cuda.synchronize()
    cpu = None
    if not args.no_cpu_baseline and args.gather == "two-ops" and args.valid == "per-chunk":
        cpu = cpu_baseline_gather(torch, wl, bank, inp, args.cpu_seconds, cfg_name)
    K = args.steps if args.steps is not None else 20
    ops = dict(idx1=inp["idx1"], w1=inp["w1"], out1=out1) if two else {}

    def launch_one(i):
        if compact:
            sdm_gather_compact(bank, inp["idx0"], inp["w0"], kpos, chunk=wl.chunk, valid=valid, chunk_valid=cv,
                               out0=out0, stash=stash, **ops)
        else:
            sdm_gather(bank, inp["idx0"], inp["w0"], chunk=wl.chunk, valid=valid, chunk_valid=cv, out0=out0,
                       stash=stash, with_stash=with_stash, **ops)

    ms = _run_steps(torch, args, launch_one, K)
    ms_step = ms / K
    width_read = wl.width0 + (wl.width1 if two else 0)
    stash_rows = compact_rows if compact else (T * wl.width0 if with_stash else 0)
    row_bytes = (live * width_read + stash_rows) * wl.head_dim * es
    gbps = row_bytes / (ms_step * 1e-3) / 1e9
    name = f"{cfg_name}: {wl.name}" + ("" if args.gather == "two-ops" else f" [{args.gather}]")
    if args.tokens is not None or args.valid != "per-chunk":
        name += f" [{T} tokens, valid {args.valid}]"
    if args.head_dim is not None or args.bank_dtype is not None:
        name += f" [head_dim {wl.head_dim}, {str(wl.bank_dtype).replace('torch.', '')} bank]"
    if args.outputs_apart is not None:
        name += f" [outputs {args.outputs_apart} rows apart]"
    config = {"workload": name, "tokens": T, "live_tokens": live, "valid": args.valid, "chunk": wl.chunk,
              "head_dim": wl.head_dim, "widths": [wl.width0, wl.width1 if two else 0],
              "stash": "compact" if compact else with_stash, "stash_rows": stash_rows,
              "slots": wl.num_slots, "bank_dtype": str(wl.bank_dtype).replace("torch.", ""),
              "launch": args.launch, "seed": args.seed}
    if args.outputs_apart is not None:
        config["outputs_apart_rows"] = args.outputs_apart
    value = T * K / (ms * 1e-3)
    return dict(value=value, unit="tokens/s", ms_step=ms_step, K=K, config=config, gbps=gbps,
                row_bytes=row_bytes, cpu=cpu, tokens_per_s=value, tokens_per_launch=T, live_tokens=live)


def calibrate_copy(torch):
    """A plain elementwise copy of 1 GiB (reads 1 GiB, writes 1 GiB), for counter scaling."""
    dev = torch.device("cuda", 0)
    n = (1 << 30) // 4
    src = torch.ones(n, device=dev)
    dst = torch.empty(n, device=dev)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    ms = _timed(torch, torch.cuda.current_stream(), lambda: torch.mul(src, 1.0, out=dst))
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "ms": ms,
                      "gbps": 2 * n * 4 / (ms * 1e-3) / 1e9}), flush=True)


def dtype_fields(wl) -> dict:
    """The arithmetic type (every sum, product and update is float32, on bfloat16 and
    float32 banks alike) and the bank's storage type."""
    return {"dtype": "f32", "storage_dtype": STORAGE_DTYPE[str(wl.bank_dtype)]}


def streaming_copy_gbps(torch, mib: int = 1024, reps: int = 5) -> float:
    """Bandwidth of a plain streaming device copy (torch's elementwise kernel copying
    ``mib`` MiB, bytes read + written per second, best of ``reps``): what sequential traffic
    reaches on this device, the yardstick the random-row rates are also given against."""
    dev = torch.device("cuda", 0)
    n = mib * (1 << 20) // 4
    src = torch.ones(n, device=dev)
    dst = torch.empty(n, device=dev)
    for _ in range(2):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    best = min(_timed(torch, torch.cuda.current_stream(), lambda: torch.mul(src, 1.0, out=dst)) for _ in range(reps))
    del src, dst
    return 2 * n * 4 / (best * 1e-3) / 1e9


# ------------------------------------------------------------------ ceiling
CEILING_LAUNCHES = 8
CEILING_KERNEL = {"read": "ceiling_rows_kernel<0", "stash": "ceiling_rows_kernel<1", "rmw": "ceiling_rows_kernel<2",
                  "mix": "ceiling_rows_kernel<3", "copy": "ceiling_copy_kernel<8, false",
                  "copy-nt": "ceiling_copy_kernel<8, true"}


CEILING_STREAM_SLOTS, CEILING_STREAM_UNITS = 16384, 64


def ceiling_plan(mode: str, bank_gib: float, row_bytes: int, layout: str = "uniform") -> tuple:
    """(units per launch, rows per unit list entry, bytes moved per launch) of one reference
    pattern: 2M random rows read (read, stash), 1M distinct rows rewritten (rmw), 1M
    units of one rewritten and one read row (mix), or a 1 GiB copy. Rows never repeat
    across the timed launches of rmw and mix. With the streams layout (rmw, mix) the
    bank is split into streams of CEILING_STREAM_SLOTS slots, and every stream has
    CEILING_STREAM_UNITS units per launch with distinct rows from its own slots (for
    mix on a 16 GiB bank of 256-byte rows: the decode's c2 step, 192 MiB)."""
    num_rows = int(bank_gib * (1 << 30)) // row_bytes
    if mode.startswith("copy"):
        return 0, 0, 2 << 30
    per_unit = 2 if mode == "mix" else 1
    if layout == "streams" and mode in ("rmw", "mix"):
        n = num_rows // CEILING_STREAM_SLOTS * CEILING_STREAM_UNITS
    else:
        n = {"read": 2 << 20, "stash": 2 << 20, "rmw": 1 << 20, "mix": 1 << 20}[mode]
        if mode in ("rmw", "mix"):
            n = min(n, num_rows // (per_unit * (CEILING_LAUNCHES + 2)))
    moved = {"read": 1, "stash": 2, "rmw": 2, "mix": 3}[mode] * n * row_bytes
    return n, per_unit, moved


def ceiling_stream_rows(torch, num_rows: int, per_unit: int, gen, dev):
    """One launch's row list in the streams layout: for each stream, CEILING_STREAM_UNITS
    units whose per_unit rows are distinct slots of the stream's own range (written rows
    first in each pair, as in the decode, where a stream's write and read slots are
    drawn from its range)."""
    streams = num_rows // CEILING_STREAM_SLOTS
    k = CEILING_STREAM_UNITS * per_unit
    out = torch.empty((streams, k), dtype=torch.int64, device=dev)
    step = max(1, (1 << 24) // CEILING_STREAM_SLOTS)
    for s0 in range(0, streams, step):
        m = min(step, streams - s0)
        keys = torch.rand((m, CEILING_STREAM_SLOTS), generator=gen, device=dev)
        out[s0:s0 + m] = keys.topk(k, dim=1).indices
    out += torch.arange(streams, device=dev)[:, None] * CEILING_STREAM_SLOTS
    if per_unit == 2:  # pair unit u's written row with its read row
        out = torch.stack([out[:, :CEILING_STREAM_UNITS], out[:, CEILING_STREAM_UNITS:]], dim=2)
    return out.reshape(-1).contiguous()


def bench_ceiling(torch, args) -> int:
    """Time each reference pattern on banks of the given sizes: after about 50 ms of the
    same launches untimed, CEILING_LAUNCHES launches between HIP events, each on its own
    random rows (uniform with repetition for read and
    stash; for rmw and mix, distinct rows never reused across launches, or the streams
    layout)."""
    from sparse_delta_rule_amd import ceiling
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    copy_gbps = None
    for gib in [float(x) for x in args.bank_gib.split(",")]:
        num_rows = int(gib * (1 << 30)) // args.row_bytes
        bank = torch.empty((num_rows, args.row_bytes // 4), dtype=torch.int32, device=dev)
        bank.random_()
        sink = torch.empty(ceiling.sink_words(), dtype=torch.int32, device=dev)
        gen = torch.Generator(device=dev)
        gen.manual_seed(args.seed)
        for mode in args.ceiling.split(","):
            layout = args.ceiling_layout if mode in ("rmw", "mix") else "uniform"
            n, per_unit, moved = ceiling_plan(mode, gib, args.row_bytes, layout)
            L = CEILING_LAUNCHES
            if mode.startswith("copy"):
                half = bank.view(-1)[: (1 << 30) // 4 * 2]
                src, dst = half[: (1 << 30) // 4], half[(1 << 30) // 4:]
                nt = mode == "copy-nt"
                launches = [lambda: ceiling.copy(dst, src, nontemporal=nt)] * (L + 1)
            else:
                if mode in ("read", "stash"):
                    lists = torch.randint(0, num_rows, ((L + 1), n), generator=gen, device=dev)
                elif layout == "streams":
                    lists = torch.stack([ceiling_stream_rows(torch, num_rows, per_unit, gen, dev)
                                         for _ in range(L + 1)])
                else:
                    perm = torch.randperm(num_rows, generator=gen, device=dev)
                    lists = perm[: (L + 1) * n * per_unit].view(L + 1, n * per_unit)
                    del perm
                stash = torch.empty((n, args.row_bytes // 4), dtype=torch.int32, device=dev) \
                    if mode == "stash" else None
                launches = [(lambda i=i: ceiling.rows(mode, bank, lists[i], stash=stash, sink=sink))
                            for i in range(L + 1)]
            # untimed: the pattern's first launch, then ~50 ms more of it (the device's clocks
            # settle after tens of milliseconds of load)
            launches[0]()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < 0.05:
                for f in launches[1:]:
                    f()
                torch.cuda.synchronize()
            ms = _timed(torch, stream, lambda: [f() for f in launches[1:]]) / L
            gbps = moved / (ms * 1e-3) / 1e9
            if mode.startswith("copy"):
                copy_gbps = max(copy_gbps or 0.0, gbps)
            line = {"metric": f"reference access pattern on one MI355X: {mode}", "mode": mode, "bank_gib": gib,
                    "row_bytes": args.row_bytes, "layout": layout, "units_per_launch": n, "bytes_per_launch": moved,
                    "launches": L, "us_per_launch": ms * 1e3, "achieved": gbps, "unit": "GB/s",
                    "peak": HBM_PEAK_GBPS, "frac": gbps / HBM_PEAK_GBPS,
                    "kernel": CEILING_KERNEL[mode].split("<")[0]}
            if copy_gbps and not mode.startswith("copy"):
                line["copy_frac"] = gbps / copy_gbps
            print(json.dumps(line), flush=True)
            del launches
            torch.cuda.empty_cache()
        del bank, sink
        torch.cuda.empty_cache()
    return 0


def host_call_cost(torch, calls: int = 2000) -> int:
    """Host time per call, in microseconds, of a 64-token two-operand gather (no stash)
    over c3's bank: sdm_gather from Python, the same C call through ctypes with its
    arguments prepared once, a plan launch from Python and through ctypes. The device
    work is the same for all four; this measures what a call costs the host."""
    import ctypes
    import gen
    from sparse_delta_rule_amd import sdm_gather, sdm_gather_plan, library
    from sparse_delta_rule_amd._binding import _stream_handle
    dev = torch.device("cuda", 0)
    wl = gen.WORKLOADS["c3"].replace(num_slots=1 << 20, tokens=64)
    bank = gen.gather_bank(wl, 0, dev)
    inp = gen.gather_inputs(wl, 0, dev)
    out0 = torch.empty((64, wl.head_dim), device=dev)
    out1 = torch.empty_like(out0)
    lib = library()
    stream = _stream_handle(dev)
    P = ctypes.c_void_p
    args = (P(bank.data_ptr()), 1, bank.shape[0], wl.head_dim, 64, 64, 64, None, 2, 1,
            P(inp["idx0"].data_ptr()), P(inp["w0"].data_ptr()), 64, P(out0.data_ptr()), None,
            P(inp["idx1"].data_ptr()), P(inp["w1"].data_ptr()), 64, P(out1.data_ptr()), stream)
    plan = sdm_gather_plan(bank, inp["idx0"], inp["w0"], tokens=64, chunk=64, idx1=inp["idx1"], w1=inp["w1"],
                           out0=out0, out1=out1)
    pl = ctypes.byref(plan._plan)
    ways = {
        "sdm_gather (Python)": lambda: sdm_gather(bank, inp["idx0"], inp["w0"], chunk=64, valid=64, idx1=inp["idx1"],
                                                  w1=inp["w1"], out0=out0, out1=out1, with_stash=False),
        "sdm_gather (ctypes)": lambda: lib.sdm_gather(*args),
        "plan launch (Python)": lambda: plan.launch(0, 64),
        "plan launch (ctypes)": lambda: lib.sdm_gather_plan_launch(pl, 0, 64, stream),
    }
    if lib.sdm_gather(*args) != 0 or lib.sdm_gather_plan_launch(pl, 0, 64, stream) != 0:
        raise SystemExit(f"bench.py: a gather call failed: {lib.sdm_last_error().decode()}")
    out = {}
    for name, call in ways.items():
        for _ in range(50):
            call()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(calls):
            call()
        host = (time.perf_counter() - t0) / calls * 1e6
        torch.cuda.synchronize()
        out[name] = host
    print(json.dumps({"metric": "host time per call, us (64-token two-operand gather, no stash)",
                      "calls": calls, **{k: round(v, 2) for k, v in out.items()}}), flush=True)
    return 0


# ------------------------------------------------------------------ profiles
def _csv_rows(directory: str, suffix: str):
    import csv
    paths = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not paths:
        raise SystemExit(f"bench.py: no *{suffix} under {directory}")
    with open(paths[0]) as f:
        return list(csv.DictReader(f))


def _counter_kib(directory: str, name_part: str, min_kib: float = 0.0):
    """Median per-dispatch counter value (KiB) of the kernels whose name contains name_part."""
    import statistics
    vals = [float(r["Counter_Value"]) for r in _csv_rows(directory, "counter_collection.csv")
            if name_part in r["Kernel_Name"] and float(r["Counter_Value"]) >= min_kib]
    if not vals:
        raise SystemExit(f"bench.py: no {name_part} dispatches in {directory}")
    return statistics.median(vals), len(vals)


def _counters(directory: str, name_part: str) -> dict:
    """Median per-dispatch value of every counter of a rocprofv3 --pmc run, over the
    dispatches of the kernels whose name contains name_part."""
    import statistics
    vals = {}
    for r in _csv_rows(directory, "counter_collection.csv"):
        if name_part in r["Kernel_Name"]:
            vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return {k: statistics.median(v) for k, v in vals.items()}


SQ_SHARES = ("SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_VMEM", "SQ_ACTIVE_INST_LDS",
             "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY")


def derived_counters(c: dict) -> dict:
    """L2 hit rate, latencies and shares of wave time from raw counter medians (those
    present)."""
    out = {}
    if "TCC_HIT_sum" in c and "TCC_MISS_sum" in c and c["TCC_HIT_sum"] + c["TCC_MISS_sum"] > 0:
        out["l2_hit_rate"] = c["TCC_HIT_sum"] / (c["TCC_HIT_sum"] + c["TCC_MISS_sum"])
    if "VmemLatency" in c:
        out["vmem_latency_cycles"] = c["VmemLatency"]
    if c.get("TCC_EA0_RDREQ_sum", 0) > 0 and "TCC_EA0_RDREQ_LEVEL_sum" in c:
        out["ea_read_latency_cycles"] = c["TCC_EA0_RDREQ_LEVEL_sum"] / c["TCC_EA0_RDREQ_sum"]
    if c.get("SQ_WAVE_CYCLES", 0) > 0:
        out["wave_time_shares"] = {k: c[k] / c["SQ_WAVE_CYCLES"] for k in SQ_SHARES if k in c}
    if "MeanOccupancyPerCU" in c:
        out["mean_occupancy_per_cu"] = c["MeanOccupancyPerCU"]
    return out


def algorithmic_bytes(cfg_name: str, entry: str, seed: int = 0, gather: str = "two-ops") -> tuple:
    """(bytes per launch, unit description, launch shape) of the row traffic the method
    needs, for the launch the benchmark runs with these arguments (gather: the launch
    shape, one of GATHER_SHAPES). The shape holds the launch's tokens per stream
    (decode) or its live-token count (gather); the live count comes from the same
    draw the benchmark launches (gen draws the per-chunk counts on the CPU for every
    device)."""
    import gen
    import torch
    wl = gen.WORKLOADS[cfg_name]
    es = torch.empty((), dtype=wl.bank_dtype).element_size()
    if isinstance(wl, gen.DecodeWorkload):
        per = wl.streams * (2 * wl.W + wl.R) * wl.head_dim * es
        tokens = wl.steps if entry == "steps" else 1
        return (per * tokens,
                f"{tokens} token(s) x {wl.streams} streams x (2W+R)={2 * wl.W + wl.R} rows x {wl.head_dim * es} B",
                {"tokens_per_launch": tokens})
    two, with_stash = GATHER_SHAPES[gather]
    live = gen.live_tokens(wl, gen.gather_inputs(wl.replace(width0=1, width1=0), seed)["chunk_valid"])
    read = wl.width0 + (wl.width1 if two else 0)
    stash_rows = wl.tokens * wl.width0 if with_stash else 0
    rows = (live * read + stash_rows) * wl.head_dim * es
    return (rows, f"{live} live tokens x {read} rows read + {stash_rows} stash rows, x {wl.head_dim * es} B",
            {"tokens_per_launch": wl.tokens, "live_tokens": live})


def ingest_profile(args) -> int:
    trace, fetch, write, copy_fetch, copy_write = args.ingest_profile
    if args.config == "c3" and (args.gather not in GATHER_SHAPES or args.valid != "per-chunk" or args.tokens
                                or args.head_dim is not None or args.bank_dtype is not None
                                or args.outputs_apart is not None):
        raise SystemExit("bench.py: gather profiles are summarised for c3's own tokens and per-chunk counts, "
                         f"in the launch shapes {sorted(GATHER_SHAPES)}")
    kind = launch_kind(args.config, args.entry, args.gather)
    pattern = kernel_pattern(kind)
    stats = [r for r in _csv_rows(trace, "kernel_stats.csv") if pattern in r["Name"]]
    if not stats:
        raise SystemExit(f"bench.py: no {pattern} kernel in the trace under {trace}")
    names = {re.search(r"(sdm_\w+_kernel)", r["Name"]).group(1) for r in stats}
    if len(names) != 1:
        raise SystemExit(f"bench.py: several kernels ({sorted(names)}) in one launch kind's trace")
    kernel = names.pop()
    calls = sum(int(r["Calls"]) for r in stats)
    avg_ns = sum(float(r["AverageNs"]) * int(r["Calls"]) for r in stats) / calls
    f_kib, f_n = _counter_kib(fetch, kernel)
    w_kib, w_n = _counter_kib(write, kernel)
    gib_kib = float(1 << 20)  # the calibration copy moves 1 GiB each way
    cf_kib, _ = _counter_kib(copy_fetch, "elementwise", min_kib=gib_kib / 8)
    cw_kib, _ = _counter_kib(copy_write, "elementwise", min_kib=gib_kib / 8)
    f_scale, w_scale = gib_kib / cf_kib, gib_kib / cw_kib
    fetch_b, write_b = f_kib * 1024 * f_scale, w_kib * 1024 * w_scale
    alg, alg_desc, shape = algorithmic_bytes(args.config, args.entry, args.seed, args.gather)
    raw = {}
    for d in args.extra_counters:
        raw.update(_counters(d, kernel))
    derived = derived_counters(raw)
    traffic_path = os.path.join(PROFILES, "traffic.json")
    data = {}
    if os.path.exists(traffic_path):
        with open(traffic_path) as f:
            data = json.load(f)
    data[f"{args.config}/{kind}"] = {
        "kernel_source_hash": kernel_source_hash(kind), "bytes_per_launch": fetch_b + write_b,
        "fetch_bytes": fetch_b, "write_bytes": write_b, "fetch_scale": f_scale, "write_scale": w_scale,
        "algorithmic_bytes_per_launch": alg, "avg_kernel_ns": avg_ns, "calls": calls, "kernel": kernel,
        "counters": raw, **shape, **derived}
    os.makedirs(PROFILES, exist_ok=True)
    with open(traffic_path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    shape_tag = "" if kind in ("gather", "steps", "step") else "_" + kind[len("gather-"):]
    md = os.path.join(PROFILES, f"{kernel}_{args.config}{shape_tag}.md")
    with open(md, "w") as f:
        f.write(f"# {kernel} on workload {args.config}{' [' + shape_tag[1:] + ']' if shape_tag else ''} "
                "(MI355X, rocprofv3)\n\n")
        f.write(f"Kernel sources hash {kernel_source_hash(kind)} (bench.py `kernel_source_hash` of launch kind "
                f"`{kind}`).\n\n")
        f.write("## Commands\n\n```\n" + args.profile_commands.strip() + "\n```\n\n")
        f.write("## Kernel trace (`--kernel-trace --stats`)\n\n| kernel | calls | average | min | max |\n|---|---|---|---|---|\n")
        for r in stats:
            f.write(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} us | "
                    f"{float(r['MinNs']) / 1e3:.2f} us | {float(r['MaxNs']) / 1e3:.2f} us |\n")
        f.write(f"\nAlgorithmic row bytes per launch: {alg / 2**20:.1f} MiB ({alg_desc}); at the average "
                f"duration that is {alg / avg_ns:.0f} GB/s, {alg / avg_ns / HBM_PEAK_GBPS:.3f} of the 8 TB/s peak.\n\n")
        f.write("## HBM bytes (`--pmc FETCH_SIZE`, `--pmc WRITE_SIZE`, one pass each)\n\n")
        f.write(f"| counter | KiB per dispatch (median of {f_n}/{w_n}) | scale (1 GiB copy) | bytes per launch |\n|---|---|---|---|\n")
        f.write(f"| FETCH_SIZE | {f_kib:.0f} | {f_scale:.4f} (copy read {cf_kib:.0f} KiB for 1048576) | {fetch_b / 2**20:.1f} MiB |\n")
        f.write(f"| WRITE_SIZE | {w_kib:.0f} | {w_scale:.4f} (copy wrote {cw_kib:.0f} KiB for 1048576) | {write_b / 2**20:.1f} MiB |\n")
        f.write(f"\nMeasured HBM traffic {(fetch_b + write_b) / 2**20:.1f} MiB per launch against "
                f"{alg / 2**20:.1f} MiB of algorithmic row bytes (ratio {(fetch_b + write_b) / alg:.3f}; "
                "the excess is slots, weights, values and outputs).\n")
        if raw:
            f.write("\n## Cache and latency counters (one `--pmc` pass per group)\n\n| counter | median per dispatch |\n|---|---|\n")
            for k in sorted(raw):
                f.write(f"| {k} | {raw[k]:.6g} |\n")
            f.write("\n")
            if "l2_hit_rate" in derived:
                f.write(f"L2 hit rate TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum) = {derived['l2_hit_rate']:.3f}. ")
            if "vmem_latency_cycles" in derived:
                f.write(f"Average VMEM instruction latency (VmemLatency: accumulated SQ_INST_LEVEL_VMEM / "
                        f"SQ_INSTS_VMEM) = {derived['vmem_latency_cycles']:.0f} cycles. ")
            if "ea_read_latency_cycles" in derived:
                f.write(f"Average L2-to-memory read latency TCC_EA0_RDREQ_LEVEL_sum / TCC_EA0_RDREQ_sum = "
                        f"{derived['ea_read_latency_cycles']:.0f} cycles. ")
            if "mean_occupancy_per_cu" in derived:
                f.write(f"Mean occupancy {derived['mean_occupancy_per_cu']:.1f} waves per CU (MeanOccupancyPerCU). ")
            f.write("\n")
            if "wave_time_shares" in derived:
                f.write("\nShares of wave time (counter / SQ_WAVE_CYCLES):\n\n| counter | share |\n|---|---|\n")
                for k, v in derived["wave_time_shares"].items():
                    f.write(f"| {k} | {v:.3f} |\n")
    print(json.dumps({"wrote": [traffic_path, md], "avg_kernel_us": avg_ns / 1e3,
                      "traffic_MiB": (fetch_b + write_b) / 2**20, "alg_MiB": alg / 2**20}))
    return 0


def _trace_dispatches(directory: str, name_part: str):
    """(workgroups, duration ns) of every dispatch in a rocprofv3 kernel trace whose
    kernel name contains name_part."""
    out = []
    for r in _csv_rows(directory, "kernel_trace.csv"):
        if name_part in r["Kernel_Name"]:
            wgs = (int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))) * int(r["Grid_Size_Y"])
            out.append((wgs, int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    return out


def fit_line(xs, ys):
    """Least-squares (intercept, slope) of ys against xs."""
    n = len(xs)
    mx, my = sum(xs) / n, sum(ys) / n
    sxx = sum((x - mx) ** 2 for x in xs)
    slope = sum((x - mx) * (y - my) for x, y in zip(xs, ys)) / sxx
    return my - slope * mx, slope


def ingest_stream_sweep(args) -> int:
    """Kernel durations of a --streams sweep, per stream count, and their fit as a fixed
    cost per launch plus a cost per stream (whose bytes give the marginal bandwidth)."""
    import statistics
    import gen
    import torch
    wl = gen.WORKLOADS[args.config]
    if not isinstance(wl, gen.DecodeWorkload):
        raise SystemExit("bench.py: a stream sweep is a decode measurement")
    kind = launch_kind(args.config, args.entry)
    pattern = kernel_pattern(kind)
    disp = _trace_dispatches(args.ingest_stream_sweep, pattern)
    if not disp:
        raise SystemExit(f"bench.py: no {pattern} dispatch in {args.ingest_stream_sweep}")
    tokens = wl.steps if kind == "steps" else 1
    es = torch.empty((), dtype=wl.bank_dtype).element_size()
    per_stream = (2 * wl.W + wl.R) * wl.head_dim * es * tokens
    by_wgs = {}
    for wgs, ns in disp:
        by_wgs.setdefault(wgs, []).append(ns)
    # launch sizes in workgroups, matched in order to the sweep's stream counts
    counts = sorted(int(x) for x in args.streams.split(",")) if args.streams else None
    groups = sorted(by_wgs)
    if counts is None or len(counts) != len(groups):
        raise SystemExit(f"bench.py: pass the sweep's --streams list ({len(groups)} launch sizes in the trace)")
    rows = [(n, wg, statistics.median(by_wgs[wg]), len(by_wgs[wg])) for n, wg in zip(counts, groups)]
    icpt, slope = fit_line([r[0] for r in rows], [r[2] for r in rows])
    marginal = per_stream / slope  # bytes per ns = GB/s
    md = os.path.join(PROFILES, f"{re.sub(r'[^a-z_]', '', pattern)}_{args.config}_stream_sweep.md")
    os.makedirs(PROFILES, exist_ok=True)
    with open(md, "w") as f:
        f.write(f"# {pattern} on workload {args.config} over stream counts (MI355X, rocprofv3 kernel trace)\n\n")
        f.write(f"Kernel sources hash {kernel_source_hash(kind)} (bench.py `kernel_source_hash` of launch kind "
                f"`{kind}`). Each stream keeps "
                f"its {wl.slots_per_stream} slots, so the bank grows with the stream count; {tokens} token(s) per "
                f"launch, {per_stream} algorithmic row bytes per stream per launch.\n\n")
        f.write("## Command\n\n```\n" + args.profile_commands.strip() + "\n```\n\n")
        f.write("## Median kernel duration per launch size\n\n| streams | workgroups | launches | median duration "
                "| row bytes | rate | fraction of 8 TB/s |\n|---|---|---|---|---|---|---|\n")
        for n, wg, med, k in rows:
            b = n * per_stream
            f.write(f"| {n} | {wg} | {k} | {med / 1e3:.2f} us | {b / 2**20:.1f} MiB | {b / med:.0f} GB/s | "
                    f"{b / med / HBM_PEAK_GBPS:.3f} |\n")
        f.write(f"\nLeast-squares fit: duration = {icpt / 1e3:.2f} us + streams x {slope:.2f} ns. The fixed part is "
                f"the cost of a launch whatever its size; the part per stream moves {per_stream} row bytes, a "
                f"marginal rate of {marginal:.0f} GB/s ({marginal / HBM_PEAK_GBPS:.3f} of the 8 TB/s peak).\n")
    print(json.dumps({"wrote": md, "fixed_us": icpt / 1e3, "ns_per_stream": slope, "marginal_gbps": marginal,
                      "rows": rows}))
    return 0


def ingest_ceiling(args) -> int:
    """Kernel durations and HBM bytes of one --ceiling run (one bank size): per pattern,
    the rate its algorithmic bytes reach in the kernel trace and the counters' bytes."""
    trace, fetch, write, copy_fetch, copy_write = args.ingest_ceiling
    gib = float(args.bank_gib)
    stats = [r for r in _csv_rows(trace, "kernel_stats.csv") if "ceiling_" in r["Name"]]
    gib_kib = float(1 << 20)
    cf_kib, _ = _counter_kib(copy_fetch, "elementwise", min_kib=gib_kib / 8)
    cw_kib, _ = _counter_kib(copy_write, "elementwise", min_kib=gib_kib / 8)
    f_scale, w_scale = gib_kib / cf_kib, gib_kib / cw_kib
    out = {}
    for mode, frag in CEILING_KERNEL.items():
        rows = [r for r in stats if frag in r["Name"]]
        if not rows:
            continue
        calls = sum(int(r["Calls"]) for r in rows)
        avg_ns = sum(float(r["AverageNs"]) * int(r["Calls"]) for r in rows) / calls
        n, _, moved = ceiling_plan(mode, gib, args.row_bytes,
                                   args.ceiling_layout if mode in ("rmw", "mix") else "uniform")
        f_kib, _ = _counter_kib(fetch, frag)
        w_kib, _ = _counter_kib(write, frag)
        out[mode] = {"avg_kernel_ns": avg_ns, "calls": calls, "bytes_per_launch": moved, "units_per_launch": n,
                     "frac": moved / avg_ns / HBM_PEAK_GBPS, "fetch_bytes": f_kib * 1024 * f_scale,
                     "write_bytes": w_kib * 1024 * w_scale}
    if not out:
        raise SystemExit(f"bench.py: no ceiling kernel in {trace}")
    path = os.path.join(PROFILES, "ceiling.json")
    data = {}
    if os.path.exists(path):
        with open(path) as f:
            data = json.load(f)
    data[f"{gib:g}GiB/{args.row_bytes}B/{args.ceiling_layout}"] = out
    os.makedirs(PROFILES, exist_ok=True)
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    md = os.path.join(PROFILES, f"sdm_ceiling_bank_{gib:g}gib_rows_{args.row_bytes}b_{args.ceiling_layout}.md")
    with open(md, "w") as f:
        f.write(f"# Reference access patterns over a {gib:g} GiB bank of {args.row_bytes}-byte rows "
                "(MI355X, rocprofv3)\n\n")
        f.write("Kernels of `sparse_delta_rule_amd/ceiling/sdm_ceiling.hip` (libsdm_ceiling): rows at uniformly "
                "random slots, 16-byte vectors on consecutive lanes, a batch of rows in flight per lane group. "
                "read: rows read (2M per launch, with repetition); stash: rows read and written to a sequential "
                "stash; rmw: distinct rows read and written back in place; mix: per unit one row read and "
                "written back and one other row read (the decode's mix of two row reads per row write); copy: a "
                "sequential 1 GiB copy (copy-nt: non-temporal loads and stores). Layout of the rmw and mix rows: "
                f"{args.ceiling_layout} (uniform: over the whole bank, never reused across launches; streams: "
                f"runs of {CEILING_STREAM_UNITS} units draw distinct rows from their own {CEILING_STREAM_SLOTS} "
                "slots, as the decode's streams do).\n\n")
        f.write("## Commands\n\n```\n" + args.profile_commands.strip() + "\n```\n\n")
        f.write("| pattern | launches | average duration | bytes moved per launch | rate | fraction of 8 TB/s | "
                "FETCH_SIZE bytes | WRITE_SIZE bytes | counted / moved |\n|---|---|---|---|---|---|---|---|---|\n")
        for mode, e in out.items():
            cnt = e["fetch_bytes"] + e["write_bytes"]
            f.write(f"| {mode} | {e['calls']} | {e['avg_kernel_ns'] / 1e3:.1f} us | {e['bytes_per_launch'] / 2**20:.0f} "
                    f"MiB | {e['bytes_per_launch'] / e['avg_kernel_ns']:.0f} GB/s | {e['frac']:.3f} | "
                    f"{e['fetch_bytes'] / 2**20:.0f} MiB | {e['write_bytes'] / 2**20:.0f} MiB | "
                    f"{cnt / e['bytes_per_launch']:.3f} |\n")
        f.write(f"\nCounter scales from a plain 1 GiB copy measured the same way: FETCH_SIZE x {f_scale:.4f}, "
                f"WRITE_SIZE x {w_scale:.4f}.\n")
    print(json.dumps({"wrote": [path, md], **{m: round(e["frac"], 4) for m, e in out.items()}}))
    return 0


def main(argv=None):
    args = parse_args(argv)
    if (args.head_dim is not None or args.bank_dtype is not None) and args.config != "c3":
        raise SystemExit("bench.py: --head-dim and --bank-dtype change the gather's bank (--config c3)")
    if args.outputs_apart is not None and args.config != "c3":
        raise SystemExit("bench.py: --outputs-apart places the gather's outputs (--config c3)")
    if args.ingest_profile:
        sys.path.insert(0, ROOT)
        return ingest_profile(args)
    if args.ingest_stream_sweep:
        sys.path.insert(0, ROOT)
        return ingest_stream_sweep(args)
    if args.ingest_ceiling:
        sys.path.insert(0, ROOT)
        return ingest_ceiling(args)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: the benchmark measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}); a step is one GPU's share of streams or tokens, which needs no exchange.",
              file=sys.stderr, flush=True)
        return 2
    sys.path.insert(0, ROOT)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    if args.calibrate_copy:
        calibrate_copy(torch)
        return 0
    if args.ceiling:
        return bench_ceiling(torch, args)
    if args.host_call_cost:
        return host_call_cost(torch)
    import gen
    wl = gen.WORKLOADS[args.config]
    if args.streams is not None:
        if not isinstance(wl, gen.DecodeWorkload):
            raise SystemExit("bench.py: --streams applies to the decode workloads")
        counts = [int(x) for x in args.streams.split(",")]
        if len(counts) > 1:
            for n in counts:
                sub = argparse.Namespace(**{**vars(args), "streams": str(n)})
                rc = main_one(torch, gen, sub, wl.replace(streams=n))
                torch.cuda.empty_cache()
                if rc:
                    return rc
            return 0
        wl = wl.replace(streams=counts[0])
    return main_one(torch, gen, args, wl)


def main_one(torch, gen, args, wl) -> int:
    """One benchmark line for one workload."""
    if isinstance(wl, gen.DecodeWorkload):
        r = bench_decode(torch, args, args.config, wl)
    else:
        r = bench_gather(torch, args, args.config, wl)
    kind = launch_kind(args.config, args.entry, args.gather)
    traffic, kernel = stored_traffic(args.config, kind, r["tokens_per_launch"], r["live_tokens"])
    if (getattr(args, "head_dim", None) is not None or getattr(args, "bank_dtype", None) is not None
            or getattr(args, "outputs_apart", None) is not None):
        traffic, kernel = None, None  # the stored figures are for the workload's own launch
    copy_gbps = streaming_copy_gbps(torch)
    out = {
        "metric": METRIC,
        "value": r["value"],
        "unit": r["unit"],
        "n_gpus": 1,
        "steps": r["K"],
        "warmup": args.warmup,
        "ms_per_step": r["ms_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        **dtype_fields(wl),
        "data": "synthetic (seeded; gen/workloads.py)",
        "config": r["config"],
        "roofline": {"bound": "hbm", "achieved": r["gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": r["gbps"] / HBM_PEAK_GBPS, "traffic": traffic,
                     "kernel": kernel or kernel_pattern(kind), "algorithmic_bytes_per_launch": r["row_bytes"],
                     "tokens_per_launch": r["tokens_per_launch"], "copy_gbps": copy_gbps,
                     "copy_frac": r["gbps"] / copy_gbps},
        "cpu_baseline": r["cpu"],
        "tokens_per_s": r["tokens_per_s"],
        "row_gbps": r["gbps"],
    }
    if r.get("single"):
        single = dict(r["single"])
        traffic1, kernel1 = stored_traffic(args.config, "step", 1)
        single.update({"kernel": kernel1 or kernel_pattern("step"), "traffic": traffic1,
                       "copy_frac": single["achieved"] / copy_gbps})
        out["single_token"] = single
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
