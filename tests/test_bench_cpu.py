"""Host logic of bench.py that needs no GPU: the one-GPU guard, and turning
rocprofv3 output (kernel trace and byte counters) into the stored HBM-traffic
figures the benchmark line reports."""

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

WIDE = "void sdm::(anonymous namespace)::sdm_decode_steps_wide_kernel<unsigned short, 16, 4, 1, 1>(sdm::DecodeParams)"
COMPACT = "void sdm::(anonymous namespace)::sdm_decode_steps_kernel<unsigned short, 16, 4, 1, 1>(sdm::DecodeParams)"
COPY = "void at::native::elementwise_kernel<128, 4>(int, float)"


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def _trace(d, kernels):
    _write_csv(os.path.join(d, "run_kernel_stats.csv"), ["Name", "Calls", "AverageNs", "MinNs", "MaxNs"],
               [[k, calls, avg, avg - 1, avg + 1] for k, calls, avg in kernels])


def _counter(d, rows):
    _write_csv(os.path.join(d, "run_counter_collection.csv"), ["Kernel_Name", "Counter_Value"], rows)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_launch_kinds():
    assert bench.launch_kind("c3", "steps") == "gather"
    assert bench.launch_kind("c1", "steps") == "steps"
    assert bench.launch_kind("c2", "step") == "step"
    # the gather's other launch shapes never pick up the workload's stored traffic
    assert bench.launch_kind("c3", "steps", "one-op") == "gather-one-op"
    assert bench.launch_kind("c3", "steps", "compact") == "gather-compact"
    assert bench.kernel_pattern("gather-no-stash") == "sdm_gather_kernel"
    assert bench.kernel_pattern("gather-compact") == "sdm_gather_kernel"


def test_ingest_scales_counters_and_keys_by_launch_kind(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    t, f, w, cf, cw = (str(tmp_path / n) for n in ("trace", "fetch", "write", "cfetch", "cwrite"))
    _trace(t, [(WIDE, 10, 300000.0), (COPY, 3, 5000.0)])
    # FETCH_SIZE counts half the bytes on this part (a 1 GiB copy reads 524288 KiB): scale 2
    _counter(f, [(WIDE, 500000.0), (WIDE, 500000.0), (COPY, 10.0)])
    _counter(w, [(WIDE, 400000.0), (WIDE, 400000.0)])
    _counter(cf, [(COPY, 524288.0), (COPY, 1.0)])
    _counter(cw, [(COPY, 1048576.0)])
    assert bench.main(["--config", "c1", "--ingest-profile", t, f, w, cf, cw, "--profile-commands", "cmds"]) == 0
    with open(tmp_path / "profiles" / "traffic.json") as fh:
        data = json.load(fh)
    e = data["c1/steps"]
    assert e["kernel"] == "sdm_decode_steps_wide_kernel"
    assert e["fetch_scale"] == pytest.approx(2.0) and e["write_scale"] == pytest.approx(1.0)
    assert e["bytes_per_launch"] == pytest.approx((500000.0 * 2 + 400000.0) * 1024)
    assert e["avg_kernel_ns"] == pytest.approx(300000.0)
    alg, _ = bench.algorithmic_bytes("c1", "steps")
    assert e["algorithmic_bytes_per_launch"] == alg == 64 * 1024 * 96 * 256
    assert (tmp_path / "profiles" / "sdm_decode_steps_wide_kernel_c1.md").exists()
    # the stored figures apply while the kernel sources are unchanged
    assert bench.stored_traffic("c1", "steps") == (e["bytes_per_launch"], "sdm_decode_steps_wide_kernel")
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.stored_traffic("c1", "steps") == (None, None)


def test_ingest_rejects_a_trace_with_both_decode_loops(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    t = str(tmp_path / "trace")
    _trace(t, [(WIDE, 5, 300000.0), (COMPACT, 5, 310000.0)])
    with pytest.raises(SystemExit, match="several kernels"):
        bench.main(["--config", "c1", "--ingest-profile", t, t, t, t, t])


def test_cache_and_latency_counters_are_summarised(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    t, f, w, cf, cw, hit, lat = (str(tmp_path / n) for n in ("t", "f", "w", "cf", "cw", "hit", "lat"))
    _trace(t, [(WIDE, 4, 300000.0)])
    _counter(f, [(WIDE, 100.0)])
    _counter(w, [(WIDE, 100.0)])
    _counter(cf, [(COPY, 524288.0)])
    _counter(cw, [(COPY, 1048576.0)])
    named = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    _write_csv(os.path.join(hit, "run_counter_collection.csv"), named,
               [(WIDE, "TCC_HIT_sum", 30.0), (WIDE, "TCC_MISS_sum", 70.0), (WIDE, "TCC_HIT_sum", 30.0),
                (WIDE, "TCC_MISS_sum", 70.0), (COPY, "TCC_HIT_sum", 1e9)])
    _write_csv(os.path.join(lat, "run_counter_collection.csv"), named,
               [(WIDE, "VmemLatency", 2500.0), (WIDE, "TCC_EA0_RDREQ_LEVEL_sum", 9000.0),
                (WIDE, "TCC_EA0_RDREQ_sum", 10.0)])
    assert bench.main(["--config", "c1", "--ingest-profile", t, f, w, cf, cw, "--extra-counters", hit, lat]) == 0
    with open(tmp_path / "profiles" / "traffic.json") as fh:
        e = json.load(fh)["c1/steps"]
    assert e["l2_hit_rate"] == pytest.approx(0.3)
    assert e["vmem_latency_cycles"] == pytest.approx(2500.0)
    assert e["ea_read_latency_cycles"] == pytest.approx(900.0)
    md = (tmp_path / "profiles" / "sdm_decode_steps_wide_kernel_c1.md").read_text()
    assert "L2 hit rate" in md and "0.300" in md


def test_kernel_hash_follows_code_not_comments(tmp_path, monkeypatch):
    src = tmp_path / "sparse_delta_rule_amd" / "csrc"
    src.mkdir(parents=True)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (src / "k.hip").write_text("// a kernel\nint f(int x) { return x + 1; }  /* one */\n")
    h0 = bench.kernel_source_hash()
    (src / "k.hip").write_text("// the kernel, reworded\n\nint f(int x) {\n  return x + 1;  // one\n}\n")
    assert bench.kernel_source_hash() == h0
    (src / "k.hip").write_text("int f(int x) { return x + 2; }\n")
    assert bench.kernel_source_hash() != h0


# ------------------------------------------------------------ CPU baseline legs
def test_host_threads_is_bounded(monkeypatch):
    monkeypatch.setenv("OMP_NUM_THREADS", "3")
    assert bench.host_threads() == min(3, len(os.sched_getaffinity(0)))
    monkeypatch.delenv("OMP_NUM_THREADS")
    assert 1 <= bench.host_threads() <= 16


def test_decode_groups_give_the_whole_runs_bits():
    """The all-cores oracle run steps contiguous stream groups on their own bank rows
    (slots renumbered): its readings and rows equal one run over all the streams."""
    import numpy as np
    import torch
    import gen
    wl = gen.WORKLOADS["c1"].replace(streams=11, slots_per_stream=64, steps=3)
    bank = gen.decode_bank(wl, 0)
    seq = [gen.decode_step_inputs(wl, 0, t) for t in range(wl.steps)]
    whole = bench.decode_groups(torch, wl, bank, seq, 11, 1)
    split = bench.decode_groups(torch, wl, bank, seq, 11, 4)
    assert len(split) == 4
    r_whole = bench.run_decode_groups(whole)[0]
    r_split = bench.run_decode_groups(split)
    for t in range(wl.steps):
        got = np.concatenate([r[t] for r in r_split])
        assert np.array_equal(got.view(np.uint16), r_whole[t].view(np.uint16)), f"step {t}"
    banks = np.concatenate([g[0] for g in split])
    assert np.array_equal(banks.view(np.uint16), whole[0][0].view(np.uint16))


def test_gather_ranges_give_the_whole_runs_bits():
    import numpy as np
    import torch
    import gen
    wl = gen.WORKLOADS["c3"].replace(num_slots=3000, tokens=7 * 16, chunk=16, width0=9, width1=5, valid_low=2,
                                     valid_high=16)
    bank = gen.gather_bank(wl, 2)
    inp = gen.gather_inputs(wl, 2)
    sub, whole = bench.gather_ranges(torch, wl, bank, inp, wl.tokens, 1)
    sub2, split = bench.gather_ranges(torch, wl, bank, inp, wl.tokens, 3)
    assert len(split) == 3 and np.array_equal(sub, sub2)
    (w0, ws, w1), = bench.run_gather_ranges(wl, sub, whole)
    parts = bench.run_gather_ranges(wl, sub, split)
    assert np.array_equal(np.concatenate([p[0] for p in parts]).view(np.uint32), w0.view(np.uint32))
    assert np.array_equal(np.concatenate([p[1] for p in parts]).view(np.uint16), ws.view(np.uint16))
    assert np.array_equal(np.concatenate([p[2] for p in parts]).view(np.uint32), w1.view(np.uint32))
