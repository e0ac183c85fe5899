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
    assert bench.kernel_pattern("gather-no-stash") == "sdm_gather_"
    assert "sdm_gather_" in "sdm_gather_kernel" and "sdm_gather_" in "sdm_gather_pair_kernel"
    assert bench.kernel_pattern("gather-compact") == "sdm_gather_"


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
    alg, _, shape = bench.algorithmic_bytes("c1", "steps")
    assert e["algorithmic_bytes_per_launch"] == alg == 64 * 1024 * 96 * 256
    assert e["tokens_per_launch"] == shape["tokens_per_launch"] == 64
    assert (tmp_path / "profiles" / "sdm_decode_steps_wide_kernel_c1.md").exists()
    # the stored figures apply while the kernel sources are unchanged, scaled to the
    # launch's token count
    assert bench.stored_traffic("c1", "steps", 64) == (e["bytes_per_launch"], "sdm_decode_steps_wide_kernel")
    b20, k20 = bench.stored_traffic("c1", "steps", 20)
    assert b20 == pytest.approx(e["bytes_per_launch"] * 20 / 64) and k20 == "sdm_decode_steps_wide_kernel"
    # a multi-token figure never stands for a single-token launch (another kernel)
    assert bench.stored_traffic("c1", "steps", 1) == (None, None)
    assert bench.stored_traffic("c1", "step", 1) == (None, None)
    monkeypatch.setattr(bench, "kernel_source_hash", lambda kind=None: "0" * 16)
    assert bench.stored_traffic("c1", "steps", 64) == (None, None)


def test_traffic_of_the_timed_launch_matches_its_algorithmic_bytes(tmp_path, monkeypatch):
    """The traffic reported for a launch of K tokens is the per-token counter bytes times
    K: its ratio to that launch's algorithmic bytes is the profiled ratio, whatever K."""
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    t, f, w, cf, cw = (str(tmp_path / n) for n in ("trace", "fetch", "write", "cfetch", "cwrite"))
    alg, _, _ = bench.algorithmic_bytes("c1", "steps")
    _trace(t, [(WIDE, 10, 300000.0)])
    # 1.04 x the algorithmic bytes over the 64-token launch, split 2:1 between reads and writes
    _counter(f, [(WIDE, alg * 1.04 * 2 / 3 / 1024 / 2)])
    _counter(w, [(WIDE, alg * 1.04 / 3 / 1024)])
    _counter(cf, [(COPY, 524288.0)])
    _counter(cw, [(COPY, 1048576.0)])
    assert bench.main(["--config", "c1", "--ingest-profile", t, f, w, cf, cw]) == 0
    per_token = alg // 64
    for k in (2, 20, 64):
        traffic, _ = bench.stored_traffic("c1", "steps", k)
        assert traffic / (per_token * k) == pytest.approx(1.04)


def test_gather_traffic_needs_the_same_live_tokens(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    g = "void sdm::(anonymous namespace)::sdm_gather_kernel<unsigned short, 16, 2, false, int, unsigned short>(sdm::GatherParams)"
    t, f, w, cf, cw = (str(tmp_path / n) for n in ("trace", "fetch", "write", "cfetch", "cwrite"))
    _trace(t, [(g, 10, 250000.0)])
    _counter(f, [(g, 700000.0)])
    _counter(w, [(g, 600000.0)])
    _counter(cf, [(COPY, 524288.0)])
    _counter(cw, [(COPY, 1048576.0)])
    assert bench.main(["--config", "c3", "--ingest-profile", t, f, w, cf, cw]) == 0
    with open(tmp_path / "profiles" / "traffic.json") as fh:
        e = json.load(fh)["c3/gather"]
    _, _, shape = bench.algorithmic_bytes("c3", "steps")
    assert e["live_tokens"] == shape["live_tokens"]
    assert bench.stored_traffic("c3", "gather", 32768, shape["live_tokens"])[0] == pytest.approx(
        (700000.0 * 2 + 600000.0) * 1024)
    assert bench.stored_traffic("c3", "gather", 32768, shape["live_tokens"] - 1) == (None, None)


def test_gather_shapes_profile_under_their_own_kind(tmp_path, monkeypatch):
    """A launch shape without a stash runs the pair layout: its profile is stored under
    its own kind, with the shape's algorithmic bytes, in a summary named for the shape."""
    import gen
    import torch
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    g = "void sdm::(anonymous namespace)::sdm_gather_pair_kernel<unsigned short, 16, 2, int, unsigned short>(sdm::GatherParams)"
    t, f, w, cf, cw = (str(tmp_path / n) for n in ("trace", "fetch", "write", "cfetch", "cwrite"))
    _trace(t, [(g, 10, 150000.0)])
    _counter(f, [(g, 300000.0)])
    _counter(w, [(g, 20000.0)])
    _counter(cf, [(COPY, 524288.0)])
    _counter(cw, [(COPY, 1048576.0)])
    assert bench.main(["--config", "c3", "--gather", "no-stash", "--ingest-profile", t, f, w, cf, cw]) == 0
    with open(tmp_path / "profiles" / "traffic.json") as fh:
        data = json.load(fh)
    assert set(data) == {"c3/gather-no-stash"}
    e = data["c3/gather-no-stash"]
    assert e["kernel"] == "sdm_gather_pair_kernel"
    wl = gen.WORKLOADS["c3"]
    row = wl.head_dim * torch.empty((), dtype=wl.bank_dtype).element_size()
    live = e["live_tokens"]
    assert e["algorithmic_bytes_per_launch"] == live * (wl.width0 + wl.width1) * row
    assert (tmp_path / "profiles" / "sdm_gather_pair_kernel_c3_no-stash.md").exists()
    assert bench.stored_traffic("c3", "gather-no-stash", wl.tokens, live)[1] == "sdm_gather_pair_kernel"
    assert bench.stored_traffic("c3", "gather", wl.tokens, live) == (None, None)
    # the other shapes' bytes
    assert bench.algorithmic_bytes("c3", "steps", 0, "one-op-no-stash")[0] == live * wl.width0 * row
    assert bench.algorithmic_bytes("c3", "steps", 0, "one-op")[0] == (live + wl.tokens) * wl.width0 * row
    assert bench.algorithmic_bytes("c3", "steps", 0, "two-ops")[0] == (
        live * (wl.width0 + wl.width1) + wl.tokens * wl.width0) * row
    # compact stashes and other paddings are not summarised
    with pytest.raises(SystemExit):
        bench.main(["--config", "c3", "--gather", "compact", "--ingest-profile", t, f, w, cf, cw])
    with pytest.raises(SystemExit):
        bench.main(["--config", "c3", "--gather", "no-stash", "--valid", "all", "--ingest-profile", t, f, w, cf, cw])


def test_gather_live_count_does_not_depend_on_the_device():
    """The profile's algorithmic bytes and the benchmark's launch count the same live
    tokens: the per-chunk counts are drawn on the CPU for every device."""
    import gen
    wl = gen.WORKLOADS["c3"]
    a = gen.gather_inputs(wl.replace(width0=1, width1=0), 0)["chunk_valid"]
    b = gen.gather_inputs(wl.replace(width0=2, width1=3), 0)["chunk_valid"]
    assert a.dtype == torch_int32() and a.equal(b)
    _, _, shape = bench.algorithmic_bytes("c3", "steps")
    assert shape["live_tokens"] == gen.live_tokens(wl, a) == int(a.long().sum())
    with open(os.path.join(ROOT, "gen", "workloads.py")) as fh:
        src = fh.read()
    assert 'generator=_gen("cpu", seed, "valid")' in src


def torch_int32():
    import torch
    return torch.int32


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


def test_kernel_hash_of_a_kind_covers_its_own_sources(tmp_path, monkeypatch):
    """A gather-only change leaves the decode kinds' stored figures valid, and the
    reverse; the shared header and the C ABI count for both."""
    src = tmp_path / "sparse_delta_rule_amd" / "csrc"
    src.mkdir(parents=True)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    for n in ("sdm_decode.hip", "sdm_gather.hip", "sdm_kernels.h", "sdm_api.hip", "sdm_convert.hip"):
        (src / n).write_text(f"int {n.split('.')[0]}() {{ return 0; }}\n")
    h = {k: bench.kernel_source_hash(k) for k in ("step", "steps", "gather", "gather-no-stash")}
    assert h["step"] == h["steps"] and h["gather"] == h["gather-no-stash"] and h["step"] != h["gather"]

    def changed(name, text):
        (src / name).write_text(text)
        return {k: bench.kernel_source_hash(k) != v for k, v in h.items()}
    assert changed("sdm_gather.hip", "int g() { return 1; }\n") == {
        "step": False, "steps": False, "gather": True, "gather-no-stash": True}
    (src / "sdm_gather.hip").write_text("int sdm_gather() { return 0; }\n")
    assert changed("sdm_decode.hip", "int d() { return 1; }\n") == {
        "step": True, "steps": True, "gather": False, "gather-no-stash": False}
    (src / "sdm_decode.hip").write_text("int sdm_decode() { return 0; }\n")
    assert not any(changed("sdm_convert.hip", "int c() { return 1; }\n").values())
    assert all(changed("sdm_kernels.h", "int k() { return 1; }\n").values())


# ------------------------------------------------------------ CPU baseline legs
def test_host_threads_is_bounded(monkeypatch):
    monkeypatch.setenv("OMP_NUM_THREADS", "3")
    assert bench.host_threads() == min(3, len(os.sched_getaffinity(0)))
    monkeypatch.delenv("OMP_NUM_THREADS")
    assert 1 <= bench.host_threads() <= bench.THREAD_CAP == 16


def test_host_record_names_the_cpu_and_the_cap():
    h = bench.host_record()
    assert h["nproc"] == os.cpu_count() and h["affinity_cpus"] == len(os.sched_getaffinity(0))
    assert isinstance(h["model"], str) and h["model"]
    assert h["thread_cap"] == 16 and "16" in h["thread_cap_reason"]


def test_single_thread_leg_is_pinned_and_restored():
    before = os.sched_getaffinity(0)
    seen = []
    with bench.pinned_to_one_cpu() as pin:
        seen.append(os.sched_getaffinity(0))
        import threading
        th = threading.Thread(target=lambda: seen.append(os.sched_getaffinity(0)))
        th.start()
        th.join()
    assert seen[0] == {pin.cpu} and seen[1] == {pin.cpu}  # threads started meanwhile inherit it
    assert os.sched_getaffinity(0) == before


def test_oracle_sample_is_bounded_in_host_memory():
    import gen
    wl = gen.WORKLOADS["c2"]
    n = bench.sample_streams(wl, 10 ** 9)
    # every touched row of every sampled stream fits the cap
    assert n * (wl.W + wl.R) * wl.steps * wl.head_dim * 2 <= 2 << 30
    assert bench.sample_streams(wl, 3) == 3 and bench.sample_streams(wl, 0) == 1
    c1 = gen.WORKLOADS["c1"]
    assert bench.sample_streams(c1, 10 ** 9) == c1.streams


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


def test_dtype_fields():
    """dtype is the arithmetic type (float32 on every bank); the bank's storage type is
    reported beside it."""
    import gen
    assert bench.dtype_fields(gen.WORKLOADS["c2"]) == {"dtype": "f32", "storage_dtype": "bf16"}
    assert bench.dtype_fields(gen.WORKLOADS["c4"]) == {"dtype": "f32", "storage_dtype": "f32"}


def test_stream_sweep_fit(tmp_path, monkeypatch):
    """A kernel trace of a stream sweep is grouped by launch size and fitted as a fixed
    cost per launch plus a cost per stream."""
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    name = "void sdm::(anonymous namespace)::sdm_decode_kernel<unsigned short, 16, 4, 1, 1>(sdm::DecodeParams)"
    hdr = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Workgroup_Size_X", "Grid_Size_X", "Grid_Size_Y"]
    rows = []
    t = 0
    for n in (512, 1024, 2048):
        for _ in range(3):
            dur = 5000 + 10 * n  # 5 us fixed + 10 ns per stream
            rows.append([name, t, t + dur, 256, n * 256, 1])
            rows.append(["other_kernel", t, t + 7, 64, 64, 1])
            t += dur + 100
    d = tmp_path / "trace"
    _write_csv(str(d / "run_kernel_trace.csv"), hdr, rows)
    assert bench.main(["--config", "c2", "--entry", "step", "--streams", "2048,512,1024",
                       "--ingest-stream-sweep", str(d)]) == 0
    md = (tmp_path / "profiles" / "sdm_decode_kernel_c2_stream_sweep.md").read_text()
    assert "5.00 us + streams x 10.00 ns" in md
    # c2 moves (2*64 + 64) rows of 256 bytes per stream per token: 49152 B per 10 ns
    assert "marginal rate of 4915 GB/s" in md
    with pytest.raises(SystemExit, match="--streams list"):
        bench.main(["--config", "c2", "--entry", "step", "--streams", "512,1024", "--ingest-stream-sweep", str(d)])


def test_gather_bank_overrides_are_for_the_gather_and_never_profiled(tmp_path, monkeypatch):
    with pytest.raises(SystemExit, match="--config c3"):
        bench.main(["--config", "c2", "--head-dim", "256"])
    with pytest.raises(SystemExit, match="--config c3"):
        bench.main(["--config", "c1", "--bank-dtype", "f32"])
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    t, f, w, cf, cw = (str(tmp_path / n) for n in ("trace", "fetch", "write", "cfetch", "cwrite"))
    for flags in (["--head-dim", "256"], ["--bank-dtype", "f32"]):
        with pytest.raises(SystemExit, match="c3's own tokens"):
            bench.main(["--config", "c3", *flags, "--ingest-profile", t, f, w, cf, cw])


def test_output_placement_is_for_the_gather_and_never_profiled(tmp_path, monkeypatch):
    with pytest.raises(SystemExit, match="--config c3"):
        bench.main(["--config", "c2", "--outputs-apart", "0"])
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    t, f, w, cf, cw = (str(tmp_path / n) for n in ("trace", "fetch", "write", "cfetch", "cwrite"))
    with pytest.raises(SystemExit, match="c3's own tokens"):
        bench.main(["--config", "c3", "--outputs-apart", "0", "--ingest-profile", t, f, w, cf, cw])
    assert bench.parse_args(["--config", "c3", "--outputs-apart", "2048"]).outputs_apart == 2048
    assert bench.parse_args([]).outputs_apart is None
