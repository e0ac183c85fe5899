"""Parity of the HIP decode step (sdm_decode_step through the C ABI) with the oracle.

Two checks on every case:
  * free-running over all steps, bit for bit against the oracle run in the
    summation order include/sdm.h documents for the kernel (RG row groups);
  * per step, within the stated tolerance of the oracle in plain ascending
    order (groups = 1), with the GPU bank of the checked streams set to the
    oracle's own state before each step (the oracle's state is the GPU's input,
    never the other way round). Untouched rows are compared bit for bit.
The float32 tolerance is 1e-5 max(|ref|, M), the bfloat16 one 1 ulp +
2^-8 max(|ref|, M), M being the sum of the magnitudes of the terms (from the
float64 brute force).
"""

import numpy as np
import pytest
import torch

import gen
import oracle
from sparse_delta_rule_amd import sdm_decode_step
from tests.helpers import (bits_equal, decode_tolerance_ok, documented_decode_groups, from_np_bank,
                           step_to_numpy, stream_rows, sub_inputs, to_np_bank)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def _say(*a):
    print(*a, flush=True)


def check_decode(wl: gen.DecodeWorkload, seed: int, free_streams, sync_streams, device_inputs=False,
                 steps=None, drift_streams=()):
    """Run ``wl`` on the GPU over all streams and check the sampled streams both ways.

    drift_streams: streams the GPU runs free that are compared, every step, with the
    oracle run free in plain ascending order from the same starting bank; the
    largest error as a multiple of the per-step bound (magnitudes from the float64
    brute force on the oracle's state) is returned as worst["drift_read"] and
    worst["drift_row"], and no bound is asserted here (two correct orders drift
    apart as errors compound)."""
    steps = wl.steps if steps is None else steps
    P = wl.slots_per_stream
    bf16 = wl.bank_dtype == torch.bfloat16
    gen_dev = DEV if device_inputs else "cpu"
    bank = gen.decode_bank(wl, seed, gen_dev).to(DEV)
    free_streams = np.asarray(free_streams, dtype=np.int64)
    sync_streams = np.asarray(sync_streams, dtype=np.int64)
    drift_streams = np.asarray(drift_streams, dtype=np.int64)
    assert not set(free_streams) & set(sync_streams) and not set(drift_streams) & set(sync_streams)
    drift_rows = torch.from_numpy(stream_rows(drift_streams, P)).to(DEV)
    bank_drift = to_np_bank(bank[drift_rows])    # oracle, ascending order, free-running
    free_rows = torch.from_numpy(stream_rows(free_streams, P)).to(DEV)
    sync_rows = torch.from_numpy(stream_rows(sync_streams, P)).to(DEV)
    bank_free = to_np_bank(bank[free_rows])      # oracle, kernel order, free-running
    bank_sync = to_np_bank(bank[sync_rows])      # oracle, ascending order, resynced into the GPU
    rg = documented_decode_groups(wl.W, wl.R)
    worst = {"read": 0.0, "row": 0.0, "drift_read": 0.0, "drift_row": 0.0}
    for t in range(steps):
        inp = gen.decode_step_inputs(wl, seed, t, gen_dev)
        inp = {k: v.to(DEV) for k, v in inp.items()}
        npin = step_to_numpy(inp)
        # the streams checked per step start from the oracle's state
        if len(sync_streams):
            bank[sync_rows] = from_np_bank(bank_sync).to(DEV)
        readings = sdm_decode_step(bank, **inp)
        torch.cuda.synchronize()
        # free-running streams: bit for bit against the kernel's documented order
        if len(free_streams):
            sub = sub_inputs(npin, free_streams, P)
            ref = oracle.decode_step(bank_free, **sub, groups=rg)
            got = to_np_bank(readings[torch.from_numpy(free_streams).to(DEV)])
            assert bits_equal(got, ref), f"step {t}: readings differ from the oracle (RG={rg})"
        # resynced streams: stated tolerance against the ascending order
        if len(sync_streams):
            sub = sub_inputs(npin, sync_streams, P)
            _, _, row_mag, _, read_mag = oracle.decode_step_f64(bank_sync.copy(), **sub)
            before = bank_sync.copy()
            ref = oracle.decode_step(bank_sync, **sub, groups=1)
            got = to_np_bank(readings[torch.from_numpy(sync_streams).to(DEV)])
            ok, ratio = decode_tolerance_ok(got, ref, read_mag, bf16)
            worst["read"] = max(worst["read"], ratio)
            assert ok, f"step {t}: readings outside tolerance (worst {ratio:.3g} of the bound)"
            got_bank = to_np_bank(bank[sync_rows])
            ok, ratio = decode_tolerance_ok(got_bank[sub["k_idx"]], bank_sync[sub["k_idx"]], row_mag, bf16)
            worst["row"] = max(worst["row"], ratio)
            assert ok, f"step {t}: written rows outside tolerance (worst {ratio:.3g} of the bound)"
            untouched = np.setdiff1d(np.arange(bank_sync.shape[0]), sub["k_idx"].ravel())
            assert bits_equal(got_bank[untouched], before[untouched]), f"step {t}: untouched rows changed"
        # free-running streams against the free-running ascending-order oracle
        if len(drift_streams):
            sub = sub_inputs(npin, drift_streams, P)
            _, _, row_mag, _, read_mag = oracle.decode_step_f64(bank_drift.copy(), **sub)
            ref = oracle.decode_step(bank_drift, **sub, groups=1)
            got = to_np_bank(readings[torch.from_numpy(drift_streams).to(DEV)])
            _, ratio = decode_tolerance_ok(got, ref, read_mag, bf16)
            worst["drift_read"] = max(worst["drift_read"], ratio)
            got_bank = to_np_bank(bank[drift_rows])
            _, ratio = decode_tolerance_ok(got_bank[sub["k_idx"]], bank_drift[sub["k_idx"]], row_mag, bf16)
            worst["drift_row"] = max(worst["drift_row"], ratio)
    if len(free_streams):
        assert bits_equal(to_np_bank(bank[free_rows]), bank_free), "final bank differs from the oracle"
    return worst


# ------------------------------------------------------------ small workloads
def test_config_c0_all_steps():
    wl = gen.WORKLOADS["c0"]
    _say("c0:", wl.name)
    for seed in (0, 1, 2):
        worst = check_decode(wl, seed, free_streams=[0, 2], sync_streams=[1, 3])
        _say(f"  seed {seed}: worst readings {worst['read']:.3g}, rows {worst['row']:.3g} of the bound")


EDGE = [
    # name, bank dtype, streams, slots/stream, hd, W, R, G, k idx, q idx, val dtype
    ("w1r1 hd1 f32", torch.float32, 5, 8, 1, 1, 1, 1, torch.int64, torch.int64, torch.float32),
    ("hd3 bf16 elem vectors", torch.bfloat16, 6, 40, 3, 5, 3, 5, torch.int32, torch.int64, torch.float32),
    ("hd8 bf16 G=W", torch.bfloat16, 9, 64, 8, 7, 9, 7, torch.int64, torch.int32, torch.float32),
    ("hd100 f32 W=R=256", torch.float32, 4, 600, 100, 256, 256, 1, torch.int64, torch.int64, torch.float32),
    ("hd100 bf16 (200-B rows)", torch.bfloat16, 5, 300, 100, 33, 17, 33, torch.int32, torch.int32, torch.float32),
    ("hd101 f32 odd", torch.float32, 3, 300, 101, 64, 64, 64, torch.int64, torch.int64, torch.float32),
    ("hd127 bf16 odd", torch.bfloat16, 3, 300, 127, 16, 48, 1, torch.int32, torch.int32, torch.bfloat16),
    ("hd128 bf16 W=1 R=256", torch.bfloat16, 4, 300, 128, 1, 256, 1, torch.int32, torch.int32, torch.float32),
    ("hd128 f32 W=256 R=1", torch.float32, 4, 300, 128, 256, 1, 256, torch.int64, torch.int32, torch.float32),
    ("hd129 f32 two slices", torch.float32, 3, 100, 129, 9, 12, 1, torch.int64, torch.int64, torch.float32),
    ("hd300 bf16 wide", torch.bfloat16, 3, 100, 300, 20, 20, 20, torch.int32, torch.int32, torch.bfloat16),
    ("hd512 f32 four slices", torch.float32, 2, 80, 512, 40, 8, 1, torch.int64, torch.int64, torch.float32),
    ("hd64 bf16 bf16 values", torch.bfloat16, 17, 128, 64, 12, 12, 12, torch.int32, torch.int32, torch.bfloat16),
]


@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_edge_shapes(case):
    name, dt, S, P, hd, W, R, G, kd, qd, vd = case
    wl = gen.DecodeWorkload(name=name, bank_dtype=dt, streams=S, slots_per_stream=P, head_dim=hd, W=W,
                            R=R, G=G, steps=3, idx_dtype=kd, weights="normal_sqrtw", beta="sigmoid",
                            g_low=-0.2, bank_std=0.5, val_dtype=vd)
    _say("edge:", name)
    half = S // 2
    # mixed index dtypes: k from wl.idx_dtype, q converted after generation
    if qd != kd:
        orig = gen.decode_step_inputs

        def patched(w, seed, step, device="cpu"):
            d = orig(w, seed, step, device)
            d["q_idx"] = d["q_idx"].to(qd)
            return d

        gen.decode_step_inputs = patched
        try:
            worst = check_decode(wl, 5, free_streams=list(range(half)), sync_streams=list(range(half, S)))
        finally:
            gen.decode_step_inputs = orig
    else:
        worst = check_decode(wl, 5, free_streams=list(range(half)), sync_streams=list(range(half, S)))
    _say(f"  worst readings {worst['read']:.3g}, rows {worst['row']:.3g} of the bound")


# ----------------------------------------------------------- read after write
@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_reads_see_this_steps_writes(dt):
    """q_idx = k_idx and one-hot q_val: each reading is the row just written, bit for bit."""
    S, P, hd, W = 64, 512, 128, 64
    wl = gen.DecodeWorkload(name="raw", bank_dtype=dt, streams=S, slots_per_stream=P, head_dim=hd, W=W,
                            R=W, G=W, steps=1, idx_dtype=torch.int64, weights="normal", beta="sigmoid",
                            g_low=-0.1)
    bank = gen.decode_bank(wl, 3).to(DEV)
    inp = {k: v.to(DEV) for k, v in gen.decode_step_inputs(wl, 3, 0).items()}
    inp["q_idx"] = inp["k_idx"].clone()
    hot = torch.randint(0, W, (S,), generator=torch.Generator().manual_seed(9)).to(DEV)
    inp["q_val"] = torch.nn.functional.one_hot(hot, W).float()
    readings = sdm_decode_step(bank, **inp)
    rows = bank[inp["k_idx"][torch.arange(S, device=DEV), hot]]
    assert torch.equal(readings.view(torch.uint8), rows.contiguous().view(torch.uint8))
    # and the readings are not the rows as they were before the write
    bank0 = gen.decode_bank(wl, 3).to(DEV)
    old = bank0[inp["k_idx"][torch.arange(S, device=DEV), hot]]
    assert not torch.equal(readings, old)


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_reads_of_written_slots_permuted_and_repeated(dt):
    """Reads drawn from this step's write slots (permuted, some repeated, mixed with
    unwritten slots): against the oracle bit for bit."""
    wl = gen.WORKLOADS["c1"].replace(streams=48, slots_per_stream=256, bank_dtype=dt)
    bank = gen.decode_bank(wl, 12).to(DEV)
    inp = {k: v.to(DEV) for k, v in gen.decode_step_inputs(wl, 12, 0).items()}
    g = torch.Generator().manual_seed(13)
    for s in range(wl.streams):
        perm = torch.randperm(wl.W, generator=g)
        take = torch.randint(0, 3, (wl.R,), generator=g)  # 0: a written slot, 1: repeat, 2: keep
        q = inp["q_idx"][s].clone()
        k = inp["k_idx"][s]
        q[take == 0] = k[perm.to(DEV)][take == 0]
        q[take == 1] = k[0]
        inp["q_idx"][s] = q
    npin = step_to_numpy(inp)
    ref_bank = to_np_bank(bank)
    ref = oracle.decode_step(ref_bank, **npin, groups=documented_decode_groups(wl.W, wl.R))
    readings = sdm_decode_step(bank, **inp)
    assert bits_equal(to_np_bank(readings), ref)
    assert bits_equal(to_np_bank(bank), ref_bank)


def test_heavy_read_write_overlap_c4_shape():
    """Config c4's shape (fp32, hd 100, W = R = 256 of 2048 slots: ~32 read slots per stream
    coincide with written ones) with q drawn from the written slots for half the streams."""
    wl = gen.WORKLOADS["c4"].replace(streams=16)
    bank = gen.decode_bank(wl, 4).to(DEV)
    inp = {k: v.to(DEV) for k, v in gen.decode_step_inputs(wl, 4, 0).items()}
    inp["q_idx"][:8] = inp["k_idx"][:8].flip(1)
    npin = step_to_numpy(inp)
    ref_bank = to_np_bank(bank)
    ref = oracle.decode_step(ref_bank, **npin, groups=documented_decode_groups(256, 256))
    readings = sdm_decode_step(bank, **inp)
    assert bits_equal(to_np_bank(readings), ref)
    assert bits_equal(to_np_bank(bank), ref_bank)


# ------------------------------------------------------------ GPU properties
def test_stream_subset_and_repeat_are_bit_identical():
    wl = gen.WORKLOADS["c2"].replace(streams=96, slots_per_stream=1024)
    bank0 = gen.decode_bank(wl, 7).to(DEV)
    inp = {k: v.to(DEV) for k, v in gen.decode_step_inputs(wl, 7, 0).items()}
    a, b, c = bank0.clone(), bank0.clone(), bank0.clone()
    ra = sdm_decode_step(a, **inp)
    rb = sdm_decode_step(b, **inp)
    assert torch.equal(ra.view(torch.int16), rb.view(torch.int16)) and torch.equal(a.view(torch.int16), b.view(torch.int16))
    sub = {k: v[10:50].contiguous() for k, v in inp.items()}
    rc = sdm_decode_step(c, **sub)
    assert torch.equal(rc.view(torch.int16), ra[10:50].view(torch.int16))
    rows = slice(10 * 1024, 50 * 1024)
    assert torch.equal(c[rows].view(torch.int16), a[rows].view(torch.int16))


def test_power_of_two_scaling_is_exact():
    """Scaling the bank and v by 2^k scales new rows and readings by 2^k exactly."""
    wl = gen.WORKLOADS["c1"].replace(streams=64, slots_per_stream=512)
    bank = gen.decode_bank(wl, 8).to(DEV)
    inp = {k: v.to(DEV) for k, v in gen.decode_step_inputs(wl, 8, 0).items()}
    b1, b2 = bank.clone(), bank.clone() * 4
    r1 = sdm_decode_step(b1, **inp)
    inp2 = dict(inp)
    inp2["v"] = inp["v"] * 4
    r2 = sdm_decode_step(b2, **inp2)
    assert torch.equal(r2, r1 * 4) and torch.equal(b2, b1 * 4)


def test_graph_of_single_steps_matches_eager():
    """A sequence of single-step launches captured in one HIP graph (the benchmark's
    --entry step path): every replay, from the same starting bank, equals eager steps."""
    wl = gen.WORKLOADS["c1"].replace(streams=96, slots_per_stream=512, steps=6)
    bank0 = gen.decode_bank(wl, 14).to(DEV)
    seq = [{k: v.to(DEV) for k, v in gen.decode_step_inputs(wl, 14, t).items()} for t in range(wl.steps)]
    ref_bank = bank0.clone()
    ref = [sdm_decode_step(ref_bank, **inp) for inp in seq]
    bank = bank0.clone()
    outs = [torch.empty_like(r) for r in ref]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for inp, o in zip(seq, outs):
            sdm_decode_step(bank, **inp, readings=o)
    for i in range(3):
        bank.copy_(bank0)
        for o in outs:
            o.zero_()
        junk = torch.randn(1 << 20, device=DEV).sum()  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o.view(torch.int16), r.view(torch.int16)), f"replay {i}, step {t}"
        assert torch.equal(bank.view(torch.int16), ref_bank.view(torch.int16)), f"replay {i}"
        del junk


def test_zero_streams_and_errors_from_python():
    from sparse_delta_rule_amd import SdmError
    bank = torch.zeros(64, 8, device=DEV)
    e = torch.zeros(0, 2, dtype=torch.int64, device=DEV)
    f = torch.zeros(0, 2, device=DEV)
    r = sdm_decode_step(bank, e, f, torch.zeros(0, 8, device=DEV), torch.zeros(0, 1, device=DEV),
                        torch.zeros(0, 1, device=DEV), e, f)
    assert r.shape == (0, 8)
    idx = torch.zeros(1, 300, dtype=torch.int64, device=DEV)
    val = torch.zeros(1, 300, device=DEV)
    with pytest.raises(SdmError, match="SDM_E_RANGE"):
        sdm_decode_step(bank, idx, val, torch.zeros(1, 8, device=DEV), torch.zeros(1, 1, device=DEV),
                        torch.zeros(1, 1, device=DEV), idx, val)
    z = torch.zeros(2, 0, dtype=torch.int64, device=DEV)  # W = R = 0
    with pytest.raises(SdmError, match="SDM_E_RANGE"):
        sdm_decode_step(bank, z, torch.zeros(2, 0, device=DEV), torch.zeros(2, 8, device=DEV),
                        torch.zeros(2, 1, device=DEV), torch.zeros(2, 1, device=DEV), z, torch.zeros(2, 0, device=DEV))


def test_debug_validation_catches_broken_preconditions():
    """SDM_DEBUG_VALIDATE=1 in a child process: a repeated write slot, a slot out of
    range and a slot shared by two streams are reported before any launch."""
    import subprocess
    import sys
    code = r'''
import torch, sparse_delta_rule_amd as sdm
dev = torch.device("cuda", 0)
bank = torch.zeros(64, 8, device=dev)
def call(k, q):
    k = torch.tensor(k, dtype=torch.int64, device=dev); q = torch.tensor(q, dtype=torch.int32, device=dev)
    S, W = k.shape; R = q.shape[1]
    try:
        sdm.sdm_decode_step(bank, k, torch.ones(S, W, device=dev), torch.ones(S, 8, device=dev),
                            torch.ones(S, 1, device=dev), torch.zeros(S, 1, device=dev), q, torch.ones(S, R, device=dev))
        return "ok"
    except sdm.SdmError as e:
        return str(e)
print(call([[1, 2], [3, 4]], [[1], [4]]))
print(call([[1, 1], [3, 4]], [[1], [4]]))
print(call([[1, 2], [3, 64]], [[1], [4]]))
print(call([[1, 2], [3, 4]], [[1], [2]]))
'''
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, SDM_DEBUG_VALIDATE="1")
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120,
                         cwd=root)
    lines = out.stdout.strip().splitlines()
    assert lines[0] == "ok", out.stderr
    assert "writes slot 1 twice" in lines[1]
    assert "outside [0, 64)" in lines[2]
    assert "used by streams 0 and 1" in lines[3]


# ----------------------------------------------------------- full-size workloads
@pytest.mark.slow
@pytest.mark.parametrize("name,free,sync", [
    ("c1", [0, 511, 1023], [1, 700]),
    ("c2", [0, 2047, 4095], [5, 3000]),
    ("c4", [0, 300, 511], [7, 256]),
])
def test_full_size_configs(name, free, sync):
    wl = gen.WORKLOADS[name]
    _say(f"{name}: {wl.name}")
    worst = check_decode(wl, 0, free_streams=free, sync_streams=sync, device_inputs=True)
    _say(f"  worst readings {worst['read']:.3g}, rows {worst['row']:.3g} of the bound")
    torch.cuda.empty_cache()


# The largest error of the GPU path run free over a whole sequence against the
# oracle run free in plain ascending order, as a multiple of the per-step bound,
# must stay below this many times the sequence length: the errors of two correct
# summation orders compound from step to step, but stay within a fixed multiple
# of the per-step bound per step.
DRIFT_PER_STEP = 1.0


@pytest.mark.slow
@pytest.mark.parametrize("name,drift", [
    ("c1", [2, 512, 1022]),
    ("c2", [1, 2048, 4094]),
    ("c4", [1, 299, 510]),
])
def test_full_size_free_running_drift(name, drift):
    """Free-running error growth of the GPU path against the plain ascending order over
    the whole sequence of c1, c2 and c4 (sampled streams), reported and bounded."""
    wl = gen.WORKLOADS[name]
    worst = check_decode(wl, 0, free_streams=[], sync_streams=[], device_inputs=True, drift_streams=drift)
    _say(f"{name} free-running over {wl.steps} steps against the ascending-order oracle: readings up to "
         f"{worst['drift_read']:.3g}, written rows up to {worst['drift_row']:.3g} times the per-step bound")
    assert max(worst["drift_read"], worst["drift_row"]) <= DRIFT_PER_STEP * wl.steps
    torch.cuda.empty_cache()
