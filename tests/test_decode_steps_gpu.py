"""Parity of the multi-token decode (sdm_decode_steps through the C ABI).

One launch advances every stream by T tokens; the result must equal T
single-step calls bit for bit, and the oracle stepped T times in the kernel's
documented summation order. Cases stress the pipelining across tokens: rows a
token writes that the next token reads or writes, and prefetch geometries with
one and with several metadata items per thread. The library has two loops for
this call (chosen by how many waves the grid puts on a SIMD); each case runs
with the automatic choice and with each loop pinned through SDM_STEPS_LOOP.
"""

import numpy as np
import pytest
import torch

import gen
import oracle
from sparse_delta_rule_amd import sdm_decode_step, sdm_decode_steps
from tests.helpers import (bits_equal, documented_decode_groups, step_to_numpy, stream_rows, sub_inputs,
                           to_np_bank)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def _say(*a):
    print(*a, flush=True)


@pytest.fixture(params=["auto", "compact", "wide"])
def loop(request, monkeypatch):
    """Pin the multi-step loop (the wide one runs only where a workgroup has at most
    256 threads; elsewhere "wide" falls back to the compact loop)."""
    if request.param == "auto":
        monkeypatch.delenv("SDM_STEPS_LOOP", raising=False)
    else:
        monkeypatch.setenv("SDM_STEPS_LOOP", request.param)
    return request.param


def _sequence(wl, seed, device, steps):
    return {k: v.to(DEV) for k, v in gen.decode_sequence(wl, seed, device, steps).items()}


def check_steps(wl: gen.DecodeWorkload, seed: int, streams_checked, *, steps=None, device="cpu",
                also_single=True, edit=None):
    """Run ``steps`` tokens of ``wl`` in one launch; compare the checked streams with the
    oracle (free-running, kernel order) and, optionally, with single-step launches."""
    steps = wl.steps if steps is None else steps
    P = wl.slots_per_stream
    bank0 = gen.decode_bank(wl, seed, device).to(DEV)
    seq = _sequence(wl, seed, device, steps)
    if edit is not None:
        edit(seq)
    checked = np.asarray(streams_checked, dtype=np.int64)
    rows = torch.from_numpy(stream_rows(checked, P)).to(DEV)
    ref_bank = to_np_bank(bank0[rows])
    bank = bank0.clone()
    readings = sdm_decode_steps(bank, **seq)
    torch.cuda.synchronize()
    rg = documented_decode_groups(wl.W, wl.R)
    sel = torch.from_numpy(checked).to(DEV)
    for t in range(steps):
        npin = step_to_numpy({k: v[t] for k, v in seq.items()})
        ref = oracle.decode_step(ref_bank, **sub_inputs(npin, checked, P), groups=rg)
        assert bits_equal(to_np_bank(readings[t][sel]), ref), f"token {t}: readings differ from the oracle"
    assert bits_equal(to_np_bank(bank[rows]), ref_bank), "bank differs from the oracle after the last token"
    if also_single:
        b1 = bank0.clone()
        for t in range(steps):
            r1 = sdm_decode_step(b1, **{k: v[t] for k, v in seq.items()})
            assert torch.equal(r1.view(torch.uint8), readings[t].contiguous().view(torch.uint8)), f"token {t}"
        assert torch.equal(b1.view(torch.uint8), bank.view(torch.uint8))
    return bank, readings


def test_config_c0_all_tokens(loop):
    wl = gen.WORKLOADS["c0"]
    for seed in (0, 1):
        check_steps(wl, seed, [0, 1, 2, 3])


CASES = [
    # name, bank dtype, streams, slots/stream, hd, W, R, G, idx dtype, val dtype, steps
    ("c1 shape small", torch.bfloat16, 40, 256, 128, 32, 32, 1, torch.int32, torch.float32, 9),
    ("two tokens", torch.bfloat16, 7, 100, 128, 16, 16, 16, torch.int64, torch.float32, 2),
    ("hd100 f32 W=R=256", torch.float32, 3, 520, 100, 256, 256, 1, torch.int64, torch.float32, 4),
    ("hd3 bf16", torch.bfloat16, 9, 40, 3, 5, 7, 5, torch.int32, torch.bfloat16, 6),
    ("hd1 f32 W=R=256 (widened lane group)", torch.float32, 3, 300, 1, 256, 200, 1, torch.int64,
     torch.float32, 3),
    ("hd129 f32 two slices", torch.float32, 5, 64, 129, 9, 33, 9, torch.int64, torch.float32, 5),
    ("hd300 bf16 three slices", torch.bfloat16, 4, 64, 300, 12, 12, 1, torch.int32, torch.bfloat16, 4),
    ("hd64 f32 W=1 R=64", torch.float32, 11, 128, 64, 1, 64, 1, torch.int32, torch.float32, 7),
    # 64-thread workgroups for 128 columns: several metadata items per thread, over 5 tokens
    ("hd128 bf16 W=R=16 G=W, 4 metadata items per thread", torch.bfloat16, 8, 64, 128, 16, 16, 16, torch.int32,
     torch.float32, 5),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_shapes(case, loop):
    name, dt, S, P, hd, W, R, G, idt, vdt, T = case
    wl = gen.DecodeWorkload(name=name, bank_dtype=dt, streams=S, slots_per_stream=P, head_dim=hd, W=W, R=R,
                            G=G, steps=T, idx_dtype=idt, weights="normal_sqrtw", beta="sigmoid", g_low=-0.2,
                            bank_std=0.5, val_dtype=vdt)
    _say("steps:", name, "loop:", loop)
    check_steps(wl, 3, list(range(S)))


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_every_token_rewrites_the_same_rows(dt, loop):
    """Each stream owns exactly W slots, written and read by every token: token t + 1's
    row loads must see token t's writes (the loads issued right after the barrier)."""
    W = 32
    wl = gen.DecodeWorkload(name="same rows", bank_dtype=dt, streams=24, slots_per_stream=W, head_dim=128,
                            W=W, R=W, G=W, steps=12, idx_dtype=torch.int32, weights="normal_sqrtw",
                            beta="sigmoid", g_low=-0.1, bank_std=0.5)
    check_steps(wl, 5, list(range(24)))


def test_reads_of_next_tokens_writes_are_not_early(loop):
    """Token t reads exactly the slots token t + 1 writes: those reads must see token t's
    state (token t + 1's writes come later), while token t + 1's rows are already loading."""
    W = 16

    def edit(seq):
        seq["q_idx"][:-1] = seq["k_idx"][1:]

    wl = gen.DecodeWorkload(name="next writes", bank_dtype=torch.float32, streams=32, slots_per_stream=48,
                            head_dim=64, W=W, R=W, G=1, steps=10, idx_dtype=torch.int64, weights="normal",
                            beta="sigmoid", g_low=-0.1, bank_std=0.5)
    check_steps(wl, 6, list(range(32)), edit=edit)


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_misaligned_bank_view_takes_narrow_vectors(dt, loop):
    """A bank view one element past 16-byte alignment: the kernels read and write
    rows with narrower vectors (element-wide here) and stay exact, multi-token
    and single-token."""
    wl = gen.DecodeWorkload(name="misaligned", bank_dtype=dt, streams=12, slots_per_stream=64, head_dim=128,
                            W=16, R=16, G=16, steps=3, idx_dtype=torch.int64, weights="normal_sqrtw",
                            beta="sigmoid", g_low=-0.1, bank_std=0.5)
    bank0 = gen.decode_bank(wl, 61, "cpu")
    seq = _sequence(wl, 61, "cpu", wl.steps)

    def view():
        full = torch.zeros(bank0.numel() + 1, dtype=dt, device=DEV)
        b = full[1:].view(bank0.shape)
        b.copy_(bank0.to(DEV))
        assert b.data_ptr() % 16 != 0
        return b

    ref_bank = to_np_bank(bank0)
    refs = [oracle.decode_step(ref_bank, **step_to_numpy({k: v[t] for k, v in seq.items()}),
                               groups=documented_decode_groups(wl.W, wl.R)) for t in range(wl.steps)]
    bank = view()
    readings = sdm_decode_steps(bank, **seq)
    for t in range(wl.steps):
        assert bits_equal(to_np_bank(readings[t]), refs[t]), f"token {t}: readings differ from the oracle"
    assert bits_equal(to_np_bank(bank), ref_bank), "bank differs from the oracle"
    b1 = view()
    for t in range(wl.steps):
        r1 = sdm_decode_step(b1, **{k: v[t] for k, v in seq.items()})
        assert bits_equal(to_np_bank(r1), refs[t]), f"single step {t}"
    assert bits_equal(to_np_bank(b1), ref_bank)


def test_zero_tokens_and_errors():
    from sparse_delta_rule_amd import SdmError
    bank = torch.zeros(64, 8, device=DEV)
    e = torch.zeros(0, 3, 2, dtype=torch.int64, device=DEV)
    f = torch.zeros(0, 3, 2, device=DEV)
    r = sdm_decode_steps(bank, e, f, torch.zeros(0, 3, 8, device=DEV), torch.zeros(0, 3, 1, device=DEV),
                         torch.zeros(0, 3, 1, device=DEV), e, f)
    assert r.shape == (0, 3, 8)
    idx = torch.zeros(2, 1, 300, dtype=torch.int64, device=DEV)
    val = torch.zeros(2, 1, 300, device=DEV)
    with pytest.raises(SdmError, match="SDM_E_RANGE"):
        sdm_decode_steps(bank, idx, val, torch.zeros(2, 1, 8, device=DEV), torch.zeros(2, 1, 1, device=DEV),
                         torch.zeros(2, 1, 1, device=DEV), idx, val)
    z = torch.zeros(2, 3, 0, dtype=torch.int64, device=DEV)  # W = R = 0
    with pytest.raises(SdmError, match="SDM_E_RANGE"):
        sdm_decode_steps(bank, z, torch.zeros(2, 3, 0, device=DEV), torch.zeros(2, 3, 8, device=DEV),
                         torch.zeros(2, 3, 1, device=DEV), torch.zeros(2, 3, 1, device=DEV), z,
                         torch.zeros(2, 3, 0, device=DEV))


def test_unknown_loop_name_is_rejected(monkeypatch):
    from sparse_delta_rule_amd import SdmError
    monkeypatch.setenv("SDM_STEPS_LOOP", "fastest")
    bank = torch.zeros(64, 8, device=DEV)
    idx = torch.zeros(2, 1, 2, dtype=torch.int64, device=DEV)
    idx[:, :, 1] = 1
    val = torch.zeros(2, 1, 2, device=DEV)
    with pytest.raises(SdmError, match="SDM_STEPS_LOOP"):
        sdm_decode_steps(bank, idx, val, torch.zeros(2, 1, 8, device=DEV), torch.zeros(2, 1, 1, device=DEV),
                         torch.zeros(2, 1, 1, device=DEV), idx, val)
    monkeypatch.setenv("SDM_STEPS_LOOP", "compact")
    sdm_decode_steps(bank, idx, val, torch.zeros(2, 1, 8, device=DEV), torch.zeros(2, 1, 1, device=DEV),
                     torch.zeros(2, 1, 1, device=DEV), idx, val)
    torch.cuda.synchronize()


def test_debug_validation_spans_tokens():
    """SDM_DEBUG_VALIDATE=1 in a child process: a slot one stream uses at token 0
    and another at token 1 is reported (the streams' tokens are not ordered
    against one another), as are a repeated write slot and a slot out of range
    at a later token; slots that stay with one stream across tokens pass."""
    import os
    import subprocess
    import sys
    code = r'''
import torch, sparse_delta_rule_amd as sdm
dev = torch.device("cuda", 0)
bank = torch.zeros(64, 8, device=dev)
def call(k, q):
    k = torch.tensor(k, dtype=torch.int32, device=dev); q = torch.tensor(q, dtype=torch.int64, device=dev)
    T, S, W = k.shape; R = q.shape[2]
    try:
        sdm.sdm_decode_steps(bank, k, torch.ones(T, S, W, device=dev), torch.ones(T, S, 8, device=dev),
                             torch.ones(T, S, 1, device=dev), torch.zeros(T, S, 1, device=dev), q,
                             torch.ones(T, S, R, device=dev))
        torch.cuda.synchronize()
        return "ok"
    except sdm.SdmError as e:
        return str(e)
print(call([[[1, 2], [3, 4]], [[2, 5], [4, 6]]], [[[1], [4]], [[5], [6]]]))
print(call([[[1, 2], [3, 4]], [[2, 5], [4, 6]]], [[[1], [4]], [[5], [2]]]))
print(call([[[1, 2], [3, 4]], [[2, 2], [4, 6]]], [[[1], [4]], [[5], [6]]]))
print(call([[[1, 2], [3, 4]], [[2, 5], [4, 6]]], [[[1], [4]], [[64], [6]]]))
'''
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, SDM_DEBUG_VALIDATE="1")
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120,
                         cwd=root)
    lines = out.stdout.strip().splitlines()
    assert len(lines) == 4, out.stderr
    assert lines[0] == "ok", lines[0]
    assert "token 1: slot 2 is used by streams 0 and 1" in lines[1]
    assert "token 1: stream 0 writes slot 2 twice" in lines[2]
    assert "token 1: q_idx[0, 0] = 64 outside [0, 64)" in lines[3]


def test_graph_replays_match_eager(loop):
    """The benchmark's launch path: sdm_decode_steps captured in a HIP graph. Every
    replay, with eager torch work and synchronisations between replays, must equal an
    eager launch from the same starting bank."""
    wl = gen.WORKLOADS["c1"].replace(streams=128, slots_per_stream=512, steps=8)
    bank0 = gen.decode_bank(wl, 2).to(DEV)
    seq = _sequence(wl, 2, "cpu", 8)
    ref_bank = bank0.clone()
    ref = sdm_decode_steps(ref_bank, **seq)
    bank = bank0.clone()
    out = torch.empty_like(ref)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sdm_decode_steps(bank, **seq, readings=out)
    for i in range(3):
        bank.copy_(bank0)
        out.zero_()
        junk = torch.randn(1 << 20, device=DEV).sum()  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {i}"
        assert torch.equal(bank.view(torch.int16), ref_bank.view(torch.int16)), f"replay {i}"
        del junk


@pytest.mark.slow
@pytest.mark.parametrize("name,checked,pin", [
    ("c1", [0, 333, 1023], None),       # automatic choice: wide (two waves per SIMD)
    ("c1", [0, 333, 1023], "compact"),
    ("c2", [0, 2047, 4095], None),      # automatic choice: compact
    ("c2", [0, 2047, 4095], "wide"),
    ("c4", [0, 255, 511], None),        # 1024-thread workgroups: compact only
])
def test_full_size_configs(name, checked, pin, monkeypatch):
    if pin is None:
        monkeypatch.delenv("SDM_STEPS_LOOP", raising=False)
    else:
        monkeypatch.setenv("SDM_STEPS_LOOP", pin)
    wl = gen.WORKLOADS[name]
    _say(f"steps {name}: {wl.name}, loop {pin or 'auto'}")
    check_steps(wl, 0, checked, device=DEV, also_single=False)
    torch.cuda.empty_cache()


@pytest.mark.slow
@pytest.mark.parametrize("name,checked", [
    ("c1", [0, 1, 511, 700, 1023]),
    ("c2", [0, 17, 2048, 4095]),
    ("c4", [0, 3, 256, 511]),
])
def test_full_size_graph_replays(name, checked, monkeypatch):
    """A full-size workload in the benchmark's launch path: its whole token sequence as
    one sdm_decode_steps launch captured in a HIP graph, replayed twice from the same
    starting bank (restored between replays); sampled streams against the oracle, bit
    for bit, on every replay."""
    monkeypatch.delenv("SDM_STEPS_LOOP", raising=False)
    wl = gen.WORKLOADS[name]
    checked = np.asarray(checked, dtype=np.int64)
    P = wl.slots_per_stream
    bank0 = gen.decode_bank(wl, 0, DEV)
    seq = _sequence(wl, 0, DEV, wl.steps)
    rows = torch.from_numpy(stream_rows(checked, P)).to(DEV)
    ref_bank = to_np_bank(bank0[rows])
    rg = documented_decode_groups(wl.W, wl.R)
    refs = []
    for t in range(wl.steps):
        npin = step_to_numpy({k: v[t] for k, v in seq.items()})
        refs.append(oracle.decode_step(ref_bank, **sub_inputs(npin, checked, P), groups=rg))
    bank = bank0.clone()
    readings = torch.empty(seq["v"].shape, dtype=bank.dtype, device=DEV)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sdm_decode_steps(bank, **seq, readings=readings)
    sel = torch.from_numpy(checked).to(DEV)
    for i in range(2):
        bank.copy_(bank0)
        readings.view(torch.int16).fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _say(f"  replay {i}")
        for t in range(wl.steps):
            assert bits_equal(to_np_bank(readings[t][sel]), refs[t]), f"replay {i}, token {t}"
        assert bits_equal(to_np_bank(bank[rows]), ref_bank), f"replay {i}: bank differs from the oracle"
    del bank, bank0, graph
    torch.cuda.empty_cache()
