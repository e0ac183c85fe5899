"""The gather plan (sdm_gather_plan_init / sdm_gather_plan_launch through the C
ABI) on the GPU: a launch at (row0, valid) must equal sdm_gather on rows
[row0, row0 + tokens) of the slot and weight arrays with that valid, bit for bit,
and the oracle's gather of the same window.
"""

import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import gen
import oracle
from sparse_delta_rule_amd import SdmError, sdm_gather, sdm_gather_plan
from tests.helpers import bits_equal, to_np_bank

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def _np(t):
    t = t.detach().cpu()
    return t.float().numpy() if t.dtype == torch.bfloat16 else t.numpy()


CASES = [
    # name, bank dtype, slots, hd, index rows, tokens, chunk, width0, width1, idx dtype, w dtype
    ("hd128 bf16 two ops", torch.bfloat16, 20000, 128, 1024, 256, 64, 64, 64, torch.int32, torch.bfloat16),
    ("hd100 f32 one op", torch.float32, 3000, 100, 200, 48, 16, 31, 0, torch.int64, torch.float32),
    ("hd3 bf16 element vectors", torch.bfloat16, 300, 3, 90, 40, 5, 7, 2, torch.int32, torch.float32),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_plan_launches_equal_gathers_of_the_window(case):
    name, dt, slots, hd, rows, T, chunk, W0, W1, idt, wdt = case
    wl = gen.GatherWorkload(name=name, bank_dtype=dt, num_slots=slots, head_dim=hd, tokens=rows, chunk=1,
                            valid_low=1, valid_high=1, width0=W0, width1=W1, idx_dtype=idt, w_dtype=wdt,
                            bank_std=0.5)
    bank = gen.gather_bank(wl, 31).to(DEV)
    inp = {k: v.to(DEV) for k, v in gen.gather_inputs(wl, 31).items()}
    two = W1 > 0
    ops = dict(idx1=inp["idx1"], w1=inp["w1"]) if two else {}
    plan = sdm_gather_plan(bank, inp["idx0"], inp["w0"], tokens=T, chunk=chunk, **ops)
    bank_np = to_np_bank(bank)
    row0_max = rows - T
    for row0, valid in ((0, chunk), (row0_max // 3, chunk // 2), (row0_max, 0), (row0_max, chunk - 1), (7, 1)):
        o0, o1 = plan.launch(row0, valid)
        win = slice(row0, row0 + T)
        wops = dict(idx1=inp["idx1"][win], w1=inp["w1"][win]) if two else {}
        g0, _, g1 = sdm_gather(bank, inp["idx0"][win], inp["w0"][win], chunk=chunk, valid=valid, with_stash=False,
                               **wops)
        torch.cuda.synchronize()
        r0, _, r1 = oracle.gather(bank_np, _np(inp["idx0"][win]), _np(inp["w0"][win]), chunk=chunk, valid=valid,
                                  idx1=_np(inp["idx1"][win]) if two else None,
                                  w1=_np(inp["w1"][win]) if two else None, stash=False)
        assert bits_equal(_np(o0), _np(g0)) and bits_equal(_np(o0), r0), f"operand 0 at row0 {row0}, valid {valid}"
        if two:
            assert bits_equal(_np(o1), _np(g1)) and bits_equal(_np(o1), r1), f"operand 1 at row0 {row0}"


def test_plan_launch_errors():
    wl = gen.WORKLOADS["c3"].replace(num_slots=1000, tokens=128, width1=0)
    bank = gen.gather_bank(wl, 32, DEV)
    inp = gen.gather_inputs(wl, 32, DEV)
    plan = sdm_gather_plan(bank, inp["idx0"], inp["w0"], tokens=64, chunk=16)
    with pytest.raises(SdmError, match="row0 = 65 outside"):
        plan.launch(65, 16)
    with pytest.raises(SdmError, match="valid = 17 outside"):
        plan.launch(0, 17)
    with pytest.raises(ValueError, match="tokens"):
        sdm_gather_plan(bank, inp["idx0"], inp["w0"], tokens=129, chunk=16)
    with pytest.raises(SdmError, match="SDM_E_SHAPE"):
        sdm_gather_plan(bank, inp["idx0"], inp["w0"], tokens=60, chunk=16)


def test_captured_plan_launches_replay_exactly():
    """Two plan launches at different windows captured in one HIP graph, each followed
    by a copy of its outputs: every replay, with eager work in between and the
    buffers cleared first, equals the eager launches."""
    wl = gen.WORKLOADS["c3"].replace(num_slots=50000, tokens=1024)
    bank = gen.gather_bank(wl, 33, DEV)
    inp = gen.gather_inputs(wl, 33, DEV)
    plan = sdm_gather_plan(bank, inp["idx0"], inp["w0"], tokens=256, chunk=64, idx1=inp["idx1"], w1=inp["w1"])
    want = []
    for row0, valid in ((128, 64), (700, 40)):
        o0, o1 = plan.launch(row0, valid)
        want.append((o0.clone(), o1.clone()))
    saved = [torch.empty_like(want[0][0]) for _ in range(4)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for k, (row0, valid) in enumerate(((128, 64), (700, 40))):
            o0, o1 = plan.launch(row0, valid)
            saved[2 * k].copy_(o0)
            saved[2 * k + 1].copy_(o1)
    for i in range(3):
        for t in saved + [plan.out0, plan.out1]:
            t.fill_(7.0)
        junk = torch.randn(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in range(2):
            assert torch.equal(saved[2 * k].view(torch.int32), want[k][0].view(torch.int32)), f"replay {i}, launch {k}"
            assert torch.equal(saved[2 * k + 1].view(torch.int32), want[k][1].view(torch.int32)), f"replay {i}"
        del junk


def test_debug_validation_covers_every_window():
    """SDM_DEBUG_VALIDATE=1 in a child process: a slot out of range in a row only a later
    window uses is reported when the plan is made."""
    code = r'''
import torch, sparse_delta_rule_amd as sdm
dev = torch.device("cuda", 0)
bank = torch.zeros(100, 8, device=dev)
idx = torch.zeros(40, 2, dtype=torch.int32, device=dev)
w = torch.ones(40, 2, device=dev)
try:
    sdm.sdm_gather_plan(bank, idx, w, tokens=8, chunk=4)
    print("ok")
except sdm.SdmError as e:
    print(e)
idx[35, 1] = 100
try:
    sdm.sdm_gather_plan(bank, idx, w, tokens=8, chunk=4)
    print("ok")
except sdm.SdmError as e:
    print(e)
'''
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, SDM_DEBUG_VALIDATE="1")
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120,
                         cwd=root)
    lines = out.stdout.strip().splitlines()
    assert len(lines) == 2, out.stderr
    assert lines[0] == "ok", lines[0]
    assert "idx0[35, 1] = 100 outside [0, 100)" in lines[1]
