"""Parity of the compact-stash gather (sdm_gather_compact through the C ABI)
with the oracle.

The outputs are sdm_gather's (compared bit for bit with the oracle's gather);
the stash is one block of chunk * width0 rows per chunk, into which each live
entry with a position copies its raw row. Stashes start filled with a byte
pattern no copied row has, so rows the kernel must leave alone (unused
positions, negative positions, padding tokens) are checked too. Small slot
ranges make many entries of a chunk share a slot, and so a position.
"""

import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import gen
import oracle
from sparse_delta_rule_amd import SdmError, sdm_gather_compact
from tests.helpers import bits_equal, to_np_bank

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)
PATTERN = 0x7E


def _np(t):
    t = t.detach().cpu()
    return t.float().numpy() if t.dtype == torch.bfloat16 else t.numpy()


def _patterned(shape, dtype, device):
    n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    return torch.full((n,), PATTERN, dtype=torch.uint8, device=device).view(dtype).view(shape)


def run_compact(wl: gen.GatherWorkload, seed: int, *, per_chunk=True, valid=None, drop=0.0, positions_for_all=False):
    """positions_for_all: build the map as if every token were live, so padding tokens carry
    positions the kernel must not use. drop: fraction of entries whose position is set to -1."""
    bank = gen.gather_bank(wl, seed).to(DEV)
    inp = gen.gather_inputs(wl, seed)
    T, chunk = wl.tokens, wl.chunk
    two = wl.width1 > 0
    cv = inp["chunk_valid"] if per_chunk else None
    counts = cv if per_chunk else torch.full((T // chunk,), chunk if valid is None else valid, dtype=torch.int32)
    kpos = gen.compact_positions(inp["idx0"], chunk, torch.full_like(counts, chunk) if positions_for_all else counts)
    if drop > 0:
        g = torch.Generator().manual_seed(seed + 1)
        kpos[torch.rand(kpos.shape, generator=g) < drop] = -1
    shape = (T // chunk, chunk * wl.width0, wl.head_dim)
    stash0 = _patterned(shape, wl.bank_dtype, "cpu")
    d = {k: v.to(DEV) for k, v in inp.items()}
    out0, st, out1 = sdm_gather_compact(bank, d["idx0"], d["w0"], kpos.to(DEV), chunk=chunk, valid=valid,
                                        chunk_valid=None if cv is None else d["chunk_valid"],
                                        idx1=d.get("idx1"), w1=d.get("w1"), stash=stash0.to(DEV))
    torch.cuda.synchronize()
    bank_np = to_np_bank(bank)
    ref0, _, ref1 = oracle.gather(bank_np, _np(inp["idx0"]), _np(inp["w0"]), chunk=chunk, valid=valid,
                                  chunk_valid=None if cv is None else _np(cv),
                                  idx1=_np(inp["idx1"]) if two else None, w1=_np(inp["w1"]) if two else None,
                                  stash=False)
    ref_st = oracle.gather_compact_stash(bank_np, _np(inp["idx0"]), kpos.numpy(), to_np_bank(stash0), chunk=chunk,
                                         valid=valid, chunk_valid=None if cv is None else _np(cv))
    assert bits_equal(_np(out0), ref0), "operand 0 outputs differ"
    if two:
        assert bits_equal(_np(out1), ref1), "operand 1 outputs differ"
    assert bits_equal(to_np_bank(st), ref_st), "compact stash differs"
    return kpos


CASES = [
    # name, bank dtype, slots, hd, tokens, chunk, width0, width1, idx dtype, w dtype
    ("hd128 bf16 two ops, few repeats", torch.bfloat16, 5000, 128, 256, 64, 64, 64, torch.int32, torch.bfloat16),
    ("hd128 bf16 two ops, many repeats", torch.bfloat16, 150, 128, 256, 64, 64, 64, torch.int32, torch.bfloat16),
    ("hd1 f32 one op", torch.float32, 20, 1, 48, 8, 3, 0, torch.int64, torch.float32),
    ("hd3 bf16 element vectors", torch.bfloat16, 30, 3, 40, 5, 7, 2, torch.int32, torch.float32),
    ("hd100 f32 400-B rows", torch.float32, 300, 100, 64, 16, 31, 0, torch.int64, torch.float32),
    ("hd127 bf16 odd", torch.bfloat16, 100, 127, 30, 10, 12, 9, torch.int32, torch.bfloat16),
    ("hd128 bf16 width 255", torch.bfloat16, 400, 128, 16, 4, 255, 33, torch.int64, torch.bfloat16),
    ("hd600 bf16 two slices", torch.bfloat16, 60, 600, 16, 8, 9, 4, torch.int32, torch.float32),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("padding", ["per_chunk", "scalar", "none", "all"])
def test_small_cases(case, padding):
    name, dt, slots, hd, T, chunk, W0, W1, idt, wdt = case
    wl = gen.GatherWorkload(name=name, bank_dtype=dt, num_slots=slots, head_dim=hd, tokens=T, chunk=chunk,
                            valid_low=0, valid_high=chunk, width0=W0, width1=W1, idx_dtype=idt, w_dtype=wdt,
                            bank_std=0.5)
    valid = {"per_chunk": None, "scalar": max(1, chunk // 2), "none": chunk, "all": 0}[padding]
    kpos = run_compact(wl, 21, per_chunk=padding == "per_chunk", valid=valid)
    if padding == "none" and slots < chunk * W0:
        first = kpos[:chunk]
        assert (first >= 0).all() and first.unique().numel() < first.numel(), "the case should repeat slots"


@pytest.mark.parametrize("drop", [0.3, 1.0])
def test_negative_positions_store_nothing(drop):
    wl = gen.WORKLOADS["c3"].replace(num_slots=3000, tokens=512)
    run_compact(wl, 22, drop=drop)


def test_padding_tokens_ignore_their_positions():
    wl = gen.WORKLOADS["c3"].replace(num_slots=3000, tokens=512, valid_low=0, valid_high=48)
    kpos = run_compact(wl, 23, positions_for_all=True)
    assert (kpos >= 0).all()


def test_c3_shape_4096_tokens():
    wl = gen.WORKLOADS["c3"].replace(tokens=4096, num_slots=1 << 20)
    run_compact(wl, 24)


def test_graph_replays_match_eager():
    """sdm_gather_compact captured in a HIP graph: every replay, with eager torch work and
    synchronisations between replays and the outputs and stash refilled first (rows
    no entry names must come back as they were put), equals an eager launch bit for bit."""
    wl = gen.WORKLOADS["c3"].replace(num_slots=2000, tokens=1024)
    bank = gen.gather_bank(wl, 25, DEV)
    inp = gen.gather_inputs(wl, 25, DEV)
    kpos = gen.compact_positions(inp["idx0"], wl.chunk, inp["chunk_valid"])
    kw = dict(chunk=wl.chunk, chunk_valid=inp["chunk_valid"], idx1=inp["idx1"], w1=inp["w1"])
    shape = (wl.tokens // wl.chunk, wl.chunk * wl.width0, wl.head_dim)
    r0, rs, r1 = sdm_gather_compact(bank, inp["idx0"], inp["w0"], kpos, **kw,
                                    stash=_patterned(shape, wl.bank_dtype, DEV))
    out0, out1 = torch.empty_like(r0), torch.empty_like(r1)
    stash = _patterned(shape, wl.bank_dtype, DEV)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sdm_gather_compact(bank, inp["idx0"], inp["w0"], kpos, **kw, out0=out0, out1=out1, stash=stash)
    for i in range(3):
        out0.fill_(7.0)
        out1.fill_(7.0)
        stash.view(torch.uint8).fill_(PATTERN)
        junk = torch.randn(1 << 20, device=DEV).sum()  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out0.view(torch.int32), r0.view(torch.int32)), f"replay {i}"
        assert torch.equal(out1.view(torch.int32), r1.view(torch.int32)), f"replay {i}"
        assert torch.equal(stash.view(torch.int16), rs.view(torch.int16)), f"replay {i}"
        del junk


def test_errors_from_python():
    bank = torch.zeros(10, 4, device=DEV)
    idx = torch.zeros(6, 2, dtype=torch.int32, device=DEV)
    w = torch.zeros(6, 2, device=DEV)
    kp = torch.zeros(6, 2, dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError, match="kpos must be int32"):
        sdm_gather_compact(bank, idx, w, kp.long(), chunk=3)
    with pytest.raises(ValueError, match="stash must be"):
        sdm_gather_compact(bank, idx, w, kp, chunk=3, stash=torch.zeros(6, 2, 4, device=DEV))
    with pytest.raises(SdmError, match="SDM_E_OVERLAP"):
        sdm_gather_compact(bank, idx, w, kp, chunk=3, out0=bank.view(-1)[:24].view(6, 4))
    o, s, _ = sdm_gather_compact(bank, idx[:0], w[:0], kp[:0], chunk=3)
    assert o.shape == (0, 4) and s.shape == (0, 6, 4)


def test_debug_validation_of_positions():
    """SDM_DEBUG_VALIDATE=1 in a child process: a position past the block and a
    position two slots share are reported; a padding token's conflict is not."""
    code = r'''
import torch, sparse_delta_rule_amd as sdm
dev = torch.device("cuda", 0)
bank = torch.zeros(64, 8, device=dev)
idx = torch.tensor([[0, 1], [2, 3], [4, 5], [6, 7]], dtype=torch.int32, device=dev)
w = torch.ones(4, 2, device=dev)
cv = torch.tensor([2, 1], dtype=torch.int32, device=dev)
def call(kp):
    try:
        sdm.sdm_gather_compact(bank, idx, w, torch.tensor(kp, dtype=torch.int32, device=dev), chunk=2, chunk_valid=cv)
        torch.cuda.synchronize()
        return "ok"
    except sdm.SdmError as e:
        return str(e)
print(call([[0, 1], [2, 3], [0, 1], [0, 0]]))
print(call([[0, 1], [2, 4], [0, 1], [0, 0]]))
print(call([[0, 1], [1, 3], [0, 1], [0, 0]]))
'''
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, SDM_DEBUG_VALIDATE="1")
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120,
                         cwd=root)
    lines = out.stdout.strip().splitlines()
    assert len(lines) == 3, out.stderr
    assert lines[0] == "ok", lines[0]
    assert "kpos[1, 1] = 4 outside [-1, 4)" in lines[1]
    assert "chunk 0: position 1 is named by slots 1 and 2" in lines[2]
