"""Parity of the HIP token gather (sdm_gather through the C ABI) with the oracle.

The kernel sums each output in plain ascending order (include/sdm.h), the
oracle's groups = 1 order, so outputs are compared bit for bit, and so are the
stash rows (raw copies) and the padding zeros.
"""

import numpy as np
import pytest
import torch

import gen
import oracle
from sparse_delta_rule_amd import SdmError, sdm_gather
from tests.helpers import bits_equal, to_np_bank

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def _say(*a):
    print(*a, flush=True)


def _np(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.float().numpy()
    return t.numpy()


def run_case(wl: gen.GatherWorkload, seed: int, *, per_chunk: bool, valid=None, stash=True):
    bank = gen.gather_bank(wl, seed).to(DEV)
    inp = {k: v.to(DEV) for k, v in gen.gather_inputs(wl, seed).items()}
    two = wl.width1 > 0
    cv = inp["chunk_valid"] if per_chunk else None
    out0, st, out1 = sdm_gather(bank, inp["idx0"], inp["w0"], chunk=wl.chunk, valid=valid, chunk_valid=cv,
                                idx1=inp.get("idx1"), w1=inp.get("w1"), with_stash=stash)
    torch.cuda.synchronize()
    ref0, ref_st, ref1 = oracle.gather(
        to_np_bank(bank), _np(inp["idx0"]), _np(inp["w0"]), chunk=wl.chunk, valid=valid,
        chunk_valid=None if cv is None else _np(cv), idx1=_np(inp["idx1"]) if two else None,
        w1=_np(inp["w1"]) if two else None, stash=stash)
    assert bits_equal(_np(out0), ref0), "operand 0 outputs differ"
    if two:
        assert bits_equal(_np(out1), ref1), "operand 1 outputs differ"
    if stash:
        assert bits_equal(to_np_bank(st), ref_st), "stash differs"
    else:
        assert st is None


CASES = [
    # name, bank dtype, slots, hd, tokens, chunk, width0, width1, idx dtype, w dtype
    ("hd128 bf16 two ops (c3 shape, small)", torch.bfloat16, 5000, 128, 256, 64, 64, 64, torch.int32, torch.bfloat16),
    ("hd1 f32 one op", torch.float32, 100, 1, 48, 8, 3, 0, torch.int64, torch.float32),
    ("hd3 bf16 element vectors", torch.bfloat16, 300, 3, 40, 5, 7, 2, torch.int32, torch.float32),
    ("hd8 f32 w=1", torch.float32, 64, 8, 32, 32, 1, 1, torch.int64, torch.bfloat16),
    ("hd64 f32 widths 256/5", torch.float32, 2000, 64, 24, 4, 256, 5, torch.int32, torch.float32),
    ("hd100 bf16 200-B rows", torch.bfloat16, 3000, 100, 60, 6, 17, 33, torch.int64, torch.bfloat16),
    ("hd100 f32 400-B rows", torch.float32, 3000, 100, 64, 16, 31, 0, torch.int32, torch.float32),
    ("hd127 bf16 odd", torch.bfloat16, 1000, 127, 30, 10, 12, 9, torch.int32, torch.bfloat16),
    ("hd129 f32 odd", torch.float32, 1000, 129, 30, 3, 10, 0, torch.int64, torch.float32),
    ("hd256 bf16 32 lanes", torch.bfloat16, 1000, 256, 40, 20, 20, 256, torch.int32, torch.bfloat16),
    ("hd600 bf16 two slices", torch.bfloat16, 500, 600, 16, 8, 9, 4, torch.int32, torch.float32),
    ("hd1000 f32 four slices", torch.float32, 200, 1000, 8, 4, 5, 3, torch.int64, torch.float32),
    ("hd128 bf16 widths 255/97", torch.bfloat16, 4000, 128, 40, 8, 255, 97, torch.int32, torch.bfloat16),
    # rows of 9 to 16 vectors (16-lane groups) with lanes past the row, narrow widths
    ("hd120 bf16 15 vectors", torch.bfloat16, 3000, 120, 96, 16, 40, 23, torch.int32, torch.bfloat16),
    ("hd40 f32 10 vectors", torch.float32, 2000, 40, 64, 8, 9, 16, torch.int64, torch.float32),
    ("hd9 bf16 2-B vectors", torch.bfloat16, 500, 9, 64, 16, 7, 8, torch.int32, torch.float32),
    ("hd30 bf16 4-B vectors", torch.bfloat16, 700, 30, 48, 12, 11, 5, torch.int64, torch.bfloat16),
    ("hd36 bf16 8-B vectors", torch.bfloat16, 900, 36, 80, 20, 16, 24, torch.int32, torch.bfloat16),
    ("hd18 f32 8-B vectors", torch.float32, 600, 18, 36, 9, 8, 0, torch.int32, torch.float32),
    ("hd128 bf16 widths 3/1", torch.bfloat16, 2000, 128, 70, 7, 3, 1, torch.int64, torch.bfloat16),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("padding", ["per_chunk", "scalar", "none", "all"])
@pytest.mark.parametrize("stash", [True, False], ids=["stash", "no-stash"])
def test_small_cases(case, padding, stash):
    name, dt, slots, hd, T, chunk, W0, W1, idt, wdt = case
    wl = gen.GatherWorkload(name=name, bank_dtype=dt, num_slots=slots, head_dim=hd, tokens=T, chunk=chunk,
                            valid_low=0, valid_high=chunk, width0=W0, width1=W1, idx_dtype=idt, w_dtype=wdt,
                            bank_std=0.5)
    valid = {"per_chunk": None, "scalar": max(1, chunk // 2), "none": chunk, "all": 0}[padding]
    run_case(wl, 11, per_chunk=padding == "per_chunk", valid=valid, stash=stash)


@pytest.mark.parametrize("stash", [True, False])
def test_without_stash(stash):
    wl = gen.WORKLOADS["c3"].replace(num_slots=20000, tokens=512)
    run_case(wl, 12, per_chunk=True, stash=stash)


def test_misaligned_views_take_narrow_vectors():
    """Outputs and bank views offset by one element: still exact (narrower vectors)."""
    wl = gen.WORKLOADS["c3"].replace(num_slots=4000, tokens=64, chunk=16, valid_low=4, valid_high=16)
    bank_full = gen.gather_bank(wl.replace(num_slots=4001), 13).to(DEV)
    bank = bank_full.view(-1)[1:1 + 4000 * 128].view(4000, 128)  # 2 bytes past 16-B alignment
    inp = {k: v.to(DEV) for k, v in gen.gather_inputs(wl, 13).items()}
    out_buf = torch.empty(64 * 128 + 1, device=DEV)
    out0 = out_buf[1:].view(64, 128)
    o0, st, o1 = sdm_gather(bank, inp["idx0"], inp["w0"], chunk=16, chunk_valid=inp["chunk_valid"][:4],
                            idx1=inp["idx1"], w1=inp["w1"], out0=out0)
    ref0, ref_st, ref1 = oracle.gather(to_np_bank(bank.contiguous()), _np(inp["idx0"]), _np(inp["w0"]), chunk=16,
                                       chunk_valid=_np(inp["chunk_valid"][:4]), idx1=_np(inp["idx1"]),
                                       w1=_np(inp["w1"]))
    assert bits_equal(_np(o0), ref0) and bits_equal(_np(o1), ref1) and bits_equal(to_np_bank(st), ref_st)


@pytest.mark.parametrize("with_stash", [True, False], ids=["stash", "no-stash"])
def test_misaligned_outputs_take_element_stores(with_stash):
    """Outputs one float past 16-byte alignment on an aligned bank (the pair layout
    without a stash): the outputs are stored element by element, the bits unchanged."""
    wl = gen.WORKLOADS["c3"].replace(num_slots=4000, tokens=128, chunk=16, valid_low=3, valid_high=16)
    bank = gen.gather_bank(wl, 14).to(DEV)
    inp = {k: v.to(DEV) for k, v in gen.gather_inputs(wl, 14).items()}
    buf0 = torch.full((128 * 128 + 1,), float("nan"), device=DEV)
    buf1 = torch.full((128 * 128 + 1,), float("nan"), device=DEV)
    out0, out1 = buf0[1:].view(128, 128), buf1[1:].view(128, 128)
    o0, st, o1 = sdm_gather(bank, inp["idx0"], inp["w0"], chunk=16, chunk_valid=inp["chunk_valid"],
                            idx1=inp["idx1"], w1=inp["w1"], out0=out0, out1=out1, with_stash=with_stash)
    torch.cuda.synchronize()
    ref0, ref_st, ref1 = oracle.gather(to_np_bank(bank), _np(inp["idx0"]), _np(inp["w0"]), chunk=16,
                                       chunk_valid=_np(inp["chunk_valid"]), idx1=_np(inp["idx1"]),
                                       w1=_np(inp["w1"]), stash=with_stash)
    assert bits_equal(_np(o0), ref0) and bits_equal(_np(o1), ref1)
    assert torch.isnan(buf0[0]) and torch.isnan(buf1[0])  # nothing written before the views
    if with_stash:
        assert bits_equal(to_np_bank(st), ref_st)


def test_errors_from_python():
    bank = torch.zeros(10, 4, device=DEV)
    idx = torch.zeros(6, 2, dtype=torch.int32, device=DEV)
    w = torch.zeros(6, 2, device=DEV)
    with pytest.raises(SdmError, match="SDM_E_SHAPE"):
        sdm_gather(bank, idx, w, chunk=4)
    with pytest.raises(SdmError, match="SDM_E_OVERLAP"):
        sdm_gather(bank, idx, w, chunk=3, out0=bank.view(-1)[:24].view(6, 4), with_stash=False)
    e = torch.zeros(0, 2, dtype=torch.int32, device=DEV)
    o, s, _ = sdm_gather(bank, e, torch.zeros(0, 2, device=DEV), chunk=4)
    assert o.shape == (0, 4) and s.shape == (0, 2, 4)


def check_c3(wl, bank, inp, out0, stash, out1):
    """c3's outputs: sampled tokens against the oracle bit for bit; every padding token
    zero and every live stash row equal to its bank row (stash None: no stash; out1
    None: operand 0 only)."""
    T = wl.tokens
    two = out1 is not None
    t = torch.arange(T, device=DEV)
    live = (t % wl.chunk) < inp["chunk_valid"].long()[t // wl.chunk]
    _say(f"  live tokens {int(live.sum())} of {T}")
    # padding: zero bits everywhere
    assert not out0[~live].view(torch.int32).any()
    if two:
        assert not out1[~live].view(torch.int32).any()
    if stash is not None:
        assert not stash[~live].view(torch.int16).any()
        # stash: raw rows of operand 0 for every live token (checked in slices)
        lt = t[live]
        for i in range(0, lt.numel(), 2048):
            sel = lt[i:i + 2048]
            rows = bank[inp["idx0"][sel].long()]
            assert torch.equal(stash[sel].view(torch.int16), rows.view(torch.int16))
    # sampled tokens against the oracle (bank rows they touch, renumbered)
    g = torch.Generator().manual_seed(1)
    sample = torch.cat([torch.randperm(T, generator=g)[:1024], torch.arange(0, 128)]).unique().to(DEV)
    idx0 = inp["idx0"][sample].long()
    idx1 = inp["idx1"][sample].long() if two else idx0[:, :0]
    uniq, inv = torch.unique(torch.cat([idx0.ravel(), idx1.ravel()]), return_inverse=True)
    sub_bank = to_np_bank(bank[uniq])
    n0 = idx0.numel()
    i0 = inv[:n0].view_as(idx0).cpu().numpy()
    i1 = inv[n0:].view_as(idx1).cpu().numpy()
    live_s = live[sample].cpu().numpy().astype(np.int32)
    # one-token chunks whose valid count is the token's liveness reproduce the padding rule
    ref0, ref_st, ref1 = oracle.gather(sub_bank, i0, _np(inp["w0"][sample]), chunk=1, chunk_valid=live_s,
                                       idx1=i1 if two else None, w1=_np(inp["w1"][sample]) if two else None,
                                       stash=stash is not None)
    assert bits_equal(_np(out0[sample]), ref0)
    if two:
        assert bits_equal(_np(out1[sample]), ref1)
    if stash is not None:
        assert bits_equal(to_np_bank(stash[sample]), ref_st)


@pytest.mark.slow
def test_full_size_c3():
    """Config c3 at full size, one eager launch."""
    wl = gen.WORKLOADS["c3"]
    _say("c3:", wl.name)
    bank = gen.gather_bank(wl, 0, DEV)
    inp = gen.gather_inputs(wl, 0, DEV)
    out0, stash, out1 = sdm_gather(bank, inp["idx0"], inp["w0"], chunk=wl.chunk, chunk_valid=inp["chunk_valid"],
                                   idx1=inp["idx1"], w1=inp["w1"])
    torch.cuda.synchronize()
    check_c3(wl, bank, inp, out0, stash, out1)
    del bank, stash
    torch.cuda.empty_cache()


@pytest.mark.slow
@pytest.mark.parametrize("two", [True, False], ids=["two-ops", "one-op"])
def test_full_size_c3_without_stash(two):
    """Config c3's tokens at full size with no stash, both operands or operand 0
    only, one eager launch (the launch shapes that take the pair layout)."""
    wl = gen.WORKLOADS["c3"]
    bank = gen.gather_bank(wl, 0, DEV)
    inp = gen.gather_inputs(wl, 0, DEV)
    kw = dict(idx1=inp["idx1"], w1=inp["w1"]) if two else {}
    out0, stash, out1 = sdm_gather(bank, inp["idx0"], inp["w0"], chunk=wl.chunk, chunk_valid=inp["chunk_valid"],
                                   with_stash=False, **kw)
    torch.cuda.synchronize()
    assert stash is None and (out1 is not None) == two
    check_c3(wl, bank, inp, out0, None, out1)
    del bank
    torch.cuda.empty_cache()


@pytest.mark.slow
def test_full_size_c3_graph_replays():
    """Config c3 at full size in the benchmark's launch path: the launch captured in a
    HIP graph, outputs cleared between replays, every replay checked."""
    wl = gen.WORKLOADS["c3"]
    bank = gen.gather_bank(wl, 0, DEV)
    inp = gen.gather_inputs(wl, 0, DEV)
    out0 = torch.empty((wl.tokens, wl.head_dim), dtype=torch.float32, device=DEV)
    out1 = torch.empty_like(out0)
    stash = torch.empty((wl.tokens, wl.width0, wl.head_dim), dtype=bank.dtype, device=DEV)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sdm_gather(bank, inp["idx0"], inp["w0"], chunk=wl.chunk, chunk_valid=inp["chunk_valid"], idx1=inp["idx1"],
                   w1=inp["w1"], out0=out0, stash=stash, out1=out1)
    for i in range(2):
        out0.fill_(float("nan"))
        out1.fill_(float("nan"))
        stash.view(torch.int16).fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _say(f"  replay {i}")
        check_c3(wl, bank, inp, out0, stash, out1)
    del bank, stash, graph
    torch.cuda.empty_cache()


@pytest.mark.parametrize("with_stash", [True, False], ids=["stash", "no-stash"])
def test_graph_replays_match_eager(with_stash):
    """The benchmark's launch path: sdm_gather captured in a HIP graph. Every replay, with
    eager torch work and synchronisations between replays and the outputs cleared
    first, must equal an eager launch bit for bit."""
    wl = gen.WORKLOADS["c3"].replace(num_slots=50000, tokens=1024)
    bank = gen.gather_bank(wl, 21, DEV)
    inp = gen.gather_inputs(wl, 21, DEV)
    kw = dict(chunk=wl.chunk, chunk_valid=inp["chunk_valid"], idx1=inp["idx1"], w1=inp["w1"])
    r0, rs, r1 = sdm_gather(bank, inp["idx0"], inp["w0"], **kw, with_stash=with_stash)
    out0, out1 = torch.empty_like(r0), torch.empty_like(r1)
    stash = torch.empty_like(rs) if with_stash else None
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sdm_gather(bank, inp["idx0"], inp["w0"], **kw, out0=out0, out1=out1, stash=stash, with_stash=with_stash)
    for i in range(3):
        out0.fill_(7.0)
        out1.fill_(7.0)
        if with_stash:
            stash.fill_(7.0)
        junk = torch.randn(1 << 20, device=DEV).sum()  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out0.view(torch.int32), r0.view(torch.int32)), f"replay {i}"
        assert torch.equal(out1.view(torch.int32), r1.view(torch.int32)), f"replay {i}"
        if with_stash:
            assert torch.equal(stash.view(torch.int16), rs.view(torch.int16)), f"replay {i}"
        del junk


def test_debug_validation_catches_broken_preconditions():
    """SDM_DEBUG_VALIDATE=1 in a child process: a slot outside the bank and a per-chunk
    valid count above the chunk are reported before any launch."""
    import os
    import subprocess
    import sys
    code = r'''
import torch, sparse_delta_rule_amd as sdm
dev = torch.device("cuda", 0)
bank = torch.zeros(100, 8, device=dev)
def call(idx, cv):
    idx = torch.tensor(idx, dtype=torch.int32, device=dev)
    cv = torch.tensor(cv, dtype=torch.int32, device=dev)
    try:
        sdm.sdm_gather(bank, idx, torch.ones(idx.shape, device=dev), chunk=2, chunk_valid=cv)
        torch.cuda.synchronize()
        return "ok"
    except sdm.SdmError as e:
        return str(e)
print(call([[1, 2], [3, 4]], [2]))
print(call([[1, 2], [3, 100]], [2]))
print(call([[1, 2], [3, 4]], [3]))
print(call([[1, 2], [-1, 100]], [1]))  # token 1 is padding: its slots are never read
def call2(idx1, cv):
    idx = torch.tensor([[1, 2], [3, 4], [5, 6], [7, 8]], dtype=torch.int32, device=dev)
    idx1 = torch.tensor(idx1, dtype=torch.int32, device=dev)
    cv = torch.tensor(cv, dtype=torch.int32, device=dev)
    try:
        sdm.sdm_gather(bank, idx, torch.ones(idx.shape, device=dev), chunk=2, chunk_valid=cv, idx1=idx1,
                       w1=torch.ones(idx1.shape, device=dev))
        torch.cuda.synchronize()
        return "ok"
    except sdm.SdmError as e:
        return str(e)
print(call2([[1], [-5], [9], [9]], [1, 2]))
print(call2([[1], [2], [9], [-5]], [1, 2]))
'''
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, SDM_DEBUG_VALIDATE="1")
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120, cwd=root)
    lines = out.stdout.strip().splitlines()
    assert lines[0] == "ok", out.stderr
    assert "outside [0, 100)" in lines[1]
    assert "chunk_valid[0] = 3 outside [0, 2]" in lines[2]
    assert lines[3] == "ok", lines[3]
    assert lines[4] == "ok", lines[4]  # operand 1's padding follows chunk_valid too
    assert "idx1[3, 0] = -5 outside [0, 100)" in lines[5]


@pytest.mark.parametrize("per_chunk", [True, False])
@pytest.mark.parametrize("idt", [torch.int32, torch.int64])
@pytest.mark.parametrize("with_stash", [True, False], ids=["stash", "no-stash"])
def test_padding_slots_are_never_read(per_chunk, idt, with_stash):
    """Slots of padding tokens set to -1 or far past the bank: the kernel reads no row
    for them (padding outputs are zeros, stash rows zero), so every result equals
    the oracle's on the same arrays, bit for bit."""
    wl = gen.GatherWorkload(name="padding junk", bank_dtype=torch.bfloat16, num_slots=3000, head_dim=128,
                            tokens=256, chunk=32, valid_low=0, valid_high=32, width0=40, width1=24, idx_dtype=idt,
                            w_dtype=torch.bfloat16, bank_std=0.5)
    bank = gen.gather_bank(wl, 61).to(DEV)
    inp = {k: v.to(DEV) for k, v in gen.gather_inputs(wl, 61).items()}
    valid = None if per_chunk else 9
    limit = inp["chunk_valid"].repeat_interleave(wl.chunk) if per_chunk else torch.full((wl.tokens,), 9, device=DEV)
    pad = torch.arange(wl.tokens, device=DEV) % wl.chunk >= limit
    assert 0 < int(pad.sum()) < wl.tokens
    far = torch.iinfo(idt).max
    for name in ("idx0", "idx1"):
        junk = torch.where(torch.arange(inp[name].shape[1], device=DEV) % 2 == 0, -1, far).to(idt)
        inp[name][pad] = junk
    cv = inp["chunk_valid"] if per_chunk else None
    out0, st, out1 = sdm_gather(bank, inp["idx0"], inp["w0"], chunk=wl.chunk, valid=valid, chunk_valid=cv,
                                idx1=inp["idx1"], w1=inp["w1"], with_stash=with_stash)
    torch.cuda.synchronize()
    ref0, ref_st, ref1 = oracle.gather(
        to_np_bank(bank), _np(inp["idx0"]), _np(inp["w0"]), chunk=wl.chunk, valid=valid,
        chunk_valid=None if cv is None else _np(cv), idx1=_np(inp["idx1"]), w1=_np(inp["w1"]), stash=with_stash)
    assert bits_equal(_np(out0), ref0) and bits_equal(_np(out1), ref1)
    assert not _np(out0)[pad.cpu().numpy()].any()
    if with_stash:
        assert bits_equal(to_np_bank(st), ref_st)
        assert not to_np_bank(st)[pad.cpu().numpy()].any()
