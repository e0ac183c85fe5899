"""Parity with the oracle on non-finite values: NaN and infinity in the bank, in
the values and weights, and results that overflow the bank dtype on store.

Sums are compared position by position: the same elements are NaN on both sides
and every other element (infinities and signed zeros included) is equal bit for
bit. Which NaN an operation on NaNs returns is not fixed by IEEE 754, so NaN
payloads of computed values are not compared; the stash is a raw copy and is
compared bit for bit, NaN payloads included.
"""

import numpy as np
import pytest
import torch

import gen
import oracle
from sparse_delta_rule_amd import sdm_decode_step, sdm_gather
from tests.helpers import documented_decode_groups, step_to_numpy, to_np_bank, widen

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def same_values(got: np.ndarray, ref: np.ndarray) -> bool:
    """Equal NaN positions, and equal bits everywhere else."""
    assert got.dtype == ref.dtype and got.shape == ref.shape
    gf, rf = widen(got), widen(ref)
    nan_g, nan_r = np.isnan(gf), np.isnan(rf)
    if not np.array_equal(nan_g, nan_r):
        return False
    bits = np.uint16 if got.dtype == np.uint16 else np.uint32
    return np.array_equal(got.view(bits)[~nan_g], ref.view(bits)[~nan_r])


def _poison(bank_np: np.ndarray, rows, vals):
    """Set whole bank rows to special values (float32 values, or their bfloat16 bits)."""
    out = bank_np.copy()
    for r, x in zip(rows, vals):
        if out.dtype == np.uint16:
            out[r] = np.array([x], np.float32).view(np.uint32)[0] >> 16
        else:
            out[r] = x
    return out


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_decode_with_nan_and_inf(dt):
    wl = gen.WORKLOADS["c1"].replace(streams=24, slots_per_stream=96, head_dim=64, W=16, R=16, G=16, steps=1,
                                     bank_dtype=dt)
    bank_np = to_np_bank(gen.decode_bank(wl, 51))
    inp = gen.decode_step_inputs(wl, 51, 0)
    k = inp["k_idx"].numpy()
    # stream 0: a written row holds NaN; stream 1: a written row holds +inf; stream 2: a
    # read-only row holds -inf; stream 3: a row no slot of this step names holds NaN
    untouched = next(r for r in range(3 * 96, 4 * 96) if r not in set(k[3]) | set(inp["q_idx"].numpy()[3]))
    bank_np = _poison(bank_np, [k[0, 3], k[1, 0], inp["q_idx"].numpy()[2, 5], untouched],
                      [np.nan, np.inf, -np.inf, np.nan])
    v = inp["v"].clone()
    v[4, 7] = float("nan")      # stream 4: delta_v of one column is NaN
    v[5, 0] = float("inf")      # stream 5: delta_v of one column is infinite
    v[6] = 3.0e38               # stream 6: large values; new rows overflow the bank dtype
    inp["v"] = v
    kv = inp["k_val"].clone()
    kv[6] = 1.0e30              # stream 6, with v = 3e38: k_val * delta_v overflows
    kv[7, 2] = float("-inf")    # stream 7: an infinite write weight
    inp["k_val"] = kv
    qv = inp["q_val"].clone()
    qv[8, 1] = float("nan")     # stream 8: a NaN read weight
    inp["q_val"] = qv
    npin = step_to_numpy(inp)
    ref_bank = bank_np.copy()
    ref = oracle.decode_step(ref_bank, **npin, groups=documented_decode_groups(wl.W, wl.R))
    bank = torch.from_numpy(bank_np.view(np.int16) if dt == torch.bfloat16 else bank_np)
    bank = (bank.view(torch.bfloat16) if dt == torch.bfloat16 else bank).to(DEV)
    readings = sdm_decode_step(bank, **{k_: x.to(DEV) for k_, x in inp.items()})
    torch.cuda.synchronize()
    got_bank, got = to_np_bank(bank), to_np_bank(readings)
    assert np.isnan(widen(ref)).any() and np.isinf(widen(ref_bank)).any()  # the cases bite
    assert same_values(got, ref), "readings differ from the oracle"
    assert same_values(got_bank, ref_bank), "bank differs from the oracle"
    assert np.isfinite(widen(got[3])).all(), "a row no slot names reached stream 3's readings"


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_gather_with_nan_and_inf(dt):
    wl = gen.WORKLOADS["c3"].replace(num_slots=4000, tokens=96, chunk=32, width0=24, width1=16, valid_low=10,
                                     valid_high=32, bank_dtype=dt)
    bank_np = to_np_bank(gen.gather_bank(wl, 52))
    inp = gen.gather_inputs(wl, 52)
    cv = inp["chunk_valid"].numpy()
    live = np.arange(wl.tokens) % wl.chunk < cv[np.arange(wl.tokens) // wl.chunk]
    pad_t = int(np.flatnonzero(~live)[0])
    live_t = np.flatnonzero(live)
    idx0, idx1 = inp["idx0"].numpy().copy(), inp["idx1"].numpy().copy()
    nan_row, inf_row, ninf_row = 1, 2, 3
    idx0[live_t[0], 4] = nan_row          # a live token sums a NaN row (and stashes its bits)
    idx0[live_t[1], 0] = inf_row          # +inf row
    idx1[live_t[1], 3] = ninf_row         # -inf in the other operand
    idx0[pad_t, :] = nan_row              # a padding token pointing at NaN rows reads none
    idx1[pad_t, :] = nan_row
    bank_np = _poison(bank_np, [nan_row, inf_row, ninf_row], [np.nan, np.inf, -np.inf])
    if dt == torch.float32:  # a NaN with a payload, to check the stash copies bits
        bank_np[nan_row, 0] = np.array([0x7fc01234], np.uint32).view(np.float32)[0]
    else:
        bank_np[nan_row, 0] = 0x7fd3
    w0 = inp["w0"].clone()
    w0[live_t[2], 5] = float("inf")       # an infinite weight
    w0[live_t[3], 6] = float("nan")       # a NaN weight
    inp["idx0"], inp["idx1"], inp["w0"] = torch.from_numpy(idx0), torch.from_numpy(idx1), w0
    bank = torch.from_numpy(bank_np.view(np.int16) if dt == torch.bfloat16 else bank_np)
    bank = (bank.view(torch.bfloat16) if dt == torch.bfloat16 else bank).to(DEV)
    out0, st, out1 = sdm_gather(bank, inp["idx0"].to(DEV), inp["w0"].to(DEV), chunk=wl.chunk,
                                chunk_valid=inp["chunk_valid"].to(DEV), idx1=inp["idx1"].to(DEV),
                                w1=inp["w1"].to(DEV))
    torch.cuda.synchronize()
    ref0, ref_st, ref1 = oracle.gather(bank_np, idx0, inp["w0"].float().numpy(), chunk=wl.chunk, chunk_valid=cv,
                                       idx1=idx1, w1=inp["w1"].float().numpy())
    assert np.isnan(ref0).any() and np.isinf(ref0).any()
    assert same_values(out0.cpu().numpy(), ref0) and same_values(out1.cpu().numpy(), ref1)
    st_np = to_np_bank(st)
    bits = np.uint16 if st_np.dtype == np.uint16 else np.uint32
    assert np.array_equal(st_np.view(bits), ref_st.view(bits)), "stash bits differ"
    assert not out0.cpu().numpy()[pad_t].view(np.uint32).any(), "padding output not +0"
