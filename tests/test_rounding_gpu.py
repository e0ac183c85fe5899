"""Rounding to a bfloat16 bank at exact ties, on the GPU against the oracle.

Random inputs almost never land exactly halfway between two bfloat16 values,
so these inputs are built to: bank rows and v on the bfloat16 grid in [1, 2),
k_val = 1, g = 0 (decay 1) and beta = 1/2 make every written value
row + (v - row) / 2, an exact tie whenever the two mantissas differ by an odd
count (about half of all elements). The value read back is q_val times a
written row, a product that ties for some mantissa pairs, and q_val arrives in
float32 with low halves 0x8000 (a tie), 0x7fff, 0x8001 and 0xffff, so its
rounding to the bank dtype on the way in sees ties as well. The rounding is
the one the pages fix for the bank (round to nearest, ties to even); the
oracle implements it bit by bit, and the comparison is bit for bit.

Five worked float32 cases sit on ties of the other rounding points (the
summation order, coef = k_val * d rounded first, delta_v's two roundings, the
fused update): the kernel must reproduce the oracle there as well.
"""

import numpy as np
import pytest
import torch

import oracle
from sparse_delta_rule_amd import sdm_decode_step, sdm_decode_steps
from tests.helpers import bits_equal, step_to_numpy, to_np_bank

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)
S, P, HD = 512, 4, 64


def _grid(gen, shape):
    """bfloat16-exact values 1 + m / 128, m in 0..127."""
    return 1.0 + torch.randint(0, 128, shape, generator=gen).float() / 128.0


def _inputs(gen, read_written: bool):
    k_idx = (torch.arange(S, dtype=torch.int64) * P).view(S, 1)
    q_idx = k_idx if read_written else k_idx + 1 + torch.randint(0, P - 1, (S, 1), generator=gen)
    hi = (_grid(gen, (S, 1)).view(torch.int32) >> 16) << 16
    lo = torch.tensor([0x0000, 0x8000, 0x7FFF, 0x8001, 0xFFFF], dtype=torch.int32)
    q_val = (hi | lo[torch.randint(0, 5, (S, 1), generator=gen)]).view(torch.float32)
    return {"k_idx": k_idx, "k_val": torch.ones(S, 1), "v": _grid(gen, (S, HD)), "beta": torch.full((S, 1), 0.5),
            "g": torch.zeros(S, 1), "q_idx": q_idx, "q_val": q_val}


def _ties_in_writes(bank_rows: np.ndarray, v: np.ndarray) -> int:
    """Written values row + (v - row) / 2 that lie exactly halfway between bfloat16 values."""
    row = (bank_rows.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    val = (row + (v.astype(np.float64) - row) / 2).astype(np.float32)  # exact: 9 significant bits
    return int(np.count_nonzero((val.view(np.uint32) & 0xFFFF) == 0x8000))


@pytest.fixture(params=["auto", "compact", "wide"])
def loop(request, monkeypatch):
    if request.param == "auto":
        monkeypatch.delenv("SDM_STEPS_LOOP", raising=False)
    else:
        monkeypatch.setenv("SDM_STEPS_LOOP", request.param)
    return request.param


@pytest.mark.parametrize("read_written", [True, False], ids=["read-written", "read-other"])
def test_single_step_ties(read_written):
    gen = torch.Generator().manual_seed(17)
    bank = _grid(gen, (S * P, HD)).to(torch.bfloat16)
    ref_bank = to_np_bank(bank)
    inp = _inputs(gen, read_written)
    npin = step_to_numpy(inp)
    ties = _ties_in_writes(ref_bank[npin["k_idx"].ravel()], npin["v"])
    assert ties > 0.3 * S * HD, f"only {ties} ties among the written values"
    bank = bank.to(DEV)
    readings = sdm_decode_step(bank, **{k: t.to(DEV) for k, t in inp.items()})
    ref = oracle.decode_step(ref_bank, **npin, groups=1)
    assert bits_equal(to_np_bank(readings), ref), "readings differ from the oracle"
    assert bits_equal(to_np_bank(bank), ref_bank), "bank differs from the oracle"


def test_multi_step_ties(loop):
    gen = torch.Generator().manual_seed(23)
    T = 4
    bank = _grid(gen, (S * P, HD)).to(torch.bfloat16)
    ref_bank = to_np_bank(bank)
    per = [_inputs(gen, t % 2 == 0) for t in range(T)]
    seq = {k: torch.stack([p[k] for p in per]) for k in per[0]}
    bank = bank.to(DEV)
    readings = sdm_decode_steps(bank, **{k: t.to(DEV) for k, t in seq.items()})
    for t in range(T):
        ref = oracle.decode_step(ref_bank, **step_to_numpy(per[t]), groups=1)
        assert bits_equal(to_np_bank(readings[t]), ref), f"token {t}: readings differ from the oracle"
    assert bits_equal(to_np_bank(bank), ref_bank), "bank differs from the oracle"


# Worked float32 cases on rounding ties (each settles one rounding point the pages
# leave open: summation order, coef = k_val * d rounded first, delta_v's two
# roundings, the fused update); hd 1, one stream. Fields: bank rows, k_idx,
# k_val, g, beta, v, q_idx, q_val, expected bank rows after the step.
_BIG = 2.0 ** 24
WORKED = {
    "ascending chain": ([_BIG, 1, 1, _BIG, 1, 1], [0, 1, 2], [1, 1, 1], 0.0, 1.0, 0.0, [3, 4, 5], [1, 1, 1],
                        [0.0, -16777215.0, -16777215.0, _BIG, 1, 1]),
    "cancelling chain": ([_BIG, 1, -_BIG, 1], [0, 1, 2, 3], [1, 1, 1, 1], 0.0, 1.0, 0.0, [0], [1],
                         [16777215.0, 0.0, -16777216.0, 0.0]),
    "fused update": ([-1.0], [0], [1 + 2.0 ** -12], 0.0, 1.0, 0.0, [0], [1], [2.0 ** -11 + 2.0 ** -24]),
    "delta roundings": ([-(2.0 ** -24), 0.0], [0, 1], [1, 1], 0.0, 1 + 2.0 ** -23, 1.0, [1], [1],
                        [1.0, 1 + 2.0 ** -23]),
    "coef rounded first": ([-(1 + 2.0 ** -23), 0.0], [0, 1], [1 + 2.0 ** -12, 1], 2.0 ** -12, 1.0, 0.0, [1], [1],
                           [None, 1 + 2.0 ** -11 + 2.0 ** -23]),
}


@pytest.mark.parametrize("name", list(WORKED))
def test_worked_float32_ties(name):
    rows, k, kv, g, beta, v, q, qv, expect = WORKED[name]
    bank = torch.tensor([[x] for x in rows], dtype=torch.float32)
    inp = {"k_idx": torch.tensor([k], dtype=torch.int64), "k_val": torch.tensor([kv], dtype=torch.float32),
           "v": torch.tensor([[v]], dtype=torch.float32), "beta": torch.tensor([[beta]], dtype=torch.float32),
           "g": torch.tensor([[g]], dtype=torch.float32), "q_idx": torch.tensor([q], dtype=torch.int64),
           "q_val": torch.tensor([qv], dtype=torch.float32)}
    ref_bank = bank.numpy().copy()
    ref = oracle.decode_step(ref_bank, **step_to_numpy(inp), groups=1)
    for i, e in enumerate(expect):
        if e is not None:
            assert ref_bank[i, 0] == np.float32(e), f"oracle row {i}"
    dbank = bank.to(DEV)
    readings = sdm_decode_step(dbank, **{key: t.to(DEV) for key, t in inp.items()})
    assert bits_equal(readings.cpu().numpy(), ref), "readings differ from the oracle"
    assert bits_equal(dbank.cpu().numpy(), ref_bank), "bank differs from the oracle"


@pytest.mark.slow
def test_bf16_conversion_over_every_float32():
    """The library's float32 -> bfloat16 conversion (sdm_round_bf16, the one every kernel
    uses on a bfloat16 store) against the oracle's round-to-nearest-even, bit for bit,
    on all 2^32 float32 bit patterns: 16 batches of 2^28, each generated on the device
    and on the host from the same counter, the oracle's part split over host threads."""
    from concurrent.futures import ThreadPoolExecutor
    from sparse_delta_rule_amd import sdm_round_bf16

    batch = 1 << 28
    threads = 16
    x = torch.empty(batch, dtype=torch.int32, device=DEV)
    out = torch.empty(batch, dtype=torch.bfloat16, device=DEV)
    host = np.empty(batch, dtype=np.uint32)
    iota = np.arange(batch, dtype=np.uint32)
    want = np.empty(batch, dtype=np.uint16)

    def ref(i):
        a, b = batch * i // threads, batch * (i + 1) // threads
        want[a:b] = oracle.float_to_bf16_array(host[a:b].view(np.float32))

    with ThreadPoolExecutor(threads) as ex:
        for k in range(16):
            base = k * batch
            lo = base - (1 << 32) if base >= 1 << 31 else base  # the same 32 bits as int32
            x.copy_(torch.arange(lo, lo + batch, dtype=torch.int64, device=DEV))
            sdm_round_bf16(x.view(torch.float32), out)
            got = out.view(torch.int16).cpu().numpy().view(np.uint16)
            np.add(iota, np.uint32(base), out=host)
            list(ex.map(ref, range(threads)))
            bad = np.flatnonzero(got != want)
            assert bad.size == 0, (f"batch {k}: {bad.size} differences, first at bits "
                                   f"{int(host[bad[0]]):#010x}: {int(got[bad[0]]):#06x} vs {int(want[bad[0]]):#06x}")
            print(f"bfloat16 conversion: bit patterns {base:#010x}..{base + batch - 1:#010x} agree", flush=True)
