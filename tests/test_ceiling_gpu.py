"""libsdm_ceiling on the GPU: every reference pattern touches exactly the rows it
names, with the bits stated in include/sdm_ceiling.h (checked against plain
torch operations on the same rows)."""

import pytest
import torch

pytestmark = pytest.mark.gpu

from sparse_delta_rule_amd import ceiling  # noqa: E402

DEV = torch.device("cuda", 0)


def _bank(rows, row_bytes, seed=0):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return torch.randint(-2**31, 2**31 - 1, (rows, row_bytes // 4), generator=g, device=DEV, dtype=torch.int64) \
        .to(torch.int32)


def _xor_all(t):
    import numpy as np
    return int(np.bitwise_xor.reduce(t.reshape(-1).cpu().numpy().view(np.uint32)))


@pytest.mark.parametrize("row_bytes", [16, 48, 256, 400, 1024])
@pytest.mark.parametrize("n", [1, 7, 1000, 5000])
def test_read_folds_every_word_of_the_named_rows(row_bytes, n):
    bank = _bank(3000, row_bytes)
    idx = torch.randint(0, 3000, (n,), device=DEV)
    sink = torch.zeros(ceiling.sink_words(), dtype=torch.int32, device=DEV)
    ceiling.rows("read", bank, idx, sink=sink)
    torch.cuda.synchronize()
    # threads past the launch's grid leave their zero words
    assert _xor_all(sink) == _xor_all(bank[idx])


@pytest.mark.parametrize("row_bytes", [16, 256, 400])
@pytest.mark.parametrize("n", [1, 33, 4100])
def test_stash_copies_the_named_rows(row_bytes, n):
    bank = _bank(5000, row_bytes, 1)
    idx = torch.randint(0, 5000, (n,), device=DEV)
    stash = torch.full((n, row_bytes // 4), 7, dtype=torch.int32, device=DEV)
    ceiling.rows("stash", bank, idx, stash=stash)
    assert torch.equal(stash, bank[idx])


@pytest.mark.parametrize("row_bytes", [16, 256, 400])
def test_rmw_flips_exactly_the_named_rows_and_twice_restores(row_bytes):
    bank = _bank(6000, row_bytes, 2)
    before = bank.clone()
    idx = torch.randperm(6000, device=DEV)[:2500]
    ceiling.rows("rmw", bank, idx)
    want = before.clone()
    want[idx] ^= 0x00010001
    assert torch.equal(bank, want)
    ceiling.rows("rmw", bank, idx)
    assert torch.equal(bank, before)


def test_mix_writes_the_even_rows_and_reads_the_odd_ones():
    bank = _bank(4000, 256, 3)
    before = bank.clone()
    pairs = torch.randperm(4000, device=DEV)[:3000]
    sink = torch.empty(ceiling.sink_words(), dtype=torch.int32, device=DEV)
    sink.zero_()
    ceiling.rows("mix", bank, pairs, sink=sink)
    torch.cuda.synchronize()
    want = before.clone()
    want[pairs[0::2]] ^= 0x00010001
    assert torch.equal(bank, want)
    assert _xor_all(sink) == _xor_all(before[pairs[1::2]])


@pytest.mark.parametrize("nt", [False, True])
@pytest.mark.parametrize("nbytes", [16, 4096, 3 << 20, (64 << 20) + 48])
def test_copy(nbytes, nt):
    src = torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device=DEV)
    dst = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    ceiling.copy(dst, src, nontemporal=nt)
    assert torch.equal(dst, src)
