"""Slots at and above 2^31 (int64 indices), on the GPU against the oracle.

Both kernels form 64-bit row offsets from 64-bit slots; these banks have more
than 2^31 rows (bfloat16, 2^31 + 4096 rows of one or of eight elements: about
4.3 and 34 GB), and the touched rows straddle and pass row 2^31. The oracle
runs on the touched rows alone, with the slots renumbered, which changes no
arithmetic; everything is compared bit for bit, and rows outside the touched
range must stay as they were.
"""

import numpy as np
import pytest
import torch

import oracle
from sparse_delta_rule_amd import sdm_decode_step, sdm_decode_steps, sdm_gather
from tests.helpers import bits_equal, documented_decode_groups, from_np_bank, to_np_bank

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)
ROWS = (1 << 31) + 4096


def _bf16_bits(rng, shape, std):
    x = torch.from_numpy((rng.standard_normal(shape) * std).astype(np.float32))
    return to_np_bank(x.to(torch.bfloat16))


@pytest.fixture(params=[1, 8], ids=["hd1", "hd8"])
def big_bank(request):
    hd = request.param
    bank = torch.zeros((ROWS, hd), dtype=torch.bfloat16, device=DEV)
    yield bank
    del bank
    torch.cuda.empty_cache()


def test_decode_slots_past_2_31(big_bank):
    bank = big_bank
    hd = bank.shape[1]
    rng = np.random.default_rng(31)
    S, P, W, R, T = 3, 64, 16, 16, 3
    base = (1 << 31) - 32  # stream 0's slots straddle row 2^31; streams 1 and 2 lie above it
    init = _bf16_bits(rng, (S * P, hd), 0.5)
    bank[base:base + S * P] = from_np_bank(init).to(DEV)
    steps = []
    for _ in range(T):
        k = np.stack([base + s * P + rng.choice(P, W, replace=False) for s in range(S)]).astype(np.int64)
        q = np.stack([base + s * P + rng.choice(P, R, replace=True) for s in range(S)]).astype(np.int64)
        steps.append({"k_idx": k, "k_val": (rng.standard_normal((S, W)) / 4).astype(np.float32),
                      "v": rng.standard_normal((S, hd)).astype(np.float32),
                      "beta": (1 / (1 + np.exp(-rng.standard_normal((S, 1))))).astype(np.float32),
                      "g": rng.uniform(-0.2, 0.0, (S, 1)).astype(np.float32), "q_idx": q,
                      "q_val": (rng.standard_normal((S, R)) / 4).astype(np.float32)})
    assert steps[0]["k_idx"].max() >= 1 << 31 and steps[0]["k_idx"].min() < 1 << 31

    # oracle on the touched rows, slots renumbered from base
    ref_bank = init.copy()
    refs = []
    for st in steps:
        local = dict(st, k_idx=st["k_idx"] - base, q_idx=st["q_idx"] - base)
        refs.append(oracle.decode_step(ref_bank, **local, groups=documented_decode_groups(W, R)))

    dev = [{k: torch.from_numpy(v).to(DEV) for k, v in st.items()} for st in steps]
    saved = bank[base:base + S * P].clone()
    # one token per launch, then the same tokens again in one multi-token launch
    for t in range(T):
        r = sdm_decode_step(bank, **dev[t])
        assert bits_equal(to_np_bank(r), refs[t]), f"single step {t}: readings differ from the oracle"
    assert bits_equal(to_np_bank(bank[base:base + S * P]), ref_bank), "bank differs after single steps"
    bank[base:base + S * P] = saved
    seq = {k: torch.stack([d[k] for d in dev]) for k in dev[0]}
    r = sdm_decode_steps(bank, **seq)
    for t in range(T):
        assert bits_equal(to_np_bank(r[t]), refs[t]), f"token {t}: readings differ from the oracle"
    assert bits_equal(to_np_bank(bank[base:base + S * P]), ref_bank), "bank differs after the multi-token launch"
    for lo, hi in ((0, 64), (base - 64, base), (base + S * P, base + S * P + 64), (ROWS - 64, ROWS)):
        assert not bank[lo:hi].any(), f"rows {lo}..{hi} outside the streams' ranges changed"


def test_gather_slots_past_2_31(big_bank):
    gather_past_2_31(big_bank, with_stash=True)


def test_gather_pair_layout_slots_past_2_31():
    """Rows of nine bfloat16 elements (nine 2-byte vectors, one 16-lane group per
    pair) and no stash: the launch shape of the pair layout."""
    bank = torch.zeros((ROWS, 9), dtype=torch.bfloat16, device=DEV)
    gather_past_2_31(bank, with_stash=False)
    del bank
    torch.cuda.empty_cache()


def test_gather_pair_layout_32_lane_groups_slots_past_2_31():
    """Rows of seventeen bfloat16 elements (17 two-byte vectors: 32-lane groups, whose
    slots are read into scalar registers, 64-bit here) and no stash (a 73 GB bank)."""
    bank = torch.zeros((ROWS, 17), dtype=torch.bfloat16, device=DEV)
    gather_past_2_31(bank, with_stash=False)
    del bank
    torch.cuda.empty_cache()


def gather_past_2_31(bank, with_stash):
    hd = bank.shape[1]
    rng = np.random.default_rng(32)
    lo = (1 << 31) - 1024  # slots drawn from [lo, ROWS): a fifth below row 2^31
    init = _bf16_bits(rng, (ROWS - lo, hd), 0.5)
    bank[lo:] = from_np_bank(init).to(DEV)
    T, chunk, W0, W1 = 128, 64, 48, 20
    cv = np.array([40, 64], dtype=np.int32)
    idx0 = rng.integers(lo, ROWS, (T, W0), dtype=np.int64)
    idx1 = rng.integers(lo, ROWS, (T, W1), dtype=np.int64)
    w0 = _bf16_bits(rng, (T, W0), 1.0)
    w1 = _bf16_bits(rng, (T, W1), 1.0)
    wf0 = (w0.astype(np.uint32) << 16).view(np.float32)
    wf1 = (w1.astype(np.uint32) << 16).view(np.float32)
    ref0, ref_st, ref1 = oracle.gather(init, idx0 - lo, wf0, chunk=chunk, chunk_valid=cv, idx1=idx1 - lo, w1=wf1,
                                       stash=with_stash)

    def dev(a):
        return torch.from_numpy(a).to(DEV)

    out0, stash, out1 = sdm_gather(bank, dev(idx0), from_np_bank(w0).to(DEV), chunk=chunk, chunk_valid=dev(cv),
                                   idx1=dev(idx1), w1=from_np_bank(w1).to(DEV), with_stash=with_stash)
    assert bits_equal(out0.cpu().numpy(), ref0), "operand 0 differs from the oracle"
    assert bits_equal(out1.cpu().numpy(), ref1), "operand 1 differs from the oracle"
    if with_stash:
        assert bits_equal(to_np_bank(stash), ref_st), "stash differs from the oracle"
    else:
        assert stash is None
