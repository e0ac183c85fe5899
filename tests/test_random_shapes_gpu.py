"""Seeded sweeps of random shapes against the oracle, on the GPU.

The hand-picked cases elsewhere pin the edge shapes one by one; these sweeps
draw combinations of them (bank dtype, head dim, widths, gate layout, index
and value dtypes, stream and token counts, chunking and padding) so that the
geometry choices (vector width, lanes per row, row groups, column slices,
metadata items per thread, the multi-token loop) meet in combinations no list
names. Every comparison is bit for bit, as in the other parity tests.
"""

import os

import numpy as np
import pytest
import torch

import gen
from tests.test_decode_steps_gpu import check_steps
from tests.test_gather_compact_gpu import run_compact
from tests.test_gather_gpu import run_case

pytestmark = pytest.mark.gpu

# Cases per sweep; SDM_SWEEP_CASES=<n> runs a longer sweep (same seeds, more of them).
N_CASES = int(os.environ.get("SDM_SWEEP_CASES", "0")) or None

HEAD_DIMS = [1, 2, 3, 5, 8, 16, 31, 36, 64, 72, 100, 101, 120, 127, 128, 129, 200, 255, 256, 300, 512, 700]
WIDTHS = [1, 2, 3, 4, 5, 7, 8, 16, 17, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 200, 255, 256]


def _pick(rng, xs):
    return xs[int(rng.integers(len(xs)))]


def _decode_case(i):
    rng = np.random.default_rng(1000 + i)
    W, R = _pick(rng, WIDTHS), _pick(rng, WIDTHS)
    return gen.DecodeWorkload(
        name=f"random decode {i}", bank_dtype=_pick(rng, [torch.float32, torch.bfloat16]),
        streams=int(rng.integers(1, 25)), slots_per_stream=max(W, R) + int(rng.integers(0, 64)),
        head_dim=_pick(rng, HEAD_DIMS), W=W, R=R, G=_pick(rng, [1, W]), steps=int(rng.integers(1, 6)),
        idx_dtype=_pick(rng, [torch.int32, torch.int64]), weights=_pick(rng, ["normal_sqrtw", "normal_16"]),
        beta=_pick(rng, ["sigmoid", "uniform"]), g_low=-0.2, bank_std=0.5,
        val_dtype=_pick(rng, [torch.float32, torch.bfloat16]))


@pytest.mark.parametrize("loop", ["auto", "compact", "wide"])
@pytest.mark.parametrize("i", range(N_CASES or 40))
def test_random_decode_shapes(i, loop, monkeypatch):
    """A multi-token launch on a random shape equals the oracle stepped token by token
    and equals one single-token launch per token."""
    if loop == "auto":
        monkeypatch.delenv("SDM_STEPS_LOOP", raising=False)
    else:
        monkeypatch.setenv("SDM_STEPS_LOOP", loop)
    wl = _decode_case(i)
    print(wl, flush=True)
    check_steps(wl, 7 + i, list(range(wl.streams)))


def _gather_case(i):
    rng = np.random.default_rng(2000 + i)
    chunk = int(rng.integers(1, 40))
    return gen.GatherWorkload(
        name=f"random gather {i}", bank_dtype=_pick(rng, [torch.float32, torch.bfloat16]),
        num_slots=int(rng.integers(1, 3000)), head_dim=_pick(rng, HEAD_DIMS), tokens=chunk * int(rng.integers(1, 9)),
        chunk=chunk, valid_low=0, valid_high=chunk, width0=_pick(rng, WIDTHS),
        width1=_pick(rng, [0] + WIDTHS), idx_dtype=_pick(rng, [torch.int32, torch.int64]),
        w_dtype=_pick(rng, [torch.float32, torch.bfloat16]), bank_std=0.5)


@pytest.mark.parametrize("i", range(N_CASES or 64))
def test_random_gather_shapes(i):
    """The gather (with and without the stash, per-chunk or scalar valid; rows of
    9 to 16 vectors take the pair layout without it) and the compact-stash gather on
    a random shape equal the oracle."""
    wl = _gather_case(i)
    print(wl, flush=True)
    run_case(wl, 40 + i, per_chunk=True)
    run_case(wl, 40 + i, per_chunk=True, stash=False)
    run_case(wl, 40 + i, per_chunk=False, valid=wl.chunk // 2, stash=False)
    run_compact(wl, 40 + i)
