"""Parity at the far ends of the shapes: very long rows (many column slices), the
widest widths on the narrowest rows, one chunk spanning every token and chunks of
one token. Bit for bit against the oracle, as the other parity tests."""

import pytest
import torch

import gen
from tests.test_decode_steps_gpu import check_steps
from tests.test_gather_compact_gpu import run_compact
from tests.test_gather_gpu import run_case

pytestmark = pytest.mark.gpu

DECODE = [
    # name, bank dtype, streams, slots/stream, hd, W, R, G, steps
    ("f32 hd 4096 (32 slices of 512 B)", torch.float32, 6, 64, 4096, 9, 7, 9, 3),
    ("bf16 hd 8192 (32 slices)", torch.bfloat16, 4, 40, 8192, 5, 12, 1, 2),
    ("f32 hd 1 W = R = 256", torch.float32, 5, 300, 1, 256, 256, 256, 3),
    ("bf16 hd 2 W = R = 256", torch.bfloat16, 3, 256, 2, 256, 256, 1, 2),
    ("bf16 hd 4095 odd long", torch.bfloat16, 3, 20, 4095, 3, 3, 3, 2),
    ("f32 many streams, one slot each", torch.float32, 3000, 1, 16, 1, 1, 1, 3),
    # the multi-token compact loop's largest LDS: 32 row groups of 256-column slices,
    # two partial buffers (about 83 KiB per workgroup)
    ("bf16 hd 256 W = R = 256 (largest loop LDS)", torch.bfloat16, 4, 600, 256, 256, 256, 1, 3),
]


@pytest.mark.parametrize("case", DECODE, ids=[c[0] for c in DECODE])
def test_decode_extremes(case):
    name, dt, S, P, hd, W, R, G, T = case
    wl = gen.DecodeWorkload(name=name, bank_dtype=dt, streams=S, slots_per_stream=P, head_dim=hd, W=W, R=R, G=G,
                            steps=T, idx_dtype=torch.int64, weights="normal_sqrtw", beta="sigmoid", g_low=-0.2,
                            bank_std=0.5)
    print(name, flush=True)
    check_steps(wl, 61, list(range(S)))


GATHER = [
    # name, bank dtype, slots, hd, tokens, chunk, width0, width1
    ("bf16 hd 8192 (16 slices)", torch.bfloat16, 500, 8192, 12, 4, 6, 3),
    ("f32 hd 4096", torch.float32, 300, 4096, 10, 5, 4, 0),
    ("one chunk of every token", torch.bfloat16, 3000, 128, 200, 200, 32, 32),
    ("chunks of one token", torch.bfloat16, 3000, 128, 150, 1, 16, 8),
    ("hd 1, widths 256", torch.float32, 1000, 1, 40, 8, 256, 256),
    # the most chunks a workgroup's LDS scan takes (4096), in each lane-group size of
    # the pair layout (16, 32 and 64 lanes: the deepest searches of the prefix)
    ("4096 chunks of one token", torch.bfloat16, 3000, 128, 4096, 1, 8, 4),
    ("4096 chunks of one token, 512-byte rows", torch.bfloat16, 3000, 256, 4096, 1, 4, 2),
    ("4096 chunks of one token, 1 KiB rows", torch.bfloat16, 3000, 512, 4096, 1, 4, 4),
    # past the 4096 chunks a workgroup's LDS scan takes: the token-order layout
    ("5000 chunks of one token", torch.bfloat16, 3000, 128, 5000, 1, 8, 4),
]


@pytest.mark.parametrize("case", GATHER, ids=[c[0] for c in GATHER])
def test_gather_extremes(case):
    name, dt, slots, hd, T, chunk, W0, W1 = case
    wl = gen.GatherWorkload(name=name, bank_dtype=dt, num_slots=slots, head_dim=hd, tokens=T, chunk=chunk,
                            valid_low=0, valid_high=chunk, width0=W0, width1=W1, idx_dtype=torch.int32,
                            w_dtype=torch.bfloat16, bank_std=0.5)
    print(name, flush=True)
    run_case(wl, 62, per_chunk=True)
    run_case(wl, 62, per_chunk=False, valid=max(1, chunk - 1))
    run_case(wl, 62, per_chunk=True, stash=False)
    run_case(wl, 62, per_chunk=False, valid=max(1, chunk - 1), stash=False)
    run_compact(wl, 62)


SPARSE = [
    # name, hd: chunks of 4 tokens with 0 or 1 live (runs of empty chunks, so runs of
    # equal prefix values), no stash: the pair layout's search at 16, 32 and 64 lanes
    ("hd 128", 128),
    ("hd 256", 256),
    ("hd 512", 512),
]


@pytest.mark.parametrize("case", SPARSE, ids=[c[0] for c in SPARSE])
def test_gather_mostly_empty_chunks(case):
    name, hd = case
    wl = gen.GatherWorkload(name=f"mostly empty chunks, {name}", bank_dtype=torch.bfloat16, num_slots=2000,
                            head_dim=hd, tokens=16000, chunk=4, valid_low=0, valid_high=1, width0=6, width1=3,
                            idx_dtype=torch.int32, w_dtype=torch.bfloat16, bank_std=0.5)
    print(wl.name, flush=True)
    run_case(wl, 63, per_chunk=True, stash=False)
    run_case(wl, 63, per_chunk=True)
