"""Workload definitions and seeded generators.

Every tensor is drawn from a torch.Generator seeded by ``sub_seed(seed, tag,
step, part)``, so each (tensor, step) pair can be regenerated on its own. The
same code runs on the CPU (small cases, CPU-only tests) and on the GPU (large
banks); a test always feeds both sides from one generation, so the device the
numbers were drawn on never matters for parity.

Distributions follow the workloads of the sparse-delta-memory decode step and
token gather (page "sparse_delta_memory/decode.py", docstring of
sdm_decode_step; page "sparse_delta_memory/cuda/gather_cuda.py", module
docstring): banks ~ N(0, 0.02^2), slots drawn without replacement from each
stream's private range (decode) or uniformly over the bank (gather), weights
and values as listed per workload below.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

_MASK64 = (1 << 64) - 1


def sub_seed(seed: int, *keys) -> int:
    """A 63-bit seed for one (tensor, step, part) substream.

    SplitMix64's finaliser (Steele, Lea and Flood, "Fast splittable
    pseudorandom number generators", OOPSLA 2014) folded over the keys; string
    keys are folded byte by byte.
    """

    def mix(z: int) -> int:
        z = (z + 0x9E3779B97F4A7C15) & _MASK64
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
        return z ^ (z >> 31)

    h = mix(seed & _MASK64)
    for k in keys:
        if isinstance(k, str):
            for b in k.encode():
                h = mix(h ^ b)
        else:
            h = mix(h ^ (int(k) & _MASK64))
    return h & ((1 << 63) - 1)


def _gen(device, seed: int, *keys) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(sub_seed(seed, *keys))
    return g


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """One decode sequence: ``steps`` tokens for each of ``streams`` streams.

    Stream ``s`` owns bank rows ``[s * slots_per_stream, (s + 1) * slots_per_stream)``.
    ``weights``: 'normal' N(0,1); 'softmax' softmax over the width of N(0,1);
    'normal_sqrtw' N(0,1)/sqrt(width); 'normal_16' N(0,1)/16.
    ``beta``: 'sigmoid' sigmoid(N(0,1)) or 'uniform' U(0,1). ``g`` ~ U(g_low, 0).
    """

    name: str
    bank_dtype: torch.dtype
    streams: int
    slots_per_stream: int
    head_dim: int
    W: int
    R: int
    G: int
    steps: int
    idx_dtype: torch.dtype
    weights: str
    beta: str
    g_low: float
    bank_std: float = 0.02
    val_dtype: torch.dtype = torch.float32

    @property
    def num_slots(self) -> int:
        return self.streams * self.slots_per_stream

    def row_bytes_per_stream_step(self) -> int:
        es = torch.empty((), dtype=self.bank_dtype).element_size()
        return (2 * self.W + self.R) * self.head_dim * es

    def replace(self, **kw) -> "DecodeWorkload":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class GatherWorkload:
    """One token-gather launch over a shared bank.

    Slots are uniform over the whole bank (with replacement across entries);
    weights are N(0,1) rounded to ``w_dtype``; chunk ``c`` has ``valid[c]`` live
    positions, uniform on ``[valid_low, valid_high]``.
    """

    name: str
    bank_dtype: torch.dtype
    num_slots: int
    head_dim: int
    tokens: int
    chunk: int
    valid_low: int
    valid_high: int
    width0: int
    width1: int  # 0: one operand
    idx_dtype: torch.dtype
    w_dtype: torch.dtype
    stash: bool = True
    bank_std: float = 0.02

    def replace(self, **kw) -> "GatherWorkload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "c0": DecodeWorkload(
        name="decode fp32 bank 4 streams x 256 slots, hd 64, W=R=4, G=1, 16 steps",
        bank_dtype=torch.float32, streams=4, slots_per_stream=256, head_dim=64,
        W=4, R=4, G=1, steps=16, idx_dtype=torch.int64, weights="normal",
        beta="sigmoid", g_low=-0.1),
    "c1": DecodeWorkload(
        name="decode bf16 bank 1024 streams x 4096 slots, hd 128, W=R=32, G=1, 64 steps",
        bank_dtype=torch.bfloat16, streams=1024, slots_per_stream=4096, head_dim=128,
        W=32, R=32, G=1, steps=64, idx_dtype=torch.int32, weights="softmax",
        beta="sigmoid", g_low=-0.05),
    "c2": DecodeWorkload(
        name="decode bf16 bank 4096 streams x 16384 slots (16 GiB), hd 128, W=R=64, G=W, 32 steps",
        bank_dtype=torch.bfloat16, streams=4096, slots_per_stream=16384, head_dim=128,
        W=64, R=64, G=64, steps=32, idx_dtype=torch.int64, weights="normal_sqrtw",
        beta="uniform", g_low=-0.1),
    "c3": GatherWorkload(
        name="gather bf16 bank 16M x 128, 32768 tokens, chunk 64, valid U[32,64], 2 x width 64, stash",
        bank_dtype=torch.bfloat16, num_slots=16 * 1024 * 1024, head_dim=128,
        tokens=32768, chunk=64, valid_low=32, valid_high=64, width0=64, width1=64,
        idx_dtype=torch.int32, w_dtype=torch.bfloat16),
    "c4": DecodeWorkload(
        name="decode fp32 bank 512 streams x 2048 slots, hd 100, W=R=256, G=1, 16 steps",
        bank_dtype=torch.float32, streams=512, slots_per_stream=2048, head_dim=100,
        W=256, R=256, G=1, steps=16, idx_dtype=torch.int64, weights="normal_16",
        beta="sigmoid", g_low=-0.2),
}

_BANK_CHUNK_ROWS = 1 << 20  # rows drawn per generator substream


def _fill_bank(bank: torch.Tensor, std: float, seed: int, tag: str) -> torch.Tensor:
    rows, hd = bank.shape
    for i, r0 in enumerate(range(0, rows, _BANK_CHUNK_ROWS)):
        n = min(_BANK_CHUNK_ROWS, rows - r0)
        gen = _gen(bank.device, seed, tag, i)
        x = torch.randn((n, hd), generator=gen, device=bank.device, dtype=torch.float32)
        x.mul_(std)
        bank[r0:r0 + n].copy_(x)
        del x
    return bank


def decode_bank(wl: DecodeWorkload, seed: int, device="cpu") -> torch.Tensor:
    """The bank before the first step: [num_slots, head_dim], N(0, bank_std^2)."""
    bank = torch.empty((wl.num_slots, wl.head_dim), dtype=wl.bank_dtype, device=device)
    return _fill_bank(bank, wl.bank_std, seed, "decode-bank")


def _distinct_slots(streams: int, per_stream: int, width: int, gen, device) -> torch.Tensor:
    """``width`` distinct local slots per stream, uniform without replacement."""
    out = torch.empty((streams, width), dtype=torch.int64, device=device)
    block = max(1, (1 << 24) // per_stream)
    for s0 in range(0, streams, block):
        n = min(block, streams - s0)
        keys = torch.rand((n, per_stream), generator=gen, device=device)
        out[s0:s0 + n] = keys.topk(width, dim=1).indices
    return out


def _weights(kind: str, shape, gen, device) -> torch.Tensor:
    x = torch.randn(shape, generator=gen, device=device)
    width = shape[-1]
    if kind == "normal":
        return x
    if kind == "softmax":
        return torch.softmax(x, dim=-1)
    if kind == "normal_sqrtw":
        return x / math.sqrt(width)
    if kind == "normal_16":
        return x / 16.0
    raise ValueError(f"unknown weight distribution {kind!r}")


def decode_step_inputs(wl: DecodeWorkload, seed: int, step: int, device="cpu") -> dict:
    """Inputs of one decode step for all streams (absolute slot numbers)."""
    S = wl.streams
    base = torch.arange(S, device=device, dtype=torch.int64)[:, None] * wl.slots_per_stream
    k_idx = _distinct_slots(S, wl.slots_per_stream, wl.W, _gen(device, seed, "k_idx", step), device)
    q_idx = _distinct_slots(S, wl.slots_per_stream, wl.R, _gen(device, seed, "q_idx", step), device)
    k_val = _weights(wl.weights, (S, wl.W), _gen(device, seed, "k_val", step), device)
    q_val = _weights(wl.weights, (S, wl.R), _gen(device, seed, "q_val", step), device)
    v = torch.randn((S, wl.head_dim), generator=_gen(device, seed, "v", step), device=device)
    if wl.beta == "sigmoid":
        beta = torch.sigmoid(torch.randn((S, 1), generator=_gen(device, seed, "beta", step),
                                         device=device))
    elif wl.beta == "uniform":
        beta = torch.rand((S, 1), generator=_gen(device, seed, "beta", step), device=device)
    else:
        raise ValueError(f"unknown beta distribution {wl.beta!r}")
    g = torch.rand((S, wl.G), generator=_gen(device, seed, "g", step), device=device) * wl.g_low
    return {
        "k_idx": (k_idx + base).to(wl.idx_dtype),
        "k_val": k_val.to(wl.val_dtype),
        "v": v.to(wl.val_dtype),
        "beta": beta.float(),
        "g": g.float(),
        "q_idx": (q_idx + base).to(wl.idx_dtype),
        "q_val": q_val.to(wl.val_dtype),
    }


def decode_sequence(wl: DecodeWorkload, seed: int, device="cpu", steps: Optional[int] = None) -> dict:
    """All steps' inputs stacked on a leading [steps] axis."""
    steps = wl.steps if steps is None else steps
    per = [decode_step_inputs(wl, seed, t, device) for t in range(steps)]
    return {k: torch.stack([p[k] for p in per]) for k in per[0]}


def gather_bank(wl: GatherWorkload, seed: int, device="cpu") -> torch.Tensor:
    bank = torch.empty((wl.num_slots, wl.head_dim), dtype=wl.bank_dtype, device=device)
    return _fill_bank(bank, wl.bank_std, seed, "gather-bank")


def gather_inputs(wl: GatherWorkload, seed: int, device="cpu") -> dict:
    """Slots, weights and per-chunk valid counts of one gather launch."""
    T = wl.tokens
    out = {}
    for o, width in ((0, wl.width0), (1, wl.width1)):
        if width == 0:
            continue
        idx = torch.randint(0, wl.num_slots, (T, width), generator=_gen(device, seed, "idx", o),
                            device=device, dtype=torch.int64)
        w = torch.randn((T, width), generator=_gen(device, seed, "w", o), device=device)
        out[f"idx{o}"] = idx.to(wl.idx_dtype)
        out[f"w{o}"] = w.to(wl.w_dtype)
    chunks = T // wl.chunk if wl.chunk > 0 else 0
    # Drawn on the CPU whatever the device, so a launch's live-token count (and with
    # it the rows it moves) is the same number on every device.
    out["chunk_valid"] = torch.randint(wl.valid_low, wl.valid_high + 1, (chunks,),
                                       generator=_gen("cpu", seed, "valid"),
                                       dtype=torch.int32).to(device)
    return out


def live_tokens(wl: GatherWorkload, chunk_valid: torch.Tensor) -> int:
    """Number of live (non-padding) tokens of a gather launch with these per-chunk counts."""
    return int(chunk_valid.to("cpu", torch.int64).clamp(0, wl.chunk).sum())


def compact_positions(idx0: torch.Tensor, chunk: int, chunk_valid: torch.Tensor) -> torch.Tensor:
    """A compact-stash position map for operand 0, as the pages' forward builds it:
    within each chunk, the live tokens' entries are sorted by slot, and every
    entry gets the first position of its slot in that sorted list (entries with
    one slot share a position; later positions of a repeated slot stay unused);
    padding tokens' entries get -1. int32 [tokens, width0], on idx0's device."""
    T, W0 = idx0.shape
    dev = idx0.device
    if T == 0:
        return torch.empty((0, W0), dtype=torch.int32, device=dev)
    t = torch.arange(T, device=dev)
    live = (t % chunk) < chunk_valid.to(dev).long()[t // chunk]
    c = (t // chunk)[:, None].expand(T, W0)
    slot = idx0.long()
    # Sort key: chunk, then slot; padding entries sort after every live entry of their chunk.
    big = int(slot.max()) + 2
    key = c * (big + 1) + torch.where(live[:, None], slot, torch.full_like(slot, big))
    flat = key.reshape(-1)
    order = torch.sort(flat, stable=True).values
    first = torch.searchsorted(order, flat)  # first position of the key in the sorted order
    chunk_start = torch.searchsorted(order, (c.reshape(-1) * (big + 1)))  # where the chunk's block begins
    pos = (first - chunk_start).reshape(T, W0)
    return torch.where(live[:, None], pos, torch.full_like(pos, -1)).to(torch.int32)
