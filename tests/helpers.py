"""Small array helpers shared by the tests (no method arithmetic here)."""

from __future__ import annotations

import numpy as np
import torch


def to_np_bank(t: torch.Tensor) -> np.ndarray:
    """A torch bank as numpy: float32, or uint16 bfloat16 bits."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    if t.dtype == torch.float32:
        return t.numpy().copy()
    raise TypeError(t.dtype)


def from_np_bank(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)
    return torch.from_numpy(a.copy())


def widen(a: np.ndarray) -> np.ndarray:
    """float32 values of a bank array (bfloat16 bits widen exactly)."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32)
    return a.astype(np.float32)


def f32_to_bf16_bits_torch(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits through torch's own conversion (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def round_to_bank_torch(x: np.ndarray, bf16: bool) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    return widen(f32_to_bf16_bits_torch(x)) if bf16 else x


def ulp(x: np.ndarray, bf16: bool) -> np.ndarray:
    """Spacing of the bank dtype at |x| (the larger neighbour gap)."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    mant = 8 if bf16 else 24
    e = np.floor(np.log2(np.where(x > 0, x, 1.0)))
    e = np.maximum(e, -126.0)
    return np.ldexp(1.0, (e - (mant - 1)).astype(np.int64))


def gamma(n: int) -> float:
    u = 2.0 ** -24
    return n * u / (1 - n * u)


def bits_equal(a: np.ndarray, b: np.ndarray) -> bool:
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    if a.dtype != b.dtype or a.shape != b.shape:
        return False
    return bool(np.array_equal(a.view(np.uint8), b.view(np.uint8)))


def random_decode_case(rng: np.random.Generator, *, streams, slots_per_stream, hd, W, R, G,
                       bf16, overlap="any", scale=1.0):
    """A random decode step with private slot ranges; ``overlap``: 'any' (independent k/q
    draws), 'none' (q drawn from slots not written) or 'all' (q = k)."""
    S = streams
    bank = (rng.standard_normal((S * slots_per_stream, hd)) * 0.5 * scale).astype(np.float32)
    if bf16:
        bank = f32_to_bf16_bits_torch(bank)
    k_idx = np.empty((S, W), np.int64)
    q_idx = np.empty((S, R), np.int64)
    for s in range(S):
        perm = rng.permutation(slots_per_stream)
        k_idx[s] = perm[:W] + s * slots_per_stream
        if overlap == "none":
            q_idx[s] = perm[W:W + R] + s * slots_per_stream
        elif overlap == "all":
            q_idx[s] = k_idx[s][:R]
        else:
            q_idx[s] = rng.permutation(slots_per_stream)[:R] + s * slots_per_stream
    case = dict(
        bank=bank,
        k_idx=k_idx,
        k_val=rng.standard_normal((S, W)).astype(np.float32),
        v=rng.standard_normal((S, hd)).astype(np.float32),
        beta=rng.uniform(0, 1, (S, 1)).astype(np.float32),
        g=rng.uniform(-0.3, 0, (S, G)).astype(np.float32),
        q_idx=q_idx,
        q_val=rng.standard_normal((S, R)).astype(np.float32),
    )
    return case


# ----------------------------------------------------------------- GPU runs
def documented_decode_groups(W: int, R: int) -> int:
    """The decode's row-group count as include/sdm.h states it:
    RG = min(32, next_pow2(ceil(max(W, R) / 4)))."""
    need = -(-max(W, R) // 4)
    rg = 1
    while rg < need:
        rg *= 2
    return min(32, rg)


def step_to_numpy(inp: dict) -> dict:
    """One step's inputs as the oracle takes them (indices int64, values float32)."""
    out = {}
    for k, t in inp.items():
        t = t.detach().cpu()
        if k in ("k_idx", "q_idx"):
            out[k] = t.to(torch.int64).numpy()
        else:
            out[k] = t.float().numpy()
    return out


def oracle_sequence(bank: np.ndarray, steps: list, groups: int):
    """Run the oracle over a list of numpy step inputs; returns (bank, [readings])."""
    import oracle
    readings = []
    for inp in steps:
        readings.append(oracle.decode_step(bank, inp["k_idx"], inp["k_val"], inp["v"], inp["beta"],
                                           inp["g"], inp["q_idx"], inp["q_val"], groups=groups))
    return bank, readings


def decode_tolerance_ok(x: np.ndarray, ref: np.ndarray, mag: np.ndarray, bf16: bool):
    """The stated parity bar: |x - ref| <= 1e-5 max(|ref|, M) for a float32 bank,
    <= ulp_bf16(ref) + 2^-8 max(|ref|, M) for a bfloat16 bank. Returns (ok, worst ratio)."""
    x = widen(x).astype(np.float64)
    ref = widen(ref).astype(np.float64)
    scale = np.maximum(np.abs(ref), mag)
    if bf16:
        bound = ulp(ref, True) + 2.0 ** -8 * scale
    else:
        bound = 1e-5 * scale
    err = np.abs(x - ref)
    ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1), np.where(err > 0, np.inf, 0))
    return bool(np.all(err <= bound)), float(ratio.max(initial=0.0))


def sub_inputs(inp: dict, streams: np.ndarray, P: int) -> dict:
    """One step's numpy inputs of the given streams, slots renumbered into the
    concatenation of those streams' private ranges (P slots each)."""
    out = {k: v[streams] for k, v in inp.items()}
    shift = (streams.astype(np.int64) * P - np.arange(len(streams), dtype=np.int64) * P)[:, None]
    out["k_idx"] = out["k_idx"] - shift
    out["q_idx"] = out["q_idx"] - shift
    return out


def stream_rows(streams: np.ndarray, P: int) -> np.ndarray:
    """Bank rows of the given streams' private ranges, concatenated."""
    return (np.asarray(streams)[:, None].astype(np.int64) * P + np.arange(P)[None, :]).ravel()
