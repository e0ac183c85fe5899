"""Pins of the token-gather oracle.

Definition: page "sparse_delta_memory/cuda/gather_cuda.py", module docstring:
per token and operand a float32-accumulated weighted sum of bank rows, a raw
copy of operand 0's rows (the stash), and padding positions (t mod chunk >=
valid) that read nothing and produce zeros; group g sums entries g, g+groups,
... in order and the group partials are summed in order.
"""

import json
import os

import numpy as np
import pytest

import oracle
from tests.helpers import bits_equal, f32_to_bf16_bits_torch, gamma, widen


def _bank(values, bf16):
    a = np.asarray(values, dtype=np.float32)
    return f32_to_bf16_bits_torch(a) if bf16 else a.copy()


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("groups", [1, 2, 3])
def test_handworked_gather(golden_dir, bf16, groups):
    c = json.load(open(os.path.join(golden_dir, "gather_handworked.json")))
    bank = _bank(c["bank"], bf16)
    out0, stash, out1 = oracle.gather(bank, c["idx0"], c["w0"], chunk=c["chunk"], valid=c["valid"],
                                      idx1=c["idx1"], w1=c["w1"], groups=groups)
    assert np.array_equal(out0, np.asarray(c["out0"], np.float32))
    assert np.array_equal(out1, np.asarray(c["out1"], np.float32))
    assert np.array_equal(widen(stash), np.asarray(c["stash"], np.float32))
    # padding rows are +0.0 exactly (bit pattern zero), stash rows all-zero bits
    assert not np.signbit(out0[1]).any() and not np.signbit(out1[3]).any()
    assert not stash[1].any() and not stash[3].any()


def _rand(rng, T, W, hd, slots, bf16):
    bank = (rng.standard_normal((slots, hd)) * 0.3).astype(np.float32)
    if bf16:
        bank = f32_to_bf16_bits_torch(bank)
    idx = rng.integers(0, slots, (T, W))
    w = rng.standard_normal((T, W)).astype(np.float32)
    return bank, idx, w


@pytest.mark.parametrize("bf16", [False, True])
def test_one_hot_weights_return_the_row(bf16):
    rng = np.random.default_rng(20)
    bank, idx, w = _rand(rng, 12, 9, 7, 50, bf16)
    w[:] = 0.0
    hot = rng.integers(0, 9, 12)
    w[np.arange(12), hot] = 1.0
    out, _, _ = oracle.gather(bank, idx, w, chunk=4)
    assert np.array_equal(out, widen(bank[idx[np.arange(12), hot]]))


@pytest.mark.parametrize("bf16", [False, True])
def test_width_one_is_one_product(bf16):
    rng = np.random.default_rng(21)
    bank, idx, w = _rand(rng, 16, 1, 5, 30, bf16)
    out, _, _ = oracle.gather(bank, idx, w, chunk=16)
    assert np.array_equal(out, widen(bank[idx[:, 0]]) * w[:, :1])


@pytest.mark.parametrize("bf16", [False, True])
def test_padding_and_stash(bf16):
    rng = np.random.default_rng(22)
    T, chunk = 24, 8
    bank, idx, w = _rand(rng, T, 5, 6, 40, bf16)
    cv = np.array([3, 0, 8], np.int32)
    out, stash, _ = oracle.gather(bank, idx, w, chunk=chunk, chunk_valid=cv)
    for t in range(T):
        live = (t % chunk) < cv[t // chunk]
        if live:
            assert bits_equal(stash[t], bank[idx[t]])
            assert np.any(out[t] != 0)
        else:
            assert not stash[t].any() and not out[t].any() and not np.signbit(out[t]).any()
    # a scalar valid equals the same count repeated per chunk
    o1, s1, _ = oracle.gather(bank, idx, w, chunk=chunk, valid=5)
    o2, s2, _ = oracle.gather(bank, idx, w, chunk=chunk, chunk_valid=np.full(3, 5, np.int32))
    assert bits_equal(o1, o2) and bits_equal(s1, s2)
    # valid = 0: everything is padding; valid = chunk: nothing is
    o0, st0, _ = oracle.gather(bank, idx, w, chunk=chunk, valid=0)
    assert not o0.any() and not st0.any()
    oc, stc, _ = oracle.gather(bank, idx, w, chunk=chunk, valid=chunk)
    assert bits_equal(stc, bank[idx])


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("groups", [1, 2, 4, 7])
def test_float32_within_bound_of_exact(bf16, groups):
    rng = np.random.default_rng(23 + groups)
    for W in (1, 4, 17, 64, 256):
        bank, idx, w = _rand(rng, 6, W, 9, 400, bf16)
        out, _, _ = oracle.gather(bank, idx, w, chunk=3, valid=2, groups=groups)
        exact, mag = oracle.gather_f64(bank, idx, w, chunk=3, valid=2)
        assert np.all(np.abs(out - exact) <= gamma(W + 1) * mag), (W, groups)


def test_groups_agree_on_exact_integers():
    rng = np.random.default_rng(24)
    for W in (1, 3, 16, 65, 256):
        bank = rng.integers(-8, 9, (300, 4)).astype(np.float32)
        idx = rng.integers(0, 300, (5, W))
        w = rng.integers(-4, 5, (5, W)).astype(np.float32)
        ref, _, _ = oracle.gather(bank, idx, w, chunk=5)
        exact, _ = oracle.gather_f64(bank, idx, w, chunk=5)
        assert np.array_equal(ref, exact)
        for groups in (2, 3, 8, 64):
            out, _, _ = oracle.gather(bank, idx, w, chunk=5, groups=groups)
            assert bits_equal(out, ref)


def test_grouped_order_is_the_stated_one():
    """Values chosen so that the float32 result depends on the order: group
    partials over n = g, g+groups, ... then summed in group order."""
    bank = np.array([[1.0], [2.0 ** 24], [-(2.0 ** 24)], [1.0]], np.float32)
    idx = np.array([[1, 0, 2, 3]])
    w = np.ones((1, 4), np.float32)
    # groups = 1: ((2^24 + 1) + -2^24) + 1 -> 2^24 (tie to even) - 2^24 + 1 = 1
    out1, _, _ = oracle.gather(bank, idx, w, chunk=1)
    assert out1[0, 0] == 1.0
    # groups = 2: p0 = 2^24 + -2^24 = 0, p1 = 1 + 1 = 2 -> 0 + 2 = 2
    out2, _, _ = oracle.gather(bank, idx, w, chunk=1, groups=2)
    assert out2[0, 0] == 2.0
    # groups = 3 on rows [2^24, 1, 1]: ((0 + 2^24) + 1) + 1 = 2^24 in group order,
    # while the reverse group order would give 2^24 + 2
    bank3 = np.array([[2.0 ** 24], [1.0], [1.0]], np.float32)
    out3, _, _ = oracle.gather(bank3, np.array([[0, 1, 2]]), np.ones((1, 3), np.float32), chunk=1,
                               groups=3)
    assert out3[0, 0] == 2.0 ** 24


def test_second_operand_matches_a_one_operand_gather():
    rng = np.random.default_rng(25)
    bank, idx0, w0 = _rand(rng, 10, 6, 5, 60, True)
    _, idx1, w1 = _rand(rng, 10, 11, 5, 60, True)
    cv = np.array([2, 5], np.int32)
    out0, stash, out1 = oracle.gather(bank, idx0, w0, chunk=5, chunk_valid=cv, idx1=idx1, w1=w1)
    solo, _, _ = oracle.gather(bank, idx1, w1, chunk=5, chunk_valid=cv)
    first, st, _ = oracle.gather(bank, idx0, w0, chunk=5, chunk_valid=cv)
    assert bits_equal(out1, solo) and bits_equal(out0, first) and bits_equal(stash, st)


def test_bad_arguments_are_reported():
    bank = np.zeros((4, 2), np.float32)
    idx = np.zeros((6, 2), np.int64)
    w = np.zeros((6, 2), np.float32)
    with pytest.raises(ValueError):
        oracle.gather(bank, idx, w, chunk=4)  # tokens not a multiple of chunk
    with pytest.raises(ValueError):
        oracle.gather(bank, idx, w, chunk=3, valid=4)
    idx[0, 0] = 4
    with pytest.raises(ValueError, match="out of range"):
        oracle.gather(bank, idx, w, chunk=3)


@pytest.mark.parametrize("bf16", [False, True])
def test_padding_slots_are_never_read(bf16):
    """A padding token reads no row (gather_cuda.py, module docstring: padding positions
    produce zeros), so any slot value there, in range or not, gives the same results;
    an out-of-range slot of a live token is still an error, for either operand."""
    rng = np.random.default_rng(31)
    bank, idx0, w0 = _rand(rng, 12, 9, 4, 40, bf16)
    _, idx1, w1 = _rand(rng, 12, 7, 4, 40, bf16)
    cv = np.array([1, 4, 0], np.int32)  # live tokens: 0, 4..7
    pad = np.ones(12, bool)
    pad[[0, 4, 5, 6, 7]] = False
    ref = oracle.gather(bank, idx0, w0, chunk=4, chunk_valid=cv, idx1=idx1, w1=w1)
    for junk in (-1, 40, 2**62):
        j0, j1 = idx0.copy(), idx1.copy()
        j0[pad] = junk
        j1[pad] = junk
        got = oracle.gather(bank, j0, w0, chunk=4, chunk_valid=cv, idx1=j1, w1=w1)
        for a, b in zip(got, ref):
            assert bits_equal(a, b)
        j0, j1 = idx0.copy(), idx1.copy()
        j0[np.arange(12) % 4 >= 1] = junk  # padding under valid = 1
        j1[np.arange(12) % 4 >= 1] = junk
        got = oracle.gather(bank, j0, w0, chunk=4, valid=1, idx1=j1, w1=w1)
        ref1 = oracle.gather(bank, idx0, w0, chunk=4, valid=1, idx1=idx1, w1=w1)
        for a, b in zip(got, ref1):
            assert bits_equal(a, b)
    bad = idx1.copy()
    bad[5, 3] = 40  # a live token of chunk 1
    with pytest.raises(ValueError, match="out of range"):
        oracle.gather(bank, idx0, w0, chunk=4, chunk_valid=cv, idx1=bad, w1=w1)
    bad = idx0.copy()
    bad[1, 0] = -1  # padding under chunk_valid, live when every token is
    oracle.gather(bank, bad, w0, chunk=4, chunk_valid=cv)
    with pytest.raises(ValueError, match="out of range"):
        oracle.gather(bank, bad, w0, chunk=4)


# ------------------------------------------------------------ compact stash
# Page "sparse_delta_memory/cuda/gather_cuda.py": with a position map kpos (one
# int32 per entry of operand 0: its first position in the chunk's sorted row
# list, or -1), the stash is one block of chunk * width0 rows per chunk and a
# live entry copies its row to that position of its chunk's block; nothing
# else is written.
SENTINEL = 0x7E  # a byte pattern no copied row has


def _sentinel_stash(T, W0, hd, dtype):
    return np.full(T * W0 * hd * np.dtype(dtype).itemsize, SENTINEL, np.uint8).view(dtype).reshape(T, W0, hd)


@pytest.mark.parametrize("bf16", [False, True])
def test_compact_stash_worked_example(bf16):
    """Two chunks of two tokens, width 2. Chunk 0 (both live) names slots 3, 1, 1, 0;
    sorted 0, 1, 1, 3, so the first positions are slot 0 -> 0, slot 1 -> 1,
    slot 3 -> 3, and position 2 (the second 1) is never written. Chunk 1 has one
    live token naming slot 2 twice (first position 0) and a padding token whose
    entries carry positions that must not be used."""
    bank = _bank([[1, 2], [3, 4], [5, 6], [7, 8]], bf16)
    idx0 = np.array([[3, 1], [1, 0], [2, 2], [0, 3]])
    kpos = np.array([[3, 1], [1, 0], [0, 0], [2, 3]], np.int32)
    stash = _sentinel_stash(4, 2, 2, bank.dtype).reshape(2, 4, 2)
    oracle.gather_compact_stash(bank, idx0, kpos, stash, chunk=2, chunk_valid=np.array([2, 1], np.int32))
    untouched = _sentinel_stash(1, 1, 2, bank.dtype)[0, 0]
    expect = [[bank[0], bank[1], untouched, bank[3]], [bank[2], untouched, untouched, untouched]]
    for k in range(2):
        for p in range(4):
            assert bits_equal(stash[k, p], expect[k][p]), (k, p)


@pytest.mark.parametrize("bf16", [False, True])
def test_compact_stash_with_identity_positions_is_the_full_stash(bf16):
    """kpos = (t mod chunk) * width0 + n puts every entry where the full stash has
    it: the live tokens' rows agree with the full stash, the padding tokens' rows
    keep their contents (the full stash zeroes them), and -1 entries skip."""
    rng = np.random.default_rng(41)
    T, chunk, W0, hd = 24, 8, 5, 6
    bank, idx, w = _rand(rng, T, W0, hd, 40, bf16)
    cv = np.array([3, 0, 8], np.int32)
    _, full, _ = oracle.gather(bank, idx, w, chunk=chunk, chunk_valid=cv)
    kpos = ((np.arange(T) % chunk)[:, None] * W0 + np.arange(W0)[None, :]).astype(np.int32)
    kpos[5, 2] = -1
    kpos[20, 0] = -7  # any negative position stores nothing
    stash = _sentinel_stash(T, W0, hd, bank.dtype)
    oracle.gather_compact_stash(bank, idx, kpos, stash.reshape(T // chunk, chunk * W0, hd), chunk=chunk,
                                chunk_valid=cv)
    untouched = _sentinel_stash(1, 1, hd, bank.dtype)[0, 0]
    for t in range(T):
        live = (t % chunk) < cv[t // chunk]
        for n in range(W0):
            if live and kpos[t, n] >= 0:
                assert bits_equal(stash[t, n], full[t, n]), (t, n)
            else:
                assert bits_equal(stash[t, n], untouched), (t, n)


def test_compact_stash_rejects_conflicting_and_out_of_block_positions():
    bank = np.arange(8, dtype=np.float32).reshape(4, 2)
    idx0 = np.array([[0, 1], [2, 3]])
    stash = np.zeros((1, 4, 2), np.float32)
    with pytest.raises(ValueError, match="named by two slots"):  # slots 0 and 2 at position 1
        oracle.gather_compact_stash(bank, idx0, np.array([[1, 0], [1, 2]], np.int32), stash, chunk=2)
    with pytest.raises(ValueError, match="past its block"):
        oracle.gather_compact_stash(bank, idx0, np.array([[0, 4], [1, 2]], np.int32), stash, chunk=2)
    # one slot named twice at one position is fine; a padding token's conflict is not looked at
    oracle.gather_compact_stash(bank, np.array([[0, 0], [2, 3]]), np.array([[0, 0], [0, 1]], np.int32), stash,
                                chunk=2, valid=1)
    assert bits_equal(stash[0, 0], bank[0])
