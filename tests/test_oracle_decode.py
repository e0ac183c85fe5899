"""Pins of the decode oracle against what the method's definition fixes.

Definition: page "sparse_delta_memory/decode.py", docstring of sdm_decode_step
(retrieve, delta, decay-and-write of the written rows, read after the write;
k_val, v, q_val rounded to the bank dtype; beta and g in float32). Each test
below would fail for a plausible slip in the oracle: a dropped term, a wrong
sign, a transposed operand, a wrong gate index, reads before the write, or
rounding at the wrong point.
"""

import json
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle
from tests.helpers import (bits_equal, f32_to_bf16_bits_torch, gamma, random_decode_case,
                           round_to_bank_torch, ulp, widen)


def _bank(values, bf16):
    a = np.asarray(values, dtype=np.float32)
    return f32_to_bf16_bits_torch(a) if bf16 else a.copy()


def _step(case, groups=1, bank=None):
    bank = case["bank"].copy() if bank is None else bank
    r = oracle.decode_step(bank, case["k_idx"], case["k_val"], case["v"], case["beta"], case["g"],
                           case["q_idx"], case["q_val"], groups=groups)
    return bank, r


def _step64(case, bank=None):
    bank = case["bank"].copy() if bank is None else bank
    out = oracle.decode_step_f64(bank, case["k_idx"], case["k_val"], case["v"], case["beta"],
                                 case["g"], case["q_idx"], case["q_val"])
    return (bank,) + out


# ------------------------------------------------------------ worked examples
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("groups", [1, 2, 3])
def test_handworked_cases(golden_dir, bf16, groups):
    data = json.load(open(os.path.join(golden_dir, "decode_handworked.json")))
    for c in data["cases"]:
        case = {k: np.asarray(c[k]) for k in ("k_idx", "k_val", "v", "beta", "g", "q_idx", "q_val")}
        case["bank"] = _bank(c["bank"], bf16)
        bank, readings = _step(case, groups)
        assert np.array_equal(widen(bank), np.asarray(c["bank_after"], np.float32)), c["name"]
        assert np.array_equal(widen(readings), np.asarray(c["readings"], np.float32)), c["name"]
        bank64, readings64, *_ = _step64(case)
        assert np.array_equal(widen(bank64), np.asarray(c["bank_after"], np.float32)), c["name"]
        assert np.array_equal(widen(readings64), np.asarray(c["readings"], np.float32)), c["name"]


# ------------------------------------------------------------------ identities
@pytest.mark.parametrize("bf16", [False, True])
def test_zero_gate_zero_beta_leaves_bank(bf16):
    rng = np.random.default_rng(1)
    case = random_decode_case(rng, streams=3, slots_per_stream=16, hd=7, W=5, R=4, G=1, bf16=bf16)
    case["g"][:] = 0.0
    case["beta"][:] = 0.0
    bank, readings = _step(case)
    assert np.array_equal(widen(bank), widen(case["bank"]))
    # readings are then q . (old rows), each rounded once to the bank dtype
    old = widen(case["bank"]).astype(np.float64)
    qv = round_to_bank_torch(case["q_val"], bf16).astype(np.float64)
    exact = np.einsum("sr,src->sc", qv, old[case["q_idx"]])
    mag = np.einsum("sr,src->sc", np.abs(qv), np.abs(old[case["q_idx"]]))
    err = np.abs(widen(readings) - exact)
    assert np.all(err <= gamma(6) * mag + ulp(exact, bf16))


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("G", ["one", "per_write"])
def test_beta_zero_decays_written_rows_only(bf16, G):
    rng = np.random.default_rng(2)
    W = 6
    case = random_decode_case(rng, streams=2, slots_per_stream=20, hd=5, W=W, R=3,
                              G=1 if G == "one" else W, bf16=bf16)
    case["beta"][:] = 0.0
    bank, _ = _step(case)
    d = np.exp(case["g"].astype(np.float64)).astype(np.float32)  # pinned separately below
    old = widen(case["bank"])
    for s in range(2):
        for w in range(W):
            dw = d[s, 0 if G == "one" else w]
            want = round_to_bank_torch(old[case["k_idx"][s, w]] * dw, bf16)
            assert np.array_equal(widen(bank[case["k_idx"][s, w]]), want)
    untouched = np.setdiff1d(np.arange(old.shape[0]), case["k_idx"].ravel())
    assert bits_equal(bank[untouched], case["bank"][untouched])


@pytest.mark.parametrize("bf16", [False, True])
def test_zero_key_weight_with_zero_gate_is_bit_identity(bf16):
    rng = np.random.default_rng(3)
    case = random_decode_case(rng, streams=3, slots_per_stream=12, hd=9, W=4, R=4, G=4, bf16=bf16)
    case["k_val"][:] = 0.0
    case["g"][:] = 0.0
    bank, _ = _step(case)
    assert bits_equal(bank, case["bank"])


@pytest.mark.parametrize("bf16", [False, True])
def test_zero_key_weight_decays(bf16):
    """k_val = 0: retrieved = 0 and each written row becomes rb(d * row)."""
    rng = np.random.default_rng(4)
    case = random_decode_case(rng, streams=2, slots_per_stream=12, hd=4, W=3, R=2, G=1, bf16=bf16)
    case["k_val"][:] = 0.0
    bank, _ = _step(case)
    d = np.exp(case["g"].astype(np.float64)).astype(np.float32)
    old = widen(case["bank"])
    for s in range(2):
        want = round_to_bank_torch(old[case["k_idx"][s]] * d[s, 0], bf16)
        assert np.array_equal(widen(bank[case["k_idx"][s]]), want)


@pytest.mark.parametrize("bf16", [False, True])
def test_untouched_rows_bit_identical(bf16):
    rng = np.random.default_rng(5)
    case = random_decode_case(rng, streams=4, slots_per_stream=30, hd=11, W=7, R=9, G=7, bf16=bf16)
    bank, _ = _step(case)
    untouched = np.setdiff1d(np.arange(bank.shape[0]), case["k_idx"].ravel())
    assert bits_equal(bank[untouched], case["bank"][untouched])
    assert not bits_equal(bank, case["bank"])


# ----------------------------------------------------------- read after write
@pytest.mark.parametrize("bf16", [False, True])
def test_read_after_write_is_the_stored_row(bf16):
    """q_idx = k_idx with one-hot q_val: readings are the new rows, bit for bit."""
    rng = np.random.default_rng(6)
    W = 5
    for j in range(W):
        case = random_decode_case(rng, streams=3, slots_per_stream=10, hd=6, W=W, R=W, G=1,
                                  bf16=bf16, overlap="all")
        case["q_val"][:] = 0.0
        case["q_val"][:, j] = 1.0
        bank, readings = _step(case)
        for s in range(3):
            assert np.array_equal(widen(readings[s]), widen(bank[case["k_idx"][s, j]]))
        # and they differ from the rows before the write (the read did not see the old bank)
        assert not np.array_equal(widen(readings), widen(case["bank"][case["k_idx"][:, j]]))


def test_repeated_read_slot_counts_twice():
    rng = np.random.default_rng(7)
    case = random_decode_case(rng, streams=2, slots_per_stream=8, hd=3, W=2, R=2, G=1, bf16=False,
                              overlap="none")
    case["q_idx"][:, 1] = case["q_idx"][:, 0]
    case["q_val"][:] = np.float32(0.75)
    bank, readings = _step(case)
    row = bank[case["q_idx"][:, 0]]
    assert np.allclose(readings, 1.5 * row, rtol=2 ** -22, atol=0)


# --------------------------------------------------------------- closed forms
def test_delta_rule_fixed_point():
    """g = 0, beta = 1/|k|^2: after the write, sum_w k_w row_w equals v."""
    rng = np.random.default_rng(8)
    for W in (1, 3, 8, 33):
        case = random_decode_case(rng, streams=3, slots_per_stream=64, hd=10, W=W, R=1, G=1, bf16=False)
        case["g"][:] = 0.0
        k = case["k_val"].astype(np.float64)
        case["beta"][:, 0] = (1.0 / np.sum(k * k, axis=1)).astype(np.float32)
        bank, _ = _step(case)
        new = bank[case["k_idx"]].astype(np.float64)  # [S, W, hd]
        got = np.einsum("sw,swc->sc", k, new)
        scale = np.einsum("sw,swc->sc", np.abs(k), np.abs(new)) + np.abs(case["v"])
        assert np.all(np.abs(got - case["v"]) <= 64 * W * 2 ** -24 * scale)


def test_single_write_full_strength_sets_value():
    """W = 1, k_val = 1, beta = 1, any gate: the written row becomes v."""
    rng = np.random.default_rng(9)
    case = random_decode_case(rng, streams=4, slots_per_stream=5, hd=16, W=1, R=1, G=1, bf16=False)
    case["k_val"][:] = 1.0
    case["beta"][:] = 1.0
    bank, _ = _step(case)
    new = bank[case["k_idx"][:, 0]]
    old = case["bank"][case["k_idx"][:, 0]]
    assert np.all(np.abs(new - case["v"]) <= 4 * 2 ** -24 * (np.abs(case["v"]) + np.abs(old)))


def test_decay_is_correctly_rounded_exp():
    """k_val = 0, beta = 0, row = 1: the stored row is d = exp(g), checked against a
    50-digit decimal exponential rounded to float32."""
    getcontext().prec = 50
    rng = np.random.default_rng(10)
    gs = np.concatenate([rng.uniform(-5, 0, 200), [0.0, -1e-30, -0.5, -2.0]]).astype(np.float32)
    S = gs.size
    case = dict(bank=np.ones((S, 1), np.float32), k_idx=np.arange(S)[:, None],
                k_val=np.zeros((S, 1), np.float32), v=np.zeros((S, 1), np.float32),
                beta=np.zeros((S, 1), np.float32), g=gs[:, None], q_idx=np.arange(S)[:, None],
                q_val=np.ones((S, 1), np.float32))
    bank, _ = _step(case)
    for i, gv in enumerate(gs):
        exact = Decimal(float(gv)).exp()
        got = Decimal(float(bank[i, 0]))
        spacing = Decimal(float(np.spacing(np.float32(bank[i, 0]))))
        assert abs(got - exact) <= spacing / 2 * Decimal("1.000001"), (gv, got, exact)


@pytest.mark.parametrize("bf16", [False, True])
def test_per_write_gate_uses_its_own_gate(bf16):
    """G = W: row w decays by exp(g[w]), not by exp(g[0])."""
    W = 4
    g = np.array([[0.0, np.log(0.5), np.log(0.25), np.log(0.125)]], np.float32)
    case = dict(bank=_bank(np.full((W, 1), 8.0), bf16), k_idx=np.arange(W)[None, :],
                k_val=np.zeros((1, W), np.float32), v=np.zeros((1, 1), np.float32),
                beta=np.zeros((1, 1), np.float32), g=g, q_idx=np.arange(W)[None, :],
                q_val=np.array([[1.0, 2.0, 4.0, 8.0]], np.float32))
    bank, readings = _step(case)
    assert np.array_equal(widen(bank)[:, 0], np.array([8.0, 4.0, 2.0, 1.0], np.float32))
    assert widen(readings)[0, 0] == 8.0 + 8.0 + 8.0 + 8.0


# ------------------------------------------------------- float64 brute force
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("groups", [1, 2, 4])
def test_float32_within_error_bound_of_float64(bf16, groups):
    rng = np.random.default_rng(11 + groups)
    for W, R, G in ((1, 1, 1), (3, 5, 3), (7, 4, 1), (16, 16, 16), (33, 20, 1)):
        case = random_decode_case(rng, streams=3, slots_per_stream=80, hd=6, W=W, R=R, G=G, bf16=bf16,
                                  overlap="none")
        bank32, r32 = _step(case, groups)
        bank64, r64, row_exact, row_mag, read_exact, read_mag = _step64(case)
        new32 = widen(bank32[case["k_idx"]]).astype(np.float64)
        bound_rows = gamma(W + 8) * row_mag + ulp(row_exact, bf16)
        assert np.all(np.abs(new32 - row_exact) <= bound_rows), (W, R, G)
        bound_read = gamma(R + 2) * read_mag + ulp(read_exact, bf16)
        assert np.all(np.abs(widen(r32) - read_exact) <= bound_read), (W, R, G)
        # the double path's stored values are the exact values rounded once
        assert np.all(np.abs(widen(bank64[case["k_idx"]]) - row_exact) <= ulp(row_exact, bf16) / 2)


def _order_case(rows_w, rows_r, groups):
    """float32 bank [rows_w; rows_r] (hd 1): write slots 0..W-1 with k_val = 1, g = 0,
    beta = 1, v = 0 (so delta_v = -retrieved and each written row becomes
    row - retrieved); read the untouched rows W.. with q_val = 1 (readings = their sum)."""
    W, R = len(rows_w), len(rows_r)
    bank = np.array([[x] for x in rows_w + rows_r], np.float32)
    r = oracle.decode_step(bank, np.arange(W)[None], np.ones((1, W), np.float32), np.zeros((1, 1), np.float32),
                           np.ones((1, 1), np.float32), np.zeros((1, 1), np.float32), np.arange(W, W + R)[None],
                           np.ones((1, R), np.float32), groups=groups)
    return bank[:W, 0].tolist(), float(r[0, 0])


def test_summation_order_is_the_stated_one():
    """Values for which the decode's float32 sums (over w, and over r) depend on the
    order: group j sums w = j, j + groups, ... ascending from +0, and the group
    partials are added in group order from +0. Near 2^24 adding 1 is a tie, which
    rounds to the even neighbour 2^24."""
    big = 2.0 ** 24
    # rows [2^24, 1, 1]: ((0 + 2^24) + 1) + 1 = 2^24 as one ascending chain and as three
    # groups in group order; a descending order would give (1 + 1) + 2^24 = 2^24 + 2.
    # delta_v = -2^24, so row 1 becomes 1 - 2^24 = -16777215 exactly (-16777216 after
    # a sum of 2^24 + 2).
    for groups in (1, 3):
        rows, read = _order_case([big, 1.0, 1.0], [big, 1.0, 1.0], groups)
        assert read == big
        assert rows == [0.0, -16777215.0, -16777215.0]
    # rows [2^24, 1, -2^24, 1]: one chain ((2^24 + 1) - 2^24) + 1 = 1; two strided groups
    # (2^24 - 2^24) + (1 + 1) = 2; contiguous halves would give (2^24 + 1) + (-2^24 + 1) = 1.
    rows, read = _order_case([big, 1.0, -big, 1.0], [big, 1.0, -big, 1.0], 1)
    assert read == 1.0
    # each row minus 1: 16777215, 0, -16777217 (a tie, to even: -16777216), 0
    assert rows == [16777215.0, 0.0, -16777216.0, 0.0]
    rows, read = _order_case([big, 1.0, -big, 1.0], [big, 1.0, -big, 1.0], 2)
    assert read == 2.0
    # each row minus 2: 16777214, -1, -16777218, -1 (all exact)
    assert rows == [16777214.0, -1.0, -16777218.0, -1.0]


def test_update_is_one_fused_multiply_add():
    """The new row is fma(k_val, delta_v, row * d) with row * d rounded first: one
    rounding for the k_val * delta_v term and the add. float32 bank, row = -1,
    k_val = 1 + 2^-12, g = 0, beta = 1, v = 0: retrieved = -(1 + 2^-12) and
    delta_v = 1 + 2^-12 exactly, and the exact k_val * delta_v = 1 + 2^-11 + 2^-24.
    Fused, the row becomes 2^-11 + 2^-24; a product rounded on its own (a tie,
    to the even 1 + 2^-11) would leave 2^-11."""
    kv = np.float32(1.0 + 2.0 ** -12)
    bank = np.array([[-1.0]], np.float32)
    r = oracle.decode_step(bank, np.array([[0]]), np.array([[kv]], np.float32), np.zeros((1, 1), np.float32),
                           np.ones((1, 1), np.float32), np.zeros((1, 1), np.float32), np.array([[0]]),
                           np.ones((1, 1), np.float32))
    assert bank[0, 0] == 2.0 ** -11 + 2.0 ** -24
    assert r[0, 0] == 2.0 ** -11 + 2.0 ** -24  # read after the write, q_val = 1


def test_delta_rounds_the_difference_then_the_product():
    """delta_v = beta * (v - retrieved) with two roundings, the difference first.
    float32 bank rows [-2^-24, 0] both written with k_val = 1, g = 0, v = 1,
    beta = 1 + 2^-23: retrieved = -2^-24, v - retrieved = 1 + 2^-24 rounds (a tie,
    to even) to 1, so delta_v = 1 + 2^-23, which row 1 (0 + 1 * delta_v) shows.
    One rounding of the exact beta (v - retrieved), or an fma form of it, would
    give 1 + 2^-22. Row 0 becomes -2^-24 + delta_v = 1 + 2^-24, a tie rounding to 1."""
    bank = np.array([[-(2.0 ** -24)], [0.0]], np.float32)
    r = oracle.decode_step(bank, np.array([[0, 1]]), np.ones((1, 2), np.float32), np.ones((1, 1), np.float32),
                           np.array([[1.0 + 2.0 ** -23]], np.float32), np.zeros((1, 1), np.float32),
                           np.array([[1]]), np.ones((1, 1), np.float32))
    assert bank[1, 0] == 1.0 + 2.0 ** -23
    assert bank[0, 0] == 1.0
    assert r[0, 0] == 1.0 + 2.0 ** -23


def test_coefficient_is_rounded_before_the_products():
    """coef = k_val * d is rounded to float32 before it multiplies the rows.
    g = 2^-12 gives d = 1 + 2^-12 (exp(2^-12) exceeds it by about a quarter ulp);
    k_val = 1 + 2^-12 makes k_val * d = 1 + 2^-11 + 2^-24, a tie rounding to
    coef = 1 + 2^-11. Against row 0 = -(1 + 2^-23): coef * row rounds to
    -(1 + 2^-11 + 2^-23), while one rounding of k_val * d * row, or k_val times a
    rounded d * row, gives -(1 + 2^-11 + 2^-22). With v = 0 and beta = 1 the
    second written row (0, k_val 1) becomes delta_v = -retrieved."""
    bank = np.array([[-(1.0 + 2.0 ** -23)], [0.0]], np.float32)
    oracle.decode_step(bank, np.array([[0, 1]]), np.array([[1.0 + 2.0 ** -12, 1.0]], np.float32),
                       np.zeros((1, 1), np.float32), np.ones((1, 1), np.float32),
                       np.array([[2.0 ** -12]], np.float32), np.array([[1]]), np.ones((1, 1), np.float32))
    assert bank[1, 0] == 1.0 + 2.0 ** -11 + 2.0 ** -23


def test_groups_agree_on_exact_integers():
    """Small-integer data make every sum exact: every grouping gives the same bits,
    so a term dropped by the grouped order would show."""
    rng = np.random.default_rng(12)
    for W in (1, 2, 5, 9, 64, 256):
        case = random_decode_case(rng, streams=2, slots_per_stream=300, hd=3, W=W, R=W, G=1, bf16=False)
        case["bank"] = rng.integers(-4, 5, case["bank"].shape).astype(np.float32)
        case["k_val"] = rng.integers(-3, 4, case["k_val"].shape).astype(np.float32)
        case["q_val"] = rng.integers(-3, 4, case["q_val"].shape).astype(np.float32)
        case["v"] = rng.integers(-8, 9, case["v"].shape).astype(np.float32)
        case["beta"][:] = 0.5
        case["g"][:] = 0.0
        ref_bank, ref_r = _step(case, 1)
        b64, r64, *_ = _step64(case)
        assert bits_equal(ref_bank, b64) and bits_equal(ref_r, r64)
        for groups in (2, 3, 4, 8, 32):
            bank, r = _step(case, groups)
            assert bits_equal(bank, ref_bank) and bits_equal(r, ref_r), (W, groups)


def test_streams_are_independent():
    """A run over a subset of streams gives those streams' results bit for bit."""
    rng = np.random.default_rng(13)
    P = 40
    case = random_decode_case(rng, streams=5, slots_per_stream=P, hd=8, W=6, R=6, G=6, bf16=True)
    bank, readings = _step(case)
    for s in (0, 3):
        sub = {k: case[k][s:s + 1] for k in ("k_val", "v", "beta", "g", "q_val")}
        sub["k_idx"] = case["k_idx"][s:s + 1] - s * P
        sub["q_idx"] = case["q_idx"][s:s + 1] - s * P
        sub["bank"] = case["bank"][s * P:(s + 1) * P].copy()
        b, r = _step(sub)
        assert bits_equal(b, bank[s * P:(s + 1) * P]) and bits_equal(r[0], readings[s])


def test_permuting_writes_changes_only_rounding():
    """Reordering the W (slot, weight, gate) entries leaves the exact result alone."""
    rng = np.random.default_rng(14)
    case = random_decode_case(rng, streams=3, slots_per_stream=50, hd=12, W=20, R=10, G=20, bf16=False)
    bank, readings = _step(case)
    perm = rng.permutation(20)
    p = dict(case)
    p["k_idx"], p["k_val"], p["g"] = case["k_idx"][:, perm], case["k_val"][:, perm], case["g"][:, perm]
    bank_p, readings_p = _step(p)
    _, _, row_exact, row_mag, read_exact, read_mag = _step64(case)
    new, new_p = bank[case["k_idx"]].astype(np.float64), bank_p[case["k_idx"]].astype(np.float64)
    assert np.all(np.abs(new - new_p) <= 2 * (gamma(28) * row_mag + ulp(row_exact, False)))
    assert np.all(np.abs(readings.astype(np.float64) - readings_p) <= 1e-5 * read_mag + 1e-30)
    assert not bits_equal(bank, case["bank"])


def test_preconditions_are_reported():
    rng = np.random.default_rng(15)
    case = random_decode_case(rng, streams=2, slots_per_stream=10, hd=2, W=3, R=2, G=1, bf16=False)
    dup = dict(case)
    dup["k_idx"] = case["k_idx"].copy()
    dup["k_idx"][1, 2] = dup["k_idx"][1, 0]
    with pytest.raises(ValueError, match="repeated write slot"):
        _step(dup)
    bad = dict(case)
    bad["q_idx"] = case["q_idx"].copy()
    bad["q_idx"][0, 0] = 20
    with pytest.raises(ValueError, match="out of range"):
        _step(bad)
