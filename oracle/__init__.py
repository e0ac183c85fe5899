"""CPU oracle for the sparse-delta-memory decode step and token gather.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product package. The arithmetic
lives in ``sdm_oracle.c`` (plain sequential C, float32 at the method's rounding
points, plus float64 brute-force versions); this module only marshals numpy
arrays into it.

Parity pins (the tests under ``tests/`` named ``test_oracle_*``) tie every
function here to the method's definitions: hand-worked dyadic cases, closed
forms, identities, read-after-write, a float64 brute force with an error bound,
and a library routine for the bfloat16 rounding. The decode's float32 choices
that the method leaves open (the summation order, k_val * d rounded before the
products, delta_v's two roundings, the fused update) are pinned by worked
float32 values that the other plausible choices miss, on top of the bound.
tests/test_oracle_mutants.py runs the pins against broken copies of the C
source and requires each copy to fail one of them.

Bank arrays are float32, or uint16 holding bfloat16 bits.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sdm_oracle.c")
_LIB = os.path.join(_HERE, "libsdm_oracle.so")
# SDM_ORACLE_LIBRARY names another build of sdm_oracle.c to load instead (used by
# the test that runs the pins against deliberately broken copies); it is loaded
# as it is, never rebuilt.
_LIB_OVERRIDE = os.environ.get("SDM_ORACLE_LIBRARY", "")

_lib = None

_ERRORS = {-1: "bad sizes or widths", -2: "slot out of range", -3: "repeated write slot in a stream",
           -4: "out of memory", -5: "compact-stash position past its block or named by two slots"}


def build() -> str:
    """Compile the oracle with gcc (no contraction, no fast-math)."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC", "-shared",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i64, i32 = ctypes.c_int64, ctypes.c_int
    lib.sdm_oracle_decode_step.argtypes = [P, i32, i64, i64, i64, i32, i32, i32, i32,
                                           P, P, P, P, P, P, P, P]
    lib.sdm_oracle_decode_step_f64.argtypes = [P, i32, i64, i64, i64, i32, i32, i32,
                                               P, P, P, P, P, P, P, P, P, P, P, P]
    lib.sdm_oracle_gather.argtypes = [P, i32, i64, i64, i64, i64, i64, P, P, P, i32, P, P,
                                      P, P, i32, P, i32]
    lib.sdm_oracle_gather_f64.argtypes = [P, i32, i64, i64, i64, i64, i64, P, P, P, i32, P, P]
    lib.sdm_oracle_gather_compact_stash.argtypes = [P, i32, i64, i64, i64, i64, i64, P, P, i32, P, P]
    lib.oracle_float_to_bf16.argtypes = [ctypes.c_float]
    lib.oracle_float_to_bf16.restype = ctypes.c_uint16
    lib.oracle_double_to_bf16.argtypes = [ctypes.c_double]
    lib.oracle_double_to_bf16.restype = ctypes.c_uint16
    lib.oracle_float_to_bf16_array.argtypes = [P, P, i64]
    lib.oracle_float_to_bf16_array.restype = None
    lib.oracle_bf16_to_float.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_float.restype = ctypes.c_float
    for f in (lib.sdm_oracle_decode_step, lib.sdm_oracle_decode_step_f64, lib.sdm_oracle_gather,
              lib.sdm_oracle_gather_f64, lib.sdm_oracle_gather_compact_stash):
        f.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what}: {_ERRORS.get(rc, rc)}")


def _bank_kind(bank: np.ndarray) -> int:
    if bank.dtype == np.float32:
        return 0
    if bank.dtype == np.uint16:
        return 1
    raise TypeError("bank must be float32 or uint16 (bfloat16 bits)")


def _f32(x):
    return np.ascontiguousarray(x, dtype=np.float32)


def _i64(x):
    return np.ascontiguousarray(x, dtype=np.int64)


def float_to_bf16(x: float) -> int:
    return int(_load().oracle_float_to_bf16(float(x)))


def float_to_bf16_array(x: np.ndarray) -> np.ndarray:
    """oracle_float_to_bf16 of every element of a float32 array (uint16 bits)."""
    x = _f32(x)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_float_to_bf16_array(_ptr(x), _ptr(out), x.size)
    return out


def double_to_bf16(x: float) -> int:
    return int(_load().oracle_double_to_bf16(float(x)))


def bf16_to_float(b: int) -> float:
    return float(_load().oracle_bf16_to_float(int(b)))


def decode_step(bank, k_idx, k_val, v, beta, g, q_idx, q_val, groups: int = 1):
    """One decode step for every stream, float32 path. ``bank`` changes in place.

    Shapes: bank [slots, hd]; k_idx, k_val [S, W]; v [S, hd]; beta [S] or [S, 1];
    g [S, G]; q_idx, q_val [S, R]. Returns readings [S, hd] in the bank dtype.
    ``groups`` fixes the summation order (see sdm_oracle.c).
    """
    assert bank.flags.c_contiguous
    bf = _bank_kind(bank)
    k_idx, q_idx = _i64(k_idx), _i64(q_idx)
    S, W = k_idx.shape
    R = q_idx.shape[1]
    g = _f32(g).reshape(S, -1)
    hd = bank.shape[1]
    readings = np.empty((S, hd), dtype=bank.dtype)
    k_val, v, q_val = _f32(k_val), _f32(v), _f32(q_val)
    beta = _f32(beta).reshape(S)
    rc = _load().sdm_oracle_decode_step(
        _ptr(bank), bf, bank.shape[0], hd, S, W, R, g.shape[1], groups,
        _ptr(k_idx), _ptr(k_val), _ptr(v), _ptr(beta), _ptr(g),
        _ptr(q_idx), _ptr(q_val), _ptr(readings))
    _check(rc, "decode_step")
    return readings


def decode_step_f64(bank, k_idx, k_val, v, beta, g, q_idx, q_val):
    """Float64 brute force of one step. ``bank`` changes in place (rounded from double).

    Returns (readings, row_exact [S,W,hd], row_mag [S,W,hd], read_exact [S,hd], read_mag [S,hd]).
    """
    bf = _bank_kind(bank)
    k_idx, q_idx = _i64(k_idx), _i64(q_idx)
    S, W = k_idx.shape
    R = q_idx.shape[1]
    g = _f32(g).reshape(S, -1)
    hd = bank.shape[1]
    readings = np.empty((S, hd), dtype=bank.dtype)
    row_exact = np.empty((S, W, hd)); row_mag = np.empty((S, W, hd))
    read_exact = np.empty((S, hd)); read_mag = np.empty((S, hd))
    k_val, v, q_val = _f32(k_val), _f32(v), _f32(q_val)
    beta = _f32(beta).reshape(S)
    rc = _load().sdm_oracle_decode_step_f64(
        _ptr(bank), bf, bank.shape[0], hd, S, W, R, g.shape[1],
        _ptr(k_idx), _ptr(k_val), _ptr(v), _ptr(beta), _ptr(g),
        _ptr(q_idx), _ptr(q_val), _ptr(readings),
        _ptr(row_exact), _ptr(row_mag), _ptr(read_exact), _ptr(read_mag))
    _check(rc, "decode_step_f64")
    return readings, row_exact, row_mag, read_exact, read_mag


def gather(bank, idx0, w0, *, chunk, valid=None, chunk_valid=None, idx1=None, w1=None,
           stash=True, groups: int = 1):
    """Token gather, float32 path. Returns (out0, stash or None, out1 or None).

    ``valid``: one count for every chunk; ``chunk_valid``: one count per chunk
    (takes precedence). Weights are widened to float32 exactly.
    """
    bf = _bank_kind(bank)
    idx0 = _i64(idx0)
    T, W0 = idx0.shape
    hd = bank.shape[1]
    if valid is None:
        valid = chunk
    cv = None if chunk_valid is None else np.ascontiguousarray(chunk_valid, dtype=np.int32)
    out0 = np.empty((T, hd), dtype=np.float32)
    st = np.empty((T, W0, hd), dtype=bank.dtype) if stash else None
    if idx1 is not None:
        idx1 = _i64(idx1)
        out1 = np.empty((T, hd), dtype=np.float32)
        W1 = idx1.shape[1]
        w1 = _f32(w1)
    else:
        out1, W1 = None, 0
    w0 = _f32(w0)
    rc = _load().sdm_oracle_gather(
        _ptr(bank), bf, bank.shape[0], hd, T, chunk, valid, _ptr(cv), _ptr(idx0), _ptr(w0),
        W0, _ptr(out0), _ptr(st), _ptr(idx1), _ptr(w1), W1, _ptr(out1), groups)
    _check(rc, "gather")
    return out0, st, out1


def gather_compact_stash(bank, idx0, kpos, stash, *, chunk, valid=None, chunk_valid=None):
    """The compact stash of operand 0, written into ``stash`` [tokens / chunk,
    chunk * width0, hd] (bank dtype) in place and returned: a live entry with
    kpos >= 0 copies its row to that position of its chunk's block; other rows
    keep their contents. The outputs are those of ``gather``."""
    bf = _bank_kind(bank)
    idx0 = _i64(idx0)
    T, W0 = idx0.shape
    kp = np.ascontiguousarray(kpos, dtype=np.int32)
    assert kp.shape == (T, W0)
    hd = bank.shape[1]
    assert stash.dtype == bank.dtype and stash.flags.c_contiguous and stash.size == T * W0 * hd
    if valid is None:
        valid = chunk
    cv = None if chunk_valid is None else np.ascontiguousarray(chunk_valid, dtype=np.int32)
    rc = _load().sdm_oracle_gather_compact_stash(_ptr(bank), bf, bank.shape[0], hd, T, chunk, valid, _ptr(cv),
                                                 _ptr(idx0), W0, _ptr(kp), _ptr(stash))
    _check(rc, "gather_compact_stash")
    return stash


def gather_f64(bank, idx, w, *, chunk, valid=None, chunk_valid=None):
    """Exact (double) sums of one operand and sum |w row| per output."""
    bf = _bank_kind(bank)
    idx = _i64(idx)
    T, W = idx.shape
    hd = bank.shape[1]
    if valid is None:
        valid = chunk
    cv = None if chunk_valid is None else np.ascontiguousarray(chunk_valid, dtype=np.int32)
    out = np.empty((T, hd)); mag = np.empty((T, hd))
    w = _f32(w)
    rc = _load().sdm_oracle_gather_f64(_ptr(bank), bf, bank.shape[0], hd, T, chunk, valid, _ptr(cv),
                                       _ptr(idx), _ptr(w), W, _ptr(out), _ptr(mag))
    _check(rc, "gather_f64")
    return out, mag


# ------------------------------------------------------------ array helpers
def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bits (uint16) to float32, exactly."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def bank_to_f32(bank: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(bank) if bank.dtype == np.uint16 else bank.astype(np.float32)
