"""The plain C caller (sparse_delta_rule_amd/examples/sdm_example.c) against the oracle.

The example uses libsdm through include/sdm.h alone — HIP runtime calls from C,
a caller-created stream, three sdm_decode_step calls, one sdm_gather and one
rejected call — and prints its results as raw bits. Its inputs are closed-form
integer patterns stated in its header comment; they are rebuilt here from that
statement, run through the oracle, and every printed bit is compared.
"""

import os
import subprocess

import numpy as np
import pytest

import oracle
from tests.helpers import documented_decode_groups

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "sparse_delta_rule_amd", "examples", "sdm_example")

S, P, HD, W, R, T = 3, 8, 8, 3, 2, 3
NS = S * P
GT, GW0, GW1, CHUNK, VALID = 8, 3, 2, 4, 3


def _bf16_bits(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _inputs():
    i, c = np.meshgrid(np.arange(NS), np.arange(HD), indexing="ij")
    bank = _bf16_bits(((i * 7 + c * 3) % 17 - 8) / 16.0)
    steps = []
    for t in range(T):
        s = np.arange(S)[:, None]
        w, r, cc = np.arange(W)[None, :], np.arange(R)[None, :], np.arange(HD)[None, :]
        steps.append(dict(
            k_idx=(s * P + (t * 5 + w * 3 + s) % P).astype(np.int64),
            k_val=(((t + 2 * s + w) % 5 - 2) / 4.0).astype(np.float32),
            v=(((3 * t + s + cc) % 9 - 4) / 8.0).astype(np.float32),
            beta=((1 + (t + np.arange(S)) % 3) / 4.0).astype(np.float32),
            g=(-((t + s + w) % 4) / 16.0).astype(np.float32),
            q_idx=(s * P + (t * 2 + r * 5 + 1) % P).astype(np.int64),
            q_val=(((t + s + 3 * r) % 7 - 3) / 8.0).astype(np.float32)))
    tt = np.arange(GT)[:, None]
    n0, n1 = np.arange(GW0)[None, :], np.arange(GW1)[None, :]
    gather = dict(idx0=((tt * 11 + n0 * 7) % NS).astype(np.int64), w0=(((tt + n0) % 5 - 2) / 2.0).astype(np.float32),
                  idx1=((tt * 3 + n1 * 13 + 5) % NS).astype(np.int64),
                  w1=(((2 * tt + n1) % 3 - 1) / 4.0).astype(np.float32))
    return bank, steps, gather


def _parse(text):
    arrays, status = {}, {}
    for line in text.splitlines():
        f = line.split()
        if not f:
            continue
        if f[0] == "status":
            status[f[1]] = int(f[2])
            continue
        n = int(f[1])
        vals = [int(x, 16) for x in f[2:]]
        assert len(vals) == n, line[:80]
        arrays[f[0]] = np.array(vals, np.uint32 if len(f[2]) == 8 else np.uint16)
    return arrays, status


def test_c_example_matches_the_oracle():
    assert os.path.exists(EXE), f"{EXE} is not built; run `python -m sparse_delta_rule_amd.build`"
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    got, status = _parse(r.stdout)

    bank, steps, gather = _inputs()
    rg = documented_decode_groups(W, R)
    reads = [oracle.decode_step(bank, **st, groups=rg) for st in steps]  # bank changes in place
    assert np.array_equal(got["readings"], np.concatenate([x.ravel() for x in reads]))
    assert np.array_equal(got["bank"], bank.ravel())
    out0, stash, out1 = oracle.gather(bank, gather["idx0"], gather["w0"], chunk=CHUNK, valid=VALID,
                                      idx1=gather["idx1"], w1=gather["w1"])
    assert np.array_equal(got["out0"], out0.view(np.uint32).ravel())
    assert np.array_equal(got["out1"], out1.view(np.uint32).ravel())
    assert np.array_equal(got["stash"], stash.ravel())
    assert status["width_257"] == 3  # SDM_E_RANGE
    # the patterns make the call non-trivial: rows changed, padding present, sums nonzero
    assert (out0 != 0).any() and not out0[3].any() and (got["readings"] != 0).any()
