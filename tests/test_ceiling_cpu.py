"""libsdm_ceiling without a GPU: it loads, exports what include/sdm_ceiling.h
declares, and rejects bad arguments on the host before any HIP call (fake,
never dereferenced device addresses); and bench.py's summary of a ceiling
profile."""

import ctypes
import json
import os
import re
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from sparse_delta_rule_amd import ceiling  # noqa: E402
import bench  # noqa: E402

HEADER = os.path.join(ROOT, "include", "sdm_ceiling.h")
A = 0x10000000


def _declared():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"\b(sdm_ceiling_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = ceiling.library()
    names = _declared()
    assert names == ["sdm_ceiling_copy", "sdm_ceiling_last_error", "sdm_ceiling_rows", "sdm_ceiling_sink_words"]
    for n in names:
        assert hasattr(lib, n), n
    text = open(HEADER).read()
    for name, val in (("SDM_CEIL_READ", ceiling.READ), ("SDM_CEIL_STASH", ceiling.STASH),
                      ("SDM_CEIL_RMW", ceiling.RMW), ("SDM_CEIL_MIX", ceiling.MIX)):
        assert int(re.search(rf"\b{name} = (\d+)", text).group(1)) == val
    assert ceiling.sink_words() == 2048 * 256


@pytest.mark.parametrize("args,code,msg", [
    ((7, A, 16, 256, A, 4, None, A), 2, "unknown mode"),
    ((0, A, 0, 256, A, 4, None, A), 2, "num_rows >= 1"),
    ((0, A, 16, 100, A, 4, None, A), 2, "multiple of 16"),
    ((0, A, 16, 2048, A, 4, None, A), 2, "multiple of 16"),
    ((0, A, 16, 256, A, -1, None, A), 2, "n >= 0"),
    ((0, None, 16, 256, A, 4, None, A), 6, "bank and rows"),
    ((1, A, 16, 256, A, 4, None, None), 6, "needs a stash"),
    ((3, A, 16, 256, A, 4, None, None), 6, "need a sink"),
    ((2, A + 8, 16, 256, A, 4, None, None), 2, "16-byte aligned"),
])
def test_rows_rejects_bad_arguments(args, code, msg):
    lib = ceiling.library()
    assert lib.sdm_ceiling_rows(*args, None) == code
    assert msg in lib.sdm_ceiling_last_error().decode()


def test_nothing_to_do_is_ok():
    lib = ceiling.library()
    assert lib.sdm_ceiling_rows(0, A, 16, 256, A, 0, None, None, None) == 0
    assert lib.sdm_ceiling_copy(A, A + 4096, 0, 0, None) == 0


def test_copy_rejects_bad_arguments():
    lib = ceiling.library()
    assert lib.sdm_ceiling_copy(A, A + 4096, 24, 0, None) == 2
    assert lib.sdm_ceiling_copy(None, A, 32, 1, None) == 6
    assert lib.sdm_ceiling_copy(A + 4, A + 4096, 32, 0, None) == 2


def test_plans_move_the_stated_bytes():
    for gib in (4, 16):
        assert bench.ceiling_plan("read", gib, 256) == (2 << 20, 1, (2 << 20) * 256)
        assert bench.ceiling_plan("stash", gib, 256)[2] == 2 * (2 << 20) * 256
        n, per, moved = bench.ceiling_plan("mix", gib, 256)
        assert per == 2 and moved == 3 * n * 256
        # distinct rows for every timed launch and the untimed one fit the bank
        assert n * per * (bench.CEILING_LAUNCHES + 1) <= gib * (1 << 30) // 256
    assert bench.ceiling_plan("copy", 4, 256)[2] == 2 << 30


def _write_csv(path, header, rows):
    import csv
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_ingest_ceiling(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    rd = "void (anonymous namespace)::ceiling_rows_kernel<0, 8>(HIP_vector_type<unsigned int, 4u>*, int)"
    mx = "void (anonymous namespace)::ceiling_rows_kernel<3, 4>(HIP_vector_type<unsigned int, 4u>*, int)"
    cp = "void at::native::elementwise_kernel<128, 4>(int, float)"
    t, f, w, cf, cw = (str(tmp_path / n) for n in ("t", "f", "w", "cf", "cw"))
    n_read, _, b_read = bench.ceiling_plan("read", 16, 256)
    n_mix, _, b_mix = bench.ceiling_plan("mix", 16, 256)
    _write_csv(os.path.join(t, "run_kernel_stats.csv"), ["Name", "Calls", "AverageNs", "MinNs", "MaxNs"],
               [[rd, 9, b_read / 5000.0, 0, 0], [mx, 9, b_mix / 4000.0, 0, 0]])
    _write_csv(os.path.join(f, "run_counter_collection.csv"), ["Kernel_Name", "Counter_Value"],
               [[rd, b_read / 2048.0], [mx, b_mix * 2 / 3 / 2048.0]])
    _write_csv(os.path.join(w, "run_counter_collection.csv"), ["Kernel_Name", "Counter_Value"],
               [[rd, 1.0], [mx, b_mix / 3 / 1024.0]])
    _write_csv(os.path.join(cf, "run_counter_collection.csv"), ["Kernel_Name", "Counter_Value"], [[cp, 524288.0]])
    _write_csv(os.path.join(cw, "run_counter_collection.csv"), ["Kernel_Name", "Counter_Value"], [[cp, 1048576.0]])
    assert bench.main(["--bank-gib", "16", "--ingest-ceiling", t, f, w, cf, cw]) == 0
    data = json.load(open(tmp_path / "profiles" / "ceiling.json"))["16GiB/256B/uniform"]
    assert data["read"]["frac"] == pytest.approx(5000.0 / 8000.0)
    assert data["mix"]["frac"] == pytest.approx(0.5)
    assert data["mix"]["fetch_bytes"] + data["mix"]["write_bytes"] == pytest.approx(b_mix)
    md = (tmp_path / "profiles" / "sdm_ceiling_bank_16gib_rows_256b_uniform.md").read_text()
    assert "| mix |" in md and "| read |" in md


def test_stream_layout_rows():
    """The streams layout gives each run of units distinct rows inside its own range,
    written rows paired with read rows."""
    import torch
    g = torch.Generator()
    g.manual_seed(0)
    rows = bench.ceiling_stream_rows(torch, 16384 * 3, 2, g, "cpu").view(3, 64, 2)
    for s in range(3):
        r = rows[s].reshape(-1)
        assert int(r.min()) >= s * 16384 and int(r.max()) < (s + 1) * 16384
        assert r.unique().numel() == 128
    n, per, moved = bench.ceiling_plan("mix", 16, 256, "streams")
    assert (n, per, moved) == (4096 * 64, 2, 4096 * 192 * 256)  # the c2 step's rows
