"""The C ABI without a GPU: the library loads, exports what include/sdm.h
declares, and rejects bad arguments on the host before any HIP call.

Every call here passes fake (never dereferenced) device addresses; each case
is one that the host checks turn into a status code, so no kernel is launched.
"""

import ctypes
import os
import re
import threading

import pytest

import sparse_delta_rule_amd as sdm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdm.h")

OK, E_DTYPE, E_SHAPE, E_RANGE, E_ALIGN, E_OVERLAP, E_NULL = 0, 1, 2, 3, 4, 5, 6
F32, BF16, I32, I64 = 0, 1, 2, 3

A = 0x10000000  # fake, 256-byte aligned device addresses, far apart
MB = 1 << 20


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sdm_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert _declared_functions() == ["sdm_abi_version", "sdm_decode_step", "sdm_decode_steps",
                                     "sdm_gather", "sdm_gather_compact", "sdm_gather_plan_init",
                                     "sdm_gather_plan_launch", "sdm_last_error", "sdm_round_bf16"]


@pytest.mark.parametrize("args,code,msg", [
    ((A, A + MB, -1), E_SHAPE, "n = -1 < 0"),
    ((None, A + MB, 4), E_NULL, "in and out are required"),
    ((A, None, 4), E_NULL, "in and out are required"),
    ((A + 4, A + MB, 4), E_ALIGN, "8-byte"),
    ((A, A + MB + 2, 4), E_ALIGN, "4-byte"),
    ((A, A + 8, 4), E_OVERLAP, "overlap"),
])
def test_round_bf16_rejects_bad_arguments(args, code, msg):
    lib = sdm.library()
    assert lib.sdm_round_bf16(*args, None) == code
    assert msg in lib.sdm_last_error().decode()


def test_round_bf16_of_nothing_is_ok():
    assert sdm.library().sdm_round_bf16(A, A + MB, 0, None) == OK


def test_library_exports_every_declared_symbol():
    lib = sdm.library()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    m = re.search(r"#define SDM_ABI_VERSION (\d+)", open(HEADER).read())
    assert sdm.abi_version() == int(m.group(1))


def test_constants_match_the_header():
    text = open(HEADER).read()
    for name in ("SDM_F32", "SDM_BF16", "SDM_I32", "SDM_I64"):
        m = re.search(rf"\b{name} = (\d+)", text)
        assert int(m.group(1)) == getattr(sdm, name)
    m = re.search(r"#define SDM_MAX_WIDTH (\d+)", text)
    assert int(m.group(1)) == sdm.SDM_MAX_WIDTH


# ------------------------------------------------------------------ decode
def decode_args(**kw):
    a = dict(bank=A, bank_dtype=BF16, num_slots=1024, head_dim=128, streams=8, W=4, R=4, G=1,
             k_idx=A + 1024 * MB, k_idx_dtype=I64, k_val=A + 1100 * MB, v=A + 1200 * MB,
             q_val=A + 1300 * MB, val_dtype=F32, beta=A + 1400 * MB, g=A + 1500 * MB,
             q_idx=A + 1600 * MB, q_idx_dtype=I32, readings=A + 1700 * MB, stream=None)
    a.update(kw)
    return a


def call_decode(**kw):
    a = decode_args(**kw)
    lib = sdm.library()
    rc = lib.sdm_decode_step(a["bank"], a["bank_dtype"], a["num_slots"], a["head_dim"], a["streams"],
                             a["W"], a["R"], a["G"], a["k_idx"], a["k_idx_dtype"], a["k_val"], a["v"],
                             a["q_val"], a["val_dtype"], a["beta"], a["g"], a["q_idx"], a["q_idx_dtype"],
                             a["readings"], a["stream"])
    return rc, lib.sdm_last_error().decode()


@pytest.mark.parametrize("kw,code,text", [
    (dict(bank_dtype=I32), E_DTYPE, "bank must be"),
    (dict(bank_dtype=7), E_DTYPE, "bank must be"),
    (dict(val_dtype=I64), E_DTYPE, "k_val, v, q_val"),
    (dict(k_idx_dtype=F32), E_DTYPE, "k_idx and q_idx"),
    (dict(q_idx_dtype=BF16), E_DTYPE, "k_idx and q_idx"),
    (dict(num_slots=0), E_SHAPE, "empty bank"),
    (dict(head_dim=0), E_SHAPE, "empty bank"),
    (dict(head_dim=(1 << 28) + 1, bank_dtype=F32), E_RANGE, "a bank row would exceed"),
    (dict(head_dim=(1 << 29) + 1, bank_dtype=BF16), E_RANGE, "a bank row would exceed"),
    (dict(streams=-1), E_SHAPE, "streams"),
    (dict(W=0), E_RANGE, "each width must lie in 1..256"),
    (dict(W=257), E_RANGE, "each width must lie in 1..256"),
    (dict(R=0), E_RANGE, "each width must lie in 1..256"),
    (dict(R=300), E_RANGE, "each width must lie in 1..256"),
    (dict(G=2), E_SHAPE, "G must be 1 or W"),
    (dict(W=4, G=5), E_SHAPE, "G must be 1 or W"),
    (dict(bank=None), E_NULL, "bank is NULL"),
    (dict(beta=None), E_NULL, "beta is NULL"),
    (dict(readings=None), E_NULL, "readings is NULL"),
    (dict(q_idx=None), E_NULL, "q_idx is NULL"),
    (dict(bank=A + 1), E_ALIGN, "aligned"),
    (dict(k_idx=A + 1024 * MB + 4), E_ALIGN, "aligned"),
    (dict(g=A + 1500 * MB + 2), E_ALIGN, "aligned"),
    (dict(readings=A + 2 * 128 * 100), E_OVERLAP, "overlap"),
    (dict(readings=A - 2 * 128 * 8 + 2), E_OVERLAP, "overlap"),
    (dict(num_slots=1 << 62, head_dim=1 << 10), E_SHAPE, "overflow"),
    (dict(streams=1 << 31), E_SHAPE, "2^31-1 streams"),
])
def test_decode_rejects(kw, code, text):
    rc, msg = call_decode(**kw)
    assert rc == code, msg
    assert text in msg


def test_decode_zero_streams_is_a_no_op():
    rc, msg = call_decode(streams=0, bank=None, readings=None)
    assert rc == OK and msg == ""


def call_decode_steps(steps, **kw):
    a = decode_args(**kw)
    lib = sdm.library()
    rc = lib.sdm_decode_steps(a["bank"], a["bank_dtype"], a["num_slots"], a["head_dim"], steps, a["streams"],
                              a["W"], a["R"], a["G"], a["k_idx"], a["k_idx_dtype"], a["k_val"], a["v"],
                              a["q_val"], a["val_dtype"], a["beta"], a["g"], a["q_idx"], a["q_idx_dtype"],
                              a["readings"], a["stream"])
    return rc, lib.sdm_last_error().decode()


@pytest.mark.parametrize("steps,kw,code,text", [
    (-1, {}, E_SHAPE, "steps = -1"),
    (4, dict(W=0), E_RANGE, "each width must lie in 1..256"),
    (4, dict(G=3), E_SHAPE, "G must be 1 or W"),
    (4, dict(v=None), E_NULL, "v is NULL"),
    (4, dict(q_val=A + 1300 * MB + 2, val_dtype=F32), E_ALIGN, "aligned"),
    # readings [4, 8, 128] bf16 end 2 bytes into the bank
    (4, dict(readings=A - 4 * 8 * 128 * 2 + 2), E_OVERLAP, "overlap"),
    (1 << 40, dict(streams=1 << 20), E_SHAPE, "overflow"),
])
def test_decode_steps_rejects(steps, kw, code, text):
    rc, msg = call_decode_steps(steps, **kw)
    assert rc == code, msg
    assert text in msg and msg.startswith("sdm_decode_steps")


def test_decode_steps_zero_steps_is_a_no_op():
    rc, msg = call_decode_steps(0, bank=None, readings=None)
    assert rc == OK and msg == ""


def test_readings_touching_the_last_bank_element_overlap():
    # bank [1024, 128] bf16 ends at A + 1024 * 128 * 2; readings starting one element
    # before that end share a byte range with it.
    rc, msg = call_decode(readings=A + 1024 * 128 * 2 - 2)
    assert rc == E_OVERLAP


# ------------------------------------------------------------------ gather
def gather_args(**kw):
    a = dict(bank=A, bank_dtype=BF16, num_slots=1000, head_dim=128, tokens=64, chunk=16, valid=16,
             chunk_valid=None, idx_dtype=I32, w_dtype=BF16, idx0=A + 1024 * MB, w0=A + 1100 * MB,
             width0=8, out0=A + 1200 * MB, stash=A + 1300 * MB, idx1=A + 1400 * MB,
             w1=A + 1500 * MB, width1=5, out1=A + 1600 * MB, stream=None)
    a.update(kw)
    return a


def call_gather(**kw):
    a = gather_args(**kw)
    lib = sdm.library()
    rc = lib.sdm_gather(a["bank"], a["bank_dtype"], a["num_slots"], a["head_dim"], a["tokens"], a["chunk"],
                        a["valid"], a["chunk_valid"], a["idx_dtype"], a["w_dtype"], a["idx0"], a["w0"],
                        a["width0"], a["out0"], a["stash"], a["idx1"], a["w1"], a["width1"], a["out1"],
                        a["stream"])
    return rc, lib.sdm_last_error().decode()


@pytest.mark.parametrize("kw,code,text", [
    (dict(bank_dtype=I64), E_DTYPE, "bank must be"),
    (dict(idx_dtype=F32), E_DTYPE, "indices must be"),
    (dict(w_dtype=I32), E_DTYPE, "weights must be"),
    (dict(num_slots=0), E_SHAPE, "empty bank"),
    (dict(head_dim=0), E_SHAPE, "empty bank"),
    (dict(head_dim=(1 << 28) + 1, bank_dtype=F32), E_RANGE, "a bank row would exceed"),
    (dict(head_dim=(1 << 29) + 1, bank_dtype=BF16), E_RANGE, "a bank row would exceed"),
    (dict(tokens=-16), E_SHAPE, "whole number of chunks"),
    (dict(tokens=60), E_SHAPE, "whole number of chunks"),
    (dict(chunk=0), E_SHAPE, "whole number of chunks"),
    (dict(valid=17), E_SHAPE, "valid lie in [0, chunk]"),
    (dict(valid=-1), E_SHAPE, "valid lie in [0, chunk]"),
    (dict(width0=0), E_RANGE, "width0"),
    (dict(width0=257), E_RANGE, "width0"),
    (dict(width1=0), E_RANGE, "width1"),
    (dict(width1=257), E_RANGE, "width1"),
    (dict(idx1=None), E_NULL, "given in part"),
    (dict(out1=None), E_NULL, "given in part"),
    (dict(idx1=None, w1=None, out1=None, width1=3), E_NULL, "given in part"),
    (dict(bank=None), E_NULL, "required"),
    (dict(out0=None), E_NULL, "required"),
    (dict(bank=A + 2, bank_dtype=F32), E_ALIGN, "aligned"),
    (dict(out0=A + 1200 * MB + 2), E_ALIGN, "aligned"),
    (dict(chunk_valid=A + 1700 * MB + 1), E_ALIGN, "aligned"),
    (dict(out0=A + 1000 * 128), E_OVERLAP, "shares memory with the bank"),
    (dict(stash=A - 64 * 8 * 128 * 2 + 2), E_OVERLAP, "shares memory with the bank"),
    (dict(out1=A + 128), E_OVERLAP, "shares memory with the bank"),
    (dict(out1=A + 1200 * MB + 4096), E_OVERLAP, "the stash and the outputs share memory"),
    (dict(stash=A + 1200 * MB + 4096), E_OVERLAP, "the stash and the outputs share memory"),
])
def test_gather_rejects(kw, code, text):
    rc, msg = call_gather(**kw)
    assert rc == code, msg
    assert text in msg


def test_gather_zero_tokens_is_a_no_op():
    rc, msg = call_gather(tokens=0, bank=None, out0=None)
    assert rc == OK and msg == ""


def call_gather_compact(kpos=A + 1800 * MB, **kw):
    a = gather_args(**kw)
    lib = sdm.library()
    rc = lib.sdm_gather_compact(a["bank"], a["bank_dtype"], a["num_slots"], a["head_dim"], a["tokens"], a["chunk"],
                                a["valid"], a["chunk_valid"], a["idx_dtype"], a["w_dtype"], a["idx0"], a["w0"],
                                a["width0"], a["out0"], a["stash"], kpos, a["idx1"], a["w1"], a["width1"],
                                a["out1"], a["stream"])
    return rc, lib.sdm_last_error().decode()


@pytest.mark.parametrize("kw,code,text", [
    (dict(stash=None), E_NULL, "stash and kpos are required"),
    (dict(kpos=None), E_NULL, "stash and kpos are required"),
    (dict(kpos=A + 1800 * MB + 2), E_ALIGN, "aligned"),
    (dict(tokens=60), E_SHAPE, "whole number of chunks"),
    (dict(width0=0), E_RANGE, "width0"),
    (dict(stash=A + 1200 * MB + 4096), E_OVERLAP, "the stash and the outputs share memory"),
    (dict(stash=A - 64 * 8 * 128 * 2 + 2), E_OVERLAP, "shares memory with the bank"),
])
def test_gather_compact_rejects(kw, code, text):
    rc, msg = call_gather_compact(**kw)
    assert rc == code, msg
    assert text in msg and msg.startswith("sdm_gather_compact:")


def test_gather_compact_zero_tokens_is_a_no_op():
    rc, msg = call_gather_compact(tokens=0, bank=None, out0=None, stash=None, kpos=None)
    assert rc == OK and msg == ""


class Plan(ctypes.Structure):
    _fields_ = [("opaque", ctypes.c_uint64 * 48)]


def plan_init(plan, **kw):
    a = gather_args(**kw)
    lib = sdm.library()
    rc = lib.sdm_gather_plan_init(None if plan is None else ctypes.byref(plan), a["bank"], a["bank_dtype"],
                                  a["num_slots"], a["head_dim"], a["tokens"], a["chunk"], a.get("row0_max", 100),
                                  a["idx_dtype"], a["w_dtype"], a["idx0"], a["w0"], a["width0"], a["out0"],
                                  a["idx1"], a["w1"], a["width1"], a["out1"])
    return rc, lib.sdm_last_error().decode()


def plan_launch(plan, row0, valid):
    lib = sdm.library()
    rc = lib.sdm_gather_plan_launch(None if plan is None else ctypes.byref(plan), row0, valid, None)
    return rc, lib.sdm_last_error().decode()


@pytest.mark.parametrize("kw,code,text", [
    (dict(row0_max=-1), E_SHAPE, "row0_max = -1"),
    (dict(row0_max=(1 << 63) - 10), E_SHAPE, "overflows"),
    (dict(bank_dtype=I64), E_DTYPE, "bank must be"),
    (dict(tokens=60), E_SHAPE, "whole number of chunks"),
    (dict(width0=0), E_RANGE, "width0"),
    (dict(head_dim=(1 << 29) + 1, bank_dtype=BF16), E_RANGE, "a bank row would exceed"),
    (dict(idx1=None), E_NULL, "given in part"),
    (dict(out0=A + 1000 * 128), E_OVERLAP, "shares memory with the bank"),
    (dict(out1=A + 1200 * MB + 4096), E_OVERLAP, "the stash and the outputs share memory"),
])
def test_gather_plan_init_rejects(kw, code, text):
    plan = Plan()
    plan.opaque[0] = 12345
    rc, msg = plan_init(plan, **kw)
    assert rc == code, msg
    assert text in msg and msg.startswith("sdm_gather_plan_init:")
    assert not any(plan.opaque), "a failed init leaves the plan zeroed"
    rc, msg = plan_launch(plan, 0, 0)
    assert rc == E_SHAPE and "not an initialised gather plan" in msg


def test_gather_plan_null_and_range_checks():
    rc, msg = plan_init(None)
    assert rc == E_NULL and "plan is NULL" in msg
    rc, msg = plan_launch(None, 0, 0)
    assert rc == E_NULL and "plan is NULL" in msg
    # an empty plan (tokens = 0) is made and launched without a device; its row0 and valid are still checked
    plan = Plan()
    rc, msg = plan_init(plan, tokens=0, chunk=16, row0_max=32, bank=None, out0=None)
    assert rc == OK, msg
    assert plan_launch(plan, 32, 16) == (OK, "")
    rc, msg = plan_launch(plan, 33, 0)
    assert rc == E_RANGE and "row0 = 33 outside [0, 32]" in msg
    rc, msg = plan_launch(plan, -1, 0)
    assert rc == E_RANGE and "row0 = -1" in msg
    rc, msg = plan_launch(plan, 0, 17)
    assert rc == E_RANGE and "valid = 17 outside [0, 16]" in msg
    copy = Plan()
    ctypes.memmove(ctypes.byref(copy), ctypes.byref(plan), ctypes.sizeof(Plan))
    assert plan_launch(copy, 5, 3) == (OK, ""), "a copy of the struct is the same plan"


def test_last_error_is_per_thread():
    rc, msg = call_decode(W=0)
    assert rc == E_RANGE and msg
    seen = {}

    def other():
        seen["msg"] = sdm.library().sdm_last_error().decode()

    th = threading.Thread(target=other)
    th.start()
    th.join()
    assert seen["msg"] == ""
    assert sdm.library().sdm_last_error().decode() == msg


def test_python_binding_raises_on_cpu_tensors():
    import torch
    bank = torch.zeros(16, 4)
    idx = torch.zeros(2, 1, dtype=torch.int64)
    val = torch.zeros(2, 1)
    with pytest.raises(ValueError, match="is on cpu"):
        sdm.sdm_decode_step(bank, idx, val, torch.zeros(2, 4), torch.zeros(2, 1), torch.zeros(2, 1),
                            idx, val)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    from sparse_delta_rule_amd import _binding
    monkeypatch.setattr(_binding, "_lib", None)
    monkeypatch.setenv("SDM_LIBRARY", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="not built"):
        _binding.library()


def test_python_binding_checks_the_extent_of_given_outputs():
    """The library writes through plain pointers, so the binding checks that a
    caller's output, stash and per-chunk count arrays have the extent it assumes
    (these checks come before the device check, so CPU tensors reach them)."""
    import torch
    bank = torch.zeros(16, 4)
    idx = torch.zeros(6, 2, dtype=torch.int32)
    w = torch.zeros(6, 2)
    with pytest.raises(ValueError, match="out0 must be float32"):
        sdm.sdm_gather(bank, idx, w, chunk=3, out0=torch.zeros(6, 3), with_stash=False)
    with pytest.raises(ValueError, match="out1 must be float32"):
        sdm.sdm_gather(bank, idx, w, chunk=3, idx1=idx, w1=w, out1=torch.zeros(6, 4, dtype=torch.float64),
                       with_stash=False)
    with pytest.raises(ValueError, match="stash must be"):
        sdm.sdm_gather(bank, idx, w, chunk=3, stash=torch.zeros(6, 1, 4))
    with pytest.raises(ValueError, match="stash must be"):
        sdm.sdm_gather(bank, idx, w, chunk=3, stash=torch.zeros(6, 2, 4, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="chunk_valid must be \\[2\\]"):
        sdm.sdm_gather(bank, idx, w, chunk=3, chunk_valid=torch.zeros(3, dtype=torch.int32))
    with pytest.raises(ValueError, match="is on cpu"):  # right extents: on to the device check
        sdm.sdm_gather(bank, idx, w, chunk=3, chunk_valid=torch.zeros(2, dtype=torch.int32))


# ------------------------------------------------------------ python binding checks
def _decode_tensors(S=3, W=4, R=5, G=1, hd=8, steps=None):
    import torch
    lead = (S,) if steps is None else (steps, S)
    return dict(k_idx=torch.zeros(lead + (W,), dtype=torch.int64), k_val=torch.zeros(lead + (W,)),
                v=torch.zeros(lead + (hd,)), beta=torch.zeros(lead + (1,)), g=torch.zeros(lead + (G,)),
                q_idx=torch.zeros(lead + (R,), dtype=torch.int64), q_val=torch.zeros(lead + (R,)))


@pytest.mark.parametrize("name,shape", [("k_val", (3, 5)), ("v", (3, 7)), ("beta", (3, 2)), ("q_val", (3, 4)),
                                        ("q_idx", (2, 5)), ("g", (4, 1))])
def test_binding_rejects_misshaped_decode_rows(name, shape):
    import torch
    t = _decode_tensors()
    t[name] = torch.zeros(shape, dtype=t[name].dtype)
    with pytest.raises(ValueError, match=f"{name} has shape"):
        sdm.sdm_decode_step(torch.zeros(64, 8), **t)


def test_binding_rejects_decode_dtypes_and_readings():
    import torch
    t = _decode_tensors()
    t["v"] = t["v"].to(torch.bfloat16)
    with pytest.raises(TypeError, match="share one dtype"):
        sdm.sdm_decode_step(torch.zeros(64, 8), **t)
    t = _decode_tensors()
    t["g"] = t["g"].double()
    with pytest.raises(TypeError, match="float32"):
        sdm.sdm_decode_step(torch.zeros(64, 8), **t)
    with pytest.raises(ValueError, match="readings"):
        sdm.sdm_decode_step(torch.zeros(64, 8), **_decode_tensors(), readings=torch.zeros(3, 9))
    with pytest.raises(ValueError, match="bank must be"):
        sdm.sdm_decode_step(torch.zeros(64), **_decode_tensors())
    # the multi-token form wants the token axis first on every row array
    t = _decode_tensors(steps=2)
    t["beta"] = torch.zeros(3, 1)
    with pytest.raises(ValueError, match="beta has shape"):
        sdm.sdm_decode_steps(torch.zeros(64, 8), **t)
    # on the CPU the shapes pass and the device check refuses
    with pytest.raises(ValueError, match="is on cpu"):
        sdm.sdm_decode_steps(torch.zeros(64, 8), **_decode_tensors(steps=2))


@pytest.mark.parametrize("give", ["idx1", "w1"])
def test_binding_wants_both_arrays_of_a_second_operand(give):
    import torch
    from sparse_delta_rule_amd import sdm_gather, sdm_gather_compact
    bank = torch.zeros(10, 4)
    idx = torch.zeros(4, 2, dtype=torch.int32)
    w = torch.zeros(4, 2)
    extra = {give: idx if give == "idx1" else w}
    with pytest.raises(ValueError, match="give both idx1 and w1"):
        sdm_gather(bank, idx, w, chunk=4, **extra)
    with pytest.raises(ValueError, match="give both idx1 and w1"):
        sdm_gather_compact(bank, idx, w, torch.zeros(4, 2, dtype=torch.int32), chunk=4, **extra)
