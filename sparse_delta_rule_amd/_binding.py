"""ctypes binding of libsdm (include/sdm.h): argument marshalling only.

Tensors must be CUDA (HIP) tensors on one device and contiguous; the work is
enqueued on torch's current stream of that device, so it orders with the
surrounding torch work and can be captured in a torch.cuda.CUDAGraph.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

SDM_F32, SDM_BF16, SDM_I32, SDM_I64 = 0, 1, 2, 3
SDM_MAX_WIDTH = 256

_STATUS = {1: "SDM_E_DTYPE", 2: "SDM_E_SHAPE", 3: "SDM_E_RANGE", 4: "SDM_E_ALIGN",
           5: "SDM_E_OVERLAP", 6: "SDM_E_NULL", 7: "SDM_E_DEVICE", 8: "SDM_E_HIP"}

_DTYPES = {torch.float32: SDM_F32, torch.bfloat16: SDM_BF16, torch.int32: SDM_I32,
           torch.int64: SDM_I64}

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.environ.get("SDM_LIBRARY", os.path.join(_HERE, "libsdm.so"))


class SdmError(RuntimeError):
    """A libsdm call returned a status other than SDM_OK."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def library() -> ctypes.CDLL:
    """The loaded libsdm, with argument types declared (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"libsdm is not built ({path} is missing); run "
                           "`python -m sparse_delta_rule_amd.build`")
    lib = ctypes.CDLL(path)
    P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.sdm_decode_step.argtypes = [P, i32, i64, i64, i64, i32, i32, i32, P, i32, P, P, P, i32,
                                    P, P, P, i32, P, P]
    lib.sdm_decode_step.restype = ctypes.c_int
    lib.sdm_decode_steps.argtypes = [P, i32, i64, i64, i64, i64, i32, i32, i32, P, i32, P, P, P, i32,
                                     P, P, P, i32, P, P]
    lib.sdm_decode_steps.restype = ctypes.c_int
    lib.sdm_gather.argtypes = [P, i32, i64, i64, i64, i64, i64, P, i32, i32, P, P, i32, P, P,
                               P, P, i32, P, P]
    lib.sdm_gather.restype = ctypes.c_int
    lib.sdm_gather_compact.argtypes = [P, i32, i64, i64, i64, i64, i64, P, i32, i32, P, P, i32, P, P, P,
                                       P, P, i32, P, P]
    lib.sdm_gather_compact.restype = ctypes.c_int
    lib.sdm_gather_plan_init.argtypes = [P, P, i32, i64, i64, i64, i64, i64, i32, i32, P, P, i32, P, P, P, i32, P]
    lib.sdm_gather_plan_init.restype = ctypes.c_int
    lib.sdm_gather_plan_launch.argtypes = [P, i64, i64, P]
    lib.sdm_gather_plan_launch.restype = ctypes.c_int
    lib.sdm_last_error.argtypes = []
    lib.sdm_last_error.restype = ctypes.c_char_p
    lib.sdm_abi_version.argtypes = []
    lib.sdm_abi_version.restype = ctypes.c_int
    lib.sdm_round_bf16.argtypes = [P, P, i64, P]
    lib.sdm_round_bf16.restype = ctypes.c_int
    _lib = lib
    return lib


def abi_version() -> int:
    return int(library().sdm_abi_version())


def sdm_round_bf16(x: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bfloat16 of every float32 of x, rounded as the library's kernels round what they
    store (sdm_round_bf16)."""
    if x.dtype != torch.float32 or x.device.type != "cuda" or not x.is_contiguous():
        raise ValueError("x must be a contiguous float32 device tensor")
    if out is None:
        out = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device)
    elif out.dtype != torch.bfloat16 or out.device != x.device or not out.is_contiguous() or out.numel() != x.numel():
        raise ValueError("out must be a contiguous bfloat16 tensor like x on its device")
    rc = library().sdm_round_bf16(x.data_ptr(), out.data_ptr(), x.numel(),
                                  torch.cuda.current_stream(x.device).cuda_stream)
    if rc != 0:
        _raise(rc)
    return out


def _raise(status: int):
    msg = library().sdm_last_error().decode(errors="replace")
    raise SdmError(status, msg)


def _dt(t: torch.Tensor, what: str) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"{what} has unsupported dtype {t.dtype}") from None


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev_check(device: torch.device, **tensors):
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda or t.device != device:
            raise ValueError(f"{name} is on {t.device}, the bank on {device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def _stream_handle(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


# The per-row arrays of sdm_decode_step / sdm_decode_steps in their C argument
# order, each with the width of its last axis in terms of the call's sizes.
_DECODE_ROWS = (("k_idx", "W"), ("k_val", "W"), ("v", "head_dim"), ("q_val", "R"), ("beta", "one"),
                ("g", "G"), ("q_idx", "R"))


def _decode_marshal(bank, tensors: dict, readings, first_axis_is_steps: bool):
    """Checks of the torch side of a decode call and the C call's sizes: every per-row
    array is [rows..., width] with the same leading axes, its width as _DECODE_ROWS
    states; readings is shaped like v in the bank dtype (allocated when None).
    Returns (readings, sizes) with sizes the C ABI's head_dim, steps, streams, W, R, G."""
    if bank.dim() != 2:
        raise ValueError("bank must be [num_slots, head_dim]")
    lead = tuple(tensors["k_idx"].shape[:-1])
    if first_axis_is_steps and len(lead) < 1:
        raise ValueError("k_idx must be [steps, ..., W]")
    sizes = {"head_dim": bank.shape[1], "one": 1, "W": tensors["k_idx"].shape[-1],
             "R": tensors["q_idx"].shape[-1], "G": tensors["g"].shape[-1]}
    for name, width in _DECODE_ROWS:
        shape = tuple(tensors[name].shape)
        if shape[:-1] != lead or shape[-1:] != (sizes[width],):
            raise ValueError(f"{name} has shape {shape}; the call needs {lead + (sizes[width],)} "
                             f"(leading axes of k_idx, last axis {width})")
    if not (tensors["k_val"].dtype == tensors["v"].dtype == tensors["q_val"].dtype):
        raise TypeError("k_val, v and q_val must share one dtype")
    if tensors["beta"].dtype != torch.float32 or tensors["g"].dtype != torch.float32:
        raise TypeError("beta and g must be float32")
    v = tensors["v"]
    if readings is None:
        readings = torch.empty(v.shape, dtype=bank.dtype, device=bank.device)
    elif tuple(readings.shape) != tuple(v.shape) or readings.dtype != bank.dtype:
        raise ValueError("readings must be shaped like v, in the bank dtype")
    _dev_check(bank.device, bank=bank, readings=readings, **tensors)
    rows = 1
    for n in lead:
        rows *= n
    steps = lead[0] if first_axis_is_steps else 1
    streams = rows // steps if steps else 0
    return readings, (sizes["head_dim"], steps, streams, sizes["W"], sizes["R"], sizes["G"])


def _decode_call(fn, bank, t, readings, sizes):
    hd, steps, streams, W, R, G = sizes
    head = (_ptr(bank), _dt(bank, "bank"), bank.shape[0], hd) + ((steps,) if fn == "sdm_decode_steps" else ())
    rc = getattr(library(), fn)(
        *head, streams, W, R, G, _ptr(t["k_idx"]), _dt(t["k_idx"], "k_idx"), _ptr(t["k_val"]), _ptr(t["v"]),
        _ptr(t["q_val"]), _dt(t["v"], "v"), _ptr(t["beta"]), _ptr(t["g"]), _ptr(t["q_idx"]),
        _dt(t["q_idx"], "q_idx"), _ptr(readings), _stream_handle(bank.device))
    if rc != 0:
        _raise(rc)
    return readings


def sdm_decode_step(bank: torch.Tensor, k_idx: torch.Tensor, k_val: torch.Tensor, v: torch.Tensor,
                    beta: torch.Tensor, g: torch.Tensor, q_idx: torch.Tensor, q_val: torch.Tensor,
                    readings: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One decode step for every stream (``sdm_decode_step`` of include/sdm.h).

    bank [num_slots, head_dim] (float32 or bfloat16) is updated in place;
    k_idx, k_val [..., W]; v [..., head_dim]; beta [..., 1]; g [..., 1] or [..., W];
    q_idx, q_val [..., R]; all with the same leading dims (one entry per stream).
    k_val, v and q_val share one dtype (float32 or bfloat16); beta and g are float32.
    Returns readings shaped like ``v`` in the bank dtype (``readings`` if given).
    """
    t = dict(k_idx=k_idx, k_val=k_val, v=v, beta=beta, g=g, q_idx=q_idx, q_val=q_val)
    readings, sizes = _decode_marshal(bank, t, readings, first_axis_is_steps=False)
    return _decode_call("sdm_decode_step", bank, t, readings, sizes)


def sdm_decode_steps(bank: torch.Tensor, k_idx: torch.Tensor, k_val: torch.Tensor, v: torch.Tensor,
                     beta: torch.Tensor, g: torch.Tensor, q_idx: torch.Tensor, q_val: torch.Tensor,
                     readings: Optional[torch.Tensor] = None) -> torch.Tensor:
    """``steps`` decode steps for every stream in one launch (``sdm_decode_steps``).

    Like ``sdm_decode_step`` with a leading token axis on every per-token input:
    k_idx, k_val [steps, ..., W]; v [steps, ..., head_dim]; beta [steps, ..., 1];
    g [steps, ..., G]; q_idx, q_val [steps, ..., R]. Token t of every stream is
    applied before token t + 1; the result equals ``steps`` single-step calls.
    Returns readings shaped like ``v`` in the bank dtype.
    """
    t = dict(k_idx=k_idx, k_val=k_val, v=v, beta=beta, g=g, q_idx=q_idx, q_val=q_val)
    readings, sizes = _decode_marshal(bank, t, readings, first_axis_is_steps=True)
    return _decode_call("sdm_decode_steps", bank, t, readings, sizes)


def _gather_operands(bank, idx0, w0, chunk, valid, chunk_valid, idx1, w1, out0, out1, stash, stash_shape,
                     make_stash):
    """Shared checks and output allocation of the two gathers; returns the marshalled
    argument head (bank .. out0, stash), the second operand's and the outputs."""
    if bank.dim() != 2 or idx0.dim() != 2 or tuple(w0.shape) != tuple(idx0.shape):
        raise ValueError("bank [slots, hd], idx0 and w0 [tokens, width0] expected")
    tokens, W0 = idx0.shape
    hd = bank.shape[1]
    dev = bank.device
    two = idx1 is not None
    if two != (w1 is not None):
        raise ValueError("give both idx1 and w1 for a second operand, or neither")
    W1 = 0
    if two:
        if idx1.dim() != 2 or tuple(w1.shape) != tuple(idx1.shape) or idx1.shape[0] != tokens:
            raise ValueError("idx1 and w1 must be [tokens, width1]")
        W1 = idx1.shape[1]
        if idx1.dtype != idx0.dtype or w1.dtype != w0.dtype:
            raise TypeError("both operands must share index and weight dtypes")
    if out0 is None:
        out0 = torch.empty((tokens, hd), dtype=torch.float32, device=dev)
    if two and out1 is None:
        out1 = torch.empty((tokens, hd), dtype=torch.float32, device=dev)
    if stash is None and make_stash is not None:
        stash = make_stash(stash_shape, dtype=bank.dtype, device=dev)
    # The library sees only pointers: a given output must have the extent it will write.
    for name, t in (("out0", out0), ("out1", out1)):
        if t is not None and (tuple(t.shape) != (tokens, hd) or t.dtype != torch.float32):
            raise ValueError(f"{name} must be float32 [{tokens}, {hd}], got {t.dtype} {tuple(t.shape)}")
    if stash is not None and (tuple(stash.shape) != stash_shape or stash.dtype != bank.dtype):
        raise ValueError(f"stash must be {bank.dtype} {list(stash_shape)}, got {stash.dtype} {tuple(stash.shape)}")
    if chunk_valid is not None:
        if chunk_valid.dtype != torch.int32:
            raise TypeError("chunk_valid must be int32")
        if chunk >= 1 and tokens % chunk == 0 and tuple(chunk_valid.shape) != (tokens // chunk,):
            raise ValueError(f"chunk_valid must be [{tokens // chunk}] (one count per chunk), got "
                             f"{tuple(chunk_valid.shape)}")
    _dev_check(dev, bank=bank, idx0=idx0, w0=w0, out0=out0, stash=stash, chunk_valid=chunk_valid,
               idx1=idx1, w1=w1, out1=out1)
    head = (_ptr(bank), _dt(bank, "bank"), bank.shape[0], hd, tokens, chunk, chunk if valid is None else valid,
            _ptr(chunk_valid), _dt(idx0, "idx0"), _dt(w0, "w0"), _ptr(idx0), _ptr(w0), W0, _ptr(out0))
    tail = (_ptr(idx1), _ptr(w1), W1, _ptr(out1), _stream_handle(dev))
    return head, tail, out0, stash, out1


def sdm_gather(bank: torch.Tensor, idx0: torch.Tensor, w0: torch.Tensor, *, chunk: int,
               valid: Optional[int] = None, chunk_valid: Optional[torch.Tensor] = None,
               idx1: Optional[torch.Tensor] = None, w1: Optional[torch.Tensor] = None,
               out0: Optional[torch.Tensor] = None, out1: Optional[torch.Tensor] = None,
               stash: Optional[torch.Tensor] = None, with_stash: bool = True):
    """Token gather (``sdm_gather`` of include/sdm.h). Returns (out0, stash, out1).

    idx0, w0 [tokens, width0] (idx int32 or int64, weights float32 or bfloat16);
    optional second operand idx1, w1 [tokens, width1]. ``valid`` defaults to
    ``chunk``; ``chunk_valid`` (int32 [tokens / chunk]) overrides it per chunk.
    out0/out1 [tokens, head_dim] float32 and stash [tokens, width0, head_dim] in the
    bank dtype are allocated when not given (no stash if ``with_stash`` is False).
    """
    shape = (idx0.shape[0], idx0.shape[1], bank.shape[-1]) if idx0.dim() == 2 else ()
    head, tail, out0, stash, out1 = _gather_operands(bank, idx0, w0, chunk, valid, chunk_valid, idx1, w1, out0,
                                                     out1, stash, shape, torch.empty if with_stash else None)
    rc = library().sdm_gather(*head, _ptr(stash), *tail)
    if rc != 0:
        _raise(rc)
    return out0, stash, out1


def sdm_gather_compact(bank: torch.Tensor, idx0: torch.Tensor, w0: torch.Tensor, kpos: torch.Tensor, *,
                       chunk: int, valid: Optional[int] = None, chunk_valid: Optional[torch.Tensor] = None,
                       idx1: Optional[torch.Tensor] = None, w1: Optional[torch.Tensor] = None,
                       out0: Optional[torch.Tensor] = None, out1: Optional[torch.Tensor] = None,
                       stash: Optional[torch.Tensor] = None):
    """Token gather with a compact stash (``sdm_gather_compact`` of include/sdm.h).
    Returns (out0, stash, out1).

    As ``sdm_gather``, with kpos int32 [tokens, width0]: a live entry with
    kpos >= 0 stores its row at that row of its chunk's block of the stash
    [tokens / chunk, chunk * width0, head_dim] (bank dtype; zero-filled when not
    given); other entries and padding tokens store nothing.
    """
    if idx0.dim() != 2 or kpos.dtype != torch.int32 or tuple(kpos.shape) != tuple(idx0.shape):
        raise ValueError("kpos must be int32 shaped like idx0 [tokens, width0]")
    tokens, W0 = idx0.shape
    if chunk < 1 or tokens % chunk:
        raise ValueError(f"tokens ({tokens}) must be a multiple of chunk ({chunk})")
    shape = (tokens // chunk, chunk * W0, bank.shape[-1])
    head, tail, out0, stash, out1 = _gather_operands(bank, idx0, w0, chunk, valid, chunk_valid, idx1, w1, out0,
                                                     out1, stash, shape, torch.zeros)
    _dev_check(bank.device, kpos=kpos)
    rc = library().sdm_gather_compact(*head, _ptr(stash), _ptr(kpos), *tail)
    if rc != 0:
        _raise(rc)
    return out0, stash, out1


class GatherPlan:
    """A gather checked once and launched per step (``sdm_gather_plan_init`` /
    ``sdm_gather_plan_launch`` of include/sdm.h). Holds the plan bytes and the
    tensors it names, so they stay alive while the plan does; the tensors must
    not be resized or moved."""

    _WORDS = 48

    def __init__(self, tensors: tuple, device: torch.device, outputs: tuple):
        self._plan = (ctypes.c_uint64 * self._WORDS)()
        self._keep = tensors
        self._device = device
        self.out0, self.out1 = outputs

    def launch(self, row0: int, valid: int):
        """Gather tokens whose slots and weights are rows [row0, row0 + tokens) into
        out0 (and out1), with padding (t mod chunk) >= valid; on torch's current stream."""
        rc = library().sdm_gather_plan_launch(ctypes.byref(self._plan), int(row0), int(valid),
                                              _stream_handle(self._device))
        if rc != 0:
            _raise(rc)
        return self.out0, self.out1


def sdm_gather_plan(bank: torch.Tensor, idx0: torch.Tensor, w0: torch.Tensor, *, tokens: int, chunk: int,
                    idx1: Optional[torch.Tensor] = None, w1: Optional[torch.Tensor] = None,
                    out0: Optional[torch.Tensor] = None, out1: Optional[torch.Tensor] = None) -> GatherPlan:
    """Plan a gather of ``tokens`` tokens (no stash) whose slot and weight rows are
    a window of idx0, w0 [rows, width0] (and idx1, w1): ``plan.launch(row0, valid)``
    for any 0 <= row0 <= rows - tokens equals ``sdm_gather`` on rows
    [row0, row0 + tokens) with that valid, written to the plan's out0 / out1."""
    if bank.dim() != 2 or idx0.dim() != 2 or tuple(w0.shape) != tuple(idx0.shape):
        raise ValueError("bank [slots, hd], idx0 and w0 [rows, width0] expected")
    rows, W0 = idx0.shape
    if tokens < 0 or tokens > rows:
        raise ValueError(f"tokens ({tokens}) must be in [0, {rows}] (the rows of idx0)")
    hd = bank.shape[1]
    dev = bank.device
    two = idx1 is not None
    if two != (w1 is not None):
        raise ValueError("give both idx1 and w1 for a second operand, or neither")
    W1 = 0
    if two:
        if idx1.dim() != 2 or tuple(w1.shape) != tuple(idx1.shape) or idx1.shape[0] != rows:
            raise ValueError("idx1 and w1 must be [rows, width1], with idx0's rows")
        W1 = idx1.shape[1]
        if idx1.dtype != idx0.dtype or w1.dtype != w0.dtype:
            raise TypeError("both operands must share index and weight dtypes")
    if out0 is None:
        out0 = torch.empty((tokens, hd), dtype=torch.float32, device=dev)
    if two and out1 is None:
        out1 = torch.empty((tokens, hd), dtype=torch.float32, device=dev)
    for name, t in (("out0", out0), ("out1", out1)):
        if t is not None and (tuple(t.shape) != (tokens, hd) or t.dtype != torch.float32):
            raise ValueError(f"{name} must be float32 [{tokens}, {hd}], got {t.dtype} {tuple(t.shape)}")
    _dev_check(dev, bank=bank, idx0=idx0, w0=w0, out0=out0, idx1=idx1, w1=w1, out1=out1)
    plan = GatherPlan((bank, idx0, w0, out0, idx1, w1, out1), dev, (out0, out1))
    with torch.cuda.device(dev):
        rc = library().sdm_gather_plan_init(
            ctypes.byref(plan._plan), _ptr(bank), _dt(bank, "bank"), bank.shape[0], hd, tokens, chunk,
            rows - tokens, _dt(idx0, "idx0"), _dt(w0, "w0"), _ptr(idx0), _ptr(w0), W0, _ptr(out0), _ptr(idx1),
            _ptr(w1), W1, _ptr(out1))
    if rc != 0:
        _raise(rc)
    return plan
