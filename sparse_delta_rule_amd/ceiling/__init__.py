"""ctypes binding of libsdm_ceiling (include/sdm_ceiling.h): reference access
patterns over a bank of rows, the yardstick the decode's and gather's roofline
fractions are read against. Argument marshalling only; torch tensors on one
device, work on torch's current stream.
"""

from __future__ import annotations

import ctypes
import os

import torch

READ, STASH, RMW, MIX = 0, 1, 2, 3
MODES = {"read": READ, "stash": STASH, "rmw": RMW, "mix": MIX}

_HERE = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_lib = None


def library_path() -> str:
    return os.environ.get("SDM_CEILING_LIBRARY", os.path.join(_HERE, "libsdm_ceiling.so"))


def library() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"libsdm_ceiling is not built ({path} is missing); run "
                           "`python -m sparse_delta_rule_amd.build`")
    lib = ctypes.CDLL(path)
    P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.sdm_ceiling_rows.argtypes = [i32, P, i64, i64, P, i64, P, P, P]
    lib.sdm_ceiling_rows.restype = ctypes.c_int
    lib.sdm_ceiling_sink_words.argtypes = []
    lib.sdm_ceiling_sink_words.restype = ctypes.c_int64
    lib.sdm_ceiling_copy.argtypes = [P, P, i64, i32, P]
    lib.sdm_ceiling_copy.restype = ctypes.c_int
    lib.sdm_ceiling_last_error.argtypes = []
    lib.sdm_ceiling_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(rc: int):
    if rc != 0:
        raise RuntimeError(f"libsdm_ceiling status {rc}: {library().sdm_ceiling_last_error().decode()}")


def sink_words() -> int:
    return int(library().sdm_ceiling_sink_words())


def rows(mode: str, bank: torch.Tensor, row_list: torch.Tensor, stash=None, sink=None) -> None:
    """Run one access pattern (read, stash, rmw or mix) over bank rows listed in
    row_list (int64; for mix, pairs of a written and a read row)."""
    if bank.device.type != "cuda" or not bank.is_contiguous() or bank.dim() != 2:
        raise ValueError("bank must be a contiguous 2-d device tensor")
    if row_list.dtype != torch.int64 or row_list.device != bank.device or not row_list.is_contiguous():
        raise ValueError("row_list must be a contiguous int64 tensor on the bank's device")
    m = MODES[mode]
    n = row_list.numel() // (2 if m == MIX else 1)
    for t, what in ((stash, "stash"), (sink, "sink")):
        if t is not None and (t.device != bank.device or not t.is_contiguous()):
            raise ValueError(f"{what} must be contiguous on the bank's device")
    if stash is not None and stash.numel() * stash.element_size() < n * bank.shape[1] * bank.element_size():
        raise ValueError("stash too small")
    if sink is not None and (sink.dtype != torch.int32 or sink.numel() < sink_words()):
        raise ValueError(f"sink must be int32 with at least {sink_words()} words")
    stream = torch.cuda.current_stream(bank.device).cuda_stream
    _check(library().sdm_ceiling_rows(m, bank.data_ptr(), bank.shape[0], bank.shape[1] * bank.element_size(),
                                      row_list.data_ptr(), n, None if stash is None else stash.data_ptr(),
                                      None if sink is None else sink.data_ptr(), stream))


def copy(dst: torch.Tensor, src: torch.Tensor, nontemporal: bool = False) -> None:
    """A plain streaming copy of src's bytes into dst (16-byte loads and stores)."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes or not (dst.is_contiguous() and src.is_contiguous()):
        raise ValueError("dst must be contiguous and hold src's bytes")
    stream = torch.cuda.current_stream(src.device).cuda_stream
    _check(library().sdm_ceiling_copy(dst.data_ptr(), src.data_ptr(), nbytes, int(nontemporal), stream))
