"""sparse_delta_rule_amd: the sparse-delta-memory decode step and token gather on MI355X.

The compute lives in ``libsdm.so`` (hand-written HIP kernels for gfx950 behind
the C ABI declared in ``include/sdm.h``). This package only marshals torch
tensors (device memory and streams) into those calls: it has no fallback, and
every entry point raises if the library is not built or a call fails.

    readings = sdm_decode_step(bank, k_idx, k_val, v, beta, g, q_idx, q_val)
    readings = sdm_decode_steps(bank, k_idx, k_val, v, beta, g, q_idx, q_val)  # [steps, ...] inputs
    out0, stash, out1 = sdm_gather(bank, idx0, w0, chunk=64, valid=64, idx1=..., w1=...)
    out0, stash, out1 = sdm_gather_compact(bank, idx0, w0, kpos, chunk=64, idx1=..., w1=...)
    plan = sdm_gather_plan(bank, idx0, w0, tokens=64, chunk=64); plan.launch(row0, valid)
"""

from ._binding import (  # noqa: F401
    GatherPlan,
    SDM_BF16,
    SDM_F32,
    SDM_I32,
    SDM_I64,
    SDM_MAX_WIDTH,
    SdmError,
    abi_version,
    library,
    library_path,
    sdm_decode_step,
    sdm_decode_steps,
    sdm_gather,
    sdm_gather_compact,
    sdm_gather_plan,
    sdm_round_bf16,
)
