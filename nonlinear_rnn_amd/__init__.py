"""Parallel Newton forward of diagonal GRU / LSTM recurrences on AMD MI355X.

The compute lives in libprn.so (HIP, gfx950; C ABI in include/prn.h).
``binding`` marshals torch tensors into that ABI under the same names;
``api`` adds allocation, contiguity, K schedules, the residual gate and the
agreement check.
"""
from .binding import (  # noqa: F401
    EXPORTS, PrnError, PrnUnsupportedError, lib, prn_backward_workspace_bytes, prn_input_proj, prn_last_error, prn_newton_backward,
    prn_newton_forward, prn_newton_forward_fused, prn_sequential_forward, prn_validate_cu_seqlens, prn_version,
    prn_workspace_bytes,
)
from .api import (  # noqa: F401
    AGREEMENT_ATOL, AgreementError, AgreementReport, LookbackTimeoutError, NewtonDivergenceError, RESIDUAL_FAIL,
    RESIDUAL_WARN,
    forward, forward_fused, gate_residual, input_proj, input_proj_apply, newton_apply, newton_forward, resolve_k,
    sequential_forward, validate_cu_seqlens, verify_agreement,
)
