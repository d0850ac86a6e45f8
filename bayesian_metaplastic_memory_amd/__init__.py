"""Palimpsa dual-state recurrence on MI355X (gfx950).

``fwd_chunked`` (training / prefill), ``bwd`` (its backward), ``fwd_frozen``
(the frozen-importance limit) with ``bwd_frozen``, ``fwd_blockdiag`` with
``step_blockdiag`` and ``bwd_blockdiag`` (block-diagonal precision) and
``step`` (decode) call the HIP kernels of ``libpalimpsa.so`` through its C
ABI; see ``include/palimpsa.h`` for the operation, layouts and error
behaviour.
"""
from ._binding import (BF16, F32, LIB_PATH, PalimpsaError, bwd, bwd_blockdiag, bwd_blockdiag_workspace_size,
                       bwd_frozen, check_params, bwd_workspace_size, fwd_blockdiag, fwd_chunked, fwd_chunked_noalloc,
                       fwd_frozen, load_library, noalloc_scratch_bytes,
                       status_string, step, step_blockdiag, version, workspace_size)

__all__ = ["fwd_chunked", "fwd_chunked_noalloc", "noalloc_scratch_bytes", "fwd_frozen", "fwd_blockdiag",
           "step_blockdiag", "bwd_blockdiag", "step", "bwd", "bwd_frozen", "workspace_size", "bwd_workspace_size", "bwd_blockdiag_workspace_size", "load_library",
           "check_params", "status_string", "version", "PalimpsaError", "LIB_PATH", "F32", "BF16"]
