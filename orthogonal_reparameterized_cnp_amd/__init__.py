"""POET-X orthogonal-equivalence linear layer on AMD MI355X (gfx950).

The compute lives in libpoetx.so (hand-written HIP kernels behind a C ABI,
include/poetx.h); `binding` is its ctypes binding with the same function names
`layer.PoetxLinear` owns the device buffers of one linear, and `layer.PoetxGroup`
runs the CNP work of several linears (e.g. one decoder layer) as one batch.
"""

from .binding import (  # noqa: F401
    POETX_BF16,
    POETX_F32,
    POETX_I8,
    POETX_OP_BWD,
    POETX_OP_CNP,
    POETX_OP_FWD,
    POETX_OP_MERGE,
    LayerDesc,
    PoetxError,
    desc,
    lib,
    poetx_adam_step_batch,
    poetx_cnp_backward_batch,
    poetx_cnp_batch_workspace_size,
    poetx_cnp_build,
    poetx_cnp_build_batch,
    poetx_cnp_grad_bytes,
    poetx_g_bytes,
    poetx_last_error,
    poetx_linear_bwd,
    poetx_linear_bwd_dx,
    poetx_linear_fwd,
    poetx_merge_reinit,
    poetx_packed_len,
    poetx_perm_from_seed,
    poetx_premerge,
    poetx_saved_bytes,
    poetx_spo_bwd,
    poetx_spo_fwd,
    poetx_spo_saved_bytes,
    poetx_spo_workspace_size,
    poetx_version,
    poetx_weight_bytes,
    poetx_workspace_size,
)
