"""BLASST block-sparse attention for AMD MI355X (gfx950): HIP kernels behind a C ABI
(include/blasst.h, libblasst.so) and a thin ctypes binding with the same entry-point names."""

from .blasst import (  # noqa: F401
    BlasstError,
    blasst_prefill,
    blasst_prefill_workspace_size,
    blasst_prefill_backward,
    blasst_prefill_paged,
    paged_prefill_params,
    blasst_prefill_backward_workspace_size,
    backward_params,
    blasst_decode,
    blasst_decode_workspace_size,
    blasst_decode_no_alloc,
    blasst_calib_quantile,
    blasst_calibrate,
    blasst_lambda_for,
    prefill_params,
    decode_params,
    lib,
    LIB_PATH,
    KEPT,
    SKIPPED,
    NOT_LIVE,
)
