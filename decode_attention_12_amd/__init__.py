"""Split-KV (Flash-Decoding style) decode attention for AMD MI355X (gfx950).

The compute path is libfd.so (hand-written HIP kernels behind a C ABI,
declared in include/fd.h); ``binding`` marshals torch tensors into it.
"""
from .binding import (  # noqa: F401
    EXPORTED, FD_BF16, FD_F32, FD_FP8_E4M3, FD_MODE_BALANCED, FD_MODE_SPLITS, FD_PATH_AUTO, FD_PATH_MFMA,
    FD_PATH_VALU, FdError, LIB_PATH, STATIC_WORKSPACE_BYTES, decode, fd_decode, fd_decode_combine,
    fd_decode_partial, fd_decode_static, fd_kv_layout,
    fd_last_error, fd_plan, fd_plan_splits, fd_problem, fd_status_string, fd_workspace_size, layout_of,
    make_problem, plan, problem_of, workspace_size)
