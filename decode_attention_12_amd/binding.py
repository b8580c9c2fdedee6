"""ctypes binding of libfd.so: the C-ABI entry points under the same names.

This module only marshals arguments: torch tensors supply device pointers and
the current HIP stream; every step of the decode runs in the library's
kernels. If libfd.so has not been built, importing this module raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfd.so")

FD_OK, FD_ERR_INVALID_ARG, FD_ERR_UNSUPPORTED = 0, -1, -2
FD_ERR_WORKSPACE_TOO_SMALL, FD_ERR_EMPTY_SEQUENCE, FD_ERR_HIP = -3, -4, -5
FD_F32, FD_BF16, FD_FP8_E4M3 = 0, 1, 2
FD_PATH_AUTO, FD_PATH_VALU, FD_PATH_MFMA = 0, 1, 2
FD_MODE_SPLITS, FD_MODE_BALANCED = 0, 1

_DTYPES = {torch.float32: FD_F32, torch.bfloat16: FD_BF16, torch.float8_e4m3fn: FD_FP8_E4M3}


class fd_problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "num_q_heads", "num_kv_heads", "head_dim", "max_seq_len", "page_size", "num_pages",
        "q_dtype", "kv_dtype", "out_dtype", "q_len")]


class fd_kv_layout(ctypes.Structure):
    _fields_ = [("stride_outer", ctypes.c_int64), ("stride_head", ctypes.c_int64),
                ("stride_token", ctypes.c_int64), ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p)]


class fd_plan(ctypes.Structure):
    _fields_ = [("num_splits", ctypes.c_int32), ("chunk_len", ctypes.c_int32), ("path", ctypes.c_int32),
                ("mode", ctypes.c_int32), ("workers", ctypes.c_int32), ("tile", ctypes.c_int32),
                ("lead_workers", ctypes.c_int32), ("lead_pct", ctypes.c_int32)]

    @property
    def path_name(self):
        return {FD_PATH_VALU: "valu", FD_PATH_MFMA: "mfma"}.get(self.path, str(self.path))

    def __repr__(self):
        if self.mode == FD_MODE_BALANCED:
            lead = f", lead={self.lead_workers}@{self.lead_pct}%" if self.lead_pct else ""
            return f"fd_plan(balanced, workers={self.workers}, tile={self.tile}{lead}, path={self.path_name})"
        return f"fd_plan(num_splits={self.num_splits}, chunk_len={self.chunk_len}, path={self.path_name})"


class FdError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run python decode_attention_12_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.fd_plan_splits.argtypes = [P(fd_problem), i32, i32, P(fd_plan)]
    lib.fd_plan_splits.restype = i32
    lib.fd_workspace_size.argtypes = [P(fd_problem), P(fd_plan)]
    lib.fd_workspace_size.restype = sz
    lib.fd_decode_partial.argtypes = [P(fd_problem), P(fd_plan), vp, vp, vp, P(fd_kv_layout), vp, vp, vp, i32, f32,
                                      vp, sz, vp, vp]
    lib.fd_decode_partial.restype = i32
    lib.fd_decode_combine.argtypes = [P(fd_problem), P(fd_plan), vp, sz, vp, vp, vp, vp]
    lib.fd_decode_combine.restype = i32
    lib.fd_decode.argtypes = [P(fd_problem), P(fd_plan), vp, vp, vp, P(fd_kv_layout), vp, vp, vp, i32, f32, vp, sz,
                              vp, vp, vp, vp]
    lib.fd_decode.restype = i32
    lib.fd_decode_static.argtypes = [P(fd_problem), P(fd_plan), vp, vp, vp, P(fd_kv_layout), vp, vp, vp, i32, f32,
                                     vp, vp, vp]
    lib.fd_decode_static.restype = i32
    lib.fd_status_string.argtypes = [i32]
    lib.fd_status_string.restype = ctypes.c_char_p
    lib.fd_last_error.argtypes = []
    lib.fd_last_error.restype = ctypes.c_char_p
    return lib


_lib = _load()

EXPORTED = ("fd_plan_splits", "fd_workspace_size", "fd_decode_partial", "fd_decode_combine", "fd_decode",
            "fd_decode_static", "fd_status_string", "fd_last_error")
# Bytes of the library-owned workspace of fd_decode_static (FD_STATIC_WORKSPACE_BYTES).
STATIC_WORKSPACE_BYTES = 32 << 20


def _check(status: int) -> None:
    if status != FD_OK:
        msg = _lib.fd_last_error().decode() or _lib.fd_status_string(status).decode()
        raise FdError(status, msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _device(name, t, *, dtype=None, contiguous=True):
    """A tensor handed to the library as a plain device pointer: it must live
    on a GPU, and be contiguous where the library reads it as a dense array."""
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a tensor on a GPU")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_CODES = {v: k for k, v in _DTYPES.items()}


def _check_step(problem, q, k, v, seq_lens, workspace, block_table):
    """What the C ABI cannot see from pointers, checked before anything is
    launched: q dense and of the problem's size and dtype; k and v one layout
    (the ABI takes one set of strides for both) whose dtype, KV-head count,
    head_dim and extent match the problem, so that no key the problem may
    address lies outside them (a contiguous cache holds batch sequences of
    max_seq_len keys; a paged pool holds num_pages pages of page_size keys);
    int32 lengths and block table; a dense workspace."""
    if q.dtype != _CODES.get(problem.q_dtype):
        raise ValueError(f"q must be {_CODES.get(problem.q_dtype)}, got {q.dtype}")
    if q.numel() != problem.batch * max(problem.q_len, 1) * problem.num_q_heads * problem.head_dim:
        raise ValueError("q does not hold batch x q_len x num_q_heads x head_dim elements")
    if k.shape != v.shape or k.stride() != v.stride() or k.dtype != v.dtype:
        raise ValueError("k and v must have the same shape, strides and dtype")
    if k.dtype != _CODES.get(problem.kv_dtype):
        raise ValueError(f"k and v must be {_CODES.get(problem.kv_dtype)}, got {k.dtype}")
    if k.dim() != 4 or k.shape[1] != problem.num_kv_heads or k.shape[3] != problem.head_dim:
        raise ValueError("k and v must be [outer][num_kv_heads][tokens][head_dim] views")
    if problem.page_size:
        if block_table is None:
            raise ValueError("a paged problem needs a block_table")
        if k.shape[2] != problem.page_size or k.shape[0] < problem.num_pages:
            raise ValueError("a paged pool must be [>= num_pages][Hkv][page_size][D]")
        if block_table.dim() != 2 or block_table.shape[0] < problem.batch or \
                block_table.shape[1] < -(-problem.max_seq_len // problem.page_size):
            raise ValueError("block_table must be [>= batch][>= ceil(max_seq_len / page_size)]")
        if block_table.stride(1) != 1 or block_table.dtype != torch.int32:
            raise ValueError("block_table must be int32 with contiguous rows")
    else:
        if block_table is not None:
            raise ValueError("a contiguous problem takes no block_table")
        if k.shape[0] < problem.batch or k.shape[2] < problem.max_seq_len:
            raise ValueError("a contiguous cache must be [>= batch][Hkv][>= max_seq_len][D]")
    if seq_lens.dtype != torch.int32 or seq_lens.numel() < problem.batch:
        raise ValueError("seq_lens must be int32 with one entry per sequence")
    _device("q", q)
    _device("k", k, contiguous=False)
    _device("v", v, contiguous=False)
    _device("seq_lens", seq_lens, dtype=torch.int32)
    if workspace is not None:
        _device("workspace", workspace)
    if block_table is not None:
        _device("block_table", block_table, dtype=torch.int32, contiguous=False)


def _check_out(problem, out, lse_out):
    if out.dtype != _CODES.get(problem.out_dtype):
        raise ValueError(f"out must be {_CODES.get(problem.out_dtype)}, got {out.dtype}")
    if out.numel() != problem.batch * max(problem.q_len, 1) * problem.num_q_heads * problem.head_dim:
        raise ValueError("out does not hold batch x q_len x num_q_heads x head_dim elements")
    if lse_out is not None:
        if lse_out.dtype != torch.float32 or \
                lse_out.numel() != problem.batch * max(problem.q_len, 1) * problem.num_q_heads:
            raise ValueError("lse_out needs one float32 per output row")
        _device("lse_out", lse_out, dtype=torch.float32)
    _device("out", out)


def _stream(s):
    if s is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(s, torch.cuda.Stream):
        return ctypes.c_void_p(s.cuda_stream)
    return ctypes.c_void_p(int(s))


def make_problem(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len, *, kv_dtype=FD_BF16, q_dtype=None,
                 out_dtype=None, page_size=0, num_pages=0, q_len=1) -> fd_problem:
    plain = FD_BF16 if kv_dtype == FD_FP8_E4M3 else kv_dtype
    q_dtype = plain if q_dtype is None else q_dtype
    out_dtype = plain if out_dtype is None else out_dtype
    return fd_problem(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len, page_size, num_pages,
                      q_dtype, kv_dtype, out_dtype, q_len)


def problem_of(q: torch.Tensor, k: torch.Tensor, max_seq_len: int, *, out_dtype=None, page_size=0,
               num_pages=0) -> fd_problem:
    """Problem for q [B][Hq][D] (or [B][q_len][Hq][D]) and a cache view k
    [outer][Hkv][tokens][D]."""
    out_dtype = q.dtype if out_dtype is None else out_dtype
    q_len = q.shape[1] if q.dim() == 4 else 1
    return make_problem(q.shape[0], q.shape[-2], k.shape[1], q.shape[-1], int(max_seq_len),
                        kv_dtype=_DTYPES[k.dtype], q_dtype=_DTYPES[q.dtype], out_dtype=_DTYPES[out_dtype],
                        page_size=page_size, num_pages=num_pages, q_len=q_len)


def layout_of(k: torch.Tensor, k_scale=None, v_scale=None) -> fd_kv_layout:
    """Strides of a cache view k [outer][Hkv][tokens][D]; k_scale / v_scale:
    float32 [Hkv] device tensors for an fp8 cache."""
    if k.stride(3) != 1:
        raise ValueError("the head_dim axis of the KV cache must be contiguous")
    for sc in (k_scale, v_scale):
        if sc is not None and (sc.dtype != torch.float32 or sc.numel() != k.shape[1] or not sc.is_contiguous()):
            raise ValueError("k_scale and v_scale must be contiguous float32 tensors with one entry per KV head")
    return fd_kv_layout(k.stride(0), k.stride(1), k.stride(2),
                        None if k_scale is None else k_scale.data_ptr(),
                        None if v_scale is None else v_scale.data_ptr())


def fd_plan_splits(problem: fd_problem, num_cus: int = 0, forced_splits: int = 0) -> fd_plan:
    plan = fd_plan()
    _check(_lib.fd_plan_splits(ctypes.byref(problem), int(num_cus), int(forced_splits), ctypes.byref(plan)))
    return plan


def fd_workspace_size(problem: fd_problem, plan: fd_plan) -> int:
    return int(_lib.fd_workspace_size(ctypes.byref(problem), ctypes.byref(plan)))


def fd_decode_partial(problem, plan, q, k, v, kv_layout, seq_lens, workspace, *, scale, seq_lens_host=None,
                      block_table=None, stream=None, after_stream=None) -> None:
    _check_step(problem, q, k, v, seq_lens, workspace, block_table)
    _partial_raw(problem, plan, q, k, v, kv_layout, seq_lens, workspace, scale=scale, seq_lens_host=seq_lens_host,
                 block_table=block_table, stream=stream, after_stream=after_stream)


def _partial_raw(problem, plan, q, k, v, kv_layout, seq_lens, workspace, *, scale, seq_lens_host=None,
                 block_table=None, stream=None, after_stream=None) -> None:
    """fd_decode_partial without the tensor checks above: the C library's own
    host-side validation is all that stands between these pointers and a
    launch (its tests call this with host tensors, which it must refuse)."""
    host = None
    if seq_lens_host is not None:
        host = (ctypes.c_int32 * len(seq_lens_host))(*[int(x) for x in seq_lens_host])
    bt_stride = block_table.stride(0) if block_table is not None else 0
    _check(_lib.fd_decode_partial(ctypes.byref(problem), ctypes.byref(plan), _ptr(q), _ptr(k), _ptr(v),
                                  ctypes.byref(kv_layout), _ptr(seq_lens),
                                  ctypes.cast(host, ctypes.c_void_p) if host is not None else None,
                                  _ptr(block_table), int(bt_stride), float(scale), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream),
                                  _stream(after_stream) if after_stream is not None else None))


def fd_decode_combine(problem, plan, workspace, out, lse_out=None, *, stream=None, partial_stream=None) -> None:
    _device("workspace", workspace)
    _check_out(problem, out, lse_out)
    _combine_raw(problem, plan, workspace, out, lse_out, stream=stream, partial_stream=partial_stream)


def _combine_raw(problem, plan, workspace, out, lse_out=None, *, stream=None, partial_stream=None) -> None:
    """fd_decode_combine without the tensor checks (see _partial_raw)."""
    _check(_lib.fd_decode_combine(ctypes.byref(problem), ctypes.byref(plan), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse_out),
                                  _stream(stream), _stream(partial_stream) if partial_stream is not None else None))


def fd_decode(problem, plan, q, k, v, kv_layout, seq_lens, workspace, out, lse_out=None, *, scale,
              seq_lens_host=None, block_table=None, stream=None, after_stream=None) -> None:
    """Single-launch step (partial + merge). The workspace's counter section
    must be zero before its first fd_decode (allocate it with torch.zeros)."""
    _check_step(problem, q, k, v, seq_lens, workspace, block_table)
    _check_out(problem, out, lse_out)
    host = None
    if seq_lens_host is not None:
        host = (ctypes.c_int32 * len(seq_lens_host))(*[int(x) for x in seq_lens_host])
    bt_stride = block_table.stride(0) if block_table is not None else 0
    _check(_lib.fd_decode(ctypes.byref(problem), ctypes.byref(plan), _ptr(q), _ptr(k), _ptr(v),
                          ctypes.byref(kv_layout), _ptr(seq_lens),
                          ctypes.cast(host, ctypes.c_void_p) if host is not None else None,
                          _ptr(block_table), int(bt_stride), float(scale), _ptr(workspace),
                          workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse_out), _stream(stream),
                          _stream(after_stream) if after_stream is not None else None))


def fd_decode_static(problem, plan, q, k, v, kv_layout, seq_lens, out, lse_out=None, *, scale, seq_lens_host=None,
                     block_table=None, stream=None) -> None:
    """Partial + combine with the records in the library's static device
    workspace (no workspace argument, nothing allocated). Calls that overlap
    on one GPU race on that workspace."""
    _check_step(problem, q, k, v, seq_lens, None, block_table)
    _check_out(problem, out, lse_out)
    _static_raw(problem, plan, q, k, v, kv_layout, seq_lens, out, lse_out, scale=scale, seq_lens_host=seq_lens_host,
                block_table=block_table, stream=stream)


def _static_raw(problem, plan, q, k, v, kv_layout, seq_lens, out, lse_out=None, *, scale, seq_lens_host=None,
                block_table=None, stream=None) -> None:
    """fd_decode_static without the tensor checks (see _partial_raw)."""
    host = None
    if seq_lens_host is not None:
        host = (ctypes.c_int32 * len(seq_lens_host))(*[int(x) for x in seq_lens_host])
    bt_stride = block_table.stride(0) if block_table is not None else 0
    _check(_lib.fd_decode_static(ctypes.byref(problem), ctypes.byref(plan), _ptr(q), _ptr(k), _ptr(v),
                                 ctypes.byref(kv_layout), _ptr(seq_lens),
                                 ctypes.cast(host, ctypes.c_void_p) if host is not None else None,
                                 _ptr(block_table), int(bt_stride), float(scale), _ptr(out), _ptr(lse_out),
                                 _stream(stream)))


def fd_status_string(status: int) -> str:
    return _lib.fd_status_string(int(status)).decode()


def fd_last_error() -> str:
    return _lib.fd_last_error().decode()


def plan(q, k, max_seq_len, *, splits=0, num_cus=0, page_size=0, num_pages=0, out_dtype=None, path=None):
    """Problem and plan of a decode step over q and the cache view k (shapes
    as in problem_of): the planner's choice, or splits > 0 chunks of equal
    length; path overrides the kernel path (FD_PATH_VALU / FD_PATH_MFMA).
    num_cus 0 asks the current device."""
    problem = problem_of(q, k, max_seq_len, out_dtype=out_dtype, page_size=page_size, num_pages=num_pages)
    p = fd_plan_splits(problem, num_cus, splits)
    if path is not None:
        p.path = path
    return problem, p


def workspace_size(problem: fd_problem, p: fd_plan) -> int:
    """Bytes of workspace a step with this problem and plan needs."""
    return fd_workspace_size(problem, p)


def decode(q, k, v, seq_lens, *, max_seq_len, scale=None, block_table=None, page_size=0, num_pages=0,
           splits=0, path=None, out=None, lse=None, out_dtype=None, workspace=None, seq_lens_host=None,
           num_cus=0, stream=None, k_scale=None, v_scale=None):
    """One decode step: plan, partial, combine on the current stream.

    q [B][Hq][D], or [B][q_len][Hq][D] for a multi-token step; k, v
    [outer][Hkv][tokens][D] views (outer = batch, or page for a paged pool
    with block_table [B][max_pages]); k_scale / v_scale for an fp8 cache.
    Returns (out, lse, plan); out has q's shape in out_dtype (default q's
    dtype), lse float32 q.shape[:-1] when requested (lse=True or a tensor)."""
    out_dtype = out_dtype or q.dtype
    problem, step_plan = plan(q, k, max_seq_len, splits=splits, num_cus=num_cus, page_size=page_size,
                              num_pages=num_pages, out_dtype=out_dtype, path=path)
    need = fd_workspace_size(problem, step_plan)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    if lse is True:
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    elif lse is False:
        lse = None
    scale = 1.0 / math.sqrt(q.shape[-1]) if scale is None else scale
    fd_decode_partial(problem, step_plan, q, k, v, layout_of(k, k_scale, v_scale), seq_lens, workspace, scale=scale,
                      seq_lens_host=seq_lens_host, block_table=block_table, stream=stream)
    fd_decode_combine(problem, step_plan, workspace, out, lse, stream=stream)
    return out, lse, step_plan
