"""fp64 CPU oracle for decode-step attention (one query token per sequence,
or the last q_len positions under the causal rule).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark use this package. The GPU library and its Python binding
never import it, and it imports nothing of theirs.

``attention`` is the plain definition of the result (full softmax over the
valid keys of each sequence, in fp64); ``attention_chunked`` is the
chunk-and-merge algorithm for one given partition of the keys. Both are thin
ctypes wrappers over ``fd_oracle.c``; the arithmetic lives there (each step is
cited to the pages in that file's header).

Tensors are CPU torch tensors (fp32, bf16, or float8_e4m3fn for K/V) used only
as byte containers: torch does no arithmetic here, and fp8 bytes are decoded by
the C code from the E4M3 definition.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fd_oracle.c")
_LIB = os.path.join(_HERE, "libfd_oracle.so")

F32, BF16, FP8_E4M3 = 0, 1, 2
_ERRORS = {-1: "invalid argument", -4: "empty sequence (no valid key)", -6: "out of memory"}


def build() -> str:
    """Compile fd_oracle.c with gcc (fp64, OpenMP) into libfd_oracle.so."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
           "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        i32, i64, dbl, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        common = [i32, i32, i32, i32, vp, i32, i64, i64, vp, vp, i32, i64, i64, i64,
                  vp, vp, i64, i32, dbl, i32, vp, vp, vp, i64]
        lib.fdo_attention_f64.argtypes = common + [vp, vp]
        lib.fdo_attention_f64.restype = i32
        lib.fdo_attention_chunked_f64.argtypes = common + [vp, i32, vp, vp, vp, vp]
        lib.fdo_attention_chunked_f64.restype = i32
        lib.fdo_decode_e4m3.argtypes = [vp, i64, vp]
        lib.fdo_decode_e4m3.restype = i32
        lib.fdo_num_threads.argtypes = []
        lib.fdo_num_threads.restype = i32
        lib.fdo_set_num_threads.argtypes = [i32]
        lib.fdo_set_num_threads.restype = None
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().fdo_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the oracle's row loop from now on."""
    _load().fdo_set_num_threads(int(n))


def _dtype_code(t: torch.Tensor, allow_fp8: bool = False) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if allow_fp8 and t.dtype == torch.float8_e4m3fn:
        return FP8_E4M3
    raise TypeError(f"oracle takes float32 or bfloat16 tensors (or float8_e4m3fn K/V), got {t.dtype}")


def decode_e4m3(codes) -> torch.Tensor:
    """fp64 values of E4M3 byte codes (a uint8 tensor or a list of ints)."""
    c = torch.as_tensor(codes, dtype=torch.uint8).contiguous()
    out = torch.empty(c.shape, dtype=torch.float64)
    _check(_load().fdo_decode_e4m3(c.data_ptr(), c.numel(), out.data_ptr()))
    return out


@dataclass
class _Marshalled:
    args: list
    nrows: int
    keep: list


def _marshal(q, k, v, seq_lens, scale, block_table, page_size, rows, k_scale, v_scale):
    """q: [B][Hq][D] (one token) or [B][q_len][Hq][D]; k, v: [outer][Hkv][tokens][D]
    views (D stride 1), where outer is the batch (contiguous) or the physical
    page (paged); k_scale, v_scale: float32 [Hkv] or None."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.device.type != "cpu":
            raise ValueError(f"{name} must be a CPU tensor")
        if t.stride(-1) != 1:
            raise ValueError(f"{name} needs a contiguous last dimension")
    if q.dim() not in (3, 4) or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q must be [B][Hq][D] or [B][q_len][Hq][D], k and v [outer][Hkv][tokens][D]")
    if k.stride() != v.stride() or k.shape != v.shape or k.dtype != v.dtype:
        raise ValueError("k and v must share shape, strides and dtype")
    if q.dim() == 4:
        B, q_len, Hq, D = q.shape
        q = q.contiguous().reshape(B, q_len * Hq, D)
    else:
        B, Hq, D = q.shape
        q_len = 1
    Hkv = k.shape[1]
    if k.shape[3] != D:
        raise ValueError("head_dim mismatch")
    seq = seq_lens.to(torch.int32).contiguous()
    keep = [q, k, v, seq]
    scale_ptrs = []
    for name, sc in (("k_scale", k_scale), ("v_scale", v_scale)):
        if sc is None:
            scale_ptrs.append(None)
            continue
        sc = torch.as_tensor(sc, dtype=torch.float32).cpu().contiguous()
        if sc.shape != (Hkv,):
            raise ValueError(f"{name} must hold one float per KV head")
        keep.append(sc)
        scale_ptrs.append(sc.data_ptr())
    bt_ptr, bt_stride = None, 0
    if page_size:
        bt = block_table.to(torch.int32).contiguous()
        keep.append(bt)
        bt_ptr, bt_stride = bt.data_ptr(), bt.shape[1]
    rows_ptr, nrows = None, B * q_len * Hq
    if rows is not None:
        rr = torch.as_tensor(rows, dtype=torch.int32).reshape(-1, 2).contiguous()
        keep.append(rr)
        rows_ptr, nrows = rr.data_ptr(), rr.shape[0]
    args = [B, Hq, Hkv, D, q.data_ptr(), _dtype_code(q), q.stride(0), q.stride(1),
            k.data_ptr(), v.data_ptr(), _dtype_code(k, allow_fp8=True), k.stride(0), k.stride(1), k.stride(2),
            seq.data_ptr(), bt_ptr, bt_stride, int(page_size), float(scale), int(q_len),
            scale_ptrs[0], scale_ptrs[1], rows_ptr, nrows]
    return _Marshalled(args, nrows, keep)


def _check(rc: int) -> None:
    if rc != 0:
        raise ValueError(f"oracle: {_ERRORS.get(rc, rc)}")


def attention(q, k, v, seq_lens, *, scale, block_table=None, page_size=0, rows=None, k_scale=None,
              v_scale=None):
    """Plain fp64 decode attention. Returns (out [nrows][D] f64, lse [nrows] f64).
    rows defaults to every (b, t, h) in order, else a list of (b, i) pairs with
    i = t * Hq + h (i = h for a one-token q). With a [B][q_len][Hq][D] q, token
    t of sequence b sees keys 0 .. L_b - q_len + t."""
    m = _marshal(q, k, v, seq_lens, scale, block_table, page_size, rows, k_scale, v_scale)
    D = q.shape[-1]
    out = torch.empty((m.nrows, D), dtype=torch.float64)
    lse = torch.empty((m.nrows,), dtype=torch.float64)
    _check(_load().fdo_attention_f64(*m.args, out.data_ptr(), lse.data_ptr()))
    return out, lse


def attention_chunked(q, k, v, seq_lens, cuts, *, scale, block_table=None, page_size=0, rows=None,
                      k_scale=None, v_scale=None):
    """Chunk-and-merge form for the partition given by ``cuts`` (ascending,
    cuts[0] == 0, cuts[-1] >= every L_b). Returns (out, lse, part_o, part_lse)
    with part_o [nrows][nchunks][D] and part_lse [nrows][nchunks] (-inf for an
    empty chunk)."""
    m = _marshal(q, k, v, seq_lens, scale, block_table, page_size, rows, k_scale, v_scale)
    D = q.shape[-1]
    c = torch.as_tensor(list(cuts), dtype=torch.int64).contiguous()
    nch = c.numel() - 1
    out = torch.empty((m.nrows, D), dtype=torch.float64)
    lse = torch.empty((m.nrows,), dtype=torch.float64)
    po = torch.empty((m.nrows, nch, D), dtype=torch.float64)
    pl = torch.empty((m.nrows, nch), dtype=torch.float64)
    _check(_load().fdo_attention_chunked_f64(*m.args, c.data_ptr(), nch, po.data_ptr(), pl.data_ptr(),
                                             out.data_ptr(), lse.data_ptr()))
    return out, lse, po, pl


def equal_chunk_cuts(max_len: int, chunk_len: int, num_chunks: int) -> list[int]:
    """Cuts of the fixed-length partition: chunk i covers [i*C, (i+1)*C),
    the last ones possibly short or empty."""
    if num_chunks * chunk_len < max_len:
        raise ValueError("chunks do not cover the keys")
    return [i * chunk_len for i in range(num_chunks + 1)]
