"""Packed variable-length attention for AMD MI355X (gfx950).

Thin Python binding over the C ABI in include/varlen.h.  Every function here
only checks and marshals arguments (torch tensors -> device pointers, the
current HIP stream) and calls the shared library; all computation runs in the
library's HIP kernels.  There is no fallback: if the library is not built, or
the tensors are not on the GPU, the call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "load_library", "lib_path", "cu_seqlens_from_lengths", "joint_cu_seqlens",
    "pack_by_cu_seqlens", "unpack_by_cu_seqlens", "pack_by_cu_seqlens_batched",
    "unpack_by_cu_seqlens_batched", "varlen_attn_fwd", "varlen_attn_fwd_split",
    "varlen_split_workspace_bytes", "varlen_attn_fwd_f32", "varlen_attn_fwd_noalloc",
    "pack_v_transposed", "varlen_attn_fwd_vt", "block_local_attn_fwd", "block_local_attn_fwd_f32", "varlen_launch_shape", "varlen_tile_map",
    "mixfusion_chunk_plan", "unpack_cfg_combine", "VarlenError", "validate_cu_seqlens",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libvarlen_mi355x.so"
_lib = None

_c_int = ctypes.c_int
_c_i32 = ctypes.c_int32
_c_i64 = ctypes.c_int64
_c_f32 = ctypes.c_float
_vp = ctypes.c_void_p

_SIGNATURES = {
    "vl_version": ([], _c_int),
    "vl_status_string": ([_c_int], ctypes.c_char_p),
    "cu_seqlens_from_lengths": ([_vp, _c_i32, _vp, _vp], _c_int),
    "joint_cu_seqlens": ([_vp, _c_i32, _vp, _c_i32, _vp, _vp, _vp, _vp, _vp], _c_int),
    "pack_by_cu_seqlens": ([_vp, _c_i64, _vp, _c_i32, _c_i64, _vp, _vp, _vp], _c_int),
    "unpack_by_cu_seqlens": ([_vp, _vp, _vp, _c_i32, _c_i64, _vp, _c_i64, _c_int, _vp], _c_int),
    "varlen_attn_fwd": ([_vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_f32,
                         _vp, _vp, _vp], _c_int),
    "varlen_attn_fwd_f32": ([_vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                             _c_f32, _vp, _vp, _vp], _c_int),
    "block_local_attn_fwd": ([_vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                              _c_i32, _c_f32, _vp, _vp, _vp], _c_int),
    "block_local_attn_fwd_f32": ([_vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                  _c_i32, _c_f32, _vp, _vp, _vp], _c_int),
    "varlen_attn_fwd_split": ([_vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_f32,
                               _vp, _vp, _c_i64, _vp, _c_i64, _vp], _c_int),
    "varlen_split_workspace_bytes": ([_c_i64, _c_i32, _c_i32, _c_i32, _vp], _c_int),
    "pack_v_transposed": ([_vp, _c_i32, _vp, _c_i32, _c_i32, _c_i32, _c_i64, _vp, _c_i64, _vp], _c_int),
    "varlen_attn_fwd_vt": ([_vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_f32, _vp, _vp, _c_i64,
                            _vp, _c_i64, _vp], _c_int),
    "varlen_attn_fwd_noalloc": ([_vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_f32,
                                 _vp, _vp, _vp], _c_int),
    "varlen_launch_shape": ([_c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_int, _c_int, _vp, _vp, _vp, _vp],
                            _c_int),
    "varlen_tile_map": ([_vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_int, _c_int, _vp, _c_i64, _vp],
                        _c_int),
    "mixfusion_chunk_plan": ([_vp, _c_i32, _c_i64, _c_i64, _vp, _vp], _c_int),
    "pack_by_cu_seqlens_batched": ([_vp, _c_i32, _vp], _c_int),
    "unpack_by_cu_seqlens_batched": ([_vp, _c_i32, _vp], _c_int),
    "unpack_cfg_combine": ([_vp, _vp, _vp, _vp, _vp, _c_i32, _c_i64, _vp, _c_i64, _c_int, _vp], _c_int),
}


class VarlenError(RuntimeError):
    pass


class _CopyDesc(ctypes.Structure):
    """vl_copy_desc of include/varlen.h."""
    _fields_ = [("src", _vp), ("dst", _vp), ("cu_seqlens", _vp), ("row_offsets", _vp),
                ("max_len", _c_i64), ("row_bytes", _c_i64), ("num_reqs", _c_i32), ("zero_fill", _c_i32)]


MAX_BATCH = 8  # copies per batched pack / unpack call


def lib_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def load_library():
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise VarlenError(
            f"{_LIB_NAME} is not built; run `python -m packed_variable_length_varlen_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (args, res) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(rc: int, what: str):
    if rc != 0:
        msg = load_library().vl_status_string(rc).decode()
        raise VarlenError(f"{what} failed: {msg} ({rc})")


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _row_bytes(flat: torch.Tensor) -> int:
    """Bytes of one row (all dims but the first); valid for an empty tensor too."""
    n = 1
    for x in flat.shape[1:]:
        n *= int(x)
    return n * flat.element_size()


def _gpu(t: torch.Tensor, name: str, dtype=None, contiguous: bool = True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise VarlenError(f"{name} must be a GPU tensor (there is no CPU path)")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise VarlenError(f"{name} must be contiguous")


# ------------------------------------------------------------------ boundaries


def cu_seqlens_from_lengths(lengths: torch.Tensor, out: Optional[torch.Tensor] = None,
                            stream=None) -> torch.Tensor:
    _gpu(lengths, "lengths", torch.int32)
    R = lengths.numel()
    if out is None:
        out = torch.empty(R + 1, dtype=torch.int32, device=lengths.device)
    _gpu(out, "out", torch.int32)
    _check(load_library().cu_seqlens_from_lengths(_ptr(lengths), R, _ptr(out), _stream(stream)),
           "cu_seqlens_from_lengths")
    return out


def joint_cu_seqlens(text_mask: torch.Tensor, img_hw: torch.Tensor, outs=None, stream=None):
    """Returns (cu_joint, cu_text, cu_img, img_dst), all int32 on the GPU."""
    _gpu(text_mask, "text_mask", torch.uint8)
    _gpu(img_hw, "img_hw", torch.int32)
    R, cap = text_mask.shape
    if tuple(img_hw.shape) != (R, 2):
        raise VarlenError("img_hw must be [num_reqs, 2]")
    dev = text_mask.device
    if outs is None:
        outs = (torch.empty(R + 1, dtype=torch.int32, device=dev),
                torch.empty(R + 1, dtype=torch.int32, device=dev),
                torch.empty(R + 1, dtype=torch.int32, device=dev),
                torch.empty(R, dtype=torch.int32, device=dev))
    for i, t in enumerate(outs):
        _gpu(t, f"outs[{i}]", torch.int32)
    _check(load_library().joint_cu_seqlens(_ptr(text_mask), cap, _ptr(img_hw), R, *[_ptr(t) for t in outs],
                                           _stream(stream)), "joint_cu_seqlens")
    return outs


# ------------------------------------------------------------------ pack / unpack


def pack_by_cu_seqlens(src_padded: torch.Tensor, cu_seqlens: torch.Tensor, dst_flat: torch.Tensor,
                       dst_row_offsets: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """src_padded [R, max_len, ...] -> rows of dst_flat [T, ...] (same row shape)."""
    _gpu(src_padded, "src_padded")
    _gpu(dst_flat, "dst_flat", src_padded.dtype)
    _gpu(cu_seqlens, "cu_seqlens", torch.int32)
    if dst_row_offsets is not None:
        _gpu(dst_row_offsets, "dst_row_offsets", torch.int32)
    R = cu_seqlens.numel() - 1
    if src_padded.shape[0] != R or tuple(src_padded.shape[2:]) != tuple(dst_flat.shape[1:]):
        raise VarlenError("src_padded must be [num_reqs, max_len, *row] and dst_flat [T, *row]")
    row_bytes = _row_bytes(dst_flat)
    _check(load_library().pack_by_cu_seqlens(_ptr(src_padded), src_padded.shape[1], _ptr(cu_seqlens), R,
                                             row_bytes, _ptr(dst_flat), _ptr(dst_row_offsets),
                                             _stream(stream)), "pack_by_cu_seqlens")
    return dst_flat


def unpack_by_cu_seqlens(src_flat: torch.Tensor, cu_seqlens: torch.Tensor, dst_padded: torch.Tensor,
                         src_row_offsets: Optional[torch.Tensor] = None, zero_fill: bool = True,
                         stream=None) -> torch.Tensor:
    """Rows of src_flat [T, ...] -> dst_padded [R, max_len, ...]."""
    _gpu(src_flat, "src_flat")
    _gpu(dst_padded, "dst_padded", src_flat.dtype)
    _gpu(cu_seqlens, "cu_seqlens", torch.int32)
    if src_row_offsets is not None:
        _gpu(src_row_offsets, "src_row_offsets", torch.int32)
    R = cu_seqlens.numel() - 1
    if dst_padded.shape[0] != R or tuple(dst_padded.shape[2:]) != tuple(src_flat.shape[1:]):
        raise VarlenError("dst_padded must be [num_reqs, max_len, *row] and src_flat [T, *row]")
    row_bytes = _row_bytes(src_flat)
    _check(load_library().unpack_by_cu_seqlens(_ptr(src_flat), _ptr(src_row_offsets), _ptr(cu_seqlens), R,
                                               row_bytes, _ptr(dst_padded), dst_padded.shape[1],
                                               1 if zero_fill else 0, _stream(stream)),
           "unpack_by_cu_seqlens")
    return dst_padded


def pack_by_cu_seqlens_batched(items, stream=None):
    """Several pack_by_cu_seqlens calls in one launch.  items: up to 8 tuples
    (src_padded, cu_seqlens, dst_flat, dst_row_offsets or None); destinations
    must not overlap each other or any source."""
    items = list(items)
    if len(items) > MAX_BATCH:
        raise VarlenError(f"at most {MAX_BATCH} copies per batched call")
    descs = (_CopyDesc * max(len(items), 1))()
    for i, (src, cu, dst, offs) in enumerate(items):
        _gpu(src, "src_padded")
        _gpu(dst, "dst_flat", src.dtype)
        _gpu(cu, "cu_seqlens", torch.int32)
        if offs is not None:
            _gpu(offs, "dst_row_offsets", torch.int32)
        R = cu.numel() - 1
        if src.shape[0] != R or tuple(src.shape[2:]) != tuple(dst.shape[1:]):
            raise VarlenError("src_padded must be [num_reqs, max_len, *row] and dst_flat [T, *row]")
        descs[i] = _CopyDesc(_ptr(src), _ptr(dst), _ptr(cu), _ptr(offs), src.shape[1], _row_bytes(dst), R, 0)
    _check(load_library().pack_by_cu_seqlens_batched(ctypes.cast(descs, _vp), len(items), _stream(stream)),
           "pack_by_cu_seqlens_batched")


def unpack_by_cu_seqlens_batched(items, zero_fill: bool = True, stream=None):
    """Several unpack_by_cu_seqlens calls in one launch.  items: up to 8 tuples
    (src_flat, cu_seqlens, dst_padded, src_row_offsets or None)."""
    items = list(items)
    if len(items) > MAX_BATCH:
        raise VarlenError(f"at most {MAX_BATCH} copies per batched call")
    descs = (_CopyDesc * max(len(items), 1))()
    for i, (src, cu, dst, offs) in enumerate(items):
        _gpu(src, "src_flat")
        _gpu(dst, "dst_padded", src.dtype)
        _gpu(cu, "cu_seqlens", torch.int32)
        if offs is not None:
            _gpu(offs, "src_row_offsets", torch.int32)
        R = cu.numel() - 1
        if dst.shape[0] != R or tuple(dst.shape[2:]) != tuple(src.shape[1:]):
            raise VarlenError("dst_padded must be [num_reqs, max_len, *row] and src_flat [T, *row]")
        descs[i] = _CopyDesc(_ptr(src), _ptr(dst), _ptr(cu), _ptr(offs), dst.shape[1], _row_bytes(src), R,
                             1 if zero_fill else 0)
    _check(load_library().unpack_by_cu_seqlens_batched(ctypes.cast(descs, _vp), len(items), _stream(stream)),
           "unpack_by_cu_seqlens_batched")


def unpack_cfg_combine(src_flat: torch.Tensor, seg_cu: torch.Tensor, pos_rows: torch.Tensor,
                       neg_rows: torch.Tensor, scale: torch.Tensor, dst_padded: torch.Tensor,
                       zero_fill: bool = True, stream=None) -> torch.Tensor:
    """dst_padded[r, i] = neg + scale[r] * (pos - neg) over request r's segments (bf16)."""
    _gpu(src_flat, "src_flat", torch.bfloat16)
    _gpu(dst_padded, "dst_padded", torch.bfloat16)
    for name, t in (("seg_cu", seg_cu), ("pos_rows", pos_rows), ("neg_rows", neg_rows)):
        _gpu(t, name, torch.int32)
    _gpu(scale, "scale", torch.float32)
    R = seg_cu.numel() - 1
    if pos_rows.numel() != R or neg_rows.numel() != R or scale.numel() != R or dst_padded.shape[0] != R:
        raise VarlenError("seg_cu [R+1], pos_rows / neg_rows / scale [R] and dst_padded [R, ...] must agree")
    if tuple(dst_padded.shape[2:]) != tuple(src_flat.shape[1:]):
        raise VarlenError("dst_padded must be [R, max_len, *row] and src_flat [T, *row]")
    row_elems = _row_bytes(src_flat) // src_flat.element_size()
    _check(load_library().unpack_cfg_combine(_ptr(src_flat), _ptr(seg_cu), _ptr(pos_rows), _ptr(neg_rows),
                                             _ptr(scale), R, row_elems, _ptr(dst_padded), dst_padded.shape[1],
                                             1 if zero_fill else 0, _stream(stream)), "unpack_cfg_combine")
    return dst_padded


# ------------------------------------------------------------------ attention


def _attn_prep(q, k, v, dtype):
    for name, t in (("q", q), ("k", k), ("v", v)):
        _gpu(t, name, dtype)
    if q.dim() != k.dim() or k.shape != v.shape or q.shape[-2:] != k.shape[-2:]:
        raise VarlenError("q, k, v must agree on heads and head_dim, and k, v on shape")


def validate_cu_seqlens(cu, rows: int, max_len: int, what: str = "cu_seqlens") -> None:
    """Host-side check of a cu_seqlens array the kernels take on trust:
    cu[0] = 0, non-decreasing, cu[-1] == rows (padded_tokens = 0: every row of
    the packed tensor belongs to a request), and every length <= max_len (the
    bound that sized the launch).  Raises VarlenError.  `cu` is a sequence of
    ints or a tensor (copied to the host, which synchronises with the device)."""
    c = [int(x) for x in (cu.tolist() if isinstance(cu, torch.Tensor) else cu)]
    if not c or c[0] != 0:
        raise VarlenError(f"{what}[0] must be 0")
    for i in range(len(c) - 1):
        if c[i + 1] < c[i]:
            raise VarlenError(f"{what} must be non-decreasing ({what}[{i + 1}] < {what}[{i}])")
        if c[i + 1] - c[i] > max_len:
            raise VarlenError(f"request {i} has {c[i + 1] - c[i]} rows, more than the bound {max_len}")
    if c[-1] != rows:
        raise VarlenError(f"{what}[-1] = {c[-1]} differs from the {rows} rows of the packed tensor "
                          f"(padded_tokens must be 0)")


def _varlen(fn_name, dtype, q, k, v, q_cu, kv_cu, max_q, max_kv, scale, out, lse, padded_tokens,
            attn_mask, return_lse, stream, workspace=None, check_cu_seqlens=False):
    # The flat path rejects attention masks and needs padded_tokens == 0
    # (vLLM-Omni PR #6711, "Reference / Acknowledgement").
    if attn_mask is not None:
        raise VarlenError("the flat varlen path takes no attention mask")
    if padded_tokens != 0:
        raise VarlenError("the flat varlen path requires padded_tokens == 0")
    staged = fn_name == "varlen_attn_fwd_vt"  # V comes as the V^T staged in the workspace
    _attn_prep(q, k, k if staged else v, dtype)
    if q.dim() != 3:
        raise VarlenError("q, k, v must be packed [total_tokens, heads, head_dim]")
    _gpu(q_cu, "q_cu_seqlens", torch.int32)
    _gpu(kv_cu, "kv_cu_seqlens", torch.int32)
    R = q_cu.numel() - 1
    if kv_cu.numel() != R + 1:
        raise VarlenError("q_cu_seqlens and kv_cu_seqlens disagree on the number of requests")
    if check_cu_seqlens:
        validate_cu_seqlens(q_cu, q.shape[0], int(max_q), "q_cu_seqlens")
        validate_cu_seqlens(kv_cu, k.shape[0], int(max_kv), "kv_cu_seqlens")
    T, H, D = q.shape
    if scale is None:
        scale = D ** -0.5
    if out is None:
        out = torch.empty_like(q)
    _gpu(out, "out", dtype)
    if out.shape != q.shape:
        raise VarlenError("out must have the shape of q")
    if lse is None and return_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    if lse is not None:
        _gpu(lse, "lse", torch.float32)
        if tuple(lse.shape) != (T, H):
            raise VarlenError("lse must be [total_tokens, heads]")
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(q_cu), _ptr(kv_cu), int(max_q), int(max_kv), R, H, D, float(scale),
            _ptr(out), _ptr(lse)]
    if staged:
        if workspace is None:
            raise VarlenError("varlen_attn_fwd_vt reads the V^T that pack_v_transposed staged in its workspace")
        _gpu(workspace, "workspace")
        args = [_ptr(q), _ptr(k), _ptr(q_cu), _ptr(kv_cu), int(max_q), int(max_kv), R, H, D, float(scale),
                _ptr(out), _ptr(lse), k.shape[0], _ptr(workspace), workspace.numel() * workspace.element_size()]
    elif fn_name == "varlen_attn_fwd_split":
        kv_rows = k.shape[0]
        need = varlen_split_workspace_bytes(kv_rows, R, H, D)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
            if stream is not None and stream != torch.cuda.current_stream(q.device):
                workspace.record_stream(stream)
        _gpu(workspace, "workspace")
        args += [kv_rows, _ptr(workspace), workspace.numel() * workspace.element_size()]
    rc = getattr(load_library(), fn_name)(*args, _stream(stream))
    _check(rc, fn_name)
    return (out, lse) if return_lse else out


def varlen_split_workspace_bytes(kv_rows: int, num_reqs: int, H: int, D: int) -> int:
    """Workspace bytes varlen_attn_fwd_split needs on the current device for K/V
    of kv_rows rows in num_reqs requests, H heads of size D."""
    n = ctypes.c_int64()
    _check(load_library().varlen_split_workspace_bytes(int(kv_rows), int(num_reqs), int(H), int(D),
                                                       ctypes.byref(n)), "varlen_split_workspace_bytes")
    return n.value


def varlen_attn_fwd(q, k, v, q_cu_seqlens, kv_cu_seqlens, max_q, max_kv, scale=None, out=None,
                    lse=None, padded_tokens: int = 0, attn_mask=None, return_lse: bool = False,
                    stream=None, check_cu_seqlens: bool = False):
    """bf16 packed [T, H, D] varlen attention; returns out (and lse if asked).
    check_cu_seqlens: validate both arrays on the host first (a device sync;
    the kernels take them on trust)."""
    return _varlen("varlen_attn_fwd", torch.bfloat16, q, k, v, q_cu_seqlens, kv_cu_seqlens, max_q,
                   max_kv, scale, out, lse, padded_tokens, attn_mask, return_lse, stream,
                   check_cu_seqlens=check_cu_seqlens)


def varlen_attn_fwd_split(q, k, v, q_cu_seqlens, kv_cu_seqlens, max_q, max_kv, scale=None, out=None,
                          lse=None, workspace: Optional[torch.Tensor] = None, padded_tokens: int = 0,
                          attn_mask=None, return_lse: bool = False, stream=None,
                          check_cu_seqlens: bool = False):
    """varlen_attn_fwd through a workspace: V is staged transposed there, the
    last partial round is cut along the keys, and the work items are taken
    through per-chiplet queues (counters in the workspace).  `workspace` (a device
    buffer of varlen_split_workspace_bytes(k.shape[0], num_reqs, H, D) bytes)
    is allocated when not given."""
    return _varlen("varlen_attn_fwd_split", torch.bfloat16, q, k, v, q_cu_seqlens, kv_cu_seqlens, max_q,
                   max_kv, scale, out, lse, padded_tokens, attn_mask, return_lse, stream, workspace,
                   check_cu_seqlens=check_cu_seqlens)


def pack_v_transposed(items, kv_cu_seqlens, kv_rows: int, workspace, stream=None):
    """V packed from its padded buffers straight into the V^T staging of the
    workspace launch (the pack and the staging in one pass).  items: 1 to 8
    tuples (src_padded [num_reqs, max_len, H, D] bf16, cu_seqlens,
    flat_row_offsets or None), the pieces of V as pack_by_cu_seqlens_batched
    would copy them into the flat [kv_rows, H, D] tensor; kv_cu_seqlens: the
    requests' key boundaries in that flat numbering; workspace: at least
    varlen_split_workspace_bytes(kv_rows, num_reqs, H, D) bytes, then given
    to varlen_attn_fwd_vt."""
    items = list(items)
    if not 1 <= len(items) <= MAX_BATCH:
        raise VarlenError(f"1 to {MAX_BATCH} pieces per call")
    _gpu(kv_cu_seqlens, "kv_cu_seqlens", torch.int32)
    _gpu(workspace, "workspace")
    R = kv_cu_seqlens.numel() - 1
    row = None
    descs = (_CopyDesc * len(items))()
    for i, (src, cu, offs) in enumerate(items):
        _gpu(src, "src_padded", torch.bfloat16)
        _gpu(cu, "cu_seqlens", torch.int32)
        if offs is not None:
            _gpu(offs, "flat_row_offsets", torch.int32)
            if offs.numel() < R:
                raise VarlenError("flat_row_offsets must have one entry per request")
        if src.dim() != 4 or src.shape[0] != R or cu.numel() != R + 1:
            raise VarlenError("src_padded must be [num_reqs, max_len, H, D] and cu_seqlens [num_reqs + 1]")
        if row is not None and tuple(src.shape[2:]) != row:
            raise VarlenError("every piece must have the same H and D")
        row = tuple(src.shape[2:])
        descs[i] = _CopyDesc(_ptr(src), None, _ptr(cu), _ptr(offs), src.shape[1], row[0] * row[1] * 2, R, 0)
    H, D = row
    _check(load_library().pack_v_transposed(ctypes.cast(descs, _vp), len(items), _ptr(kv_cu_seqlens), R, H, D,
                                            int(kv_rows), _ptr(workspace),
                                            workspace.numel() * workspace.element_size(), _stream(stream)),
           "pack_v_transposed")


def varlen_attn_fwd_vt(q, k, q_cu_seqlens, kv_cu_seqlens, max_q, max_kv, workspace, scale=None, out=None, lse=None,
                       padded_tokens: int = 0, attn_mask=None, return_lse: bool = False, stream=None,
                       check_cu_seqlens: bool = False):
    """varlen_attn_fwd_split with V taken from the V^T that pack_v_transposed
    staged in `workspace` (same kv_cu_seqlens; kv_rows = k.shape[0])."""
    return _varlen("varlen_attn_fwd_vt", torch.bfloat16, q, k, None, q_cu_seqlens, kv_cu_seqlens, max_q, max_kv,
                   scale, out, lse, padded_tokens, attn_mask, return_lse, stream, workspace,
                   check_cu_seqlens=check_cu_seqlens)


def varlen_attn_fwd_noalloc(q, k, v, q_cu_seqlens, kv_cu_seqlens, max_q, max_kv, scale=None, out=None,
                            lse=None, padded_tokens: int = 0, attn_mask=None, return_lse: bool = False,
                            stream=None, check_cu_seqlens: bool = False):
    """varlen_attn_fwd with the key split of the last round and no device
    allocation in the library: the split's partial results live in a static
    device array (one per GPU; overlapping calls on one GPU race).  out / lse
    are allocated here only when not given."""
    return _varlen("varlen_attn_fwd_noalloc", torch.bfloat16, q, k, v, q_cu_seqlens, kv_cu_seqlens, max_q,
                   max_kv, scale, out, lse, padded_tokens, attn_mask, return_lse, stream,
                   check_cu_seqlens=check_cu_seqlens)


def varlen_attn_fwd_f32(q, k, v, q_cu_seqlens, kv_cu_seqlens, max_q, max_kv, scale=None, out=None,
                        lse=None, padded_tokens: int = 0, attn_mask=None, return_lse: bool = False,
                        stream=None, check_cu_seqlens: bool = False):
    """float32 packed [T, H, D] varlen attention; returns out (and lse if asked)."""
    return _varlen("varlen_attn_fwd_f32", torch.float32, q, k, v, q_cu_seqlens, kv_cu_seqlens, max_q,
                   max_kv, scale, out, lse, padded_tokens, attn_mask, return_lse, stream,
                   check_cu_seqlens=check_cu_seqlens)


def _block_local(fn_name, dtype, q, k, v, block, look_back, look_ahead, scale, out, lse, return_lse,
                 stream):
    _attn_prep(q, k, v, dtype)
    if q.dim() != 4 or q.shape != k.shape:
        raise VarlenError("q, k, v must be [batch, frames, heads, head_dim] of one shape")
    B, n, H, D = q.shape
    if scale is None:
        scale = D ** -0.5
    if out is None:
        out = torch.empty_like(q)
    _gpu(out, "out", dtype)
    if out.shape != q.shape:
        raise VarlenError("out must have the shape of q")
    if lse is None and return_lse:
        lse = torch.empty((B, n, H), dtype=torch.float32, device=q.device)
    if lse is not None:
        _gpu(lse, "lse", torch.float32)
        if tuple(lse.shape) != (B, n, H):
            raise VarlenError("lse must be [batch, frames, heads]")
    rc = getattr(load_library(), fn_name)(_ptr(q), _ptr(k), _ptr(v), B, n, H, D, int(block), int(look_back),
                                          int(look_ahead), float(scale), _ptr(out), _ptr(lse),
                                          _stream(stream))
    _check(rc, fn_name)
    return (out, lse) if return_lse else out


def block_local_attn_fwd(q, k, v, block: int, look_back: int, look_ahead: int, scale=None, out=None,
                         lse=None, return_lse: bool = False, stream=None):
    """bf16 block-local attention over [B, n, H, D]."""
    return _block_local("block_local_attn_fwd", torch.bfloat16, q, k, v, block, look_back, look_ahead,
                        scale, out, lse, return_lse, stream)


def block_local_attn_fwd_f32(q, k, v, block: int, look_back: int, look_ahead: int, scale=None, out=None,
                             lse=None, return_lse: bool = False, stream=None):
    """float32 block-local attention over [B, n, H, D]."""
    return _block_local("block_local_attn_fwd_f32", torch.float32, q, k, v, block, look_back, look_ahead,
                        scale, out, lse, return_lse, stream)


# ------------------------------------------------------------------ schedule export


def varlen_launch_shape(max_q: int, num_reqs: int, H: int, D: int, f32: bool = False, max_kv: int = 0,
                        split: bool = False) -> Tuple[int, int, int, int]:
    """(block_m, chunk, blocks, slots) of the launch for these scalars."""
    bm, ch, nb, sl = _c_i32(), _c_i32(), _c_i64(), _c_i32()
    _check(load_library().varlen_launch_shape(int(max_q), int(max_kv), int(num_reqs), int(H), int(D),
                                              1 if f32 else 0, 1 if split else 0, ctypes.byref(bm),
                                              ctypes.byref(ch), ctypes.byref(nb), ctypes.byref(sl)),
           "varlen_launch_shape")
    return bm.value, ch.value, nb.value, sl.value


def varlen_tile_map(q_cu: torch.Tensor, kv_cu: torch.Tensor, max_q: int, H: int, D: int, f32: bool = False,
                    max_kv: int = 0, split: bool = False, stream=None) -> torch.Tensor:
    """[blocks, 5] int32 (request, head, q-tile, part, parts) per launched work-group, -1 if idle."""
    _gpu(q_cu, "q_cu", torch.int32)
    _gpu(kv_cu, "kv_cu", torch.int32)
    R = q_cu.numel() - 1
    _, _, G, _ = varlen_launch_shape(max_q, R, H, D, f32, max_kv, split)
    out = torch.empty((max(G, 1), 5), dtype=torch.int32, device=q_cu.device)
    _check(load_library().varlen_tile_map(_ptr(q_cu), _ptr(kv_cu), int(max_q), int(max_kv), R, H, D,
                                          1 if f32 else 0, 1 if split else 0, _ptr(out), max(G, 1),
                                          _stream(stream)), "varlen_tile_map")
    return out[:G]


# ------------------------------------------------------------------ MixFusion layout check (host)


def mixfusion_chunk_plan(token_counts, min_chunk_tokens: int = 256, max_chunks: int = 128):
    """(accepted, chunk_size, chunk_count) for a mixed-resolution batch (host-only)."""
    counts = [int(c) for c in token_counts]
    arr = (ctypes.c_int64 * max(len(counts), 1))(*counts)
    size, count = ctypes.c_int64(), ctypes.c_int64()
    rc = load_library().mixfusion_chunk_plan(ctypes.cast(arr, ctypes.c_void_p), len(counts), int(min_chunk_tokens),
                                             int(max_chunks), ctypes.byref(size), ctypes.byref(count))
    if rc < 0:
        _check(rc, "mixfusion_chunk_plan")
    return bool(rc), size.value, count.value
