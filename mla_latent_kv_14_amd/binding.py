"""ctypes binding of libmla.so: the same entry points, taking torch tensors.

Argument marshalling only: each function checks that tensors are contiguous
device tensors of the expected dtype and size (a host pointer handed to a GPU
kernel would fault the device), then calls the C function of the same name on
the current (or given) HIP stream.  Every computation runs in libmla's HIP
kernels; there is no fallback of any kind.  A missing library raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmla.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "mla.h")

MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE, MLA_ERR_HIP = 0, -1, -2, -3, -4
MLA_F32, MLA_BF16 = 0, 1


class MLAError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


class mla_dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "q_len", "num_heads", "d_c", "d_rope", "d_nope", "d_v", "block_size", "max_blocks_per_seq",
        "num_blocks", "dtype")]

    def __repr__(self):
        return "mla_dims(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


_lib = None


def load() -> ctypes.CDLL:
    """Load libmla.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m mla_latent_kv_14_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    D = ctypes.POINTER(mla_dims)
    sig = {
        "mla_absorb_q": [D, P, P, P, P, P],
        "mla_absorb_q_plan": [D, P, P, P, P, P, I32, P, SZ, P],
        "mla_absorb_q_plan_fp8": [D, P, P, P, P, P, I32, P, SZ, P],
        "mla_decode_num_splits": [D, I32, I64, ctypes.POINTER(I32)],
        "mla_choose_splits": [D, P, I32, ctypes.POINTER(I32)],
        "mla_choose_splits_fp8": [D, P, I32, ctypes.POINTER(I32)],
        "mla_decode_workspace_bytes": [D, I32, ctypes.POINTER(SZ)],
        "mla_decode": [D, P, P, P, P, F32, I32, P, SZ, P, P, P],
        "mla_decode_noalloc": [D, P, P, P, P, F32, I32, P, P, P],
        "mla_decode_plan": [D, P, I32, P, SZ, P],
        "mla_decode_planned": [D, P, P, P, F32, I32, P, SZ, P, P, P],
        "mla_decode_num_splits_fp8": [D, I32, I64, ctypes.POINTER(I32)],
        "mla_decode_plan_fp8": [D, P, I32, P, SZ, P],
        "mla_decode_planned_fp8": [D, P, P, F32, P, F32, I32, P, SZ, P, P, P],
        "mla_decode_fp8": [D, P, P, F32, P, P, F32, I32, P, SZ, P, P, P],
        "mla_combine": [D, I32, P, P, P, P, P],
        "mla_absorb_out": [D, P, P, P, P],
        "mla_combine_absorb_out": [D, I32, P, P, P, P, P, P, P],
        "mla_combine_absorb_out_fused": [D, I32],
        "mla_cache_append_workspace_bytes": [D, I32, ctypes.POINTER(SZ)],
        "mla_cache_append": [D, I32, P, P, P, F32, P, P, P, P, SZ, P],
        "mla_cache_append_fp8": [D, I32, P, P, P, F32, F32, P, P, P, P, SZ, P],
        "mla_prefill_workspace_bytes": [D, I32, ctypes.POINTER(SZ)],
        "mla_prefill": [D, I32, I32, P, P, P, P, P, P, P, F32, I32, P, P, P, SZ, P],
        "mla_fold_query_weight": [D, I32, P, P, P, P],
        "mla_fused_query": [D, I32, P, P, P, P, P],
        "mla_fold_output_weight": [D, I32, P, P, P, P],
        "mla_fused_output_workspace_bytes": [D, I32, ctypes.POINTER(SZ)],
        "mla_fused_output": [D, I32, P, P, P, P, SZ, P],
        "mla_fused_query_weight_packed": [D, I32],
        "mla_fused_output_weight_packed": [D, I32],
        "mla_version": [],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.mla_status_str.argtypes = [ctypes.c_int]
    lib.mla_status_str.restype = ctypes.c_char_p
    _lib = lib
    return lib


def header_symbols() -> list:
    """Names of the functions include/mla.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(mla_\w+)\s*\(", text, flags=re.M)))


def status_str(status: int) -> str:
    return load().mla_status_str(status).decode()


def _check(fn: str, status: int):
    if status != MLA_OK:
        raise MLAError(fn, status, status_str(status))


def make_dims(batch, q_len, num_heads, d_c, d_rope, d_nope, d_v, block_size, max_blocks_per_seq, num_blocks,
              dtype) -> mla_dims:
    if isinstance(dtype, torch.dtype):
        dtype = {torch.float32: MLA_F32, torch.bfloat16: MLA_BF16}[dtype]
    return mla_dims(batch, q_len, num_heads, d_c, d_rope, d_nope, d_v, block_size, max_blocks_per_seq, num_blocks,
                    dtype)


def _storage_dtype(dims: mla_dims) -> torch.dtype:
    return torch.float32 if dims.dtype == MLA_F32 else torch.bfloat16


def _ptr(t: Optional[torch.Tensor], name: str, dtype: torch.dtype, numel: int):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return ctypes.c_void_p(handle)


def mla_absorb_q(dims, q_nope, q_rope, w_uk, q_cat, stream=None):
    d, st = dims, _storage_dtype(dims)
    rows = d.batch * d.q_len * d.num_heads
    _check("mla_absorb_q", load().mla_absorb_q(
        ctypes.byref(d), _ptr(q_nope, "q_nope", st, rows * d.d_nope), _ptr(q_rope, "q_rope", st, rows * d.d_rope),
        _ptr(w_uk, "w_uk", st, d.num_heads * d.d_nope * d.d_c),
        _ptr(q_cat, "q_cat", st, rows * (d.d_c + d.d_rope)), _stream(stream)))


def _absorb_q_plan(fn, dims, q_nope, q_rope, w_uk, q_cat, seq_lens, num_splits, workspace, stream):
    d, st = dims, _storage_dtype(dims)
    rows = d.batch * d.q_len * d.num_heads
    if not (workspace.is_cuda and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous device tensor")
    _check(fn, getattr(load(), fn)(
        ctypes.byref(d), _ptr(q_nope, "q_nope", st, rows * d.d_nope), _ptr(q_rope, "q_rope", st, rows * d.d_rope),
        _ptr(w_uk, "w_uk", st, d.num_heads * d.d_nope * d.d_c), _ptr(q_cat, "q_cat", st, rows * (d.d_c + d.d_rope)),
        _ptr(seq_lens, "seq_lens", torch.int32, d.batch), int(num_splits), ctypes.c_void_p(workspace.data_ptr()),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def mla_absorb_q_plan(dims, q_nope, q_rope, w_uk, q_cat, seq_lens, num_splits, workspace, stream=None):
    """mla_absorb_q and mla_decode_plan in one launch."""
    _absorb_q_plan("mla_absorb_q_plan", dims, q_nope, q_rope, w_uk, q_cat, seq_lens, num_splits, workspace, stream)


def mla_absorb_q_plan_fp8(dims, q_nope, q_rope, w_uk, q_cat, seq_lens, num_splits, workspace, stream=None):
    """mla_absorb_q and mla_decode_plan_fp8 in one launch."""
    _absorb_q_plan("mla_absorb_q_plan_fp8", dims, q_nope, q_rope, w_uk, q_cat, seq_lens, num_splits, workspace,
                   stream)


def mla_decode_num_splits(dims, max_seq_len: int, total_tokens: int) -> int:
    out = ctypes.c_int32(0)
    _check("mla_decode_num_splits", load().mla_decode_num_splits(ctypes.byref(dims), int(max_seq_len),
                                                                 int(total_tokens), ctypes.byref(out)))
    return out.value


def _choose(fn: str, dims, seq_lens_host, max_seq_len: int) -> int:
    import numpy as np

    out = ctypes.c_int32(0)
    arr = None
    ptr = None
    if seq_lens_host is not None:
        arr = np.ascontiguousarray(seq_lens_host, dtype=np.int32)
        if arr.shape != (dims.batch,):
            raise ValueError(f"seq_lens_host must be a host array of {dims.batch} int32 lengths")
        ptr = arr.ctypes.data_as(ctypes.c_void_p)
    _check(fn, getattr(load(), fn)(ctypes.byref(dims), ptr, int(max_seq_len), ctypes.byref(out)))
    return out.value


def mla_choose_splits(dims, seq_lens_host=None, max_seq_len: int = 0) -> int:
    """Split count from host lengths (a numpy array or list of B int32), or from max_seq_len alone."""
    return _choose("mla_choose_splits", dims, seq_lens_host, max_seq_len)


def mla_choose_splits_fp8(dims, seq_lens_host=None, max_seq_len: int = 0) -> int:
    return _choose("mla_choose_splits_fp8", dims, seq_lens_host, max_seq_len)


def mla_decode_workspace_bytes(dims, num_splits: int) -> int:
    out = ctypes.c_size_t(0)
    _check("mla_decode_workspace_bytes",
           load().mla_decode_workspace_bytes(ctypes.byref(dims), int(num_splits), ctypes.byref(out)))
    return out.value


def mla_decode(dims, q_cat, kv_cache, block_table, seq_lens, softmax_scale, num_splits, workspace, o_partial,
               lse_partial, stream=None):
    d, st = dims, _storage_dtype(dims)
    rows = d.batch * d.q_len * d.num_heads
    D = d.d_c + d.d_rope
    if not (workspace.is_cuda and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous device tensor")
    _check("mla_decode", load().mla_decode(
        ctypes.byref(d), _ptr(q_cat, "q_cat", st, rows * D),
        _ptr(kv_cache, "kv_cache", st, d.num_blocks * d.block_size * D),
        _ptr(block_table, "block_table", torch.int32, d.batch * d.max_blocks_per_seq),
        _ptr(seq_lens, "seq_lens", torch.int32, d.batch), float(softmax_scale), int(num_splits),
        ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(),
        _ptr(o_partial, "o_partial", _storage_dtype(d), rows * num_splits * d.d_c),
        _ptr(lse_partial, "lse_partial", torch.float32, rows * num_splits), _stream(stream)))


def mla_decode_noalloc(dims, q_cat, kv_cache, block_table, seq_lens, softmax_scale, num_splits, o_partial,
                       lse_partial, stream=None):
    d, st = dims, _storage_dtype(dims)
    rows = d.batch * d.q_len * d.num_heads
    D = d.d_c + d.d_rope
    _check("mla_decode_noalloc", load().mla_decode_noalloc(
        ctypes.byref(d), _ptr(q_cat, "q_cat", st, rows * D),
        _ptr(kv_cache, "kv_cache", st, d.num_blocks * d.block_size * D),
        _ptr(block_table, "block_table", torch.int32, d.batch * d.max_blocks_per_seq),
        _ptr(seq_lens, "seq_lens", torch.int32, d.batch), float(softmax_scale), int(num_splits),
        _ptr(o_partial, "o_partial", _storage_dtype(d), rows * num_splits * d.d_c),
        _ptr(lse_partial, "lse_partial", torch.float32, rows * num_splits), _stream(stream)))


def mla_decode_plan(dims, seq_lens, num_splits, workspace, stream=None):
    d = dims
    if not (workspace.is_cuda and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous device tensor")
    _check("mla_decode_plan", load().mla_decode_plan(
        ctypes.byref(d), _ptr(seq_lens, "seq_lens", torch.int32, d.batch), int(num_splits),
        ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(), _stream(stream)))


def mla_decode_planned(dims, q_cat, kv_cache, block_table, softmax_scale, num_splits, workspace, o_partial,
                       lse_partial, stream=None):
    d, st = dims, _storage_dtype(dims)
    rows = d.batch * d.q_len * d.num_heads
    D = d.d_c + d.d_rope
    if not (workspace.is_cuda and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous device tensor")
    _check("mla_decode_planned", load().mla_decode_planned(
        ctypes.byref(d), _ptr(q_cat, "q_cat", st, rows * D),
        _ptr(kv_cache, "kv_cache", st, d.num_blocks * d.block_size * D),
        _ptr(block_table, "block_table", torch.int32, d.batch * d.max_blocks_per_seq), float(softmax_scale),
        int(num_splits), ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(),
        _ptr(o_partial, "o_partial", _storage_dtype(d), rows * num_splits * d.d_c),
        _ptr(lse_partial, "lse_partial", torch.float32, rows * num_splits), _stream(stream)))


# ---- FP8 (E4M3) latent cache: kv_cache is a uint8 tensor of codes standing for kv_scale * value

def mla_decode_num_splits_fp8(dims, max_seq_len: int, total_tokens: int) -> int:
    out = ctypes.c_int32(0)
    _check("mla_decode_num_splits_fp8", load().mla_decode_num_splits_fp8(ctypes.byref(dims), int(max_seq_len),
                                                                         int(total_tokens), ctypes.byref(out)))
    return out.value


def mla_decode_plan_fp8(dims, seq_lens, num_splits, workspace, stream=None):
    d = dims
    if not (workspace.is_cuda and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous device tensor")
    _check("mla_decode_plan_fp8", load().mla_decode_plan_fp8(
        ctypes.byref(d), _ptr(seq_lens, "seq_lens", torch.int32, d.batch), int(num_splits),
        ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(), _stream(stream)))


def mla_decode_planned_fp8(dims, q_cat, kv_cache, kv_scale, block_table, softmax_scale, num_splits, workspace,
                           o_partial, lse_partial, stream=None):
    d, st = dims, _storage_dtype(dims)
    rows = d.batch * d.q_len * d.num_heads
    D = d.d_c + d.d_rope
    if not (workspace.is_cuda and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous device tensor")
    _check("mla_decode_planned_fp8", load().mla_decode_planned_fp8(
        ctypes.byref(d), _ptr(q_cat, "q_cat", st, rows * D),
        _ptr(kv_cache, "kv_cache", torch.uint8, d.num_blocks * d.block_size * D), float(kv_scale),
        _ptr(block_table, "block_table", torch.int32, d.batch * d.max_blocks_per_seq), float(softmax_scale),
        int(num_splits), ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(),
        _ptr(o_partial, "o_partial", _storage_dtype(d), rows * num_splits * d.d_c),
        _ptr(lse_partial, "lse_partial", torch.float32, rows * num_splits), _stream(stream)))


def mla_decode_fp8(dims, q_cat, kv_cache, kv_scale, block_table, seq_lens, softmax_scale, num_splits, workspace,
                   o_partial, lse_partial, stream=None):
    d, st = dims, _storage_dtype(dims)
    rows = d.batch * d.q_len * d.num_heads
    D = d.d_c + d.d_rope
    if not (workspace.is_cuda and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous device tensor")
    _check("mla_decode_fp8", load().mla_decode_fp8(
        ctypes.byref(d), _ptr(q_cat, "q_cat", st, rows * D),
        _ptr(kv_cache, "kv_cache", torch.uint8, d.num_blocks * d.block_size * D), float(kv_scale),
        _ptr(block_table, "block_table", torch.int32, d.batch * d.max_blocks_per_seq),
        _ptr(seq_lens, "seq_lens", torch.int32, d.batch), float(softmax_scale), int(num_splits),
        ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(),
        _ptr(o_partial, "o_partial", _storage_dtype(d), rows * num_splits * d.d_c),
        _ptr(lse_partial, "lse_partial", torch.float32, rows * num_splits), _stream(stream)))


def mla_combine(dims, num_splits, o_partial, lse_partial, o_latent, lse=None, stream=None):
    d = dims
    rows = d.batch * d.q_len * d.num_heads
    _check("mla_combine", load().mla_combine(
        ctypes.byref(d), int(num_splits), _ptr(o_partial, "o_partial", _storage_dtype(d), rows * num_splits * d.d_c),
        _ptr(lse_partial, "lse_partial", torch.float32, rows * num_splits),
        _ptr(o_latent, "o_latent", torch.float32, rows * d.d_c),
        _ptr(lse, "lse", torch.float32, rows) if lse is not None else None, _stream(stream)))


def mla_absorb_out(dims, o_latent, w_uv, out, stream=None):
    d, st = dims, _storage_dtype(dims)
    rows = d.batch * d.q_len * d.num_heads
    _check("mla_absorb_out", load().mla_absorb_out(
        ctypes.byref(d), _ptr(o_latent, "o_latent", torch.float32, rows * d.d_c),
        _ptr(w_uv, "w_uv", st, d.num_heads * d.d_v * d.d_c), _ptr(out, "out", st, rows * d.d_v), _stream(stream)))


def mla_combine_absorb_out(dims, num_splits, o_partial, lse_partial, w_uv, out, o_latent=None, lse=None,
                           stream=None):
    d, st = dims, _storage_dtype(dims)
    rows = d.batch * d.q_len * d.num_heads
    _check("mla_combine_absorb_out", load().mla_combine_absorb_out(
        ctypes.byref(d), int(num_splits), _ptr(o_partial, "o_partial", _storage_dtype(d), rows * num_splits * d.d_c),
        _ptr(lse_partial, "lse_partial", torch.float32, rows * num_splits),
        _ptr(w_uv, "w_uv", st, d.num_heads * d.d_v * d.d_c), _ptr(out, "out", st, rows * d.d_v),
        _ptr(o_latent, "o_latent", torch.float32, rows * d.d_c) if o_latent is not None else None,
        _ptr(lse, "lse", torch.float32, rows) if lse is not None else None, _stream(stream)))


def mla_combine_absorb_out_fused(dims, num_splits) -> bool:
    return bool(load().mla_combine_absorb_out_fused(ctypes.byref(dims), int(num_splits)))



def mla_cache_append_workspace_bytes(dims, d_model: int) -> int:
    out = ctypes.c_size_t(0)
    _check("mla_cache_append_workspace_bytes",
           load().mla_cache_append_workspace_bytes(ctypes.byref(dims), int(d_model), ctypes.byref(out)))
    return out.value


def mla_cache_append(dims, d_model, h, w_dkv, w_kr, rope_base, block_table, seq_lens, kv_cache, workspace=None,
                     stream=None):
    d, st = dims, _storage_dtype(dims)
    D = d.d_c + d.d_rope
    if workspace is not None and not (workspace.is_cuda and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous device tensor")
    ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("mla_cache_append", load().mla_cache_append(
        ctypes.byref(d), int(d_model), _ptr(h, "h", st, d.batch * d.q_len * d_model),
        _ptr(w_dkv, "w_dkv", st, d.d_c * d_model),
        _ptr(w_kr, "w_kr", st, d.d_rope * d_model) if w_kr is not None else None, float(rope_base),
        _ptr(block_table, "block_table", torch.int32, d.batch * d.max_blocks_per_seq),
        _ptr(seq_lens, "seq_lens", torch.int32, d.batch),
        _ptr(kv_cache, "kv_cache", st, d.num_blocks * d.block_size * D), ws_ptr, ws_bytes, _stream(stream)))


def mla_cache_append_fp8(dims, d_model, h, w_dkv, w_kr, rope_base, kv_scale, block_table, seq_lens, kv_cache,
                         workspace=None, stream=None):
    d, st = dims, _storage_dtype(dims)
    D = d.d_c + d.d_rope
    if workspace is not None and not (workspace.is_cuda and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous device tensor")
    ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("mla_cache_append_fp8", load().mla_cache_append_fp8(
        ctypes.byref(d), int(d_model), _ptr(h, "h", st, d.batch * d.q_len * d_model),
        _ptr(w_dkv, "w_dkv", st, d.d_c * d_model),
        _ptr(w_kr, "w_kr", st, d.d_rope * d_model) if w_kr is not None else None, float(rope_base),
        float(kv_scale), _ptr(block_table, "block_table", torch.int32, d.batch * d.max_blocks_per_seq),
        _ptr(seq_lens, "seq_lens", torch.int32, d.batch),
        _ptr(kv_cache, "kv_cache", torch.uint8, d.num_blocks * d.block_size * D), ws_ptr, ws_bytes,
        _stream(stream)))


def mla_fold_query_weight(dims, d_in, w_in, w_uk, w_fused, stream=None):
    d, st = dims, _storage_dtype(dims)
    H = d.num_heads
    _check("mla_fold_query_weight", load().mla_fold_query_weight(
        ctypes.byref(d), int(d_in), _ptr(w_in, "w_in", st, H * d.d_nope * d_in),
        _ptr(w_uk, "w_uk", st, H * d.d_nope * d.d_c), _ptr(w_fused, "w_fused", st, H * d.d_c * d_in),
        _stream(stream)))


def mla_fused_query(dims, d_in, x, q_rope, w_fused, q_cat, stream=None):
    d, st = dims, _storage_dtype(dims)
    M, H = d.batch * d.q_len, d.num_heads
    _check("mla_fused_query", load().mla_fused_query(
        ctypes.byref(d), int(d_in), _ptr(x, "x", st, M * d_in),
        _ptr(q_rope, "q_rope", st, M * H * d.d_rope) if d.d_rope > 0 else None,
        _ptr(w_fused, "w_fused", st, H * d.d_c * d_in), _ptr(q_cat, "q_cat", st, M * H * (d.d_c + d.d_rope)),
        _stream(stream)))


def mla_fold_output_weight(dims, d_out, w_o, w_uv, w_fused, stream=None):
    d, st = dims, _storage_dtype(dims)
    H = d.num_heads
    _check("mla_fold_output_weight", load().mla_fold_output_weight(
        ctypes.byref(d), int(d_out), _ptr(w_o, "w_o", st, d_out * H * d.d_v),
        _ptr(w_uv, "w_uv", st, H * d.d_v * d.d_c), _ptr(w_fused, "w_fused", st, d_out * H * d.d_c),
        _stream(stream)))


def mla_fused_query_weight_packed(dims, d_in) -> bool:
    return bool(load().mla_fused_query_weight_packed(ctypes.byref(dims), int(d_in)))


def mla_fused_output_weight_packed(dims, d_out) -> bool:
    return bool(load().mla_fused_output_weight_packed(ctypes.byref(dims), int(d_out)))


def mla_fused_output_workspace_bytes(dims, d_out: int) -> int:
    out = ctypes.c_size_t(0)
    _check("mla_fused_output_workspace_bytes",
           load().mla_fused_output_workspace_bytes(ctypes.byref(dims), int(d_out), ctypes.byref(out)))
    return out.value


def mla_fused_output(dims, d_out, o_latent, w_fused, y, workspace=None, stream=None):
    d, st = dims, _storage_dtype(dims)
    M, H = d.batch * d.q_len, d.num_heads
    if workspace is not None and not (workspace.is_cuda and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous device tensor")
    ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("mla_fused_output", load().mla_fused_output(
        ctypes.byref(d), int(d_out), _ptr(o_latent, "o_latent", torch.float32, M * H * d.d_c),
        _ptr(w_fused, "w_fused", st, d_out * H * d.d_c), _ptr(y, "y", st, M * d_out), ws_ptr, ws_bytes,
        _stream(stream)))


def mla_prefill_workspace_bytes(dims, total_tokens: int) -> int:
    out = ctypes.c_size_t(0)
    _check("mla_prefill_workspace_bytes",
           load().mla_prefill_workspace_bytes(ctypes.byref(dims), int(total_tokens), ctypes.byref(out)))
    return out.value


def mla_prefill(dims, total_tokens, max_seqlen, cu_seqlens, q_nope, q_rope, c_kv, k_rope, w_uk, w_uv, softmax_scale,
                causal, out, workspace, lse=None, stream=None):
    d, st = dims, _storage_dtype(dims)
    T, H = int(total_tokens), d.num_heads
    if not (workspace.is_cuda and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous device tensor")
    _check("mla_prefill", load().mla_prefill(
        ctypes.byref(d), T, int(max_seqlen), _ptr(cu_seqlens, "cu_seqlens", torch.int32, d.batch + 1),
        _ptr(q_nope, "q_nope", st, T * H * d.d_nope), _ptr(q_rope, "q_rope", st, T * H * d.d_rope),
        _ptr(c_kv, "c_kv", st, T * d.d_c), _ptr(k_rope, "k_rope", st, T * d.d_rope),
        _ptr(w_uk, "w_uk", st, H * d.d_nope * d.d_c), _ptr(w_uv, "w_uv", st, H * d.d_v * d.d_c),
        float(softmax_scale), int(causal), _ptr(out, "out", st, T * H * d.d_v),
        _ptr(lse, "lse", torch.float32, T * H) if lse is not None else None,
        ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(), _stream(stream)))
