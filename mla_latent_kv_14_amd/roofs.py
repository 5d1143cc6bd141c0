"""ctypes binding of libmla_roofs.so: the benchmark's measurement kernels
(cache flush, streaming HBM read, register-only bf16 matrix-core loop, empty
kernel).  Argument marshalling only; a missing library raises."""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmla_roofs.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "mla_roofs.h")

_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m mla_latent_kv_14_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.mla_roofs_flush.argtypes = [P, SZ, P]
    lib.mla_roofs_hbm_read.argtypes = [P, SZ, I32, P, SZ, P]
    lib.mla_roofs_mfma_bf16.argtypes = [I32, P, SZ, ctypes.POINTER(ctypes.c_double), P]
    lib.mla_roofs_empty.argtypes = [P]
    lib.mla_roofs_read_grid.argtypes = []
    lib.mla_roofs_mfma_grid.argtypes = []
    for fn in ("mla_roofs_flush", "mla_roofs_hbm_read", "mla_roofs_mfma_bf16", "mla_roofs_empty",
               "mla_roofs_read_grid", "mla_roofs_mfma_grid"):
        getattr(lib, fn).restype = ctypes.c_int
    _lib = lib
    return lib


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t: torch.Tensor, what: str):
    if not (t.is_cuda and t.is_contiguous()):
        raise ValueError(f"{what} must be a contiguous device tensor")
    return ctypes.c_void_p(t.data_ptr())


def _ok(fn, st):
    if st != 0:
        raise RuntimeError(f"{fn} failed with status {st}")


def flush(buf: torch.Tensor, stream=None):
    """Overwrite the whole of buf (its byte size a multiple of 16)."""
    _ok("mla_roofs_flush", load().mla_roofs_flush(_dev(buf, "buf"), buf.numel() * buf.element_size(),
                                                  _stream(stream)))


def read_grid() -> int:
    return int(load().mla_roofs_read_grid())


def mfma_grid() -> int:
    return int(load().mla_roofs_mfma_grid())


def hbm_read(buf: torch.Tensor, sink: torch.Tensor, nontemporal=False, stream=None):
    """Stream buf once; sink is an int32 device tensor of at least read_grid() words."""
    _ok("mla_roofs_hbm_read", load().mla_roofs_hbm_read(_dev(buf, "buf"), buf.numel() * buf.element_size(),
                                                        1 if nontemporal else 0, _dev(sink, "sink"), sink.numel(),
                                                        _stream(stream)))


def mfma_bf16(iters: int, sink: torch.Tensor, stream=None) -> float:
    """Launch the matrix-core loop; returns its flop count.  sink: int32, at least 4 * mfma_grid() words."""
    flops = ctypes.c_double(0.0)
    _ok("mla_roofs_mfma_bf16", load().mla_roofs_mfma_bf16(int(iters), _dev(sink, "sink"), sink.numel(),
                                                          ctypes.byref(flops), _stream(stream)))
    return flops.value


def empty(stream=None):
    _ok("mla_roofs_empty", load().mla_roofs_empty(_stream(stream)))
