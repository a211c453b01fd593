"""ctypes binding of libnf4calib.so (include/nf4calib.h): the measurement
kernels behind the achievable ceilings the benchmark quotes -- a plain
streaming read of device memory, a loop of bf16 MFMA instructions, and that
loop fed like the fused GEMM's inner loop.
Argument marshalling only."""

from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnf4calib.so")
if not os.path.exists(LIB_PATH):
    raise ImportError("libnf4calib.so is not built; run `python -m bit_nf4_quantized_04_amd.build`")
_lib = C.CDLL(LIB_PATH)
_P = C.c_void_p
_lib.nf4calib_read.restype = C.c_int
_lib.nf4calib_read.argtypes = [_P, C.c_size_t, _P, C.c_int, _P]
_lib.nf4calib_mfma.restype = C.c_int
_lib.nf4calib_mfma.argtypes = [C.c_int, C.c_int, C.c_int, _P, _P]
_lib.nf4calib_mfma_tile.restype = C.c_int
_lib.nf4calib_mfma_tile.argtypes = [C.c_int, C.c_int, C.c_int, _P, _P]
_lib.nf4calib_default_workgroups.restype = C.c_int
_lib.nf4calib_default_workgroups.argtypes = [C.c_int]

EXPORTS = ("nf4calib_read", "nf4calib_mfma", "nf4calib_mfma_tile", "nf4calib_default_workgroups")
MFMA_FLOPS_PER_INSTR = 32 * 32 * 16 * 2
MFMA_INSTR_PER_ITER = 8


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def default_workgroups(which: int) -> int:
    return int(_lib.nf4calib_default_workgroups(which))


def read(buf: torch.Tensor, sink: torch.Tensor, workgroups: int = 0) -> None:
    """Read every byte of `buf` once (a contiguous device tensor); `sink` has
    one int32 per workgroup (default_workgroups(0) of them for 0)."""
    rc = _lib.nf4calib_read(C.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                            C.c_void_p(sink.data_ptr()), workgroups, _stream())
    if rc:
        raise RuntimeError("nf4calib_read failed (%d)" % rc)


def mfma(iters: int, sink: torch.Tensor, workgroups: int, waves: int) -> int:
    """Run the MFMA loop; returns the flops it performs."""
    rc = _lib.nf4calib_mfma(iters, workgroups, waves, C.c_void_p(sink.data_ptr()), _stream())
    if rc:
        raise RuntimeError("nf4calib_mfma failed (%d)" % rc)
    return workgroups * waves * iters * MFMA_INSTR_PER_ITER * MFMA_FLOPS_PER_INSTR


def mfma_tile(iters: int, sink: torch.Tensor, workgroups: int, dequant: bool) -> int:
    """Run the GEMM-structure loop (8 waves per workgroup, one LDS fragment
    per MFMA, with or without the dequantizing lookups); `sink` holds 8
    floats per workgroup.  Returns the flops it performs."""
    rc = _lib.nf4calib_mfma_tile(iters, workgroups, int(bool(dequant)), C.c_void_p(sink.data_ptr()), _stream())
    if rc:
        raise RuntimeError("nf4calib_mfma_tile failed (%d)" % rc)
    return workgroups * 8 * iters * MFMA_INSTR_PER_ITER * MFMA_FLOPS_PER_INSTR
