"""ctypes binding of libnf4qlora.so: argument marshalling only.

The names follow the C ABI in include/nf4qlora.h.  Every computation runs in
the library's HIP kernels; torch is used for device memory (output and
workspace allocation) and for the current stream.  Importing this module
loads the library and raises ImportError when it has not been built.
"""

from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnf4qlora.so")

# torch first: its HIP runtime is the one the library must share.
import torch  # noqa: E402,F401

if not os.path.exists(LIB_PATH):
    raise ImportError("libnf4qlora.so is not built; run `python -m bit_nf4_quantized_04_amd.build`")
_lib = C.CDLL(LIB_PATH)

NF4_OK, NF4_EINVAL, NF4_ESHAPE, NF4_EUNSUPPORTED, NF4_EWORKSPACE, NF4_ELAUNCH, NF4_ETOOLARGE = range(7)
QLORA_NOALLOC_SCRATCH_BYTES = 64 << 20
NF4_QUANT_NF4, NF4_QUANT_FP4 = 0, 1
QUANT_TYPES = {"nf4": NF4_QUANT_NF4, "fp4": NF4_QUANT_FP4}
QLORA_OP_FORWARD, QLORA_OP_BACKWARD, QLORA_OP_FORWARD_MULTI = 1, 2, 3
QLORA_OP_BLOCK128 = 0x100  # OR'ed into a workspace query for a weight with 128-element blocks
QLORA_OP_DROPOUT = 0x200   # OR'ed into a workspace query for the *_dropout calls


class nf4_config(C.Structure):
    _fields_ = [("block_size", C.c_int32), ("double_quant", C.c_int32), ("dq_group", C.c_int32),
                ("quant_type", C.c_int32)]


class nf4_tensor(C.Structure):
    _fields_ = [
        ("codes", C.c_void_p),
        ("absmax", C.c_void_p),
        ("scale_codes", C.c_void_p),
        ("group_absmax", C.c_void_p),
        ("rows", C.c_int64),
        ("cols", C.c_int64),
        ("cfg", nf4_config),
    ]


class qlora_dropout(C.Structure):
    _fields_ = [("p", C.c_float), ("pad", C.c_uint32), ("seed", C.c_uint64)]


_P = C.c_void_p
_I64 = C.c_int64
_SIGS = {
    "nf4_table": (C.POINTER(C.c_float), []),
    "nf4_levels": (C.POINTER(C.c_float), [C.c_int32]),
    "nf4_strerror": (C.c_char_p, [C.c_int]),
    "nf4_version": (C.c_int, []),
    "nf4_last_hip_error": (C.c_int, []),
    "nf4_profile_events": (C.c_int, [_P, _P, C.c_int]),
    "nf4_storage_sizes": (C.c_int, [_I64, _I64, C.POINTER(nf4_config), C.POINTER(C.c_size_t),
                                    C.POINTER(C.c_size_t), C.POINTER(C.c_size_t)]),
    "nf4_quantize": (C.c_int, [_P, _I64, _I64, C.POINTER(nf4_config), _P, _P, _P, _P, _P]),
    "nf4_quantize_bf16": (C.c_int, [_P, _I64, _I64, C.POINTER(nf4_config), _P, _P, _P, _P, _P]),
    "nf4_dequantize": (C.c_int, [C.POINTER(nf4_tensor), _P, _P]),
    "nf4_dequantize_bf16": (C.c_int, [C.POINTER(nf4_tensor), _P, _P]),
    "qlora_workspace_bytes": (C.c_size_t, [C.c_int, _I64, _I64, _I64, C.c_int32, C.c_int32]),
    "qlora_linear_forward": (C.c_int, [C.POINTER(nf4_tensor), _P, _I64, _P, _P, C.c_int32,
                                       C.c_float, _P, _P, _P, C.c_size_t, _P]),
    "qlora_linear_forward_noalloc": (C.c_int, [C.POINTER(nf4_tensor), _P, _I64, _P, _P, C.c_int32,
                                               C.c_float, _P, _P, _P]),
    "qlora_linear_forward_multi": (C.c_int, [C.POINTER(nf4_tensor), _P, _I64, _P, _P, C.c_int32,
                                             C.c_int32, _P, _P, _P, _P, C.c_size_t, _P]),
    "qlora_linear_backward": (C.c_int, [C.POINTER(nf4_tensor), _P, _P, _I64, _P, _P, C.c_int32,
                                        C.c_float, _P, _P, _P, _P, _P, C.c_size_t, _P]),
    "qlora_linear_forward_dropout": (C.c_int, [C.POINTER(nf4_tensor), _P, _I64, _P, _P, C.c_int32, C.c_float,
                                               C.POINTER(qlora_dropout), _P, _P, _P, C.c_size_t, _P]),
    "qlora_linear_backward_dropout": (C.c_int, [C.POINTER(nf4_tensor), _P, _P, _I64, _P, _P, C.c_int32,
                                                C.c_float, C.POINTER(qlora_dropout), _P, _P, _P, _P, _P,
                                                C.c_size_t, _P]),
    "qlora_merge": (C.c_int, [C.POINTER(nf4_tensor), _P, _P, C.c_int32, C.c_float, _P, _P]),
    "qlora_adamw_step": (C.c_int, [_P, _P, _P, _P, _P, _I64, C.c_int32, C.c_float, C.c_float, C.c_float,
                                   C.c_float, C.c_float, _P]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTS = tuple(_SIGS)


class NF4Error(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = _lib.nf4_strerror(code).decode()
        if code == NF4_ELAUNCH:
            msg += " (hipError %d)" % _lib.nf4_last_hip_error()
        super().__init__("%s: %s" % (where, msg))


def _check(rc: int, where: str) -> None:
    if rc != NF4_OK:
        raise NF4Error(rc, where)


def _stream(stream=None):
    import torch

    if stream is None:  # the current stream's raw handle (no Stream object made)
        return C.c_void_p(torch._C._cuda_getCurrentRawStream(torch.cuda.current_device()))
    return C.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


# ------------------------------------------------------------------ host-only
def nf4_table() -> np.ndarray:
    p = _lib.nf4_table()
    return np.ctypeslib.as_array(p, shape=(16,)).copy()


def nf4_levels(quant_type: str = "nf4") -> np.ndarray:
    """The 16 levels of a quant type, index = 4-bit code."""
    p = _lib.nf4_levels(QUANT_TYPES[quant_type])
    return np.ctypeslib.as_array(p, shape=(16,)).copy()


def nf4_version() -> int:
    return _lib.nf4_version()


def nf4_strerror(code: int) -> str:
    return _lib.nf4_strerror(code).decode()


def nf4_storage_sizes(rows: int, cols: int, double_quant: bool, dq_group: int = 256,
                      block_size: int = 64):
    cfg = nf4_config(block_size, int(double_quant), dq_group)
    a, b, c = C.c_size_t(), C.c_size_t(), C.c_size_t()
    _check(_lib.nf4_storage_sizes(rows, cols, C.byref(cfg), C.byref(a), C.byref(b), C.byref(c)),
           "nf4_storage_sizes")
    return a.value, b.value, c.value


def qlora_workspace_bytes(op: int, rows: int, cols: int, M: int, r: int, n_adapters: int = 0) -> int:
    return int(_lib.qlora_workspace_bytes(op, rows, cols, M, r, n_adapters))


def nf4_profile_events(start=None, stop=None, mode: int = 0) -> None:
    """Record a pair of raw hipEvent_t handles (ints) around the dominant
    kernel of later layer calls (None, None disables); mode 0 attaches both
    to that kernel's dispatch, mode 1 starts at the end of the kernel before."""
    _check(_lib.nf4_profile_events(None if start is None else C.c_void_p(start),
                                   None if stop is None else C.c_void_p(stop), int(mode)),
           "nf4_profile_events")


class HipEvents:
    """Minimal raw HIP event helper (the runtime torch loaded), for timing
    kernels that the library launches on the current stream."""

    def __init__(self):
        import glob

        import torch as _t

        cands = glob.glob(os.path.join(os.path.dirname(_t.__file__), "lib", "libamdhip64.so*"))
        self.rt = C.CDLL(cands[0])
        self.rt.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.rt.hipEventDestroy.argtypes = [C.c_void_p]
        self.rt.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]

    def create(self) -> int:
        e = C.c_void_p()
        if self.rt.hipEventCreate(C.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e.value

    def record(self, ev: int, stream=None) -> None:
        if self.rt.hipEventRecord(C.c_void_p(ev), _stream(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a: int, b: int) -> float:
        f = C.c_float()
        if self.rt.hipEventElapsedTime(C.byref(f), C.c_void_p(a), C.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return f.value

    def destroy(self, ev: int) -> None:
        self.rt.hipEventDestroy(C.c_void_p(ev))


# ---------------------------------------------------------------- quantized W
@dataclass
class NF4Weight:
    """Device buffers of a quantized [rows, cols] weight (torch tensors)."""

    codes: object
    absmax: object
    scale_codes: object
    group_absmax: object
    rows: int
    cols: int
    double_quant: bool
    dq_group: int = 256
    block_size: int = 64
    quant_type: str = "nf4"  # or "fp4"

    @property
    def op_flags(self) -> int:
        """Flag for the workspace queries of the layer calls on this weight."""
        return QLORA_OP_BLOCK128 if self.block_size == 128 else 0

    def c_struct(self) -> nf4_tensor:
        return nf4_tensor(
            _ptr(self.codes) or None, _ptr(self.absmax) or None,
            _ptr(self.scale_codes) if self.double_quant else None,
            _ptr(self.group_absmax) if self.double_quant else None,
            self.rows, self.cols,
            nf4_config(self.block_size, int(self.double_quant), self.dq_group, QUANT_TYPES[self.quant_type]))


def nf4_quantize(W, double_quant: bool, dq_group: int = 256, block_size: int = 64, stream=None,
                 quant_type: str = "nf4") -> NF4Weight:
    """Quantize a contiguous fp32 or bf16 CUDA tensor [rows, cols] in blocks of
    64 or 128 (bf16 through nf4_quantize_bf16: the same codes as its exact fp32
    values); quant_type "nf4" or "fp4"."""
    import torch

    rows, cols = W.shape
    n = rows * cols
    dev = W.device
    nb = n // block_size
    codes = torch.empty(max(n // 2, 16), dtype=torch.uint8, device=dev)
    absmax = torch.empty(max(nb, 4), dtype=torch.float32, device=dev)
    sc = gab = None
    if double_quant:
        sc = torch.empty(max(nb, 16), dtype=torch.int8, device=dev)
        gab = torch.empty(max((nb + dq_group - 1) // dq_group, 4), dtype=torch.float32, device=dev)
    cfg = nf4_config(block_size, int(double_quant), dq_group, QUANT_TYPES[quant_type])
    fn, name = ((_lib.nf4_quantize_bf16, "nf4_quantize_bf16") if W.dtype == torch.bfloat16
                else (_lib.nf4_quantize, "nf4_quantize"))
    _check(fn(_ptr(W), rows, cols, C.byref(cfg), _ptr(codes), _ptr(absmax), _ptr(sc), _ptr(gab),
              _stream(stream)), name)
    return NF4Weight(codes[: n // 2], absmax[:nb], None if sc is None else sc[:nb],
                     None if gab is None else gab[: (nb + dq_group - 1) // dq_group],
                     rows, cols, double_quant, dq_group, block_size, quant_type)


def nf4_dequantize(w: NF4Weight, stream=None):
    import torch

    out = torch.empty((w.rows, w.cols), dtype=torch.float32, device=w.codes.device)
    t = w.c_struct()
    _check(_lib.nf4_dequantize(C.byref(t), _ptr(out), _stream(stream)), "nf4_dequantize")
    return out


def nf4_dequantize_bf16(w: NF4Weight, stream=None):
    import torch

    out = torch.empty((w.rows, w.cols), dtype=torch.bfloat16, device=w.codes.device)
    t = w.c_struct()
    _check(_lib.nf4_dequantize_bf16(C.byref(t), _ptr(out), _stream(stream)), "nf4_dequantize_bf16")
    return out


def _workspace(nbytes: int, device):
    import torch

    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def qlora_linear_forward(w: NF4Weight, x, A, B, scale: float, want_u: bool = False, ws=None,
                         out=None, stream=None, dropout=None):
    """h = x Wb^T + scale (dropout(x) A^T) B^T; x, A, B bf16 CUDA tensors.
    dropout: None, or (p, seed) for dropout on the adapter input.  Returns h
    (and u = dropout(x) A^T)."""
    import torch

    M = x.shape[0]
    r = 0 if A is None else A.shape[0]
    h = out if out is not None else torch.empty((M, w.rows), dtype=torch.bfloat16, device=x.device)
    u = torch.empty((M, r), dtype=torch.float32, device=x.device) if (want_u and r) else None
    if ws is None:  # (a given workspace is checked by the library)
        flags = w.op_flags | (QLORA_OP_DROPOUT if dropout is not None else 0)
        ws = _workspace(qlora_workspace_bytes(QLORA_OP_FORWARD | flags, w.rows, w.cols, M, r), x.device)
    t = w.c_struct()
    if dropout is None:
        _check(_lib.qlora_linear_forward(C.byref(t), _ptr(x), M, _ptr(A), _ptr(B), r, float(scale),
                                         _ptr(h), _ptr(u), _ptr(ws), ws.numel(), _stream(stream)),
               "qlora_linear_forward")
    else:
        d = qlora_dropout(float(dropout[0]), 0, int(dropout[1]))
        _check(_lib.qlora_linear_forward_dropout(C.byref(t), _ptr(x), M, _ptr(A), _ptr(B), r, float(scale),
                                                 C.byref(d), _ptr(h), _ptr(u), _ptr(ws), ws.numel(),
                                                 _stream(stream)), "qlora_linear_forward_dropout")
    return (h, u) if want_u else h


def qlora_linear_forward_noalloc(w: NF4Weight, x, A, B, scale: float, want_u: bool = False, out=None, u_out=None,
                                 stream=None):
    """qlora_linear_forward on the library's own device scratch (the C call
    allocates nothing; pass `out` and `u_out` to allocate nothing here
    either).  Returns h (and u)."""
    import torch

    M = x.shape[0]
    r = 0 if A is None else A.shape[0]
    h = out if out is not None else torch.empty((M, w.rows), dtype=torch.bfloat16, device=x.device)
    u = u_out
    if u is None and want_u and r:
        u = torch.empty((M, r), dtype=torch.float32, device=x.device)
    t = w.c_struct()
    _check(_lib.qlora_linear_forward_noalloc(C.byref(t), _ptr(x), M, _ptr(A), _ptr(B), r, float(scale), _ptr(h),
                                             _ptr(u), _stream(stream)), "qlora_linear_forward_noalloc")
    return (h, u) if want_u else h


def qlora_linear_forward_multi(w: NF4Weight, x, A_bank, B_bank, scales, ids, ws=None, out=None,
                               stream=None):
    """Per-token adapter forward; scales fp32 CUDA [n], ids int32 CUDA [M]."""
    import torch

    M = x.shape[0]
    n, r = A_bank.shape[0], A_bank.shape[1]
    h = out if out is not None else torch.empty((M, w.rows), dtype=torch.bfloat16, device=x.device)
    need = qlora_workspace_bytes(QLORA_OP_FORWARD_MULTI | w.op_flags, w.rows, w.cols, M, r, n)
    if ws is None:
        ws = _workspace(need, x.device)
    t = w.c_struct()
    _check(_lib.qlora_linear_forward_multi(C.byref(t), _ptr(x), M, _ptr(A_bank), _ptr(B_bank), n, r,
                                           _ptr(scales), _ptr(ids), _ptr(h), _ptr(ws), ws.numel(),
                                           _stream(stream)), "qlora_linear_forward_multi")
    return h


def qlora_linear_backward(w: NF4Weight, x, dH, A, B, scale: float, u=None, want_dx: bool = True,
                          ws=None, stream=None, dropout=None):
    """Returns (dX or None, dA fp32 [r, in], dB fp32 [out, r]); dropout as in
    qlora_linear_forward (the same (p, seed) regenerates the same mask)."""
    import torch

    M = x.shape[0]
    r = A.shape[0]
    dev = x.device
    dX = torch.empty((M, w.cols), dtype=torch.bfloat16, device=dev) if want_dx else None
    dA = torch.empty((r, w.cols), dtype=torch.float32, device=dev)
    dB = torch.empty((w.rows, r), dtype=torch.float32, device=dev)
    flags = w.op_flags | (QLORA_OP_DROPOUT if dropout is not None else 0)
    need = qlora_workspace_bytes(QLORA_OP_BACKWARD | flags, w.rows, w.cols, M, r)
    if ws is None:
        ws = _workspace(need, dev)
    t = w.c_struct()
    if dropout is None:
        _check(_lib.qlora_linear_backward(C.byref(t), _ptr(x), _ptr(dH), M, _ptr(A), _ptr(B), r,
                                          float(scale), _ptr(u), _ptr(dX), _ptr(dA), _ptr(dB), _ptr(ws),
                                          ws.numel(), _stream(stream)), "qlora_linear_backward")
    else:
        d = qlora_dropout(float(dropout[0]), 0, int(dropout[1]))
        _check(_lib.qlora_linear_backward_dropout(C.byref(t), _ptr(x), _ptr(dH), M, _ptr(A), _ptr(B), r,
                                                  float(scale), C.byref(d), _ptr(u), _ptr(dX), _ptr(dA), _ptr(dB),
                                                  _ptr(ws), ws.numel(), _stream(stream)),
               "qlora_linear_backward_dropout")
    return dX, dA, dB


def qlora_merge(w: NF4Weight, A, B, scale: float, out=None, stream=None):
    """The merged bf16 weight [rows, cols] = Wb + scale * B A."""
    import torch

    r = A.shape[0]
    if out is None:
        out = torch.empty((w.rows, w.cols), dtype=torch.bfloat16, device=A.device)
    t = w.c_struct()
    _check(_lib.qlora_merge(C.byref(t), _ptr(A), _ptr(B), r, float(scale), _ptr(out), _stream(stream)),
           "qlora_merge")
    return out


def qlora_adamw_step(p, g, m, v, step: int, lr: float, beta1: float = 0.9, beta2: float = 0.999,
                     eps: float = 1e-8, weight_decay: float = 0.0, p_bf16=None, stream=None):
    """One AdamW step in place on fp32 p, m, v (m, v may be pinned host
    tensors); g fp32; p_bf16 (optional) receives bf16(p)."""
    n = p.numel()
    _check(_lib.qlora_adamw_step(_ptr(p), _ptr(g), _ptr(m), _ptr(v), _ptr(p_bf16), n, int(step), float(lr),
                                 float(beta1), float(beta2), float(eps), float(weight_decay), _stream(stream)),
           "qlora_adamw_step")
