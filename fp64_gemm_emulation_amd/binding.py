"""ctypes binding of liboz2.so (the C ABI in include/oz2.h).

Argument marshalling only: every step of the computation runs in the HIP library.
The functions named like the C entry points take plain integers / device pointers;
``dgemm`` and ``dgemm_debug`` are conveniences over torch tensors (PyTorch supplies
device memory and the current stream, nothing else).

Loading fails loudly if the library has not been built: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "liboz2.so")

OZ2_FAST, OZ2_ACCU = 0, 1
OZ2_OK, OZ2_ERR_ARG, OZ2_ERR_UNSUPPORTED, OZ2_ERR_WORKSPACE, OZ2_ERR_HIP = 0, 1, 2, 3, 4
OZ2_MIN_S, OZ2_MAX_S, OZ2_MAX_Q, OZ2_MAX_Q_P_DUMP, OZ2_X_LIMBS = 2, 20, 524287, 131071, 5
OZ2_OP_N, OZ2_OP_T = 0, 1
OZ2_FLAG_NONFINITE = 1
OZ2_NOALLOC_SCRATCH_BYTES = 256 << 20
MODES = {"fast": OZ2_FAST, "accu": OZ2_ACCU}


class Oz2Error(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {ozaki2_status_string(status)} (status {status})")
        self.status = status


class OZ2Dump(ctypes.Structure):
    """Mirror of oz2_dump_t: device pointers (0 = skip)."""

    _fields_ = [(name, ctypes.c_void_p) for name in
                ("d", "b", "Ap", "Bp", "At", "Bt", "P", "R", "X",
                 "e", "f", "Abar", "Bbar", "rho", "gamma")]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it first (python -m fp64_gemm_emulation_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    i, vp, sz = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    sig = {
        "ozaki2_dgemm": (i, [i, i, i, vp, i, vp, i, vp, i, i, i, vp]),
        "ozaki2_dgemm_noalloc": (i, [i, i, i, vp, i, vp, i, vp, i, i, i, vp]),
        "ozaki2_dgemm_ex": (i, [i, i, i, i, i, ctypes.c_double, vp, i, vp, i, ctypes.c_double, vp, i, i, i, vp]),
        "ozaki2_dgemm_debug": (i, [i, i, i, vp, i, vp, i, vp, i, i, i, vp, ctypes.POINTER(OZ2Dump)]),
        "ozaki2_workspace_size": (sz, [i, i, i, i, i]),
        "ozaki2_set_workspace": (i, [vp, sz]),
        "ozaki2_release": (i, []),
        "ozaki2_timing_begin": (i, [i]),
        "ozaki2_timing_end": (i, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i)]),
        "ozaki2_get_stage_ms": (i, [ctypes.POINTER(ctypes.c_float)]),
        "ozaki2_get_flags": (i, [ctypes.POINTER(ctypes.c_uint)]),
        "ozaki2_moduli": (i, [i, ctypes.POINTER(i)]),
        "ozaki2_tau": (i, [i]),
        "ozaki2_status_string": (ctypes.c_char_p, [i]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_LIB = _load()


# --- entry points with the C names -------------------------------------------------
def ozaki2_dgemm(p, q, r, A, lda, B, ldb, C, ldc, s, mode, stream) -> int:
    return _LIB.ozaki2_dgemm(p, q, r, A, lda, B, ldb, C, ldc, s, mode, stream)


def ozaki2_dgemm_noalloc(p, q, r, A, lda, B, ldb, C, ldc, s, mode, stream) -> int:
    return _LIB.ozaki2_dgemm_noalloc(p, q, r, A, lda, B, ldb, C, ldc, s, mode, stream)


def ozaki2_dgemm_ex(transa, transb, p, q, r, alpha, A, lda, B, ldb, beta, C, ldc, s, mode, stream) -> int:
    return _LIB.ozaki2_dgemm_ex(transa, transb, p, q, r, alpha, A, lda, B, ldb, beta, C, ldc, s, mode, stream)


def ozaki2_dgemm_debug(p, q, r, A, lda, B, ldb, C, ldc, s, mode, stream, dump: OZ2Dump | None) -> int:
    return _LIB.ozaki2_dgemm_debug(p, q, r, A, lda, B, ldb, C, ldc, s, mode, stream,
                                   ctypes.byref(dump) if dump is not None else None)


def ozaki2_workspace_size(p, q, r, s, mode) -> int:
    return _LIB.ozaki2_workspace_size(p, q, r, s, mode)


def ozaki2_set_workspace(ptr, nbytes) -> int:
    return _LIB.ozaki2_set_workspace(ptr, nbytes)


def ozaki2_release() -> int:
    return _LIB.ozaki2_release()


def ozaki2_timing_begin(max_calls: int) -> int:
    return _LIB.ozaki2_timing_begin(max_calls)


def ozaki2_timing_end():
    """Returns (status, [scaling, residues, gemm, crt] ms summed, ncalls)."""
    ms = (ctypes.c_double * 4)()
    n = ctypes.c_int(0)
    rc = _LIB.ozaki2_timing_end(ms, ctypes.byref(n))
    return rc, list(ms), n.value


def ozaki2_get_stage_ms():
    """Returns (status, [scaling, residues, gemm, crt] ms of the most recent timed call)."""
    ms = (ctypes.c_float * 4)()
    rc = _LIB.ozaki2_get_stage_ms(ms)
    return rc, list(ms)


def ozaki2_get_flags():
    v = ctypes.c_uint(0)
    rc = _LIB.ozaki2_get_flags(ctypes.byref(v))
    return rc, v.value


def ozaki2_moduli(s: int):
    out = (ctypes.c_int * max(s, 1))()
    rc = _LIB.ozaki2_moduli(s, out)
    return rc, list(out)[:s]


def ozaki2_tau(s: int) -> int:
    return _LIB.ozaki2_tau(s)


def ozaki2_status_string(status: int) -> str:
    return _LIB.ozaki2_status_string(status).decode()


# --- torch conveniences --------------------------------------------------------------
def _colmajor_ld(t, name):
    import torch
    if t.dtype != torch.float64 or not t.is_cuda or t.dim() != 2:
        raise ValueError(f"{name} must be a 2-D float64 CUDA tensor")
    rows, cols = t.shape
    if rows == 0 or cols == 0:
        return max(1, rows)
    if t.stride(0) != 1 or (cols > 1 and t.stride(1) < rows):
        raise ValueError(f"{name} must be column-major (stride (1, ld >= rows)); use colmajor()")
    return t.stride(1) if cols > 1 else max(1, rows)


def colmajor(t):
    """Column-major copy of a 2-D tensor (same values, Fortran layout)."""
    return t.t().contiguous().t()


def empty_colmajor(rows, cols, device="cuda", dtype=None):
    import torch
    return torch.empty((cols, rows), dtype=dtype or torch.float64, device=device).t()


def _stream_ptr(stream, device):
    import torch
    st = stream if stream is not None else torch.cuda.current_stream(device)
    return st.cuda_stream


def _on_device(*tensors):
    """The operands' common device, made current for the call (the library works on the
    current device)."""
    import torch
    dev = tensors[0].device
    for t in tensors[1:]:
        if t is not None and t.device != dev:
            raise ValueError("all operands must be on the same device")
    return torch.cuda.device(dev)


def dgemm(A, B, s: int = 14, mode: str = "fast", out=None, stream=None):
    """C = A B (FP64, emulated) for column-major CUDA tensors; returns C (column-major)."""
    p, q = A.shape
    q2, r = B.shape
    if q != q2:
        raise ValueError("inner dimensions differ")
    C = out if out is not None else empty_colmajor(p, r, device=A.device)
    if tuple(C.shape) != (p, r):
        raise ValueError("out has the wrong shape")
    with _on_device(A, B, C):
        rc = ozaki2_dgemm(p, q, r, A.data_ptr(), _colmajor_ld(A, "A"), B.data_ptr(), _colmajor_ld(B, "B"),
                          C.data_ptr(), _colmajor_ld(C, "C"), s, MODES[mode], _stream_ptr(stream, A.device))
    if rc != OZ2_OK:
        raise Oz2Error(rc, "ozaki2_dgemm")
    return C


def dgemm_ex(A, B, transa: bool = False, transb: bool = False, alpha: float = 1.0, beta: float = 0.0,
             C=None, s: int = 14, mode: str = "fast", stream=None):
    """C = alpha op(A) op(B) + beta C for column-major CUDA tensors (op = transpose when
    transa / transb); C is created (and beta must be 0) when not given.  Returns C."""
    p, q = (A.shape[1], A.shape[0]) if transa else tuple(A.shape)
    q2, r = (B.shape[1], B.shape[0]) if transb else tuple(B.shape)
    if q != q2:
        raise ValueError("inner dimensions differ")
    if C is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs C")
        C = empty_colmajor(p, r, device=A.device)
    if tuple(C.shape) != (p, r):
        raise ValueError("C has the wrong shape")
    with _on_device(A, B, C):
        rc = ozaki2_dgemm_ex(OZ2_OP_T if transa else OZ2_OP_N, OZ2_OP_T if transb else OZ2_OP_N, p, q, r,
                             float(alpha), A.data_ptr(), _colmajor_ld(A, "A"), B.data_ptr(), _colmajor_ld(B, "B"),
                             float(beta), C.data_ptr(), _colmajor_ld(C, "C"), s, MODES[mode],
                             _stream_ptr(stream, A.device))
    if rc != OZ2_OK:
        raise Oz2Error(rc, "ozaki2_dgemm_ex")
    return C


DUMP_FIELDS = ("d", "b", "Ap", "Bp", "At", "Bt", "P", "R", "X", "e", "f", "Abar", "Bbar", "rho", "gamma")


def dgemm_debug(A, B, s: int = 14, mode: str = "fast", want=DUMP_FIELDS, stream=None):
    """Run ozaki2_dgemm_debug; returns dict with C and the requested intermediates as
    device tensors in the layouts documented in include/oz2.h."""
    import torch
    p, q = A.shape
    _, r = B.shape
    dev = A.device
    C = empty_colmajor(p, r, device=dev)
    shapes = {
        "d": ((p,), torch.int32), "b": ((r,), torch.int32),
        "Ap": ((q, p), torch.float64), "Bp": ((r, q), torch.float64),   # column-major p x q / q x r
        "At": ((s, p, q), torch.int8), "Bt": ((s, r, q), torch.int8),
        "P": ((s, r, p), torch.int32), "R": ((s, r, p), torch.uint8),
        "X": ((r, p, OZ2_X_LIMBS), torch.int32),
        "e": ((p,), torch.int32), "f": ((r,), torch.int32),
        "Abar": ((p, q), torch.int8), "Bbar": ((r, q), torch.int8),
        "rho": ((p,), torch.int32), "gamma": ((r,), torch.int32),
    }
    bufs = {k: torch.zeros(*shapes[k][0], dtype=shapes[k][1], device=dev) for k in want}
    dump = OZ2Dump(**{k: (bufs[k].data_ptr() if bufs[k].numel() else None) for k in want})
    with _on_device(A, B, C):
        rc = ozaki2_dgemm_debug(p, q, r, A.data_ptr(), _colmajor_ld(A, "A"), B.data_ptr(), _colmajor_ld(B, "B"),
                                C.data_ptr(), _colmajor_ld(C, "C"), s, MODES[mode], _stream_ptr(stream, dev), dump)
    if rc != OZ2_OK:
        raise Oz2Error(rc, "ozaki2_dgemm_debug")
    if "Ap" in bufs:
        bufs["Ap"] = bufs["Ap"].t()
    if "Bp" in bufs:
        bufs["Bp"] = bufs["Bp"].t()
    bufs["C"] = C
    return bufs
