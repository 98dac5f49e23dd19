"""Thin Python binding of libpirscan (include/pirscan.h).

Argument marshalling only: every step of the scan runs in the HIP kernels of
``libpirscan.so``.  PyTorch supplies device memory and the current HIP stream;
uint32 data travels in ``torch.int32`` (or ``torch.uint32``) tensors as raw
bits.  If the library is not built, every call raises -- there is no CPU
fallback.

Function names follow the C entry points (``pirscan_<name>``).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpirscan.so")
MAX_R = 8

OK, EINVAL, EDEVICE, EUNSUPPORTED = 0, -1, -2, -3


class RowselShape(ctypes.Structure):
    """pirscan_rowsel_shape: N points per limb, R limbs with moduli q, D0 (k), D1 (n)."""

    _fields_ = [("N", ctypes.c_uint32), ("R", ctypes.c_uint32), ("q", ctypes.c_uint32 * MAX_R),
                ("D0", ctypes.c_uint32), ("D1", ctypes.c_uint32)]

    @classmethod
    def make(cls, N: int, q, D0: int, D1: int) -> "RowselShape":
        q = [int(v) for v in q]
        if not 1 <= len(q) <= MAX_R:
            raise ValueError(f"need 1..{MAX_R} moduli")
        s = cls()
        s.N, s.R, s.D0, s.D1 = N, len(q), D0, D1
        for i, v in enumerate(q):
            s.q[i] = v
        return s

    @property
    def P(self) -> int:
        return self.N * self.R


class PirscanError(RuntimeError):
    def __init__(self, fn: str, status: int):
        lib = _load()
        msg = lib.pirscan_strerror(status).decode()
        if status == EDEVICE:
            msg += f" (hipError {lib.pirscan_last_device_error()})"
        super().__init__(f"{fn}: {msg} [{status}]")
        self.status = status


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libpirscan is not built ({LIB_PATH}); run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, u32, u64, sz = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_size_t
        shp = ctypes.POINTER(RowselShape)
        L.pirscan_layout_db_bytes.argtypes = [shp]
        L.pirscan_layout_db_bytes.restype = sz
        L.pirscan_layout_db.argtypes = [shp, vp, vp, vp]
        L.pirscan_layout_db.restype = ctypes.c_int
        L.pirscan_rowsel_workspace_bytes.argtypes = [shp, u32]
        L.pirscan_rowsel_workspace_bytes.restype = sz
        L.pirscan_rowsel_modgemm.argtypes = [shp, u32, vp, vp, vp, vp, sz, vp]
        L.pirscan_rowsel_modgemm.restype = ctypes.c_int
        L.pirscan_scalar_workspace_bytes.argtypes = [u64, u64, u32]
        L.pirscan_scalar_workspace_bytes.restype = sz
        L.pirscan_scalar_gemm_u32.argtypes = [vp, vp, vp, u64, u64, u32, vp, sz, vp]
        L.pirscan_scalar_gemm_u32.restype = ctypes.c_int
        L.pirscan_strerror.argtypes = [ctypes.c_int]
        L.pirscan_strerror.restype = ctypes.c_char_p
        L.pirscan_version.argtypes = []
        L.pirscan_version.restype = ctypes.c_int
        L.pirscan_last_device_error.argtypes = []
        L.pirscan_last_device_error.restype = ctypes.c_int
        _lib = L
    return _lib


def lib():
    """The loaded ctypes library (raises if it is not built)."""
    return _load()


def _check(fn: str, status: int):
    if status != OK:
        raise PirscanError(fn, status)


def _ptr(t) -> ctypes.c_void_p:
    if t is None:
        return ctypes.c_void_p(0)
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, name: str, elem: int, numel: int):
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.element_size() != elem or t.numel() != numel:
        raise ValueError(f"{name}: expected {numel} elements of {elem} bytes, got "
                         f"{t.numel()} of {t.element_size()}")


# ---- entry points -----------------------------------------------------------

def version() -> int:
    return int(_load().pirscan_version())


def strerror(status: int) -> str:
    return _load().pirscan_strerror(status).decode()


def layout_db_bytes(shape: RowselShape) -> int:
    return int(_load().pirscan_layout_db_bytes(ctypes.byref(shape)))


def layout_db(shape: RowselShape, db_pmajor, db_tiled, stream=None) -> None:
    """db_pmajor [D0][D1][P] (uint32 bits) -> db_tiled (same word count)."""
    n = shape.D0 * shape.D1 * shape.P
    _dev(db_pmajor, "db_pmajor", 4, n)
    _dev(db_tiled, "db_tiled", 4, n)
    _check("pirscan_layout_db",
           _load().pirscan_layout_db(ctypes.byref(shape), _ptr(db_pmajor), _ptr(db_tiled), _stream(stream)))


def rowsel_workspace_bytes(shape: RowselShape, m: int) -> int:
    return int(_load().pirscan_rowsel_workspace_bytes(ctypes.byref(shape), m))


def rowsel_modgemm(shape: RowselShape, m: int, ct, db_tiled, out, workspace=None, stream=None) -> None:
    """out[m][D1][P] = RowSel(ct[m][D0][P], db) mod q, on device.

    ``workspace``: a device buffer of at least ``rowsel_workspace_bytes(shape, m)``
    bytes (any dtype; may be None when that size is 0), owned by the caller.
    """
    P = shape.P
    _dev(ct, "ct", 4, m * shape.D0 * P)
    _dev(db_tiled, "db_tiled", 4, shape.D0 * shape.D1 * P)
    _dev(out, "out", 4, m * shape.D1 * P)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pirscan_rowsel_modgemm",
           _load().pirscan_rowsel_modgemm(ctypes.byref(shape), m, _ptr(ct), _ptr(db_tiled), _ptr(out),
                                          _ptr(workspace), wbytes, _stream(stream)))


def scalar_workspace_bytes(M: int, K: int, B: int) -> int:
    return int(_load().pirscan_scalar_workspace_bytes(M, K, B))


def scalar_gemm_u32(db, query, out, workspace=None, stream=None) -> None:
    """out[M][B] = sext(db[M][K]) @ query[K][B] mod 2^32, on device.

    ``workspace``: a device buffer of at least ``scalar_workspace_bytes(M, K, B)``
    bytes (any dtype), owned by the caller.
    """
    M, K = db.shape
    B = query.shape[1] if query.dim() == 2 else 1
    _dev(db, "db", 1, M * K)
    _dev(query, "query", 4, K * B)
    _dev(out, "out", 4, M * B)
    need = scalar_workspace_bytes(M, K, B)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pirscan_scalar_gemm_u32",
           _load().pirscan_scalar_gemm_u32(_ptr(db), _ptr(query), _ptr(out), M, K, B,
                                           _ptr(workspace) if need else ctypes.c_void_p(0),
                                           wbytes, _stream(stream)))
