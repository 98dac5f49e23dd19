"""Thin Python binding of libpirscan (include/pirscan.h).

Argument marshalling only: every step of the scan runs in the HIP kernels of
``libpirscan.so``.  PyTorch supplies device memory and the current HIP stream;
uint32 data travels in ``torch.int32`` (or ``torch.uint32``) tensors as raw
bits.  If the library is not built, every call raises -- there is no CPU
fallback.

Function names follow the C entry points (``pirscan_<name>``).  The module
functions call the product library; :class:`Library` binds any build of it,
such as ``libpirscan_bench.so`` -- the same sources compiled with the
benchmark's timing hooks, which also exports include/pirscan_bench.h
(:meth:`Library.kernel_timer_begin`, :meth:`Library.bench_read`).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpirscan.so")
BENCH_LIB_PATH = os.path.join(_HERE, "libpirscan_bench.so")
MAX_R = 8

OK, EINVAL, EDEVICE, EUNSUPPORTED, ESCRATCH = 0, -1, -2, -3, -4
NOALLOC_SCRATCH_BYTES = 72 << 20   # PIRSCAN_NOALLOC_SCRATCH_BYTES
SCAN_AUTO, SCAN_VALU = 0, 1   # PIRSCAN_SCAN_*: which scan kernel (and stored layout) a shape uses


class RowselShape(ctypes.Structure):
    """pirscan_rowsel_shape: N points per limb, R limbs with moduli q, D0 (k),
    D1 (n), and the scan kind (SCAN_AUTO or SCAN_VALU)."""

    _fields_ = [("N", ctypes.c_uint32), ("R", ctypes.c_uint32), ("q", ctypes.c_uint32 * MAX_R),
                ("D0", ctypes.c_uint32), ("D1", ctypes.c_uint32), ("scan", ctypes.c_uint32)]

    @classmethod
    def make(cls, N: int, q, D0: int, D1: int, scan: int = SCAN_AUTO) -> "RowselShape":
        q = [int(v) for v in q]
        if not 1 <= len(q) <= MAX_R:
            raise ValueError(f"need 1..{MAX_R} moduli")
        s = cls()
        s.N, s.R, s.D0, s.D1, s.scan = N, len(q), D0, D1, scan
        for i, v in enumerate(q):
            s.q[i] = v
        return s

    @property
    def P(self) -> int:
        return self.N * self.R


class ExppackShape(ctypes.Structure):
    """pirscan_exppack_shape: N points per limb, R limbs with moduli q, Dr output
    ciphertexts (rows of H and G), n LWE dimension (columns of H, rows of C),
    and the scan kind (SCAN_AUTO or SCAN_VALU)."""

    _fields_ = [("N", ctypes.c_uint32), ("R", ctypes.c_uint32), ("q", ctypes.c_uint32 * MAX_R),
                ("Dr", ctypes.c_uint32), ("n", ctypes.c_uint32), ("scan", ctypes.c_uint32)]

    @classmethod
    def make(cls, N: int, q, Dr: int, n: int, scan: int = SCAN_AUTO) -> "ExppackShape":
        q = [int(v) for v in q]
        if not 1 <= len(q) <= MAX_R:
            raise ValueError(f"need 1..{MAX_R} moduli")
        s = cls()
        s.N, s.R, s.Dr, s.n, s.scan = N, len(q), Dr, n, scan
        for i, v in enumerate(q):
            s.q[i] = v
        return s

    @property
    def P(self) -> int:
        return self.N * self.R


class NttShape(ctypes.Structure):
    """pirscan_ntt_shape: degree N (power of two), R limbs with primes q and
    primitive 2N-th roots of unity psi."""

    _fields_ = [("N", ctypes.c_uint32), ("R", ctypes.c_uint32), ("q", ctypes.c_uint32 * MAX_R),
                ("psi", ctypes.c_uint32 * MAX_R)]

    @classmethod
    def make(cls, N: int, q, psi) -> "NttShape":
        q = [int(v) for v in q]
        psi = [int(v) for v in psi]
        if not 1 <= len(q) <= MAX_R or len(psi) != len(q):
            raise ValueError(f"need 1..{MAX_R} moduli and one psi per modulus")
        s = cls()
        s.N, s.R = N, len(q)
        for i, (v, w) in enumerate(zip(q, psi)):
            s.q[i] = v
            s.psi[i] = w
        return s


class PirscanError(RuntimeError):
    def __init__(self, fn: str, status: int, lib=None):
        L = lib if lib is not None else default()._load()
        msg = L.pirscan_strerror(status).decode()
        if status == EDEVICE:
            msg += f" (hipError {L.pirscan_last_device_error()})"
        super().__init__(f"{fn}: {msg} [{status}]")
        self.status = status


def _init_torch_device():
    """torch and libpirscan each carry a HIP runtime.  The library's must start
    after torch's has opened the device: loaded first, it later finds no
    device (hipErrorNoDevice on its first call).  So torch's comes up first
    wherever a GPU is present."""
    try:
        import torch
    except ImportError:
        return
    if torch.cuda.is_available():
        torch.cuda.init()


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


def _dev_bytes(t, name: str, nbytes: int):
    """A contiguous device buffer of any dtype holding at least nbytes."""
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous() or t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name}: expected a contiguous buffer of at least {nbytes} bytes, got "
                         f"{t.numel() * t.element_size()}")


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


class Library:
    """One build of libpirscan, loaded on first use."""

    def __init__(self, path: str):
        self.path = path
        self._L = None

    def _load(self):
        if self._L is None:
            if not os.path.exists(self.path):
                raise RuntimeError(f"{os.path.basename(self.path)} is not built ({self.path}); "
                                   "run __graft_entry__.build()")
            _init_torch_device()
            L = ctypes.CDLL(self.path)
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
            ehp = ctypes.POINTER(ExppackShape)
            L.pirscan_exppack_layout_h_bytes.argtypes = [ehp]
            L.pirscan_exppack_layout_h_bytes.restype = sz
            L.pirscan_exppack_layout_h.argtypes = [ehp, vp, vp, vp]
            L.pirscan_exppack_layout_h.restype = ctypes.c_int
            L.pirscan_exppack_workspace_bytes.argtypes = [ehp, u32]
            L.pirscan_exppack_workspace_bytes.restype = sz
            L.pirscan_exppack_modgemm.argtypes = [ehp, u32, vp, vp, vp, vp, vp, sz, vp]
            L.pirscan_exppack_modgemm.restype = ctypes.c_int
            L.pirscan_scalar_workspace_bytes.argtypes = [u64, u64, u32]
            L.pirscan_scalar_workspace_bytes.restype = sz
            L.pirscan_scalar_gemm_u32.argtypes = [vp, vp, vp, u64, u64, u32, vp, sz, vp]
            L.pirscan_scalar_gemm_u32.restype = ctypes.c_int
            L.pirscan_scalar_gemm_u32_noalloc.argtypes = [vp, vp, vp, u64, u64, u32, vp]
            L.pirscan_scalar_gemm_u32_noalloc.restype = ctypes.c_int
            L.pirscan_scalar_layout_db_bytes.argtypes = [u64, u64]
            L.pirscan_scalar_layout_db_bytes.restype = sz
            L.pirscan_scalar_layout_db.argtypes = [vp, vp, u64, u64, vp]
            L.pirscan_scalar_layout_db.restype = ctypes.c_int
            L.pirscan_scalar_tiled_workspace_bytes.argtypes = [u64, u64, u32]
            L.pirscan_scalar_tiled_workspace_bytes.restype = sz
            L.pirscan_scalar_gemm_u32_tiled.argtypes = [vp, vp, vp, u64, u64, u32, vp, sz, vp]
            L.pirscan_scalar_gemm_u32_tiled.restype = ctypes.c_int
            nsp = ctypes.POINTER(NttShape)
            L.pirscan_ntt_plan_bytes.argtypes = [nsp]
            L.pirscan_ntt_plan_bytes.restype = sz
            L.pirscan_ntt_plan_init.argtypes = [nsp, vp, sz, vp]
            L.pirscan_ntt_plan_init.restype = ctypes.c_int
            for name in ("pirscan_ntt_forward", "pirscan_ntt_inverse", "pirscan_ntt_rns_forward"):
                f = getattr(L, name)
                f.argtypes = [nsp, vp, vp, vp, u64, vp]
                f.restype = ctypes.c_int
            L.pirscan_strerror.argtypes = [ctypes.c_int]
            L.pirscan_strerror.restype = ctypes.c_char_p
            L.pirscan_version.argtypes = []
            L.pirscan_version.restype = ctypes.c_int
            L.pirscan_last_device_error.argtypes = []
            L.pirscan_last_device_error.restype = ctypes.c_int
            if hasattr(L, "pirscan_kernel_timer_begin"):  # the benchmark build
                L.pirscan_kernel_timer_begin.argtypes = [u32]
                L.pirscan_kernel_timer_begin.restype = ctypes.c_int
                L.pirscan_kernel_timer_end.argtypes = [ctypes.POINTER(ctypes.c_float), u32, ctypes.POINTER(u32)]
                L.pirscan_kernel_timer_end.restype = ctypes.c_int
                L.pirscan_bench_read.argtypes = [vp, sz, vp, vp]
                L.pirscan_bench_read.restype = ctypes.c_int
            self._L = L
        return self._L

    def lib(self):
        """The loaded ctypes library (raises if it is not built)."""
        return self._load()

    def _check(self, fn: str, status: int):
        if status != OK:
            raise PirscanError(fn, status, self._load())

    @property
    def has_bench_hooks(self) -> bool:
        return hasattr(self._load(), "pirscan_kernel_timer_begin")

    # ---- entry points -------------------------------------------------------

    def version(self) -> int:
        return int(self._load().pirscan_version())

    def strerror(self, status: int) -> str:
        return self._load().pirscan_strerror(status).decode()

    def layout_db_bytes(self, shape: RowselShape) -> int:
        return int(self._load().pirscan_layout_db_bytes(ctypes.byref(shape)))

    def layout_db(self, shape: RowselShape, db_pmajor, db_tiled, stream=None) -> None:
        """db_pmajor [D0][D1][P] (uint32 bits) -> db_tiled, a device buffer of at
        least ``layout_db_bytes(shape)`` bytes (any dtype)."""
        _dev(db_pmajor, "db_pmajor", 4, shape.D0 * shape.D1 * shape.P)
        _dev_bytes(db_tiled, "db_tiled", self.layout_db_bytes(shape))
        self._check("pirscan_layout_db",
                    self._load().pirscan_layout_db(ctypes.byref(shape), _ptr(db_pmajor), _ptr(db_tiled),
                                                   _stream(stream)))

    def rowsel_workspace_bytes(self, shape: RowselShape, m: int) -> int:
        return int(self._load().pirscan_rowsel_workspace_bytes(ctypes.byref(shape), m))

    def rowsel_modgemm(self, shape: RowselShape, m: int, ct, db_tiled, out, workspace=None, stream=None) -> None:
        """out[m][D1][P] = RowSel(ct[m][D0][P], db) mod q, on device.

        ``workspace``: a device buffer of at least ``rowsel_workspace_bytes(shape, m)``
        bytes (any dtype), owned by the caller.
        """
        P = shape.P
        _dev(ct, "ct", 4, m * shape.D0 * P)
        _dev_bytes(db_tiled, "db_tiled", self.layout_db_bytes(shape))
        _dev(out, "out", 4, m * shape.D1 * P)
        self._check("pirscan_rowsel_modgemm",
                    self._load().pirscan_rowsel_modgemm(ctypes.byref(shape), m, _ptr(ct), _ptr(db_tiled), _ptr(out),
                                                        _ptr(workspace), _nbytes(workspace), _stream(stream)))

    def exppack_layout_h_bytes(self, shape: ExppackShape) -> int:
        return int(self._load().pirscan_exppack_layout_h_bytes(ctypes.byref(shape)))

    def exppack_layout_h(self, shape: ExppackShape, h_pmajor, h_tiled, stream=None) -> None:
        """h_pmajor [Dr][n][P] (uint32 bits) -> h_tiled, a device buffer of at
        least ``exppack_layout_h_bytes(shape)`` bytes (any dtype)."""
        _dev(h_pmajor, "h_pmajor", 4, shape.Dr * shape.n * shape.P)
        _dev_bytes(h_tiled, "h_tiled", self.exppack_layout_h_bytes(shape))
        self._check("pirscan_exppack_layout_h",
                    self._load().pirscan_exppack_layout_h(ctypes.byref(shape), _ptr(h_pmajor), _ptr(h_tiled),
                                                          _stream(stream)))

    def exppack_workspace_bytes(self, shape: ExppackShape, B: int) -> int:
        return int(self._load().pirscan_exppack_workspace_bytes(ctypes.byref(shape), B))

    def exppack_modgemm(self, shape: ExppackShape, B: int, C, h_tiled, G, out, workspace=None,
                        stream=None) -> None:
        """out[Dr][2B][P] = H*C + (0|G) mod q, on device (VIPIR section 3.5.2).

        C [n][2B][P], G [Dr][B][P] or None, all uint32 bits in 4-byte tensors.
        ``workspace``: at least ``exppack_workspace_bytes(shape, B)`` bytes, owned
        by the caller.
        """
        P = shape.P
        _dev(C, "C", 4, shape.n * 2 * B * P)
        _dev_bytes(h_tiled, "h_tiled", self.exppack_layout_h_bytes(shape))
        if G is not None:
            _dev(G, "G", 4, shape.Dr * B * P)
        _dev(out, "out", 4, shape.Dr * 2 * B * P)
        self._check("pirscan_exppack_modgemm",
                    self._load().pirscan_exppack_modgemm(ctypes.byref(shape), B, _ptr(C), _ptr(h_tiled), _ptr(G),
                                                         _ptr(out), _ptr(workspace), _nbytes(workspace),
                                                         _stream(stream)))

    def scalar_workspace_bytes(self, M: int, K: int, B: int) -> int:
        return int(self._load().pirscan_scalar_workspace_bytes(M, K, B))

    def scalar_gemm_u32(self, db, query, out, workspace=None, stream=None) -> None:
        """out[M][B] = sext(db[M][K]) @ query[K][B] mod 2^32, on device.

        ``workspace``: a device buffer of at least ``scalar_workspace_bytes(M, K, B)``
        bytes (any dtype), owned by the caller.
        """
        M, K = db.shape
        B = query.shape[1] if query.dim() == 2 else 1
        _dev(db, "db", 1, M * K)
        _dev(query, "query", 4, K * B)
        _dev(out, "out", 4, M * B)
        need = self.scalar_workspace_bytes(M, K, B)
        self._check("pirscan_scalar_gemm_u32",
                    self._load().pirscan_scalar_gemm_u32(_ptr(db), _ptr(query), _ptr(out), M, K, B,
                                                         _ptr(workspace) if need else ctypes.c_void_p(0),
                                                         _nbytes(workspace), _stream(stream)))

    def scalar_gemm_u32_noalloc(self, db, query, out, stream=None) -> None:
        """As :meth:`scalar_gemm_u32`, with the library's built-in scratch buffer
        instead of a workspace: for callers that cannot allocate.  Calls that
        overlap in time on one GPU share that buffer and race."""
        M, K = db.shape
        B = query.shape[1] if query.dim() == 2 else 1
        _dev(db, "db", 1, M * K)
        _dev(query, "query", 4, K * B)
        _dev(out, "out", 4, M * B)
        self._check("pirscan_scalar_gemm_u32_noalloc",
                    self._load().pirscan_scalar_gemm_u32_noalloc(_ptr(db), _ptr(query), _ptr(out), M, K, B,
                                                                 _stream(stream)))

    def scalar_layout_db_bytes(self, M: int, K: int) -> int:
        return int(self._load().pirscan_scalar_layout_db_bytes(M, K))

    def scalar_layout_db(self, db, db_tiled, stream=None) -> None:
        """db [M][K] int8 (row-major) -> db_tiled, a device buffer of at least
        ``scalar_layout_db_bytes(M, K)`` bytes (any dtype)."""
        M, K = db.shape
        _dev(db, "db", 1, M * K)
        _dev_bytes(db_tiled, "db_tiled", self.scalar_layout_db_bytes(M, K))
        self._check("pirscan_scalar_layout_db",
                    self._load().pirscan_scalar_layout_db(_ptr(db), _ptr(db_tiled), M, K, _stream(stream)))

    def scalar_tiled_workspace_bytes(self, M: int, K: int, B: int) -> int:
        return int(self._load().pirscan_scalar_tiled_workspace_bytes(M, K, B))

    def scalar_gemm_u32_tiled(self, db_tiled, M: int, K: int, query, out, workspace, stream=None) -> None:
        """out[M][B] = sext(db) @ query[K][B] mod 2^32 on the tiled DB, on device.

        ``workspace``: at least ``scalar_tiled_workspace_bytes(M, K, B)`` bytes,
        owned by the caller.
        """
        B = query.shape[1] if query.dim() == 2 else 1
        _dev_bytes(db_tiled, "db_tiled", self.scalar_layout_db_bytes(M, K))
        _dev(query, "query", 4, K * B)
        _dev(out, "out", 4, M * B)
        self._check("pirscan_scalar_gemm_u32_tiled",
                    self._load().pirscan_scalar_gemm_u32_tiled(_ptr(db_tiled), _ptr(query), _ptr(out), M, K, B,
                                                               _ptr(workspace), _nbytes(workspace),
                                                               _stream(stream)))

    def ntt_plan_bytes(self, shape: NttShape) -> int:
        return int(self._load().pirscan_ntt_plan_bytes(ctypes.byref(shape)))

    def ntt_plan_init(self, shape: NttShape, plan, stream=None) -> None:
        """Fills ``plan`` (a device buffer of at least ``ntt_plan_bytes(shape)``
        bytes) with the shape's twiddle factors."""
        if plan.device.type != "cuda":
            raise ValueError("plan must be a device tensor")
        self._check("pirscan_ntt_plan_init",
                    self._load().pirscan_ntt_plan_init(ctypes.byref(shape), _ptr(plan), _nbytes(plan),
                                                       _stream(stream)))

    def _ntt_call(self, name: str, shape: NttShape, plan, x, out, in_words_per_poly: int, stream):
        N, R = shape.N, shape.R
        if x.numel() % in_words_per_poly:
            raise ValueError(f"input of {x.numel()} words is not a whole number of polynomials")
        count = x.numel() // in_words_per_poly
        _dev(x, "input", 4, count * in_words_per_poly)
        _dev(out, "out", 4, count * R * N)
        self._check(name, getattr(self._load(), name)(ctypes.byref(shape), _ptr(plan), _ptr(x), _ptr(out), count,
                                                      _stream(stream)))

    def ntt_forward(self, shape: NttShape, plan, x, out, stream=None) -> None:
        """out[c][r][:] = NTT of x[c][r][:] mod q[r] (x, out: [count][R][N] uint32
        bits; out may be x)."""
        self._ntt_call("pirscan_ntt_forward", shape, plan, x, out, shape.R * shape.N, stream)

    def ntt_inverse(self, shape: NttShape, plan, x, out, stream=None) -> None:
        """Inverse of :meth:`ntt_forward` (out may be x)."""
        self._ntt_call("pirscan_ntt_inverse", shape, plan, x, out, shape.R * shape.N, stream)

    def ntt_rns_forward(self, shape: NttShape, plan, coeffs, out, stream=None) -> None:
        """out[c][r][:] = NTT of (coeffs[c][:] mod q[r]): coeffs [count][N] integers
        in [0, 2^32) as uint32 bits, out [count][R][N]."""
        self._ntt_call("pirscan_ntt_rns_forward", shape, plan, coeffs, out, shape.N, stream)

    # ---- the benchmark build only (include/pirscan_bench.h) ---------------

    def _bench_lib(self, fn: str):
        L = self._load()
        if not hasattr(L, "pirscan_kernel_timer_begin"):
            raise RuntimeError(f"{fn}: {os.path.basename(self.path)} is not the benchmark build "
                               f"(use {os.path.basename(BENCH_LIB_PATH)})")
        return L

    def bench_read(self, buf, sink, stream=None) -> None:
        """Benchmark reference: one non-temporal read pass over the device buffer
        ``buf`` (16-byte aligned, a multiple of 16 bytes); ``sink`` is a device
        buffer of at least 4 bytes whose contents become unspecified."""
        L = self._bench_lib("pirscan_bench_read")
        _dev_bytes(sink, "sink", 4)
        if buf.device.type != "cuda":
            raise ValueError("buf must be a device tensor")
        self._check("pirscan_bench_read", L.pirscan_bench_read(_ptr(buf), _nbytes(buf), _ptr(sink), _stream(stream)))

    def kernel_timer_begin(self, capacity: int) -> None:
        """Benchmark hook: time the main kernel of the next ``capacity`` scan calls
        of this thread with HIP events on their stream."""
        L = self._bench_lib("pirscan_kernel_timer_begin")
        self._check("pirscan_kernel_timer_begin", L.pirscan_kernel_timer_begin(capacity))

    def kernel_timer_end(self, max_count: int) -> list:
        """Waits for the recorded events; returns each call's main-kernel time (ms)."""
        L = self._bench_lib("pirscan_kernel_timer_end")
        buf = (ctypes.c_float * max(1, max_count))()
        n = ctypes.c_uint32(0)
        self._check("pirscan_kernel_timer_end", L.pirscan_kernel_timer_end(buf, max_count, ctypes.byref(n)))
        return [float(buf[i]) for i in range(n.value)]


# ---- module-level entry points: the default library ---------------------------

_default = Library(LIB_PATH)


def default() -> Library:
    """The library the module functions call (the product build unless
    :func:`use_library` chose another)."""
    return _default


def use_library(path: str) -> Library:
    """Make the module functions call the build at ``path`` (for instance
    BENCH_LIB_PATH, so that the scans and the timing hooks are one library).
    Only before the default library has been loaded."""
    global _default
    if _default._L is not None and _default.path != path:
        raise RuntimeError(f"{os.path.basename(_default.path)} is already loaded")
    _default = Library(path)
    return _default


def bench_library() -> Library:
    """The benchmark build (libpirscan_bench.so) as its own :class:`Library`."""
    return _default if _default.path == BENCH_LIB_PATH else Library(BENCH_LIB_PATH)


def lib():
    """The default library's ctypes handle (raises if it is not built)."""
    return _default._load()


def _forward(name):
    def call(*args, **kwargs):
        return getattr(_default, name)(*args, **kwargs)

    call.__name__ = name
    call.__doc__ = getattr(Library, name).__doc__
    return call


for _name in ("version", "strerror", "layout_db_bytes", "layout_db", "rowsel_workspace_bytes", "rowsel_modgemm",
              "exppack_layout_h_bytes", "exppack_layout_h", "exppack_workspace_bytes", "exppack_modgemm",
              "scalar_workspace_bytes", "scalar_gemm_u32", "scalar_gemm_u32_noalloc", "scalar_layout_db_bytes",
              "scalar_layout_db",
              "scalar_tiled_workspace_bytes", "scalar_gemm_u32_tiled", "ntt_plan_bytes", "ntt_plan_init",
              "ntt_forward", "ntt_inverse", "ntt_rns_forward", "bench_read", "kernel_timer_begin",
              "kernel_timer_end"):
    globals()[_name] = _forward(_name)
del _name
