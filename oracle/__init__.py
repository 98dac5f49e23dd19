"""CPU oracle for the PIR database-multiplication scan -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product package
(``he_database_scan_amd``) never imports it, and the oracle shares no code with
the GPU path.

This module is argument marshalling around ``liboracle.so`` (plain C, built by
``make -C oracle``); every definition lives in ``oracle.c``:

* :func:`rowsel` -- GPIR's RowSel, ``out[p,m,n] = sum_k ct[p,m,k] * DB[p,k,n]
  mod q_r`` (GPIR, the RowSel formulation paragraph; VIPIR section 4 and 2.3),
  in p-major layouts, exact 128-bit accumulation.
* :func:`exppack` -- VIPIR's ExpPack packing GEMM ``H*C + (0|G) mod q_r``
  (VIPIR section 3.5.2), the (#RNS*N)-parallel modular GEMM with the body
  term added to each client's second column.
* :func:`scalar` -- VIPIR's INT8 x INT32 database GEMM mod 2^32 (VIPIR section
  2.5 and section 4), sign-extended DB bytes.
* :func:`ntt_batch`, :func:`ntt_rns` -- the negacyclic NTT / INTT of every
  RNS limb of a batch of polynomials by direct evaluation, and the RNS
  decomposition of integer coefficients followed by the NTT (VIPIR sections
  2.3, 3.5.2 and 4.3).
* number-theory helpers (prime search, primitive roots, direct-evaluation
  negacyclic NTT/INTT, schoolbook negacyclic product) and the signed-digit
  split, used by the tests that pin the oracle.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_u32p = ctypes.POINTER(ctypes.c_uint32)
_i8p = ctypes.POINTER(ctypes.c_int8)


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (``make -C oracle``)."""
    import subprocess

    cmd = ["make", "-C", _HERE] + (["-B"] if force else [])
    subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_default_threads.restype = ctypes.c_int
        L.oracle_rowsel.argtypes = [_u32p, _u32p, _u32p, ctypes.c_uint32, ctypes.c_uint32, _u32p,
                                    ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int]
        L.oracle_rowsel.restype = ctypes.c_int
        L.oracle_exppack.argtypes = [_u32p, _u32p, _u32p, _u32p, ctypes.c_uint32, ctypes.c_uint32,
                                     _u32p, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                                     ctypes.c_int]
        L.oracle_exppack.restype = ctypes.c_int
        L.oracle_scalar.argtypes = [_i8p, _u32p, _u32p, ctypes.c_uint64, ctypes.c_uint64,
                                    ctypes.c_uint32, ctypes.c_int]
        L.oracle_scalar.restype = ctypes.c_int
        L.oracle_signed_digits_batch.argtypes = [_u32p, _i8p, ctypes.c_uint64]
        L.oracle_signed_digits_batch.restype = None
        L.oracle_is_prime_u32.argtypes = [ctypes.c_uint32]
        L.oracle_is_prime_u32.restype = ctypes.c_int
        L.oracle_ntt_primes.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int, _u32p]
        L.oracle_ntt_primes.restype = ctypes.c_int
        L.oracle_primitive_root.argtypes = [ctypes.c_uint32]
        L.oracle_primitive_root.restype = ctypes.c_uint32
        L.oracle_psi.argtypes = [ctypes.c_uint32, ctypes.c_uint32]
        L.oracle_psi.restype = ctypes.c_uint32
        L.oracle_powmod.argtypes = [ctypes.c_uint32, ctypes.c_uint64, ctypes.c_uint32]
        L.oracle_powmod.restype = ctypes.c_uint32
        for name in ("oracle_ntt", "oracle_intt"):
            f = getattr(L, name)
            f.argtypes = [_u32p, _u32p, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32]
            f.restype = None
        L.oracle_ntt_batch.argtypes = [_u32p, _u32p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                       _u32p, _u32p, ctypes.c_int, ctypes.c_int]
        L.oracle_ntt_batch.restype = ctypes.c_int
        L.oracle_ntt_rns.argtypes = [_u32p, _u32p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                     _u32p, _u32p, ctypes.c_int]
        L.oracle_ntt_rns.restype = ctypes.c_int
        L.oracle_negacyclic_mul.argtypes = [_u32p, _u32p, _u32p, ctypes.c_uint32, ctypes.c_uint32]
        L.oracle_negacyclic_mul.restype = None
        _lib = L
    return _lib


def _u32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.uint32))


def _ptr(a: np.ndarray, t):
    return a.ctypes.data_as(t)


def default_threads() -> int:
    return int(lib().oracle_default_threads())


def rowsel(ct, db, N: int, q, nthreads: int = 0) -> np.ndarray:
    """RowSel on p-major arrays: ct [m][D0][P], db [D0][D1][P] -> out [m][D1][P].

    Point p uses modulus q[p // N]; P = len(q) * N.
    """
    ct = _u32(ct)
    db = _u32(db)
    q = _u32(q)
    m, D0, P = ct.shape
    D0b, D1, Pb = db.shape
    if D0b != D0 or Pb != P or P != len(q) * N:
        raise ValueError("rowsel: inconsistent shapes")
    out = np.empty((m, D1, P), dtype=np.uint32)
    rc = lib().oracle_rowsel(_ptr(ct, _u32p), _ptr(db, _u32p), _ptr(out, _u32p), N, len(q),
                             _ptr(q, _u32p), m, D0, D1, int(nthreads))
    if rc != 0:
        raise ValueError("oracle_rowsel failed (zero modulus?)")
    return out


def exppack(H, C, G, N: int, q, nthreads: int = 0) -> np.ndarray:
    """ExpPack's H*C + (0|G) on p-major arrays (VIPIR section 3.5.2).

    H [Dr][n][P], C [n][2B][P], G [Dr][B][P] or None -> out [Dr][2B][P];
    point p uses modulus q[p // N].
    """
    H = _u32(H)
    C = _u32(C)
    q = _u32(q)
    Dr, n, P = H.shape
    nb, cols, Pb = C.shape
    if nb != n or Pb != P or cols % 2 or P != len(q) * N:
        raise ValueError("exppack: inconsistent shapes")
    B = cols // 2
    gp = None
    if G is not None:
        G = _u32(G)
        if G.shape != (Dr, B, P):
            raise ValueError("exppack: G must be [Dr][B][P]")
        gp = _ptr(G, _u32p)
    out = np.empty((Dr, cols, P), dtype=np.uint32)
    rc = lib().oracle_exppack(_ptr(H, _u32p), _ptr(C, _u32p), gp, _ptr(out, _u32p), N, len(q),
                              _ptr(q, _u32p), Dr, n, B, int(nthreads))
    if rc != 0:
        raise ValueError("oracle_exppack failed (zero modulus?)")
    return out


def scalar(db, Q, nthreads: int = 0) -> np.ndarray:
    """out[M][B] = sext(db[M][K]) @ Q[K][B] mod 2^32 (uint32)."""
    db = np.ascontiguousarray(np.asarray(db, dtype=np.int8))
    Q = _u32(Q)
    if Q.ndim == 1:
        Q = Q.reshape(-1, 1)
    M, K = db.shape
    Kb, B = Q.shape
    if Kb != K:
        raise ValueError("scalar: inconsistent shapes")
    out = np.empty((M, B), dtype=np.uint32)
    rc = lib().oracle_scalar(_ptr(db, _i8p), _ptr(Q, _u32p), _ptr(out, _u32p), M, K, B, int(nthreads))
    if rc != 0:
        raise ValueError("oracle_scalar failed")
    return out


def signed_digits(x) -> np.ndarray:
    """[n] uint32 -> [n][4] int8 signed digits (sum_j s_j 2^(8j) == x mod 2^32)."""
    x = _u32(x).reshape(-1)
    s = np.empty((x.size, 4), dtype=np.int8)
    lib().oracle_signed_digits_batch(_ptr(x, _u32p), _ptr(s, _i8p), x.size)
    return s


def is_prime(n: int) -> bool:
    return bool(lib().oracle_is_prime_u32(n))


def ntt_primes(bits: int, two_n: int, count: int) -> list[int]:
    out = np.zeros(count, dtype=np.uint32)
    k = lib().oracle_ntt_primes(bits, two_n, count, _ptr(out, _u32p))
    return [int(v) for v in out[:k]]


def primitive_root(q: int) -> int:
    return int(lib().oracle_primitive_root(q))


def psi(q: int, N: int) -> int:
    return int(lib().oracle_psi(q, N))


def powmod(a: int, e: int, q: int) -> int:
    return int(lib().oracle_powmod(a, e, q))


def ntt(a, q: int, psi_: int) -> np.ndarray:
    a = _u32(a)
    A = np.empty_like(a)
    lib().oracle_ntt(_ptr(a, _u32p), _ptr(A, _u32p), a.size, q, psi_)
    return A


def intt(A, q: int, psi_: int) -> np.ndarray:
    A = _u32(A)
    a = np.empty_like(A)
    lib().oracle_intt(_ptr(A, _u32p), _ptr(a, _u32p), A.size, q, psi_)
    return a


def ntt_batch(x, q, psis, inverse: bool = False, nthreads: int = 0) -> np.ndarray:
    """Forward (or inverse) NTT of every limb of [count][R][N] residue
    polynomials; limb r uses q[r], psis[r]."""
    x = _u32(x)
    R = len(q)
    if x.ndim != 3 or x.shape[1] != R:
        raise ValueError("expected [count][R][N]")
    out = np.empty_like(x)
    qa, pa = _u32(q), _u32(psis)
    rc = lib().oracle_ntt_batch(_ptr(x, _u32p), _ptr(out, _u32p), x.shape[0], x.shape[2], R,
                                _ptr(qa, _u32p), _ptr(pa, _u32p), int(bool(inverse)), nthreads)
    if rc != 0:
        raise ValueError("oracle_ntt_batch failed")
    return out


def ntt_rns(coeffs, q, psis, nthreads: int = 0) -> np.ndarray:
    """RNS decomposition of integer coefficients [count][N] (uint32, read as
    integers in [0, 2^32)) followed by the NTT: [count][R][N]."""
    c = _u32(coeffs)
    if c.ndim != 2:
        raise ValueError("expected [count][N]")
    R = len(q)
    out = np.empty((c.shape[0], R, c.shape[1]), dtype=np.uint32)
    qa, pa = _u32(q), _u32(psis)
    rc = lib().oracle_ntt_rns(_ptr(c, _u32p), _ptr(out, _u32p), c.shape[0], c.shape[1], R,
                              _ptr(qa, _u32p), _ptr(pa, _u32p), nthreads)
    if rc != 0:
        raise ValueError("oracle_ntt_rns failed")
    return out


def negacyclic_mul(a, b, q: int) -> np.ndarray:
    a = _u32(a)
    b = _u32(b)
    c = np.empty_like(a)
    lib().oracle_negacyclic_mul(_ptr(a, _u32p), _ptr(b, _u32p), _ptr(c, _u32p), a.size, q)
    return c
