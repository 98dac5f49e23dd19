"""Seeded synthetic inputs for the PIR scan -- shared by the oracle side and
the GPU side, and holding none of the scan's arithmetic.

The generator is counter-based SplitMix64 (Steele, Lea and Flood, "Fast
splittable pseudorandom number generators", OOPSLA 2014; the 64-bit finaliser
with the constants of Vigna's public-domain ``splitmix64.c``):

    mix64(z):  z ^= z >> 30; z *= 0xBF58476D1CE4E5B9
               z ^= z >> 27; z *= 0x94D049BB133111EB
               z ^= z >> 31
    value(state0, i) = mix64(state0 + (i + 1) * 0x9E3779B97F4A7C15)  (mod 2^64)

i.e. the i-th output of SplitMix64 started from ``state0``.  Every element is a
pure function of (seed, stream, index), so any slice of a 64 GiB input can be
regenerated on the host without materialising the rest.  ``state0`` is derived
on the host only and handed to the device filler, so the device implements
just ``mix64`` and the counter.

Derived element types (the shapes and distributions of the pages' workloads:
uniform residues for NTT-domain points, uniform int8 records, uniform
Z_{2^32} query words):

* residue mod q:  ``value % q`` where the element at linear index ``i`` of a
  p-major ``[X][P]`` array uses ``q[(i % P) // N]``;
* int8:           byte ``i % 8`` (little-endian) of ``value(i // 8)``;
* uint32:         the high 32 bits of ``value(i)``.

Streams: RowSel DB 1, RowSel ct 2, scalar DB 3, scalar query 4, ExpPack hint H 5,
ExpPack special ciphertexts C 6, ExpPack body G 7, NTT input 8.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1

STREAM_ROWSEL_DB = 1
STREAM_ROWSEL_CT = 2
STREAM_SCALAR_DB = 3
STREAM_SCALAR_Q = 4
STREAM_EXPPACK_H = 5
STREAM_EXPPACK_C = 6
STREAM_EXPPACK_G = 7
STREAM_NTT_IN = 8


def mix64_int(z: int) -> int:
    z &= MASK64
    z ^= z >> 30
    z = (z * _M1) & MASK64
    z ^= z >> 27
    z = (z * _M2) & MASK64
    z ^= z >> 31
    return z


def state0(seed: int, stream: int) -> int:
    """Start state of one (seed, stream) sequence."""
    return mix64_int(seed) ^ mix64_int((stream + 0x632BE59BD9B4E019) & MASK64)


def mix64(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.uint64).copy()
    with np.errstate(over="ignore"):
        z ^= z >> np.uint64(30)
        z *= np.uint64(_M1)
        z ^= z >> np.uint64(27)
        z *= np.uint64(_M2)
        z ^= z >> np.uint64(31)
    return z


def values(st: int, idx) -> np.ndarray:
    """SplitMix64 outputs number ``idx`` (0-based) from start state ``st``."""
    idx = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(st) + (idx + np.uint64(1)) * np.uint64(GAMMA)
    return mix64(z)


# ---- element types -------------------------------------------------------

def residues(seed: int, stream: int, idx, P: int, N: int, q) -> np.ndarray:
    """Residues at linear indices ``idx`` of a p-major [X][P] array."""
    idx = np.asarray(idx, dtype=np.uint64)
    qv = np.asarray(q, dtype=np.uint64)[(idx % np.uint64(P)) // np.uint64(N)]
    return (values(state0(seed, stream), idx) % qv).astype(np.uint32)


def residue_array(seed: int, stream: int, shape, N: int, q) -> np.ndarray:
    """A full p-major array of the given shape (last axis = P = len(q)*N)."""
    P = shape[-1]
    assert P == len(q) * N
    n = int(np.prod(shape))
    return residues(seed, stream, np.arange(n, dtype=np.uint64), P, N, q).reshape(shape)


def int8_bytes(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """Bytes [start, start+count) of the int8 stream."""
    if count == 0:
        return np.zeros(0, dtype=np.int8)
    w0 = start // 8
    w1 = (start + count + 7) // 8
    v = values(state0(seed, stream), np.arange(w0, w1, dtype=np.uint64))
    b = v.astype("<u8").view(np.int8)
    off = start - 8 * w0
    return b[off:off + count].copy()


def int8_rows(seed: int, stream: int, K: int, rows) -> np.ndarray:
    """Rows of a row-major [M][K] int8 matrix drawn from the int8 stream."""
    rows = list(rows)
    out = np.empty((len(rows), K), dtype=np.int8)
    for r, i in enumerate(rows):
        out[r] = int8_bytes(seed, stream, int(i) * K, K)
    return out


def uint32_words(seed: int, stream: int, idx) -> np.ndarray:
    idx = np.asarray(idx, dtype=np.uint64)
    return (values(state0(seed, stream), idx) >> np.uint64(32)).astype(np.uint32)


def uint32_array(seed: int, stream: int, shape) -> np.ndarray:
    n = int(np.prod(shape))
    return uint32_words(seed, stream, np.arange(n, dtype=np.uint64)).reshape(shape)


# ---- device filler (libpirsynth.so) --------------------------------------

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libpirsynth.so")
_dev = None


def _device_lib():
    global _dev
    if _dev is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built (run __graft_entry__.build())")
        # torch's bundled HIP runtime must open the device before the one this
        # library links comes up (loaded first, the library's runtime later
        # finds no device), so torch's starts first
        import torch

        if torch.cuda.is_available():
            torch.cuda.init()
        L = ctypes.CDLL(_LIB_PATH)
        vp, u64, u32 = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32
        L.pirsynth_fill_residues.argtypes = [vp, u64, u64, u64, u32, u32, ctypes.POINTER(u32), vp]
        L.pirsynth_fill_residues.restype = ctypes.c_int
        L.pirsynth_fill_int8.argtypes = [vp, u64, u64, u64, vp]
        L.pirsynth_fill_int8.restype = ctypes.c_int
        L.pirsynth_fill_uint32.argtypes = [vp, u64, u64, u64, vp]
        L.pirsynth_fill_uint32.restype = ctypes.c_int
        _dev = L
    return _dev


def _stream_handle():
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def fill_residues_(t, seed: int, stream: int, N: int, q, first_index: int = 0):
    """Fill a contiguous device tensor (int32/uint32 bits) as a p-major array
    whose last axis is P = len(q) * N; element j gets linear index
    ``first_index + j``."""
    assert t.is_contiguous() and t.element_size() == 4
    P = len(q) * N
    qa = (ctypes.c_uint32 * 8)(*[int(v) for v in q])
    rc = _device_lib().pirsynth_fill_residues(ctypes.c_void_p(t.data_ptr()), t.numel(), state0(seed, stream),
                                              first_index, P, N, qa, _stream_handle())
    if rc != 0:
        raise RuntimeError(f"pirsynth_fill_residues failed ({rc})")
    return t


def fill_int8_(t, seed: int, stream: int, first_byte: int = 0):
    assert t.is_contiguous() and t.element_size() == 1
    rc = _device_lib().pirsynth_fill_int8(ctypes.c_void_p(t.data_ptr()), t.numel(), state0(seed, stream),
                                          first_byte, _stream_handle())
    if rc != 0:
        raise RuntimeError(f"pirsynth_fill_int8 failed ({rc})")
    return t


def fill_uint32_(t, seed: int, stream: int, first_index: int = 0):
    assert t.is_contiguous() and t.element_size() == 4
    rc = _device_lib().pirsynth_fill_uint32(ctypes.c_void_p(t.data_ptr()), t.numel(), state0(seed, stream),
                                            first_index, _stream_handle())
    if rc != 0:
        raise RuntimeError(f"pirsynth_fill_uint32 failed ({rc})")
    return t
