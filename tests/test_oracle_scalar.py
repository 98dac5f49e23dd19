"""Pins for the scalar-HE oracle (oracle.scalar): VIPIR section 2.5 (the
D1 x B x D0 INT8-INT32 GEMM of batched SimplePIR) and section 4 (mod 2^32 is
free); Regev parameters of section 2.2 / 5 (plaintext 2^8, ciphertext 2^32)."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def numpy_reference(db, Q):
    """Library routine: exact int64 matmul then mod 2^32.  |sum| <= 128 *
    (2^32-1) * K < 2^63 for K <= 2^24, so int64 is exact here."""
    return ((db.astype(np.int64) @ Q.astype(np.int64)) & 0xFFFFFFFF).astype(np.uint32)


@pytest.mark.parametrize("M,K,B", [(1, 1, 1), (3, 17, 1), (5, 64, 8), (33, 1000, 3), (64, 4096, 32)])
def test_matches_numpy_int64(M, K, B):
    rng = np.random.default_rng(M * 1000 + K + B)
    db = rng.integers(-128, 128, size=(M, K), dtype=np.int64).astype(np.int8)
    Q = rng.integers(0, 1 << 32, size=(K, B), dtype=np.uint64).astype(np.uint32)
    np.testing.assert_array_equal(oracle.scalar(db, Q), numpy_reference(db, Q))


def test_matches_python_bruteforce():
    rng = np.random.default_rng(9)
    M, K, B = 4, 13, 3
    db = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    Q = rng.integers(0, 1 << 32, size=(K, B), dtype=np.uint64).astype(np.uint32)
    out = oracle.scalar(db, Q)
    for i in range(M):
        for b in range(B):
            assert int(out[i, b]) == sum(int(db[i, k]) * int(Q[k, b]) for k in range(K)) % (1 << 32)


def test_one_hot_returns_sign_extended_column():
    M, K = 257, 300
    db = synth.int8_rows(2, synth.STREAM_SCALAR_DB, K, range(M))
    for k in (0, 1, 150, K - 1):
        Q = np.zeros((K, 1), dtype=np.uint32)
        Q[k, 0] = 1
        out = oracle.scalar(db, Q)[:, 0]
        np.testing.assert_array_equal(out, db[:, k].astype(np.int32).astype(np.uint32))
    assert (oracle.scalar(np.full((1, 1), -1, np.int8), np.ones((1, 1), np.uint32)) == 0xFFFFFFFF).all()


def test_regev_view_recovers_plaintext_byte():
    """Q = Delta * e_k with Delta = 2^24 (plaintext 2^8 in ciphertext 2^32):
    the top byte of the output is the selected record mod 256."""
    M, K = 100, 64
    db = synth.int8_rows(2, synth.STREAM_SCALAR_DB, K, range(M))
    Q = np.zeros((K, 1), dtype=np.uint32)
    Q[37, 0] = 1 << 24
    out = oracle.scalar(db, Q)[:, 0]
    np.testing.assert_array_equal((out >> 24).astype(np.uint8), db[:, 37].view(np.uint8))


@pytest.mark.parametrize("K", [1, 2, 1000, 1 << 18])
def test_closed_form_overflow(K):
    # db = -128, Q = 0xFFFFFFFF = -1 (mod 2^32): out = 128 K mod 2^32
    db = np.full((2, K), -128, dtype=np.int8)
    Q = np.full((K, 1), 0xFFFFFFFF, dtype=np.uint32)
    assert (oracle.scalar(db, Q) == (128 * K) % (1 << 32)).all()
    # db = 127, Q = 2^31: out = 127 * 2^31 * K mod 2^32 = 2^31 * (K mod 2)
    db = np.full((1, K), 127, dtype=np.int8)
    Q = np.full((K, 1), 1 << 31, dtype=np.uint32)
    assert int(oracle.scalar(db, Q)[0, 0]) == (127 * (1 << 31) * K) % (1 << 32)


def test_batched_equals_stacked_gemv():
    rng = np.random.default_rng(12)
    M, K, B = 40, 333, 8
    db = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    Q = rng.integers(0, 1 << 32, size=(K, B), dtype=np.uint64).astype(np.uint32)
    full = oracle.scalar(db, Q)
    for b in range(B):
        np.testing.assert_array_equal(full[:, b], oracle.scalar(db, Q[:, b:b + 1].copy())[:, 0])


def test_signed_digit_examples():
    cases = {0xFFFFFFFF: (-1, 0, 0, 0), 0x80808080: (-128, -127, -127, -127), 0x80: (-128, 1, 0, 0),
             0xFF: (-1, 1, 0, 0), 0x7F7F7F7F: (127, 127, 127, 127), 0x12345678: (120, 86, 52, 18), 0: (0, 0, 0, 0)}
    s = oracle.signed_digits(list(cases))
    for row, (x, want) in zip(s, cases.items()):
        assert tuple(int(v) for v in row) == want, hex(x)


def test_signed_digits_exhaustive_2_32():
    """Every 32-bit word: digits in [-128, 127] and sum_j s_j 2^(8j) == x
    (mod 2^32).  The check loop is C (tests/c/digit_exhaustive.c), linked
    against the oracle; it reconstructs each word independently."""
    src = os.path.join(ROOT, "tests", "c", "digit_exhaustive.c")
    exe = os.path.join(ROOT, "tests", "c", "digit_exhaustive")
    odir = os.path.join(ROOT, "oracle")
    subprocess.run(["gcc", "-O2", "-o", exe, src, "-I", odir, "-L", odir, "-loracle",
                    f"-Wl,-rpath,{odir}"], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "checked 4294967296" in r.stdout
