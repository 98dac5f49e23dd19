"""Pins for the oracle's batched NTT / INTT over RNS polynomials and its RNS
decomposition + NTT (VIPIR section 2.3: a polynomial is an #RNS x N matrix,
the NTT turns products in Z_q[X]/(X^N+1) into point-wise products; section
3.5.2: integer first-step outputs are read as polynomial coefficients and
transformed; section 4.3: the RNS decomposition is fused with the NTT).

The batched forms are pinned to integer polynomial algebra through the CRT
(Python big integers), to the transform's values on monomials, and to the
single-polynomial transform that test_oracle_ntt.py pins by direct
evaluation."""
import numpy as np
import pytest

import oracle

TINY_Q = [1073738753, 1073732609]
MED_Q = [536813569, 536690689, 536641537]


def crt(residues, q):
    """The integer in [0, prod q) with the given residues (Python big ints)."""
    Q = 1
    for v in q:
        Q *= v
    x = 0
    for r, qr in zip(residues, q):
        Mi = Q // qr
        x += int(r) * Mi * pow(Mi, -1, qr)
    return x % Q, Q


def negacyclic_int(a, b):
    """Exact integer product of a(X) b(X) reduced by X^N + 1."""
    N = len(a)
    c = [0] * N
    for i in range(N):
        for j in range(N):
            t = i + j
            if t < N:
                c[t] += int(a[i]) * int(b[j])
            else:
                c[t - N] -= int(a[i]) * int(b[j])
    return c


@pytest.mark.parametrize("inverse", [False, True])
def test_batch_is_the_per_limb_transform(inverse):
    N, q = 64, TINY_Q + [oracle.ntt_primes(30, 128, 3)[2]]
    psis = [oracle.psi(v, N) for v in q]
    rng = np.random.default_rng(11)
    x = np.stack([np.stack([rng.integers(0, v, size=N) for v in q]) for _ in range(5)]).astype(np.uint32)
    got = oracle.ntt_batch(x, q, psis, inverse=inverse, nthreads=3)
    f = oracle.intt if inverse else oracle.ntt
    for c in range(5):
        for r in range(3):
            np.testing.assert_array_equal(got[c, r], f(x[c, r], q[r], psis[r]))


def test_batch_roundtrip_at_n4096():
    N, q = 4096, MED_Q
    psis = [oracle.psi(v, N) for v in q]
    rng = np.random.default_rng(12)
    x = np.stack([rng.integers(0, v, size=N) for v in q])[None].astype(np.uint32)
    A = oracle.ntt_batch(x, q, psis)
    np.testing.assert_array_equal(oracle.ntt_batch(A, q, psis, inverse=True), x)
    # monomial X: its transform at output j is psi^(2j+1) (evaluation at the j-th root)
    mono = np.zeros((1, 3, N), dtype=np.uint32)
    mono[0, :, 1] = 1
    M = oracle.ntt_batch(mono, q, psis)
    for r in range(3):
        for j in (0, 1, 2, 1000, N - 1):
            assert int(M[0, r, j]) == pow(psis[r], 2 * j + 1, q[r])


def test_rns_reads_unsigned_integers_and_crt_recovers_them():
    N, q = 256, MED_Q
    psis = [oracle.psi(v, N) for v in q]
    rng = np.random.default_rng(13)
    c = rng.integers(0, 1 << 32, size=(3, N), dtype=np.uint64).astype(np.uint32)
    c[0, :4] = [0xFFFFFFFF, 0x80000000, 0, 1]
    A = oracle.ntt_rns(c, q, psis)
    back = oracle.ntt_batch(A, q, psis, inverse=True)
    for i in range(3):
        for t in range(N):
            x, _ = crt([back[i, r, t] for r in range(3)], q)
            assert x == int(c[i, t])          # the integer in [0, 2^32), not a signed reading
    # a constant polynomial evaluates to its constant at every root
    const = np.full((1, N), 0, dtype=np.uint32)
    const[0, 0] = 0xFFFFFFFF
    K = oracle.ntt_rns(const, q, psis)
    for r in range(3):
        assert (K[0, r] == (0xFFFFFFFF % q[r])).all()


def test_rns_pointwise_product_is_the_integer_negacyclic_product():
    """a, b with integer coefficients in [0, 2^32): INTT(ntt_rns(a) * ntt_rns(b))
    CRT-combined over q0*q1*q2 (about 2^87) is a*b in Z[X]/(X^N+1) exactly,
    since every coefficient is below N * 2^64 < Q/2 in absolute value."""
    N, q = 32, MED_Q
    psis = [oracle.psi(v, N) for v in q]
    rng = np.random.default_rng(14)
    ab = rng.integers(0, 1 << 32, size=(2, N), dtype=np.uint64).astype(np.uint32)
    A = oracle.ntt_rns(ab, q, psis).astype(np.uint64)
    prod = np.stack([(A[0, r] * A[1, r]) % q[r] for r in range(3)])[None].astype(np.uint32)
    back = oracle.ntt_batch(prod, q, psis, inverse=True)
    want = negacyclic_int(ab[0], ab[1])
    for t in range(N):
        x, Q = crt([back[0, r, t] for r in range(3)], q)
        if x > Q // 2:
            x -= Q
        assert x == want[t]


def test_rns_limb_is_the_transform_of_the_residues():
    N, q = 128, TINY_Q
    psis = [oracle.psi(v, N) for v in q]
    rng = np.random.default_rng(15)
    c = rng.integers(0, 1 << 32, size=(4, N), dtype=np.uint64).astype(np.uint32)
    A = oracle.ntt_rns(c, q, psis, nthreads=2)
    for i in range(4):
        for r in range(2):
            np.testing.assert_array_equal(A[i, r], oracle.ntt(c[i] % q[r], q[r], psis[r]))
