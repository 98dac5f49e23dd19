"""Pins tying RowSel's point-wise products to polynomial products (VIPIR
section 2.3: after the NTT a product in Z_q[X]/(X^N+1) is point-wise mod q_i;
an RNS row per prime), and pins for the prime / root search that fixes the
configurations' moduli."""
import numpy as np
import pytest

import oracle

TINY_Q = [1073738753, 1073732609]
MED_Q = [536813569, 536690689, 536641537]


def trial_division_is_prime(n):
    if n < 2:
        return False
    d = 2
    while d * d <= n:
        if n % d == 0:
            return False
        d += 1
    return True


def poly_negacyclic_python(a, b, q):
    """Polynomial product with Python ints, then reduction by X^N + 1."""
    N = len(a)
    full = [0] * (2 * N - 1)
    for i in range(N):
        for j in range(N):
            full[i + j] += int(a[i]) * int(b[j])
    return [(full[t] - (full[t + N] if t + N < 2 * N - 1 else 0)) % q for t in range(N)]


def test_prime_search_matches_trial_division():
    # the configurations' primes: largest q < 2^30 (== 1 mod 512) and q < 2^29 (== 1 mod 8192)
    assert oracle.ntt_primes(30, 512, 2) == TINY_Q
    assert oracle.ntt_primes(29, 8192, 3) == MED_Q
    for q, bits, two_n in [(TINY_Q, 30, 512), (MED_Q, 29, 8192)]:
        for v in q:
            assert trial_division_is_prime(v) and v % two_n == 1 and v < (1 << bits)
        # nothing larger was skipped: every candidate above the smallest is composite
        for cand in range(max(q), (1 << bits), two_n):
            if cand not in q:
                assert not trial_division_is_prime(cand)
        for cand in range(min(q), max(q), two_n):
            if cand not in q:
                assert not trial_division_is_prime(cand)


def test_miller_rabin_against_trial_division():
    rng = np.random.default_rng(1)
    samples = list(range(0, 2000)) + [int(x) for x in rng.integers(2, 1 << 32, size=300)]
    samples += [4294967291, 4294967295, 3215031751, 2152302898, 1373653]  # strong pseudoprimes to some bases
    for n in samples:
        if n < (1 << 32):
            assert oracle.is_prime(n) == trial_division_is_prime(n), n


@pytest.mark.parametrize("q,N", [(TINY_Q[0], 256), (TINY_Q[1], 256), (MED_Q[0], 4096), (MED_Q[2], 4096)])
def test_psi_is_primitive_2n_root(q, N):
    psi = oracle.psi(q, N)
    assert pow(psi, 2 * N, q) == 1
    assert pow(psi, N, q) == q - 1          # psi^N = -1: psi is a root of X^N + 1
    g = oracle.primitive_root(q)
    # g generates: g^((q-1)/f) != 1 for each prime factor f of q-1 (factored in Python)
    r, f, d = q - 1, set(), 2
    while d * d <= r:
        while r % d == 0:
            f.add(d)
            r //= d
        d += 1
    if r > 1:
        f.add(r)
    assert all(pow(g, (q - 1) // fi, q) != 1 for fi in f)


def test_ntt_direct_evaluation_tiny():
    q, N = 97, 8               # 97 == 1 mod 16
    psi = oracle.psi(q, N)
    rng = np.random.default_rng(2)
    a = rng.integers(0, q, size=N)
    A = oracle.ntt(a, q, psi)
    for j in range(N):
        x = pow(psi, 2 * j + 1, q)
        assert int(A[j]) == sum(int(a[i]) * pow(x, i, q) for i in range(N)) % q
    np.testing.assert_array_equal(oracle.intt(A, q, psi), a)


def test_ntt_of_one_is_all_ones_and_roundtrip():
    q, N = TINY_Q[0], 256
    psi = oracle.psi(q, N)
    one = np.zeros(N, dtype=np.uint32)
    one[0] = 1
    assert (oracle.ntt(one, q, psi) == 1).all()
    rng = np.random.default_rng(4)
    x = rng.integers(0, q, size=N).astype(np.uint32)
    np.testing.assert_array_equal(oracle.intt(oracle.ntt(x, q, psi), q, psi), x)


def test_schoolbook_matches_python_polynomials():
    rng = np.random.default_rng(6)
    q, N = 1073738753, 16
    a = rng.integers(0, q, size=N)
    b = rng.integers(0, q, size=N)
    assert list(oracle.negacyclic_mul(a, b, q)) == poly_negacyclic_python(a, b, q)
    # X * X^(N-1) = X^N = -1
    x1 = np.zeros(N, dtype=np.uint32); x1[1] = 1
    xn = np.zeros(N, dtype=np.uint32); xn[N - 1] = 1
    c = oracle.negacyclic_mul(x1, xn, q)
    assert c[0] == q - 1 and not c[1:].any()


def test_rowsel_is_polynomial_product_after_ntt_with_crt():
    """For each limb r: INTT(RowSel(NTT(a), NTT(b))) = sum_k a_k * b_{k,n} in
    Z_{q_r}[X]/(X^N+1); CRT-combining the two limbs equals the product mod
    Q = q0*q1 computed with Python big integers."""
    N, m, D0, D1 = 256, 2, 3, 2
    q = TINY_Q
    rng = np.random.default_rng(8)
    Qbig = q[0] * q[1]
    # polynomials with coefficients mod Q, reduced per limb (RNS decomposition)
    a = [[[int(v) for v in rng.integers(0, 1 << 62, size=N)] for _ in range(D0)] for _ in range(m)]
    b = [[[int(v) for v in rng.integers(0, 1 << 62, size=N)] for _ in range(D1)] for _ in range(D0)]
    psis = [oracle.psi(qr, N) for qr in q]
    ct = np.zeros((m, D0, 2 * N), dtype=np.uint32)
    db = np.zeros((D0, D1, 2 * N), dtype=np.uint32)
    for r, qr in enumerate(q):
        for mi in range(m):
            for k in range(D0):
                ct[mi, k, r * N:(r + 1) * N] = oracle.ntt([c % qr for c in a[mi][k]], qr, psis[r])
        for k in range(D0):
            for n in range(D1):
                db[k, n, r * N:(r + 1) * N] = oracle.ntt([c % qr for c in b[k][n]], qr, psis[r])
    out = oracle.rowsel(ct, db, N, q)
    for mi in range(m):
        for n in range(D1):
            limbs = [oracle.intt(out[mi, n, r * N:(r + 1) * N], q[r], psis[r]) for r in range(2)]
            # schoolbook per limb
            for r in range(2):
                acc = np.zeros(N, dtype=np.uint64)
                for k in range(D0):
                    acc = (acc + oracle.negacyclic_mul([c % q[r] for c in a[mi][k]],
                                                       [c % q[r] for c in b[k][n]], q[r])) % q[r]
                np.testing.assert_array_equal(limbs[r], acc.astype(np.uint32))
            # CRT against big-integer polynomial arithmetic mod Q
            big = [0] * N
            for k in range(D0):
                prod = poly_negacyclic_python(a[mi][k], b[k][n], Qbig)
                big = [(x + y) % Qbig for x, y in zip(big, prod)]
            inv = pow(q[0], -1, q[1])
            for t in range(0, N, 17):
                x0, x1 = int(limbs[0][t]), int(limbs[1][t])
                crt = (x0 + q[0] * (((x1 - x0) * inv) % q[1])) % Qbig
                assert crt == big[t]
