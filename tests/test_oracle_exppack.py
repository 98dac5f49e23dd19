"""Pins for the ExpPack packing-GEMM oracle (oracle.exppack).

VIPIR section 3.5.2: the hint rows H (Dr x n polynomials) and the first-step
outputs G (Dr x B polynomials) are taken to the NTT domain, and the packing
computes H*C + (0|G) with C the n x 2B matrix of expanded special
ciphertexts; with RNS and the NTT that is a (#RNS*N)-parallel
ceil(D1/N) x 2B x n modular GEMM.  Layouts are p-major: H [Dr][n][P],
C [n][2B][P], G [Dr][B][P], out [Dr][2B][P].

The pins tie the oracle to the polynomial algebra it stands for (NTT ->
point-wise GEMM -> INTT equals schoolbook negacyclic products, CRT-combined
against big-integer arithmetic), to closed forms, to the pinned RowSel oracle
on transposed operands, and to brute force on tiny inputs.
"""
import numpy as np
import pytest

import oracle

TINY_Q = [1073738753, 1073732609]


def rand_residues(rng, shape, N, q):
    P = shape[-1]
    qv = np.asarray(q, dtype=np.uint64)[np.arange(P) // N]
    return (rng.integers(0, 1 << 63, size=shape, dtype=np.uint64) % qv).astype(np.uint32)


def poly_negacyclic_python(a, b, Q):
    N = len(a)
    full = [0] * (2 * N - 1)
    for i in range(N):
        ai = int(a[i])
        for j in range(N):
            full[i + j] += ai * int(b[j])
    return [(full[t] - (full[t + N] if t + N < 2 * N - 1 else 0)) % Q for t in range(N)]


def test_packing_is_polynomial_algebra_after_ntt():
    """INTT(exppack(NTT h, NTT c, NTT g)) per limb, CRT-combined, equals
    sum_i h[r][i]*c[i][j] (+ g[r][b] for j = 2b+1) in Z_Q[X]/(X^N+1) computed
    with Python big integers, Q = q0*q1."""
    N, Dr, n, B = 16, 2, 3, 2
    q = [97, 193]                         # both == 1 mod 32, so 2N-th roots exist
    Qbig = q[0] * q[1]
    rng = np.random.default_rng(31)
    big = lambda: [int(v) for v in rng.integers(0, 1 << 40, size=N)]
    h = [[big() for _ in range(n)] for _ in range(Dr)]
    c = [[big() for _ in range(2 * B)] for _ in range(n)]
    g = [[big() for _ in range(B)] for _ in range(Dr)]
    psis = [oracle.psi(qr, N) for qr in q]
    P = 2 * N

    def ntt_rows(polys):
        outer, inner = len(polys), len(polys[0])
        arr = np.zeros((outer, inner, P), dtype=np.uint32)
        for r, qr in enumerate(q):
            for a in range(outer):
                for b in range(inner):
                    arr[a, b, r * N:(r + 1) * N] = oracle.ntt([x % qr for x in polys[a][b]], qr, psis[r])
        return arr

    out = oracle.exppack(ntt_rows(h), ntt_rows(c), ntt_rows(g), N, q)
    inv = pow(q[0], -1, q[1])
    for r in range(Dr):
        for j in range(2 * B):
            want = [0] * N
            for i in range(n):
                prod = poly_negacyclic_python(h[r][i], c[i][j], Qbig)
                want = [(x + y) % Qbig for x, y in zip(want, prod)]
            if j % 2 == 1:
                want = [(x + y) % Qbig for x, y in zip(want, g[r][j // 2])]
            limbs = [oracle.intt(out[r, j, t * N:(t + 1) * N], q[t], psis[t]) for t in range(2)]
            for t in range(N):
                x0, x1 = int(limbs[0][t]), int(limbs[1][t])
                assert (x0 + q[0] * (((x1 - x0) * inv) % q[1])) % Qbig == want[t]


def test_one_hot_selects_a_hint_column():
    """C = e_{i0} in column j0 returns H[:, i0] there; Dr != n so a transposed
    operand cannot pass."""
    N, Dr, n, B = 4, 3, 5, 2
    q = TINY_Q
    P = 2 * N
    rng = np.random.default_rng(32)
    H = rand_residues(rng, (Dr, n, P), N, q)
    G = rand_residues(rng, (Dr, B, P), N, q)
    for i0 in range(n):
        for j0 in range(2 * B):
            C = np.zeros((n, 2 * B, P), dtype=np.uint32)
            C[i0, j0, :] = 1
            out = oracle.exppack(H, C, G, N, q)
            qv = np.asarray(q, dtype=np.uint64)[np.arange(P) // N]
            for j in range(2 * B):
                z = G[:, j // 2, :].astype(np.uint64) if j % 2 else np.zeros((Dr, P), np.uint64)
                sel = H[:, i0, :].astype(np.uint64) if j == j0 else np.zeros((Dr, P), np.uint64)
                np.testing.assert_array_equal(out[:, j, :], ((sel + z) % qv).astype(np.uint32))


def test_all_q_minus_one_closed_form():
    """(q-1)^2 == 1 (mod q): even columns give n mod q, odd columns n + (q-1)
    == n - 1 (mod q)."""
    N, Dr, n, B = 2, 2, 1281, 1
    q = [4294967291, 536813569]
    P = 2 * N
    qv = np.asarray(q, dtype=np.uint64)[np.arange(P) // N]
    H = np.broadcast_to((qv - 1).astype(np.uint32), (Dr, n, P)).copy()
    C = np.broadcast_to((qv - 1).astype(np.uint32), (n, 2 * B, P)).copy()
    G = np.broadcast_to((qv - 1).astype(np.uint32), (Dr, B, P)).copy()
    out = oracle.exppack(H, C, G, N, q)
    np.testing.assert_array_equal(out[:, 0, :], np.broadcast_to(n % qv, (Dr, P)))
    np.testing.assert_array_equal(out[:, 1, :], np.broadcast_to((n - 1) % qv, (Dr, P)))


def test_matches_rowsel_on_transposed_operands():
    """Without G, out[r][j] = sum_i C^T[j][i] H^T[i][r]: RowSel with ct = C^T
    ([2B][n][P]) and db = H^T ([n][Dr][P]), transposed back."""
    N, Dr, n, B = 8, 5, 7, 3
    q = TINY_Q
    rng = np.random.default_rng(33)
    H = rand_residues(rng, (Dr, n, 2 * N), N, q)
    C = rand_residues(rng, (n, 2 * B, 2 * N), N, q)
    want = oracle.rowsel(C.transpose(1, 0, 2), H.transpose(1, 0, 2), N, q).transpose(1, 0, 2)
    np.testing.assert_array_equal(oracle.exppack(H, C, None, N, q), want)


@pytest.mark.parametrize("n", [1, 2, 33, 65])
def test_bruteforce_near_2_32(n):
    """Python big integers on tiny shapes with moduli near 2^32 (sums far past
    2^64)."""
    N, Dr, B = 2, 2, 2
    q = [4294967291, 4294967279]
    P = 2 * N
    rng = np.random.default_rng(40 + n)
    H = rand_residues(rng, (Dr, n, P), N, q)
    C = rand_residues(rng, (n, 2 * B, P), N, q)
    G = rand_residues(rng, (Dr, B, P), N, q)
    out = oracle.exppack(H, C, G, N, q)
    for p in range(P):
        qr = q[p // N]
        for r in range(Dr):
            for j in range(2 * B):
                s = sum(int(H[r, i, p]) * int(C[i, j, p]) for i in range(n))
                if j % 2:
                    s += int(G[r, j // 2, p])
                assert int(out[r, j, p]) == s % qr


def test_linear_in_c_and_g():
    N, Dr, n, B = 4, 3, 9, 2
    q = TINY_Q
    P = 2 * N
    qv = np.asarray(q, dtype=np.uint64)[np.arange(P) // N]
    rng = np.random.default_rng(34)
    H = rand_residues(rng, (Dr, n, P), N, q)
    C1, C2 = (rand_residues(rng, (n, 2 * B, P), N, q) for _ in range(2))
    G1, G2 = (rand_residues(rng, (Dr, B, P), N, q) for _ in range(2))
    s = lambda x, y: ((x.astype(np.uint64) + y) % qv).astype(np.uint32)
    lhs = oracle.exppack(H, s(C1, C2), s(G1, G2), N, q)
    rhs = s(oracle.exppack(H, C1, G1, N, q), oracle.exppack(H, C2, G2, N, q))
    np.testing.assert_array_equal(lhs, rhs)
