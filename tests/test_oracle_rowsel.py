"""Pins for the RowSel oracle (oracle.rowsel) against what the pages and the
mathematics fix -- never against a re-typing of the oracle's own formula.

RowSel (GPIR, RowSel formulation): out[p,m,n] = sum_k ct[p,m,k] * DB[p,k,n]
mod q_r, stored p-major (ct [m][D0][P], db [D0][D1][P], out [m][D1][P]).
"""
import numpy as np
import pytest

import oracle
import synth

TINY_Q = [1073738753, 1073732609]            # 2 largest primes < 2^30, == 1 mod 512
MED_Q = [536813569, 536690689, 536641537]    # 3 largest primes < 2^29, == 1 mod 8192


def brute_force(ct, db, N, q):
    """Python big integers, index by index (independent of the C oracle)."""
    m, D0, P = ct.shape
    D1 = db.shape[1]
    out = np.zeros((m, D1, P), dtype=np.uint32)
    for p in range(P):
        qr = int(q[p // N])
        for mi in range(m):
            for n in range(D1):
                s = 0
                for k in range(D0):
                    s += int(ct[mi, k, p]) * int(db[k, n, p])
                out[mi, n, p] = s % qr
    return out


def rand_residues(rng, shape, N, q):
    P = shape[-1]
    qv = np.asarray(q, dtype=np.uint64)[np.arange(P) // N]
    return (rng.integers(0, 1 << 63, size=shape, dtype=np.uint64) % qv).astype(np.uint32)


@pytest.mark.parametrize("D0", [1, 2, 3, 17, 33, 65])
def test_bruteforce_random_shapes(D0):
    rng = np.random.default_rng(100 + D0)
    # moduli near 2^32 stress the 128-bit accumulation; N=2 points per limb
    q = [4294967291, 3221225473, 65537]
    N, m, D1 = 2, 3, 4
    P = N * len(q)
    ct = rand_residues(rng, (m, D0, P), N, q)
    db = rand_residues(rng, (D0, D1, P), N, q)
    np.testing.assert_array_equal(oracle.rowsel(ct, db, N, q), brute_force(ct, db, N, q))


def test_bruteforce_tiny_config():
    # the tiny configuration: N=256, R=2, m=2, D0=16, D1=8 (checked on a point subset)
    N, m, D0, D1 = 256, 2, 16, 8
    ct = synth.residue_array(1, synth.STREAM_ROWSEL_CT, (m, D0, 2 * N), N, TINY_Q)
    db = synth.residue_array(1, synth.STREAM_ROWSEL_DB, (D0, D1, 2 * N), N, TINY_Q)
    out = oracle.rowsel(ct, db, N, TINY_Q)
    pts = [0, 1, 255, 256, 257, 511]
    sub = brute_force(ct[:, :, pts], db[:, :, pts], 1, [TINY_Q[p // N] for p in pts])
    np.testing.assert_array_equal(out[:, :, pts], sub)


def test_non_square_operands_not_transposed():
    # m != D0 != D1 != P so any swapped index hits a different element
    rng = np.random.default_rng(7)
    q = [97, 101]
    N, m, D0, D1 = 3, 2, 5, 7
    ct = rand_residues(rng, (m, D0, 2 * N), N, q)
    db = rand_residues(rng, (D0, D1, 2 * N), N, q)
    np.testing.assert_array_equal(oracle.rowsel(ct, db, N, q), brute_force(ct, db, N, q))


def test_one_hot_selects_db_row():
    """ct row = e_k for every point (the NTT image of an encrypted one-hot
    selector) must return DB row k exactly: 'row selection'."""
    N, m, D0, D1 = 256, 2, 16, 8
    P = 2 * N
    db = synth.residue_array(1, synth.STREAM_ROWSEL_DB, (D0, D1, P), N, TINY_Q)
    for k in range(D0):
        ct = np.zeros((m, D0, P), dtype=np.uint32)
        ct[:, k, :] = 1
        out = oracle.rowsel(ct, db, N, TINY_Q)
        for mi in range(m):
            np.testing.assert_array_equal(out[mi], db[k])


@pytest.mark.parametrize("q,D0", [(TINY_Q, 16), (MED_Q, 1024), ([4294967291], 3)])
def test_closed_form_all_max(q, D0):
    """All inputs q-1: each product is (q-1)^2 == 1 (mod q), so every output is
    D0 mod q -- the worst case for any lazy 64-bit accumulator."""
    N, m, D1 = 2, 2, 3
    P = N * len(q)
    qv = np.asarray(q, dtype=np.uint32)[np.arange(P) // N]
    ct = np.broadcast_to(qv - 1, (m, D0, P)).copy()
    db = np.broadcast_to(qv - 1, (D0, D1, P)).copy()
    out = oracle.rowsel(ct, db, N, q)
    expect = (np.uint64(D0) % qv.astype(np.uint64)).astype(np.uint32)
    for mi in range(m):
        for n in range(D1):
            np.testing.assert_array_equal(out[mi, n], expect)
    # one k zeroed out: (D0 - 1) mod q
    ct[:, D0 // 2, :] = 0
    out = oracle.rowsel(ct, db, N, q)
    expect = (np.uint64(D0 - 1) % qv.astype(np.uint64)).astype(np.uint32)
    np.testing.assert_array_equal(out[1, 2], expect)


def test_linearity_and_zero():
    rng = np.random.default_rng(3)
    N, m, D0, D1 = 4, 2, 9, 5
    q = MED_Q
    P = N * len(q)
    qv = np.asarray(q, dtype=np.uint64)[np.arange(P) // N]
    a1 = rand_residues(rng, (m, D0, P), N, q)
    a2 = rand_residues(rng, (m, D0, P), N, q)
    b1 = rand_residues(rng, (D0, D1, P), N, q)
    b2 = rand_residues(rng, (D0, D1, P), N, q)
    s = ((a1.astype(np.uint64) + a2) % qv).astype(np.uint32)
    lhs = oracle.rowsel(s, b1, N, q).astype(np.uint64)
    rhs = (oracle.rowsel(a1, b1, N, q).astype(np.uint64) + oracle.rowsel(a2, b1, N, q)) % qv
    np.testing.assert_array_equal(lhs, rhs)
    sb = ((b1.astype(np.uint64) + b2) % qv).astype(np.uint32)
    lhs = oracle.rowsel(a1, sb, N, q).astype(np.uint64)
    rhs = (oracle.rowsel(a1, b1, N, q).astype(np.uint64) + oracle.rowsel(a1, b2, N, q)) % qv
    np.testing.assert_array_equal(lhs, rhs)
    assert not oracle.rowsel(np.zeros_like(a1), b1, N, q).any()
    out = oracle.rowsel(a1, b1, N, q)
    assert (out.astype(np.uint64) < qv).all()


def test_d0_one_is_elementwise_modmul():
    rng = np.random.default_rng(11)
    q = [4294967291, 2147483647]
    N, m, D1 = 8, 3, 4
    P = N * len(q)
    qv = np.asarray(q, dtype=np.uint64)[np.arange(P) // N]
    ct = rand_residues(rng, (m, 1, P), N, q)
    db = rand_residues(rng, (1, D1, P), N, q)
    out = oracle.rowsel(ct, db, N, q)
    for mi in range(m):
        for n in range(D1):
            ref = (ct[mi, 0].astype(np.uint64) * db[0, n].astype(np.uint64)) % qv  # < 2^64
            np.testing.assert_array_equal(out[mi, n], ref.astype(np.uint32))


def test_threads_do_not_change_result():
    rng = np.random.default_rng(5)
    N, m, D0, D1 = 64, 2, 20, 6
    q = TINY_Q
    ct = rand_residues(rng, (m, D0, 2 * N), N, q)
    db = rand_residues(rng, (D0, D1, 2 * N), N, q)
    np.testing.assert_array_equal(oracle.rowsel(ct, db, N, q, nthreads=1),
                                  oracle.rowsel(ct, db, N, q, nthreads=7))
