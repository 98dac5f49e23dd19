"""ExpPack's packing GEMM H*C + (0|G) on the GPU through the C ABI,
bit-exact against the oracle (VIPIR section 3.5.2).

Element by element on shapes that cover both kernels (int8 MFMA over
centred limbs whenever every q < 2^31 and n <= 16384; the 64-bit VALU scan
for the moduli at or above 2^31), ragged Dr / n tails, multi-pass batches, G
present and absent, and the moduli extremes; at the section 3.6 size (15 GiB
hint) every output of B = 1 and B = 16."""
import numpy as np
import pytest

import oracle
import synth
from he_database_scan_amd import pirscan
from tests.fullsize import check_modgemm
from tests.gpu_util import MED_Q, TINY_Q, empty_bytes, empty_u32, release, say, to_dev_u32, to_host_u32

pytestmark = pytest.mark.gpu


def workspace(shape, B):
    import torch

    n = pirscan.exppack_workspace_bytes(shape, B)
    return torch.empty(n, dtype=torch.uint8, device="cuda:0") if n else None


def run_gpu(H, C, G, N, q, scan=pirscan.SCAN_AUTO):
    Dr, n, P = H.shape
    B = C.shape[1] // 2
    shape = pirscan.ExppackShape.make(N, q, Dr, n, scan=scan)
    d_ht = empty_bytes(pirscan.exppack_layout_h_bytes(shape))
    pirscan.exppack_layout_h(shape, to_dev_u32(H), d_ht)
    d_out = empty_u32((Dr, 2 * B, P))
    pirscan.exppack_modgemm(shape, B, to_dev_u32(C), d_ht, None if G is None else to_dev_u32(G), d_out,
                            workspace(shape, B))
    return to_host_u32(d_out)


def rand_res(rng, shape, N, q):
    qv = np.asarray(q, dtype=np.uint64)[np.arange(shape[-1]) // N]
    return (rng.integers(0, 1 << 63, size=shape, dtype=np.uint64) % qv).astype(np.uint32)


# (Dr, n, B, with_G): the MFMA scan's batch classes (2B = 2..16 rows on the
# direct kernel, 32 on the shared-ring kernel, 34 as a 32-row pass plus a
# 2-row pass), ragged Dr (partial column tiles) and n (partial 64-wide
# k-steps), and the section 3.6 aspect (Dr = 256, n = 1280) at a small N.
SHAPES = [(3, 40, 1, True), (1, 1, 1, True), (256, 1280, 1, True), (5, 130, 2, False),
          (2, 1100, 3, True), (257, 33, 7, True), (5, 130, 8, True), (17, 65, 16, True),
          (9, 33, 17, True), (64, 1280, 16, False), (1, 1, 8, True)]


@pytest.mark.parametrize("Dr,n,B,with_g", SHAPES)
def test_shapes_full(Dr, n, B, with_g):
    N, q = 16, MED_Q
    P = N * len(q)
    rng = np.random.default_rng(Dr * 100000 + n * 100 + B)
    say(f"exppack Dr={Dr} n={n} B={B} G={with_g}")
    H = rand_res(rng, (Dr, n, P), N, q)
    C = rand_res(rng, (n, 2 * B, P), N, q)
    G = rand_res(rng, (Dr, B, P), N, q) if with_g else None
    np.testing.assert_array_equal(run_gpu(H, C, G, N, q), oracle.exppack(H, C, G, N, q))


@pytest.mark.parametrize("q,B", [([4294967291, 4294967279], 1), ([2147483659, 65537], 2),
                                 ([2147483647, 2147483629], 8), ([3, 5], 16), (TINY_Q, 9),
                                 ([4294967291], 17)])
def test_extreme_moduli_and_worst_case(q, B):
    """Moduli near 2^32 (the VALU scan, shortest fold), just under 2^31 (the
    MFMA path's limit), tiny moduli, and a two-pass batch on the VALU scan
    (2B = 34 with a modulus >= 2^31); all-(q-1) inputs are the worst case of
    both the 64-bit accumulation and the limb diagonals."""
    N, Dr, n = 4, 6, 97
    P = N * len(q)
    rng = np.random.default_rng(B + q[0] % 997)
    say(f"exppack moduli {q} B={B}")
    H = rand_res(rng, (Dr, n, P), N, q)
    C = rand_res(rng, (n, 2 * B, P), N, q)
    G = rand_res(rng, (Dr, B, P), N, q)
    np.testing.assert_array_equal(run_gpu(H, C, G, N, q), oracle.exppack(H, C, G, N, q))
    qv = np.asarray(q, dtype=np.uint64)[np.arange(P) // N]
    m1 = lambda shp: np.broadcast_to((qv - 1).astype(np.uint32), shp).copy()
    Hm, Cm, Gm = m1((Dr, n, P)), m1((n, 2 * B, P)), m1((Dr, B, P))
    got = run_gpu(Hm, Cm, Gm, N, q)
    np.testing.assert_array_equal(got[:, 0::2, :], np.broadcast_to((n % qv).astype(np.uint32), (Dr, B, P)))
    np.testing.assert_array_equal(got[:, 1::2, :],
                                  np.broadcast_to(((n + qv - 1) % qv).astype(np.uint32), (Dr, B, P)))


@pytest.mark.parametrize("Dr,n,B", [(3, 40, 1), (257, 33, 7), (17, 65, 16), (9, 33, 17)])
def test_valu_scan_on_request(Dr, n, B):
    """scan = SCAN_VALU: the 64-bit VALU scan on the word-transposed hint with
    moduli below 2^31, G present."""
    N, q = 16, MED_Q
    P = N * len(q)
    rng = np.random.default_rng(900 + Dr * 10 + B)
    say(f"exppack VALU on request Dr={Dr} n={n} B={B}")
    H = rand_res(rng, (Dr, n, P), N, q)
    C = rand_res(rng, (n, 2 * B, P), N, q)
    G = rand_res(rng, (Dr, B, P), N, q)
    np.testing.assert_array_equal(run_gpu(H, C, G, N, q, scan=pirscan.SCAN_VALU), oracle.exppack(H, C, G, N, q))


@pytest.mark.parametrize("B", [1, 8])
def test_one_hot_selects_hint_column(B):
    N, Dr, n = 8, 5, 12
    q = TINY_Q
    P = N * len(q)
    rng = np.random.default_rng(70 + B)
    H = rand_res(rng, (Dr, n, P), N, q)
    shape = pirscan.ExppackShape.make(N, q, Dr, n)
    d_ht = empty_bytes(pirscan.exppack_layout_h_bytes(shape))
    pirscan.exppack_layout_h(shape, to_dev_u32(H), d_ht)
    d_out = empty_u32((Dr, 2 * B, P))
    ws = workspace(shape, B)
    say(f"exppack one-hot B={B}")
    for i0 in range(n):
        C = np.zeros((n, 2 * B, P), dtype=np.uint32)
        C[i0, :, :] = 1
        pirscan.exppack_modgemm(shape, B, to_dev_u32(C), d_ht, None, d_out, ws)
        got = to_host_u32(d_out)
        for j in range(2 * B):
            np.testing.assert_array_equal(got[:, j, :], H[:, i0, :])


def test_layout_h_is_a_permutation():
    """Every hint word survives the relayout: one-hot C over all (i, j)
    reproduces H, and distinct markers stay distinct."""
    N, Dr, n = 4, 3, 7
    q = [4294967291]
    H = np.arange(Dr * n * N, dtype=np.uint32).reshape(Dr, n, N) + 1
    for i0 in range(n):
        C = np.zeros((n, 2, N), dtype=np.uint32)
        C[i0, 0, :] = 1
        got = run_gpu(H, C, None, N, q)
        np.testing.assert_array_equal(got[:, 0, :], H[:, i0, :])
        assert not got[:, 1, :].any()


def test_section_3_6_size_every_output():
    """VIPIR section 3.6's packing at full size (N = 2^12, #RNS = 3, Dr = 2^8,
    n = 1280: a 15 GiB hint) synthesised on the device, one tiled hint for
    both batches, B = 1 and B = 16: every output.  The oracle reads the
    device's own H, C and G back in chunks."""
    N, q, Dr, n = 4096, MED_Q, 256, 1280
    P = N * len(q)
    seed = 6
    shape = pirscan.ExppackShape.make(N, q, Dr, n)
    say(f"exppack full size: synthesising {4 * P * Dr * n / 2**30:.1f} GiB hint")
    d_h = empty_u32((Dr, n, P))
    synth.fill_residues_(d_h, seed, synth.STREAM_EXPPACK_H, N, q)
    d_ht = empty_bytes(pirscan.exppack_layout_h_bytes(shape))
    pirscan.exppack_layout_h(shape, d_h, d_ht)
    for B in (1, 16):
        d_c = empty_u32((n, 2 * B, P))
        synth.fill_residues_(d_c, seed, synth.STREAM_EXPPACK_C, N, q)
        d_g = empty_u32((Dr, B, P))
        synth.fill_residues_(d_g, seed, synth.STREAM_EXPPACK_G, N, q)
        d_out = empty_u32((Dr, 2 * B, P))
        say(f"  packing B={B}")
        pirscan.exppack_modgemm(shape, B, d_c, d_ht, d_g, d_out, workspace(shape, B))
        check_modgemm("exppack", (d_h,), {B: (d_c, d_g, d_out)}, N, q, [(0, P)], f"exppack 15 GiB B={B}")
        del d_c, d_g, d_out
        release()
    del d_h, d_ht
    release()


def random_exppack_cases(n=8, seed=5003):
    """Seeded random ExpPack cases: N from 16 to 256, one to three moduli
    below 2^31 (or, one case in four, at or above 2^31: the VALU scan), Dr and
    n up to 300, B up to 20 (2B rows: multi-pass past 32), G present or
    absent, at most 1.5e8 multiply-adds each for the oracle."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        N = 1 << int(rng.integers(4, 9))
        R = int(rng.integers(1, 4))
        wide = bool(rng.integers(0, 4) == 0)
        lo, hi = (1 << 31, 1 << 32) if wide else (2, 1 << 31)
        q = [int(v) for v in rng.integers(lo, hi, size=R, dtype=np.uint64)]
        Dr, n_, B = int(rng.integers(1, 301)), int(rng.integers(1, 301)), int(rng.integers(1, 21))
        if Dr * n_ * 2 * B * N * R <= 1.5e8:
            out.append((N, tuple(q), Dr, n_, B, bool(rng.integers(0, 2)), int(rng.integers(0, 1 << 30))))
    return out


@pytest.mark.parametrize("N,q,Dr,n,B,with_g,s", random_exppack_cases())
def test_random_shapes_both_scans(N, q, Dr, n, B, with_g, s):
    q = list(q)
    P = N * len(q)
    rng = np.random.default_rng(s)
    say(f"exppack random N={N} R={len(q)} Dr={Dr} n={n} B={B} G={with_g}")
    H = rand_res(rng, (Dr, n, P), N, q)
    C = rand_res(rng, (n, 2 * B, P), N, q)
    G = rand_res(rng, (Dr, B, P), N, q) if with_g else None
    want = oracle.exppack(H, C, G, N, q)
    np.testing.assert_array_equal(run_gpu(H, C, G, N, q), want)
    np.testing.assert_array_equal(run_gpu(H, C, G, N, q, scan=pirscan.SCAN_VALU), want)
