"""RowSel on the GPU through the C ABI, bit-exact against the oracle.

Element by element at sizes the oracle finishes in seconds (several
wavefront slices, ragged column / k tails, every row-group width and every
fold period).  The full 3 GiB and 48 GiB configurations are compared in
test_gpu_rowsel_fullsize.py."""
import numpy as np
import pytest

import oracle
import synth
from he_database_scan_amd import pirscan
from tests.gpu_util import MED_Q, TINY_Q, empty_bytes, empty_u32, release, say, to_dev_u32, to_host_u32

pytestmark = pytest.mark.gpu


def run_gpu(ct, db, N, q, scan=pirscan.SCAN_AUTO):
    m, D0, P = ct.shape
    D1 = db.shape[1]
    shape = pirscan.RowselShape.make(N, q, D0, D1, scan=scan)
    d_db = to_dev_u32(db)
    d_dbt = empty_bytes(pirscan.layout_db_bytes(shape))
    pirscan.layout_db(shape, d_db, d_dbt)
    d_out = empty_u32((m, D1, P))
    pirscan.rowsel_modgemm(shape, m, to_dev_u32(ct), d_dbt, d_out, workspace(shape, m))
    return to_host_u32(d_out)


def workspace(shape, m):
    import torch

    n = pirscan.rowsel_workspace_bytes(shape, m)
    return torch.empty(n, dtype=torch.uint8, device="cuda:0") if n else None


def rand_res(rng, shape, N, q):
    qv = np.asarray(q, dtype=np.uint64)[np.arange(shape[-1]) // N]
    return (rng.integers(0, 1 << 63, size=shape, dtype=np.uint64) % qv).astype(np.uint32)


def test_tiny_config_full():
    N, m, D0, D1 = 256, 2, 16, 8
    P = 2 * N
    say("rowsel tiny")
    ct = synth.residue_array(1, synth.STREAM_ROWSEL_CT, (m, D0, P), N, TINY_Q)
    db = synth.residue_array(1, synth.STREAM_ROWSEL_DB, (D0, D1, P), N, TINY_Q)
    np.testing.assert_array_equal(run_gpu(ct, db, N, TINY_Q), oracle.rowsel(ct, db, N, TINY_Q))


def test_tiny_one_hot_rows_and_all_max():
    N, m, D0, D1 = 256, 2, 16, 8
    P = 2 * N
    db = synth.residue_array(1, synth.STREAM_ROWSEL_DB, (D0, D1, P), N, TINY_Q)
    shape = pirscan.RowselShape.make(N, TINY_Q, D0, D1)
    d_dbt = empty_bytes(pirscan.layout_db_bytes(shape))
    pirscan.layout_db(shape, to_dev_u32(db), d_dbt)
    d_out = empty_u32((m, D1, P))
    for k in range(D0):
        ct = np.zeros((m, D0, P), dtype=np.uint32)
        ct[:, k, :] = 1
        pirscan.rowsel_modgemm(shape, m, to_dev_u32(ct), d_dbt, d_out, workspace(shape, m))
        got = to_host_u32(d_out)
        for mi in range(m):
            np.testing.assert_array_equal(got[mi], db[k])
    qv = np.asarray(TINY_Q, dtype=np.uint32)[np.arange(P) // N]
    ctm = np.broadcast_to(qv - 1, (m, D0, P)).copy()
    dbm = np.broadcast_to(qv - 1, (D0, D1, P)).copy()
    got = run_gpu(ctm, dbm, N, TINY_Q)
    assert (got == (D0 % qv)[None, None, :]).all()       # (q-1)^2 == 1: out = D0 mod q
    np.testing.assert_array_equal(got, oracle.rowsel(ctm, dbm, N, TINY_Q))


# (m, D0, D1): every row-group width (2/4/8/16/32 and a multi-pass m), the
# 128/64/32-bit column paths, ragged column slices and k tails that cross the
# LDS chunk and the fold period.
SHAPES = [(2, 33, 256), (1, 7, 8), (3, 40, 300), (4, 64, 512), (6, 17, 258), (8, 65, 1024),
          (12, 9, 130), (16, 70, 256), (32, 66, 128), (34, 5, 129), (2, 1, 1), (2, 1100, 64)]


@pytest.mark.parametrize("m,D0,D1", SHAPES)
def test_multi_tile_shapes_full(m, D0, D1):
    rng = np.random.default_rng(m * 10000 + D0 * 100 + D1)
    N, q = 16, MED_Q
    P = N * len(q)
    say(f"rowsel m={m} D0={D0} D1={D1} P={P}")
    ct = rand_res(rng, (m, D0, P), N, q)
    db = rand_res(rng, (D0, D1, P), N, q)
    np.testing.assert_array_equal(run_gpu(ct, db, N, q), oracle.rowsel(ct, db, N, q))


@pytest.mark.parametrize("q", [[4294967291, 4294967279], [2147483659, 3221225473], [65537, 2],
                               [3, 1073741827], [TINY_Q[0], MED_Q[0]]])
def test_fold_periods_and_extreme_moduli(q):
    """Moduli from 2 to just under 2^32 select every fold period (1..32);
    all-(q-1) inputs are the 64-bit accumulator's worst case."""
    rng = np.random.default_rng(q[0] % 1000)
    N, m, D0, D1 = 8, 2, 97, 260
    P = N * len(q)
    say(f"rowsel moduli {q}")
    ct = rand_res(rng, (m, D0, P), N, q)
    db = rand_res(rng, (D0, D1, P), N, q)
    np.testing.assert_array_equal(run_gpu(ct, db, N, q), oracle.rowsel(ct, db, N, q))
    qv = np.asarray(q, dtype=np.uint32)[np.arange(P) // N]
    ctm = np.broadcast_to(qv - 1, (m, D0, P)).copy()
    dbm = np.broadcast_to(qv - 1, (D0, D1, P)).copy()
    np.testing.assert_array_equal(run_gpu(ctm, dbm, N, q), oracle.rowsel(ctm, dbm, N, q))


@pytest.mark.parametrize("m,D0,D1", [(1, 97, 260), (2, 1024, 64), (3, 40, 300), (6, 65, 129), (8, 17, 256),
                                     (16, 70, 100), (17, 33, 64), (32, 66, 128), (40, 9, 33)])
def test_valu_scan_on_request(m, D0, D1):
    """scan = SCAN_VALU runs the 64-bit lazy-reduction kernel on the word
    layout although every modulus is below 2^31: every row-group width, a
    multi-pass m, ragged column slices and k tails past the fold period."""
    rng = np.random.default_rng(5000 + m * 100 + D0)
    N, q = 16, MED_Q
    P = N * len(q)
    say(f"rowsel VALU on request m={m} D0={D0} D1={D1}")
    ct = rand_res(rng, (m, D0, P), N, q)
    db = rand_res(rng, (D0, D1, P), N, q)
    np.testing.assert_array_equal(run_gpu(ct, db, N, q, scan=pirscan.SCAN_VALU), oracle.rowsel(ct, db, N, q))
    qv = np.asarray(q, dtype=np.uint32)[np.arange(P) // N]
    ctm = np.broadcast_to(qv - 1, (m, D0, P)).copy()
    dbm = np.broadcast_to(qv - 1, (D0, D1, P)).copy()
    got = run_gpu(ctm, dbm, N, q, scan=pirscan.SCAN_VALU)
    assert (got == (D0 % qv)[None, None, :]).all()       # (q-1)^2 == 1: out = D0 mod q


def test_repeat_runs_identical():
    rng = np.random.default_rng(1)
    N, m, D0, D1 = 16, 2, 50, 512
    ct = rand_res(rng, (m, D0, 3 * N), N, MED_Q)
    db = rand_res(rng, (D0, D1, 3 * N), N, MED_Q)
    a = run_gpu(ct, db, N, MED_Q)
    b = run_gpu(ct, db, N, MED_Q)
    np.testing.assert_array_equal(a, b)


# Batched path (m >= 16, every q < 2^31: int8 MFMA over centred signed limbs)
@pytest.mark.parametrize("q,m,D0,D1", [([2147483647, 2147483629], 16, 100, 50),
                                       ([2147483647], 32, 130, 33), ([1073741827, 65537], 40, 64, 96),
                                       (MED_Q, 32, 1, 16), ([3, 5], 17, 257, 40)])
def test_batched_path_edges(q, m, D0, D1):
    N = 4
    P = N * len(q)
    shape = pirscan.RowselShape.make(N, q, D0, D1)
    assert pirscan.rowsel_workspace_bytes(shape, m) > 0
    rng = np.random.default_rng(m * 7 + D0)
    say(f"rowsel batched q={q} m={m} D0={D0} D1={D1}")
    ct = rand_res(rng, (m, D0, P), N, q)
    db = rand_res(rng, (D0, D1, P), N, q)
    np.testing.assert_array_equal(run_gpu(ct, db, N, q), oracle.rowsel(ct, db, N, q))
    qv = np.asarray(q, dtype=np.uint64)[np.arange(P) // N]
    # the centring boundary: values q/2 and q/2 + 1, and q - 1
    for vals in ((qv // 2), (qv // 2 + 1) % qv, qv - 1):
        ctv = np.broadcast_to(vals.astype(np.uint32), (m, D0, P)).copy()
        dbv = np.broadcast_to(((qv - 1) - vals % qv).astype(np.uint32), (D0, D1, P)).copy()
        np.testing.assert_array_equal(run_gpu(ctv, dbv, N, q), oracle.rowsel(ctv, dbv, N, q))


@pytest.mark.parametrize("N,q,m,D0,D1", [(3, [2147483647, 65537], 32, 70, 48), (5, MED_Q, 20, 130, 66),
                                         (16, [1073741827, 7681], 48, 200, 40)])
def test_batched_path_point_counts(N, q, m, D0, D1):
    """P = R*N not a multiple of 4 (the ct relayout then goes through the
    transpose + limb-split passes) and P not a multiple of the 32-point prep
    block, with one, two and three row-tile passes."""
    P = N * len(q)
    rng = np.random.default_rng(N * 1000 + m)
    say(f"rowsel batched N={N} P={P} m={m} D0={D0} D1={D1}")
    ct = rand_res(rng, (m, D0, P), N, q)
    db = rand_res(rng, (D0, D1, P), N, q)
    np.testing.assert_array_equal(run_gpu(ct, db, N, q), oracle.rowsel(ct, db, N, q))


def test_every_batch_size_on_one_layout():
    """One relaid DB serves every m: 1..17 (one 16-row tile, then two), 31..33
    (two tiles, then a second 32-row pass), on ragged D0 / D1 (partial k-step,
    partial column tile, column-tile groups that leave waves of the last
    workgroup without work)."""
    import torch

    N, q, D0, D1 = 4, MED_Q, 130, 300
    P = N * len(q)
    rng = np.random.default_rng(77)
    db = rand_res(rng, (D0, D1, P), N, q)
    shape = pirscan.RowselShape.make(N, q, D0, D1)
    d_dbt = empty_bytes(pirscan.layout_db_bytes(shape))
    pirscan.layout_db(shape, to_dev_u32(db), d_dbt)
    for m in list(range(1, 18)) + [31, 32, 33]:
        say(f"rowsel one layout m={m}")
        ct = rand_res(rng, (m, D0, P), N, q)
        d_out = empty_u32((m, D1, P))
        pirscan.rowsel_modgemm(shape, m, to_dev_u32(ct), d_dbt, d_out, workspace(shape, m))
        np.testing.assert_array_equal(to_host_u32(d_out), oracle.rowsel(ct, db, N, q))
        del d_out
    torch.cuda.synchronize()


@pytest.mark.parametrize("D1", [256, 512])
def test_whole_row_stores_on_whole_groups(D1):
    """Column counts that split into whole groups of four workgroup waves
    (D1 = 256: 16 column tiles; 512: 32) take the epilogue that gathers the
    residues in LDS and stores whole rows: every batch-size class (1-4 rows
    with one tile per wave, 5-16 with four, 17-32 on the shared ring, and a
    second pass), with a ragged k extent and enough points for several
    workgroup chunks per XCD."""
    import torch

    N, q, D0 = 64, MED_Q, 130
    P = N * len(q)
    rng = np.random.default_rng(D1 + 5)
    db = rand_res(rng, (D0, D1, P), N, q)
    shape = pirscan.RowselShape.make(N, q, D0, D1)
    d_dbt = empty_bytes(pirscan.layout_db_bytes(shape))
    pirscan.layout_db(shape, to_dev_u32(db), d_dbt)
    for m in (1, 2, 4, 5, 8, 13, 16, 17, 24, 32, 33, 48):
        say(f"rowsel whole-row stores D1={D1} m={m}")
        ct = rand_res(rng, (m, D0, P), N, q)
        d_out = empty_u32((m, D1, P))
        pirscan.rowsel_modgemm(shape, m, to_dev_u32(ct), d_dbt, d_out, workspace(shape, m))
        np.testing.assert_array_equal(to_host_u32(d_out), oracle.rowsel(ct, db, N, q))
        del d_out
    torch.cuda.synchronize()


def signed_limb_value(digits):
    return sum(int(d) << (8 * i) for i, d in enumerate(digits))


@pytest.mark.parametrize("m", [2, 32])
def test_limb_diagonals_at_the_largest_reduction(m):
    """D0 = 16384, the largest k extent of the limb path: inputs whose centred
    values have the largest digits a modulus below 2^31 allows (-128, -128,
    -128, -63) and (127, 127, 127, 63) drive every int32 diagonal sum to its
    extreme (4 pairs x D0 x 2^14 bounds it by 2^30).  D0 = 16385 takes the
    64-bit VALU scan on a word-transposed layout."""
    q = [2147483647, 2147483629]
    N, D1 = 2, 16
    P = N * len(q)
    qv = np.asarray(q, dtype=np.int64)[np.arange(P) // N]
    neg = signed_limb_value([-128, -128, -128, -63])
    pos = signed_limb_value([127, 127, 127, 63])
    assert -neg <= q[1] // 2 and pos <= q[1] // 2
    xneg = (qv + neg).astype(np.uint32)
    xpos = np.full(P, pos, dtype=np.uint32)
    for D0 in (16384, 16385):
        say(f"rowsel limb extremes m={m} D0={D0}")
        for a, b in ((xneg, xneg), (xneg, xpos), (xpos, xpos)):
            ct = np.broadcast_to(a, (m, D0, P)).copy()
            db = np.broadcast_to(b, (D0, D1, P)).copy()
            np.testing.assert_array_equal(run_gpu(ct, db, N, q), oracle.rowsel(ct, db, N, q))
        rng = np.random.default_rng(D0 + m)
        ct = np.where(rng.integers(0, 2, size=(m, D0, P)) == 1, xneg, xpos).astype(np.uint32)
        db = np.where(rng.integers(0, 2, size=(D0, D1, P)) == 1, xneg, xpos).astype(np.uint32)
        np.testing.assert_array_equal(run_gpu(ct, db, N, q), oracle.rowsel(ct, db, N, q))


def random_rowsel_cases(n=10, seed=4099):
    """Seeded random RowSel cases: N a power of two from 16 to 512, R from 1
    to 4 limbs with moduli drawn from [2, 2^31) (the int8 scan) or [2^31,
    2^32) (the VALU scan), D0 up to 300, D1 up to 300, m up to 40 (multi-pass
    past 32), at most 1.5e8 multiply-adds each for the oracle."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        N = 1 << int(rng.integers(4, 10))
        R = int(rng.integers(1, 5))
        wide = bool(rng.integers(0, 4) == 0)
        lo, hi = (1 << 31, 1 << 32) if wide else (2, 1 << 31)
        q = [int(v) for v in rng.integers(lo, hi, size=R, dtype=np.uint64)]
        D0, D1, m = int(rng.integers(1, 301)), int(rng.integers(1, 301)), int(rng.integers(1, 41))
        if m * D0 * D1 * N * R <= 1.5e8:
            out.append((N, tuple(q), D0, D1, m, int(rng.integers(0, 1 << 30))))
    return out


@pytest.mark.parametrize("N,q,D0,D1,m,s", random_rowsel_cases())
def test_random_shapes_both_scans(N, q, D0, D1, m, s):
    q = list(q)
    P = N * len(q)
    rng = np.random.default_rng(s)
    say(f"rowsel random N={N} R={len(q)} D0={D0} D1={D1} m={m}")
    ct = rand_res(rng, (m, D0, P), N, q)
    db = rand_res(rng, (D0, D1, P), N, q)
    want = oracle.rowsel(ct, db, N, q)
    np.testing.assert_array_equal(run_gpu(ct, db, N, q), want)
    np.testing.assert_array_equal(run_gpu(ct, db, N, q, scan=pirscan.SCAN_VALU), want)
