"""The scalar-HE product on the tiled DB (pirscan_scalar_layout_db +
pirscan_scalar_gemm_u32_tiled), on the GPU through the C ABI, bit-exact
against the oracle: element by element on ragged shapes (M and K not
multiples of the 16-row tile or the 64-byte step, misaligned row-major
sources), every batch width class (1, several column tiles, several 64-column
passes), closed forms past 2^31 inside one accumulator, one-hot selections,
and sampled rows of the hint and second-fold shapes (the 64 GiB configuration
is compared in full in test_gpu_scalar_fullsize.py)."""
import numpy as np
import pytest

import oracle
import synth
from he_database_scan_amd import pirscan
from tests.gpu_util import empty_bytes, empty_u32, release, say, to_dev_i8, to_dev_u32, to_host_u32

pytestmark = pytest.mark.gpu


def tiled(d_db):
    M, K = d_db.shape
    t = empty_bytes(pirscan.scalar_layout_db_bytes(M, K))
    pirscan.scalar_layout_db(d_db, t)
    return t


def scan(t, M, K, d_q):
    B = d_q.shape[1]
    d_o = empty_u32((M, B))
    pirscan.scalar_gemm_u32_tiled(t, M, K, d_q, d_o, empty_bytes(pirscan.scalar_tiled_workspace_bytes(M, K, B)))
    return d_o


def run_gpu(db, Q, offset=0):
    """offset > 0 lays out from a misaligned row-major source."""
    import torch

    M, K = db.shape
    if offset:
        raw = torch.empty(M * K + offset, dtype=torch.int8, device="cuda:0")
        raw[offset:] = to_dev_i8(db.reshape(-1))
        d_db = raw[offset:].view(M, K)
    else:
        d_db = to_dev_i8(db)
    return to_host_u32(scan(tiled(d_db), M, K, to_dev_u32(Q)))


def rand_case(seed, M, K, B):
    rng = np.random.default_rng(seed)
    db = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    Q = rng.integers(0, 1 << 32, size=(K, B), dtype=np.uint64).astype(np.uint32)
    return db, Q


# (M, K, B): one row, ragged rows and k (K % 16 != 0 takes the byte-wise
# packing), one to several 16-column tiles, a 64-column pass plus a ragged one,
# and the wide passes (up to four 128-column groups per launch) of wide batches.
SHAPES = [(1, 1, 1), (1, 16, 1), (17, 65, 1), (63, 4096, 1), (300, 4096 * 3 + 48, 1), (257, 160, 1),
          (50, 1001, 1), (100, 64, 2), (130, 1040, 3), (64, 4096, 8), (333, 20000, 8), (65, 16400, 16),
          (200, 2048, 17), (129, 33024, 32), (70, 512, 33), (40, 800, 40), (17, 33, 5), (77, 4160, 64),
          (100, 2048, 65), (31, 300, 130),
          # wide launches while more than 64 columns remain: one group (65..128), a group plus a partial
          # group of more than 64 (200), whole groups plus a narrow remainder (130, 300, 530, 1281), three
          # groups (384), four groups and a partial launch (600), ragged rows past a 128-row tile, K not a
          # multiple of 64
          (129, 4160, 128), (257, 20480, 200), (100, 4096, 1280), (37, 1040, 1281), (300, 16400, 96),
          (70, 1100, 300), (64, 4096, 384), (90, 2048, 530), (150, 4160, 600)]


@pytest.mark.parametrize("M,K,B", SHAPES)
def test_tiled_shapes_full(M, K, B):
    say(f"scalar tiled M={M} K={K} B={B}")
    db, Q = rand_case(M * 11 + K * 5 + B, M, K, B)
    np.testing.assert_array_equal(run_gpu(db, Q), oracle.scalar(db, Q))


def wide_random_shapes(n=8, seed=2027):
    """Seeded random shapes for the wide launches: B from 65 to 700 (one to
    five 128-column groups, partial groups and narrow remainders), ragged M and
    K, at most 4e8 multiply-adds each for the oracle."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M, K, B = int(rng.integers(1, 700)), int(rng.integers(1, 6000)), int(rng.integers(65, 701))
        if M * K * B <= 4e8:
            out.append((M, K, B))
    return out


@pytest.mark.parametrize("M,K,B", wide_random_shapes())
def test_tiled_wide_random(M, K, B):
    say(f"scalar tiled wide M={M} K={K} B={B}")
    db, Q = rand_case(M * 7 + K * 3 + B, M, K, B)
    np.testing.assert_array_equal(run_gpu(db, Q), oracle.scalar(db, Q))


def test_tiled_from_misaligned_source():
    db, Q = rand_case(4, 40, 4096, 3)
    np.testing.assert_array_equal(run_gpu(db, Q, offset=5), oracle.scalar(db, Q))


@pytest.mark.parametrize("B", [1, 32, 200])
def test_tiled_overflow_closed_forms(B):
    """db = -128, Q = 0x80808080 (digits -128, -127, -127, -127): every digit
    plane's int32 sum passes 2^31 in one accumulator at K = 2^17."""
    K, M = 1 << 17, 48
    say(f"scalar tiled overflow B={B}")
    db = np.full((M, K), -128, dtype=np.int8)
    Q = np.full((K, B), 0x80808080, dtype=np.uint32)
    want = (K * -128 * 0x80808080) % (1 << 32)
    assert (run_gpu(db, Q) == want).all()
    db = np.full((M, K), 127, dtype=np.int8)
    Q = np.full((K, B), 1 << 31, dtype=np.uint32)
    assert (run_gpu(db, Q) == (127 * (1 << 31) * K) % (1 << 32)).all()


def test_tiled_one_hot_and_regev_view():
    M, K = 300, 8200
    db = synth.int8_rows(2, synth.STREAM_SCALAR_DB, K, range(M))
    ks = [0, 1, 63, 64, 4095, 4096, 8191, 8199]
    Q = np.zeros((K, len(ks)), dtype=np.uint32)
    for b, k in enumerate(ks):
        Q[k, b] = 1 << 24 if b % 2 else 1
    got = run_gpu(db, Q)
    for b, k in enumerate(ks):
        if b % 2:
            np.testing.assert_array_equal((got[:, b] >> 24).astype(np.uint8), db[:, k].view(np.uint8))
        else:
            np.testing.assert_array_equal(got[:, b], db[:, k].astype(np.int32).astype(np.uint32))
    got1 = run_gpu(db, Q[:, 6:7].copy())
    np.testing.assert_array_equal(got1[:, 0], got[:, 6])     # B = 1 column == the same column at B = 8


def test_tiled_hint_and_second_fold_sampled():
    """VIPIR's offline hint (the 2^20 x 2^16 database view times the
    2^16 x 1280 matrix A: wide launches of four, four and two 128-column
    groups) and the double-packing second fold (32768 x 2^17 times
    2^17 x 1281: the same plus one narrow column, K split in four blocks) on
    tiled copies of the 64 GiB database's leading bytes, as the benchmark runs
    them.  Sampled rows: two in each eighth of the rows (each XCD's share of
    the hint's first launch) and the first and last row; every column."""
    import torch

    seed, N_LWE = 5, 1280
    say("scalar tiled hint / second fold: synthesising 64 GiB")
    d_bytes = torch.empty(1 << 36, dtype=torch.int8, device="cuda:0")
    synth.fill_int8_(d_bytes, seed, synth.STREAM_SCALAR_DB)
    def spread(M):
        eighth = M // 8
        return sorted({0, M - 1} | {x * eighth + o for x in range(8) for o in (5, eighth // 2 + 77)})

    for M, K, B, rows, qseed in (((1 << 20), (1 << 16), N_LWE, spread(1 << 20), seed + 100),
                                 (32768, 1 << 17, N_LWE + 1, spread(32768), seed + 200)):
        say(f"  M={M} K={K} B={B}")
        t = tiled(d_bytes[:M * K].view(M, K))
        d_q = empty_u32((K, B))
        synth.fill_uint32_(d_q, qseed, synth.STREAM_SCALAR_Q)
        got = to_host_u32(scan(t, M, K, d_q).index_select(0, torch.tensor(rows, device="cuda:0")))
        db_s = synth.int8_rows(seed, synth.STREAM_SCALAR_DB, K, rows)
        np.testing.assert_array_equal(got, oracle.scalar(db_s, synth.uint32_array(qseed, synth.STREAM_SCALAR_Q, (K, B))))
        del t, d_q
        release()
    del d_bytes
    release()
