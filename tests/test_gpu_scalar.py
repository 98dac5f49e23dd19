"""Scalar-HE product on the GPU through the C ABI, bit-exact against the
oracle: element by element on multi-tile ragged shapes for the GEMV (B=1),
MFMA (B>1) and generic paths; overflow closed forms and one-hot selections.
The full 1 GiB and 64 GiB configurations are compared in
test_gpu_scalar_fullsize.py."""
import numpy as np
import pytest

import oracle
import synth
from he_database_scan_amd import pirscan
from tests.gpu_util import empty_u32, release, say, to_dev_i8, to_dev_u32, to_host_u32

pytestmark = pytest.mark.gpu


def run_gpu(db, Q, offset=0):
    """offset > 0 places the DB at a misaligned address (generic path)."""
    import torch

    M, K = db.shape
    B = Q.shape[1]
    if offset:
        raw = torch.empty(M * K + offset, dtype=torch.int8, device="cuda:0")
        raw[offset:] = to_dev_i8(db.reshape(-1))
        d_db = raw[offset:].view(M, K)
    else:
        d_db = to_dev_i8(db)
    d_q = to_dev_u32(Q)
    d_o = empty_u32((M, B))
    ws = torch.empty(max(16, pirscan.scalar_workspace_bytes(M, K, B)), dtype=torch.uint8, device="cuda:0")
    pirscan.scalar_gemm_u32(d_db, d_q, d_o, ws)
    return to_host_u32(d_o)


def rand_case(seed, M, K, B):
    rng = np.random.default_rng(seed)
    db = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    Q = rng.integers(0, 1 << 32, size=(K, B), dtype=np.uint64).astype(np.uint32)
    return db, Q


# (M, K, B): GEMV with one and several k-blocks and ragged K, rows not a
# multiple of the 64-row wavefront tile; MFMA with B=2..40 (several column
# passes), K not a multiple of the 64-wide MFMA step; generic (K % 16 != 0).
SHAPES = [(1, 16, 1), (63, 4096, 1), (300, 4096 * 3 + 48, 1), (1000, 8192, 1), (257, 160, 1),
          (100, 64, 2), (130, 1040, 3), (64, 4096, 8), (333, 20000, 8), (65, 16400, 16),
          (200, 2048, 17), (129, 33024, 32), (70, 512, 33), (40, 800, 40),
          (50, 1001, 1), (17, 33, 5)]


@pytest.mark.parametrize("M,K,B", SHAPES)
def test_multi_tile_shapes_full(M, K, B):
    say(f"scalar M={M} K={K} B={B}")
    db, Q = rand_case(M * 7 + K * 3 + B, M, K, B)
    np.testing.assert_array_equal(run_gpu(db, Q), oracle.scalar(db, Q))


def test_misaligned_db_uses_generic_path():
    db, Q = rand_case(3, 40, 4096, 2)
    np.testing.assert_array_equal(run_gpu(db, Q, offset=3), oracle.scalar(db, Q))


@pytest.mark.parametrize("B", [1, 8, 32])
def test_overflow_closed_forms(B):
    """db=-128, Q=0xFFFFFFFF: out = 128*K mod 2^32; db=127, Q=2^31: out =
    127*2^31*K mod 2^32.  With K=2^17 every int8 digit product sum exceeds
    2^31 in magnitude if accumulated unsplit."""
    K, M = 1 << 17, 64
    say(f"scalar overflow B={B}")
    db = np.full((M, K), -128, dtype=np.int8)
    Q = np.full((K, B), 0xFFFFFFFF, dtype=np.uint32)
    assert (run_gpu(db, Q) == (128 * K) % (1 << 32)).all()
    db = np.full((M, K), 127, dtype=np.int8)
    Q = np.full((K, B), 1 << 31, dtype=np.uint32)
    assert (run_gpu(db, Q) == (127 * (1 << 31) * K) % (1 << 32)).all()
    # digits (-128, -127, -127, -127) of 0x80808080 against -128 bytes
    db = np.full((M, K), -128, dtype=np.int8)
    Q = np.full((K, B), 0x80808080, dtype=np.uint32)
    np.testing.assert_array_equal(run_gpu(db, Q), oracle.scalar(db[:2], Q)[[0] * M])


def test_one_hot_and_regev_view():
    M, K = 512, 8192
    db = synth.int8_rows(2, synth.STREAM_SCALAR_DB, K, range(M))
    Q = np.zeros((K, 8), dtype=np.uint32)
    for b, k in enumerate([0, 1, 100, 4095, 4096, 5000, 8190, 8191]):
        Q[k, b] = 1 << 24 if b % 2 else 1
    got = run_gpu(db, Q)
    for b, k in enumerate([0, 1, 100, 4095, 4096, 5000, 8190, 8191]):
        if b % 2:
            np.testing.assert_array_equal((got[:, b] >> 24).astype(np.uint8), db[:, k].view(np.uint8))
        else:
            np.testing.assert_array_equal(got[:, b], db[:, k].astype(np.int32).astype(np.uint32))
    got1 = run_gpu(db, Q[:, 2:3].copy())
    np.testing.assert_array_equal(got1[:, 0], got[:, 2])     # B=1 column == B>1 column


@pytest.mark.parametrize("B", [8, 32])
def test_int32_digit_sums_wrap_inside_one_k_block(B):
    """131072 rows x 2^17: the plan keeps K in one block (enough row tiles),
    so each digit-plane sum of (-128)*(-128) products reaches 2^31 inside a
    single int32 accumulator.  Q = 0x80808080 has digits (-128, -127, -127,
    -127); out = K * (-128) * 0x80808080 mod 2^32 for every element."""
    import torch

    M = K = 1 << 17
    say(f"scalar wrap M={M} K={K} B={B}")
    d_db = torch.full((M, K), -128, dtype=torch.int8, device="cuda:0")
    d_q = torch.full((K, B), 0x80808080 - (1 << 32), dtype=torch.int32, device="cuda:0")
    d_o = empty_u32((M, B))
    ws = torch.empty(pirscan.scalar_workspace_bytes(M, K, B), dtype=torch.uint8, device="cuda:0")
    pirscan.scalar_gemm_u32(d_db, d_q, d_o, ws)
    want = (K * -128 * 0x80808080) % (1 << 32)
    want_i32 = want - (1 << 32) if want >= (1 << 31) else want
    assert bool((d_o == want_i32).all())
    del d_db, d_q, d_o, ws
    release()
