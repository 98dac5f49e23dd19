"""The scalar-HE product at the pages' other shapes, on the GPU through the C
ABI, bit-exact against the oracle.

* VIPIR's offline hint: the database times the D0 x n random matrix A
  (n = 1280 LWE columns), a D1 x n result -- the same INT8 x uint32 product
  mod 2^32 with a wide query operand (VIPIR, the SimplePIR example paragraph:
  the D0 x n part of the query matrix is query-independent and precomputed).
* The double-packing protocol's second fold: an 8N x D1 INT8 intermediate
  times D1 x (n+1) scalar-HE ciphertexts (VIPIR section 4.4).
* The D/D0 aspect ratios at a fixed database size (VIPIR section 6.6: the
  (D/D0) x B x D0 GEMM does D*B multiply-adds whatever D0 is), on the same
  64 GiB of bytes viewed as 2^20 x 2^16 ... 2^17 x 2^19.

Element by element on small wide-query shapes; sampled rows at full size."""
import numpy as np
import pytest

import oracle
import synth
from he_database_scan_amd import pirscan
from tests.gpu_util import empty_u32, release, say, to_dev_i8, to_dev_u32, to_host_u32

pytestmark = pytest.mark.gpu

SEED = 5
N_LWE = 1280


@pytest.mark.parametrize("M,K,B", [(100, 4096, N_LWE), (37, 1040, N_LWE + 1), (300, 16400, 96),
                                   (65, 2048, 33), (77, 4160, 64), (100, 2048, 65), (260, 20480, 48)])
def test_wide_query_full(M, K, B):
    import torch

    say(f"scalar wide M={M} K={K} B={B}")
    rng = np.random.default_rng(M + K + B)
    db = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    Q = rng.integers(0, 1 << 32, size=(K, B), dtype=np.uint64).astype(np.uint32)
    d_o = empty_u32((M, B))
    ws = torch.empty(pirscan.scalar_workspace_bytes(M, K, B), dtype=torch.uint8, device="cuda:0")
    pirscan.scalar_gemm_u32(to_dev_i8(db), to_dev_u32(Q), d_o, ws)
    np.testing.assert_array_equal(to_host_u32(d_o), oracle.scalar(db, Q))


def scan_sampled(d_bytes, M, K, B, rows, qseed):
    """Runs the product on the first M*K bytes of d_bytes viewed as [M][K]
    and compares the given rows with the oracle."""
    import torch

    say(f"  M={M} K={K} B={B}")
    d_db = d_bytes[:M * K].view(M, K)
    d_q = empty_u32((K, B))
    synth.fill_uint32_(d_q, qseed, synth.STREAM_SCALAR_Q)
    d_o = empty_u32((M, B))
    ws = torch.empty(pirscan.scalar_workspace_bytes(M, K, B), dtype=torch.uint8, device="cuda:0")
    pirscan.scalar_gemm_u32(d_db, d_q, d_o, ws)
    got = to_host_u32(d_o.index_select(0, torch.tensor(rows, device="cuda:0")))
    db_s = synth.int8_rows(SEED, synth.STREAM_SCALAR_DB, K, rows)
    Q = synth.uint32_array(qseed, synth.STREAM_SCALAR_Q, (K, B))
    np.testing.assert_array_equal(got, oracle.scalar(db_s, Q))
    del d_q, d_o, ws


def test_64gib_aspects_hint_and_second_fold_sampled():
    import torch

    total = 1 << 36
    say("scalar shapes: synthesising 64 GiB")
    d_bytes = torch.empty(total, dtype=torch.int8, device="cuda:0")
    synth.fill_int8_(d_bytes, SEED, synth.STREAM_SCALAR_DB)
    for logm in (20, 19, 17):
        M, K = 1 << logm, total >> logm
        rows = [0, 1, 63, M // 2 + 5, M - 1]
        for B in (1, 32):
            scan_sampled(d_bytes, M, K, B, rows, SEED)
    say("scalar shapes: hint D1 x n = 2^20 x 1280 over the 64 GiB database")
    scan_sampled(d_bytes, 1 << 20, 1 << 16, N_LWE, [0, 777, (1 << 20) - 1], SEED + 100)
    say("scalar shapes: second fold 8N x D1 (4 GiB) times D1 x (n+1)")
    scan_sampled(d_bytes, 8 * 4096, 1 << 17, N_LWE + 1, [0, 4097, 32767], SEED + 200)
    del d_bytes
    release()
