"""pirscan_scalar_gemm_u32_noalloc -- the scalar-HE product without a
workspace argument (the library's built-in per-GPU scratch buffer), for
callers that cannot allocate -- against pirscan_scalar_gemm_u32 with a
caller-owned workspace, bit for bit.  Two calls in a row on the shared
buffer, the second with a smaller input, so stale contents of the first
cannot leak into the second; then the size limit."""
import ctypes

import numpy as np
import pytest

from he_database_scan_amd import pirscan
from tests.gpu_util import empty_bytes, empty_u32, say, to_dev_i8, to_dev_u32

pytestmark = pytest.mark.gpu


def both(db, Q):
    M, K = db.shape
    B = Q.shape[1]
    d_db, d_q = to_dev_i8(db), to_dev_u32(Q)
    want = empty_u32((M, B))
    pirscan.scalar_gemm_u32(d_db, d_q, want, empty_bytes(max(16, pirscan.scalar_workspace_bytes(M, K, B))))
    got = empty_u32((M, B))
    pirscan.scalar_gemm_u32_noalloc(d_db, d_q, got)
    return got.cpu().numpy(), want.cpu().numpy()


@pytest.mark.parametrize("first,second", [((2048, 65536, 1), (300, 8192, 1)),    # GEMV, split-K partials
                                          ((1024, 32768, 24), (130, 1040, 3)),   # MFMA, split-K partials
                                          ((512, 40960, 5), (70, 4096, 1))])     # MFMA then GEMV
def test_noalloc_matches_the_workspace_entry_point(first, second):
    rng = np.random.default_rng(sum(first) + sum(second))
    for M, K, B in (first, second):
        assert 0 < pirscan.scalar_workspace_bytes(M, K, B) <= pirscan.NOALLOC_SCRATCH_BYTES
        say(f"noalloc M={M} K={K} B={B}")
        db = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
        Q = rng.integers(0, 1 << 32, size=(K, B), dtype=np.uint64).astype(np.uint32)
        got, want = both(db, Q)
        np.testing.assert_array_equal(got, want)


def test_noalloc_at_the_64gib_shape_and_past_the_limit():
    """Every batch at M = K = 2^18 fits the scratch (B = 1: 1 MiB of digits +
    64 MiB of partials); twice that many rows at B = 1 does not, and is
    refused before any device work."""
    import torch

    for B in (1, 32, 64, 100):
        assert pirscan.scalar_workspace_bytes(1 << 18, 1 << 18, B) <= pirscan.NOALLOC_SCRATCH_BYTES
    assert pirscan.scalar_workspace_bytes(1 << 19, 1 << 18, 1) > pirscan.NOALLOC_SCRATCH_BYTES
    L = pirscan.lib()
    vp = ctypes.c_void_p
    rc = L.pirscan_scalar_gemm_u32_noalloc(vp(1 << 40), vp(1 << 44), vp(1 << 45), 1 << 19, 1 << 18, 1, None)
    assert rc == pirscan.ESCRATCH
    # a small call still works afterwards
    rng = np.random.default_rng(3)
    db = rng.integers(-128, 128, size=(64, 4096)).astype(np.int8)
    Q = rng.integers(0, 1 << 32, size=(4096, 2), dtype=np.uint64).astype(np.uint32)
    got, want = both(db, Q)
    np.testing.assert_array_equal(got, want)
    torch.cuda.synchronize()
