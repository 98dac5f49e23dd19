"""The scalar-HE product at the full configurations, against the oracle.

VIPIR section 2.5 defines the database product as a D1 x B x D0 INT8-INT32
GEMM: out[i][b] for every row i and query column b.  Both entry points run
on the same device bytes -- the row-major pirscan_scalar_gemm_u32 and the
tiled pirscan_scalar_gemm_u32_tiled -- and the oracle reads the device's own
row-major DB and queries back in chunks of rows.

* scalar 1 GiB (M = K = 32768), B = 1 and B = 8: every output.
* scalar 64 GiB (M = K = 262144), one tiled DB for both batches as the
  benchmark runs them: B = 1 and B = 32, every output.
"""
import pytest

import synth
from he_database_scan_amd import pirscan
from tests.fullsize import check_scalar
from tests.gpu_util import empty_bytes, empty_u32, release, say

pytestmark = pytest.mark.gpu


def synth_db(seed, M, K):
    import torch

    say(f"scalar M={M} K={K}: synthesising {M * K / 2**30:.1f} GiB, one-time layout")
    d_db = torch.empty((M, K), dtype=torch.int8, device="cuda:0")
    synth.fill_int8_(d_db, seed, synth.STREAM_SCALAR_DB)
    d_t = empty_bytes(pirscan.scalar_layout_db_bytes(M, K))
    pirscan.scalar_layout_db(d_db, d_t)
    return d_db, d_t


def run_both(d_db, d_t, seed, B):
    """Both entry points on one synthesised query; returns (Q host, {name: d_out})."""
    M, K = d_db.shape
    d_q = empty_u32((K, B))
    synth.fill_uint32_(d_q, seed, synth.STREAM_SCALAR_Q)
    say(f"  scan B={B} (row-major and tiled)")
    d_rm = empty_u32((M, B))
    ws = empty_bytes(max(16, pirscan.scalar_workspace_bytes(M, K, B)))
    pirscan.scalar_gemm_u32(d_db, d_q, d_rm, ws)
    d_tl = empty_u32((M, B))
    ws2 = empty_bytes(pirscan.scalar_tiled_workspace_bytes(M, K, B))
    pirscan.scalar_gemm_u32_tiled(d_t, M, K, d_q, d_tl, ws2)
    Q = d_q.cpu().numpy().view("uint32")
    del ws, ws2
    return {f"row-major B={B}": (Q, d_rm), f"tiled B={B}": (Q, d_tl)}


def test_scalar_1gib_every_output():
    M = K = 32768
    d_db, d_t = synth_db(2, M, K)
    for B in (1, 8):
        outs = run_both(d_db, d_t, 2, B)
        check_scalar(d_db, outs, [(0, M)], f"scalar 1 GiB B={B}")
        del outs
    del d_db, d_t
    release()


@pytest.fixture(scope="module")
def scalar64():
    M = K = 262144
    d_db, d_t = synth_db(5, M, K)
    yield d_db, d_t
    del d_db, d_t
    release()


def test_scalar_64gib_b1_every_output(scalar64):
    d_db, d_t = scalar64
    M = d_db.shape[0]
    outs = run_both(d_db, d_t, 5, 1)
    check_scalar(d_db, outs, [(0, M)], "scalar 64 GiB B=1")
    del outs
    release()


def test_scalar_64gib_b32_every_output(scalar64):
    d_db, d_t = scalar64
    M = d_db.shape[0]
    outs = run_both(d_db, d_t, 5, 32)
    check_scalar(d_db, outs, [(0, M)], "scalar 64 GiB B=32")
    del outs
    release()
