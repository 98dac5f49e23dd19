"""Work is enqueued on the caller's stream (include/pirscan.h: every call is
asynchronous on `stream`).  Each scan runs on a non-default torch stream
behind a GPU busy-wait that delays that stream, with its inputs written on
the same stream after the wait and its output read back on it: a launch on
any other stream would read the inputs before they are written, or be read
before it has run.  Every result is compared with the oracle."""
import numpy as np
import pytest

import oracle
from he_database_scan_amd import pirscan
from tests.gpu_util import MED_Q, empty_bytes, empty_u32, say, to_dev_i8, to_dev_u32

pytestmark = pytest.mark.gpu

SPIN_CYCLES = 200_000_000  # a GPU busy-wait of roughly 0.1 s at the shader clock


def delayed(stream, fill_pairs):
    """On `stream`: a busy-wait, then dst.copy_(src) for every pair, so the
    destinations hold their values only once the stream reaches that point."""
    import torch

    with torch.cuda.stream(stream):
        torch.cuda._sleep(SPIN_CYCLES)
        for dst, src in fill_pairs:
            dst.copy_(src)


def test_rowsel_on_a_side_stream():
    import torch

    rng = np.random.default_rng(21)
    N, D0, D1 = 16, 130, 300
    P = N * len(MED_Q)
    qv = np.asarray(MED_Q, dtype=np.uint64)[np.arange(P) // N]
    db = (rng.integers(0, 1 << 62, size=(D0, D1, P), dtype=np.uint64) % qv).astype(np.uint32)
    shape = pirscan.RowselShape.make(N, MED_Q, D0, D1)
    dbt = empty_bytes(pirscan.layout_db_bytes(shape))
    pirscan.layout_db(shape, to_dev_u32(db), dbt)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    for m in (2, 32):
        say(f"rowsel on a side stream m={m}")
        ct = (rng.integers(0, 1 << 62, size=(m, D0, P), dtype=np.uint64) % qv).astype(np.uint32)
        src = to_dev_u32(ct)
        d_ct = torch.zeros_like(src)
        out = torch.zeros((m, D1, P), dtype=torch.int32, device="cuda:0")
        ws = empty_bytes(pirscan.rowsel_workspace_bytes(shape, m))
        torch.cuda.synchronize()
        delayed(s, [(d_ct, src)])
        with torch.cuda.stream(s):
            pirscan.rowsel_modgemm(shape, m, d_ct, dbt, out, ws)   # the binding passes torch's current stream
            res = out.clone()
        s.synchronize()
        np.testing.assert_array_equal(res.cpu().numpy().view(np.uint32), oracle.rowsel(ct, db, N, MED_Q))


def test_scalar_on_a_side_stream():
    import torch

    rng = np.random.default_rng(22)
    M, K = 520, 8256
    db = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    d_db = to_dev_i8(db)
    tiled = empty_bytes(pirscan.scalar_layout_db_bytes(M, K))
    pirscan.scalar_layout_db(d_db, tiled)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    for B in (1, 8):
        say(f"scalar on a side stream B={B}")
        Q = rng.integers(0, 1 << 32, size=(K, B), dtype=np.uint64).astype(np.uint32)
        src = to_dev_u32(Q)
        d_q = torch.zeros_like(src)
        o1 = empty_u32((M, B))
        o2 = empty_u32((M, B))
        w1 = empty_bytes(max(16, pirscan.scalar_workspace_bytes(M, K, B)))
        w2 = empty_bytes(pirscan.scalar_tiled_workspace_bytes(M, K, B))
        torch.cuda.synchronize()
        delayed(s, [(d_q, src)])
        # explicit stream argument this time
        pirscan.scalar_gemm_u32(d_db, d_q, o1, w1, stream=s.cuda_stream)
        pirscan.scalar_gemm_u32_tiled(tiled, M, K, d_q, o2, w2, stream=s.cuda_stream)
        with torch.cuda.stream(s):
            r1, r2 = o1.clone(), o2.clone()
        s.synchronize()
        want = oracle.scalar(db, Q)
        np.testing.assert_array_equal(r1.cpu().numpy().view(np.uint32), want)
        np.testing.assert_array_equal(r2.cpu().numpy().view(np.uint32), want)
