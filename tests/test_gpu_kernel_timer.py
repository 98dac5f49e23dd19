"""The benchmark build's kernel-timer hook (pirscan_kernel_timer_begin / _end,
libpirscan_bench.so), which the benchmark uses to price each scan's main
kernel: one time per call, in call order, positive and no longer than the
whole call; and the benchmark build gives the product library's results."""
import numpy as np
import pytest

from he_database_scan_amd import pirscan
from tests.gpu_util import MED_Q, empty_bytes, empty_u32, say, to_dev_u32

pytestmark = pytest.mark.gpu

bench = pirscan.bench_library()


def test_one_time_per_call_within_the_call():
    import torch

    rng = np.random.default_rng(5)
    N, D0, D1 = 64, 256, 512
    P = N * len(MED_Q)
    shape = pirscan.RowselShape.make(N, MED_Q, D0, D1)
    dbt = empty_bytes(bench.layout_db_bytes(shape))
    bench.layout_db(shape, to_dev_u32(rng.integers(0, MED_Q[2], size=(D0, D1, P))), dbt)
    calls = []
    for m in (2, 32):
        ct = to_dev_u32(rng.integers(0, MED_Q[2], size=(m, D0, P)))
        out = empty_u32((m, D1, P))
        n = bench.rowsel_workspace_bytes(shape, m)
        ws = torch.empty(n, dtype=torch.uint8, device="cuda:0") if n else None
        calls.append(lambda ct=ct, out=out, m=m, ws=ws: bench.rowsel_modgemm(shape, m, ct, dbt, out, ws))
    db8 = torch.randint(-128, 128, (4096, 8192), dtype=torch.int8, device="cuda:0")
    for B in (1, 32):
        q = to_dev_u32(rng.integers(0, 1 << 32, size=(8192, B), dtype=np.uint64).astype(np.uint32))
        o = empty_u32((4096, B))
        ws = torch.empty(bench.scalar_workspace_bytes(4096, 8192, B), dtype=torch.uint8, device="cuda:0")
        calls.append(lambda q=q, o=o, ws=ws: bench.scalar_gemm_u32(db8, q, o, ws))
    say("kernel timer: 4 scans x 3 rounds")
    stream = torch.cuda.current_stream()
    bench.kernel_timer_begin(12)
    whole = []
    for _ in range(3):
        for fn in calls:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            whole.append((e0, e1))
    kms = bench.kernel_timer_end(12)
    torch.cuda.synchronize()
    assert len(kms) == 12
    for k, (e0, e1) in zip(kms, whole):
        assert 0.0 < k <= e0.elapsed_time(e1) * 1.05 + 0.05
    # capacity bounds what is recorded; a second begin starts afresh
    bench.kernel_timer_begin(2)
    for fn in calls:
        fn()
    assert len(bench.kernel_timer_end(100)) == 2
    # off: nothing recorded, _end without _begin is an error
    calls[0]()
    with pytest.raises(pirscan.PirscanError):
        bench.kernel_timer_end(4)


def test_read_reference_is_timed_and_reads_only():
    """The read-stream reference runs on any multiple of 16 bytes (whole
    unrolled rounds and a tail), records one kernel time per call, and leaves
    the buffer it reads untouched."""
    import torch

    rng = np.random.default_rng(11)
    for nbytes in (16, 4096 + 48, 3 << 20):
        buf = torch.from_numpy(rng.integers(0, 256, size=nbytes, dtype=np.uint8)).to("cuda:0")
        before = buf.clone()
        sink = torch.zeros(4, dtype=torch.uint8, device="cuda:0")
        say(f"read reference {nbytes} bytes")
        bench.kernel_timer_begin(2)
        bench.bench_read(buf, sink)
        bench.bench_read(buf, sink)
        kms = bench.kernel_timer_end(2)
        assert len(kms) == 2 and all(k > 0.0 for k in kms)
        assert torch.equal(buf, before)
    with pytest.raises(pirscan.PirscanError):
        bench.bench_read(buf[:20], sink)   # not a multiple of 16 bytes


def test_benchmark_build_matches_the_product_library():
    """Same sources, same kernels: the two builds give identical outputs."""
    import torch

    rng = np.random.default_rng(9)
    N, D0, D1 = 16, 130, 300
    P = N * len(MED_Q)
    db = to_dev_u32(rng.integers(0, MED_Q[2], size=(D0, D1, P)))
    for m in (2, 33):
        ct = to_dev_u32(rng.integers(0, MED_Q[2], size=(m, D0, P)))
        outs = []
        for L in (pirscan.default(), bench):
            shape = pirscan.RowselShape.make(N, MED_Q, D0, D1)
            dbt = empty_bytes(L.layout_db_bytes(shape))
            L.layout_db(shape, db, dbt)
            out = empty_u32((m, D1, P))
            L.rowsel_modgemm(shape, m, ct, dbt, out, empty_bytes(L.rowsel_workspace_bytes(shape, m)))
            outs.append(out)
        assert torch.equal(outs[0], outs[1])
    db8 = torch.randint(-128, 128, (300, 4160), dtype=torch.int8, device="cuda:0")
    for B in (1, 5):
        q = to_dev_u32(rng.integers(0, 1 << 32, size=(4160, B), dtype=np.uint64).astype(np.uint32))
        outs = []
        for L in (pirscan.default(), bench):
            o = empty_u32((300, B))
            L.scalar_gemm_u32(db8, q, o, empty_bytes(max(16, L.scalar_workspace_bytes(300, 4160, B))))
            outs.append(o)
        assert torch.equal(outs[0], outs[1])
