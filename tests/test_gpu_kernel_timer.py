"""The library's kernel-timer hook (pirscan_kernel_timer_begin / _end), which
the benchmark uses to price each scan's main kernel: one time per call, in
call order, positive and no longer than the whole call."""
import numpy as np
import pytest

from he_database_scan_amd import pirscan
from tests.gpu_util import MED_Q, empty_bytes, empty_u32, say, to_dev_u32

pytestmark = pytest.mark.gpu


def test_one_time_per_call_within_the_call():
    import torch

    rng = np.random.default_rng(5)
    N, D0, D1 = 64, 256, 512
    P = N * len(MED_Q)
    shape = pirscan.RowselShape.make(N, MED_Q, D0, D1)
    dbt = empty_bytes(pirscan.layout_db_bytes(shape))
    pirscan.layout_db(shape, to_dev_u32(rng.integers(0, MED_Q[2], size=(D0, D1, P))), dbt)
    calls = []
    for m in (2, 32):
        ct = to_dev_u32(rng.integers(0, MED_Q[2], size=(m, D0, P)))
        out = empty_u32((m, D1, P))
        n = pirscan.rowsel_workspace_bytes(shape, m)
        ws = torch.empty(n, dtype=torch.uint8, device="cuda:0") if n else None
        calls.append(lambda ct=ct, out=out, m=m, ws=ws: pirscan.rowsel_modgemm(shape, m, ct, dbt, out, ws))
    db8 = torch.randint(-128, 128, (4096, 8192), dtype=torch.int8, device="cuda:0")
    for B in (1, 32):
        q = to_dev_u32(rng.integers(0, 1 << 32, size=(8192, B), dtype=np.uint64).astype(np.uint32))
        o = empty_u32((4096, B))
        ws = torch.empty(pirscan.scalar_workspace_bytes(4096, 8192, B), dtype=torch.uint8, device="cuda:0")
        calls.append(lambda q=q, o=o, ws=ws: pirscan.scalar_gemm_u32(db8, q, o, ws))
    say("kernel timer: 4 scans x 3 rounds")
    stream = torch.cuda.current_stream()
    pirscan.kernel_timer_begin(12)
    whole = []
    for _ in range(3):
        for fn in calls:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            whole.append((e0, e1))
    kms = pirscan.kernel_timer_end(12)
    torch.cuda.synchronize()
    assert len(kms) == 12
    for k, (e0, e1) in zip(kms, whole):
        assert 0.0 < k <= e0.elapsed_time(e1) * 1.05 + 0.05
    # capacity bounds what is recorded; a second begin starts afresh
    pirscan.kernel_timer_begin(2)
    for fn in calls:
        fn()
    assert len(pirscan.kernel_timer_end(100)) == 2
    # off: nothing recorded, _end without _begin is an error
    calls[0]()
    with pytest.raises(pirscan.PirscanError):
        pirscan.kernel_timer_end(4)


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
        pirscan.kernel_timer_begin(2)
        pirscan.bench_read(buf, sink)
        pirscan.bench_read(buf, sink)
        kms = pirscan.kernel_timer_end(2)
        assert len(kms) == 2 and all(k > 0.0 for k in kms)
        assert torch.equal(buf, before)
    with pytest.raises(pirscan.PirscanError):
        pirscan.bench_read(buf[:20], sink)   # not a multiple of 16 bytes
