"""Full-size parity: every GPU output of a large configuration against the
oracle, which reads the GPU's own input bytes back from device memory.

The inputs of a full-size configuration live only on the device (tens of GiB,
synthesised there).  They are copied back in chunks of at most 1 GiB into two
pinned host buffers used in turn: while the oracle works on one chunk (on all
the host cores this process may use), a helper thread gathers and copies the
next.  Each chunk's oracle result is compared element by element with the
GPU's outputs for the same points (RowSel, ExpPack) or rows (scalar-HE).
"""
from __future__ import annotations

import os
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
from tests.gpu_util import say

CHUNK_BYTES = 1 << 30


def host_threads() -> int:
    """The host cores this process may use: its affinity set, capped by
    OMP_NUM_THREADS when that is set (the CPU share of the machine)."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def _pinned(nbytes: int):
    import torch

    return torch.empty(max(16, nbytes), dtype=torch.uint8, pin_memory=True)


def _to_host(dev_view, buf):
    """A device view (any strides) -> numpy array of its shape in `buf`
    (pinned, uint8), through a contiguous device copy."""
    import torch

    c = dev_view.contiguous()
    nbytes = c.numel() * c.element_size()
    h = buf[:nbytes].view(c.dtype).view(c.shape)
    h.copy_(c)
    torch.cuda.synchronize()
    return h.numpy()


def _stream(nchunks, fetch, consume):
    """fetch(i, slot) on a helper thread, consume(i, data) here; fetch(i + 1)
    runs while consume(i) does (slots alternate, so a slot is refilled only
    after the chunk in it has been consumed)."""
    with ThreadPoolExecutor(max_workers=1) as ex:
        fut = ex.submit(fetch, 0, 0)
        for i in range(nchunks):
            data = fut.result()
            if i + 1 < nchunks:
                fut = ex.submit(fetch, i + 1, (i + 1) % 2)
            consume(i, data)


def _first_mismatch(got, want):
    idx = np.argwhere(got != want)
    return tuple(int(v) for v in idx[0]), int(got[tuple(idx[0])]), int(want[tuple(idx[0])])


def point_chunks(ranges, N: int, width: int):
    """Split point ranges [a, b) into chunks of at most `width` points that
    never cross an RNS limb (a limb is N consecutive points)."""
    out = []
    for a, b in ranges:
        p = a
        while p < b:
            e = min(b, p + width, (p // N + 1) * N)
            out.append((p, e))
            p = e
    return out


def check_modgemm(kind, d_ops, d_outs, N, q, ranges, label):
    """Every output of the point-wise modular GEMM at the points in `ranges`.

    kind "rowsel":  d_ops = (d_db [D0][D1][P],); d_outs = {m: (d_ct [m][D0][P],
                    d_out [m][D1][P])}.
    kind "exppack": d_ops = (d_h [Dr][n][P],);   d_outs = {B: (d_c [n][2B][P],
                    d_g [Dr][B][P] or None, d_out [Dr][2B][P])}.
    The streamed operand (DB / hint) is read back in point chunks of at most
    1 GiB; the per-query operands and outputs of the chunk come with it.
    """
    d_big = d_ops[0]
    X, Y, P = d_big.shape
    per_point = 4 * X * Y
    width = max(1, min(N, CHUNK_BYTES // per_point))
    chunks = point_chunks(ranges, N, width)
    bufs = [_pinned(per_point * width) for _ in range(2)]
    threads = host_threads()
    npts = sum(b - a for a, b in chunks)
    say(f"  {label}: {npts} points in {len(chunks)} chunks of <= {width}, oracle on {threads} threads")

    def fetch(i, slot):
        a, b = chunks[i]
        big = _to_host(d_big[:, :, a:b], bufs[slot]).view(np.uint32)
        per_q = {}
        for key, tensors in d_outs.items():
            per_q[key] = tuple(None if t is None else t[:, :, a:b].contiguous().cpu().numpy().view(np.uint32)
                               for t in tensors)
        return big, per_q

    t0 = [time.perf_counter(), time.perf_counter()]

    def consume(i, data):
        a, b = chunks[i]
        big, per_q = data
        qr = [int(q[a // N])]
        for key, arrs in per_q.items():
            if kind == "rowsel":
                ct, got = arrs
                want = oracle.rowsel(ct, big, b - a, qr, nthreads=threads)
            else:
                c, g, got = arrs
                want = oracle.exppack(big, c, g, b - a, qr, nthreads=threads)
            if not np.array_equal(got, want):
                (x, y, t), gv, wv = _first_mismatch(got, want)
                raise AssertionError(f"{label} {key}: first mismatch at [{x}][{y}][p={a + t}]: "
                                     f"gpu {gv}, oracle {wv}")
        now = time.perf_counter()
        if now - t0[1] > 10 or i + 1 == len(chunks):
            say(f"    chunk {i + 1}/{len(chunks)} (points {a}..{b - 1}) ok, {now - t0[0]:.1f} s")
            t0[1] = now

    _stream(len(chunks), fetch, consume)


def check_scalar(d_db, outs, row_ranges, label):
    """Every output of the scalar-HE product at the rows in `row_ranges`.

    d_db [M][K] int8 on the device (row-major); outs = {name: (Q [K][B] host
    uint32, d_out [M][B] device)}: several products of the same DB (batch
    sizes, entry points) share each chunk of DB rows read back."""
    M, K = d_db.shape
    rows_per = max(1, CHUNK_BYTES // K)
    chunks = []
    for a, b in row_ranges:
        for r in range(a, b, rows_per):
            chunks.append((r, min(b, r + rows_per)))
    bufs = [_pinned(K * rows_per) for _ in range(2)]
    threads = host_threads()
    nrows = sum(b - a for a, b in chunks)
    say(f"  {label}: {nrows} rows in {len(chunks)} chunks of <= {rows_per}, oracle on {threads} threads")

    def fetch(i, slot):
        a, b = chunks[i]
        db = _to_host(d_db[a:b], bufs[slot]).view(np.int8)
        return db, {name: d_out[a:b].cpu().numpy().view(np.uint32) for name, (Q, d_out) in outs.items()}

    t0 = [time.perf_counter(), time.perf_counter()]
    wants = {}

    def consume(i, data):
        a, b = chunks[i]
        db, gots = data
        wants.clear()
        for name, (Q, _) in outs.items():
            key = Q.ctypes.data  # products with the same query share the oracle's result
            if key not in wants:
                wants[key] = oracle.scalar(db, Q, nthreads=threads)
            want = wants[key]
            if not np.array_equal(gots[name], want):
                (r, c), gv, wv = _first_mismatch(gots[name], want)
                raise AssertionError(f"{label} {name}: first mismatch at row {a + r}, column {c}: "
                                     f"gpu {gv}, oracle {wv}")
        now = time.perf_counter()
        if now - t0[1] > 10 or i + 1 == len(chunks):
            say(f"    chunk {i + 1}/{len(chunks)} (rows {a}..{b - 1}) ok, {now - t0[0]:.1f} s")
            t0[1] = now

    _stream(len(chunks), fetch, consume)
