"""The seeded input generator shared by both sides (synth): pinned to the
published SplitMix64 sequence, and its derived element types checked."""
import os

import numpy as np

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def golden_splitmix():
    path = os.path.join(ROOT, "tests", "golden", "splitmix64_seed0.txt")
    return [int(l, 16) for l in open(path) if l.strip() and not l.startswith("#")]


def test_published_splitmix64_vector():
    want = golden_splitmix()
    got = [int(v) for v in synth.values(0, np.arange(len(want)))]
    assert got == want
    assert [synth.mix64_int((i + 1) * synth.GAMMA) for i in range(len(want))] == want


def test_counter_based_slices_agree():
    a = synth.int8_bytes(5, 3, 0, 1000)
    for start, cnt in [(0, 1), (7, 9), (8, 16), (13, 987), (999, 1)]:
        np.testing.assert_array_equal(synth.int8_bytes(5, 3, start, cnt), a[start:start + cnt])
    rows = synth.int8_rows(5, 3, 100, [0, 3, 9])
    np.testing.assert_array_equal(rows[1], a[300:400])


def test_element_types():
    st = synth.state0(2, synth.STREAM_SCALAR_Q)
    v = synth.values(st, np.arange(10))
    np.testing.assert_array_equal(synth.uint32_words(2, synth.STREAM_SCALAR_Q, np.arange(10)),
                                  (v >> np.uint64(32)).astype(np.uint32))
    st = synth.state0(2, synth.STREAM_SCALAR_DB)
    v = synth.values(st, np.arange(2))
    b = synth.int8_bytes(2, synth.STREAM_SCALAR_DB, 0, 16)
    assert [int(x) & 0xFF for x in b[:8]] == [(int(v[0]) >> (8 * t)) & 0xFF for t in range(8)]
    q = [1073738753, 1073732609]
    r = synth.residue_array(1, synth.STREAM_ROWSEL_DB, (3, 512), 256, q)
    assert (r[:, :256] < q[0]).all() and (r[:, 256:] < q[1]).all()
    raw = synth.values(synth.state0(1, synth.STREAM_ROWSEL_DB), np.arange(3 * 512)).reshape(3, 512)
    np.testing.assert_array_equal(r[:, 300], (raw[:, 300] % np.uint64(q[1])).astype(np.uint32))


def test_streams_and_seeds_differ():
    a = synth.uint32_array(1, 1, (64,))
    assert not np.array_equal(a, synth.uint32_array(1, 2, (64,)))
    assert not np.array_equal(a, synth.uint32_array(2, 1, (64,)))
    np.testing.assert_array_equal(a, synth.uint32_array(1, 1, (64,)))


def test_int8_distribution_covers_range():
    b = synth.int8_bytes(5, 3, 0, 1 << 16)
    assert b.min() == -128 and b.max() == 127
    assert abs(float(b.astype(np.float64).mean())) < 2.0
