"""The device input filler reproduces the host generator exactly, so inputs
synthesised on the GPU for the full-size configurations are the same bytes the
oracle regenerates on the host."""
import numpy as np
import pytest

import synth
from tests.gpu_util import TINY_Q, MED_Q, empty_u32, to_host_u32, say

pytestmark = pytest.mark.gpu


def test_device_residues_match_host():
    import torch

    for (shape, N, q, first) in [((16, 8, 512), 256, TINY_Q, 0), ((3, 12288), 4096, MED_Q, 0),
                                 ((1000,), 4096, MED_Q, 12288 * 1023 + 5)]:
        say(f"residues shape={shape} first={first}")
        t = empty_u32(shape)
        synth.fill_residues_(t, 4, synth.STREAM_ROWSEL_DB, N, q, first_index=first)
        P = len(q) * N
        idx = np.arange(first, first + t.numel(), dtype=np.uint64)
        want = synth.residues(4, synth.STREAM_ROWSEL_DB, idx, P, N, q).reshape(shape)
        np.testing.assert_array_equal(to_host_u32(t), want)


def test_device_int8_and_uint32_match_host():
    import torch

    for first, count in [(0, 4096), (3, 1000), (8 * 12345 + 5, 77)]:
        say(f"int8 first={first} count={count}")
        t = torch.empty(count, dtype=torch.int8, device="cuda:0")
        synth.fill_int8_(t, 5, synth.STREAM_SCALAR_DB, first_byte=first)
        np.testing.assert_array_equal(t.cpu().numpy(), synth.int8_bytes(5, synth.STREAM_SCALAR_DB, first, count))
    t = empty_u32((333, 7))
    synth.fill_uint32_(t, 5, synth.STREAM_SCALAR_Q)
    np.testing.assert_array_equal(to_host_u32(t), synth.uint32_array(5, synth.STREAM_SCALAR_Q, (333, 7)))
