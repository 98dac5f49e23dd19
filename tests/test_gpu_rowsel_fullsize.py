"""RowSel at the full configurations, every output against the oracle.

GPIR's RowSel formulation defines out[p, m, n] for every point p, row m and
column n; the oracle reads the device's own p-major DB and ct back in chunks
and computes each of them.

* RowSel medium (N = 4096, three 29-bit primes, P = 12288, D0 = D1 = 256,
  3 GiB DB), B = 1 (m = 2): every output, on the int8 matrix-core scan and
  on the 64-bit VALU scan.
* RowSel large (D0 = D1 = 1024, 48 GiB DB), one tiled DB shared by both
  batches as the benchmark runs them: B = 1 (m = 2) and B = 16 (m = 32),
  every output (the B = 16 check split by RNS limb).
"""
import pytest

import synth
from he_database_scan_amd import pirscan
from tests.fullsize import check_modgemm
from tests.gpu_util import MED_Q, empty_bytes, empty_u32, release, say

pytestmark = pytest.mark.gpu

N = 4096
P = N * len(MED_Q)


def build_db(seed, D0, D1, scan=pirscan.SCAN_AUTO):
    shape = pirscan.RowselShape.make(N, MED_Q, D0, D1, scan=scan)
    say(f"rowsel D0={D0} D1={D1}: synthesising {4 * P * D0 * D1 / 2**30:.1f} GiB, one-time layout")
    d_db = empty_u32((D0, D1, P))
    synth.fill_residues_(d_db, seed, synth.STREAM_ROWSEL_DB, N, MED_Q)
    d_dbt = empty_bytes(pirscan.layout_db_bytes(shape))
    pirscan.layout_db(shape, d_db, d_dbt)
    return shape, d_db, d_dbt


def run_scan(shape, d_dbt, seed, m):
    d_ct = empty_u32((m, shape.D0, P))
    synth.fill_residues_(d_ct, seed, synth.STREAM_ROWSEL_CT, N, MED_Q)
    d_out = empty_u32((m, shape.D1, P))
    ws = empty_bytes(pirscan.rowsel_workspace_bytes(shape, m))
    say(f"  scan m={m}")
    pirscan.rowsel_modgemm(shape, m, d_ct, d_dbt, d_out, ws)
    del ws
    return d_ct, d_out


def test_medium_every_output():
    shape, d_db, d_dbt = build_db(3, 256, 256)
    d_ct, d_out = run_scan(shape, d_dbt, 3, 2)
    check_modgemm("rowsel", (d_db,), {2: (d_ct, d_out)}, N, MED_Q, [(0, P)], "rowsel medium 3 GiB B=1")
    del d_db, d_dbt, d_ct, d_out
    release()


def test_medium_every_output_valu_scan():
    """The same configuration on the 64-bit VALU scan (word layout, lazy
    accumulation), chosen at run time with SCAN_VALU."""
    shape, d_db, d_dbt = build_db(3, 256, 256, scan=pirscan.SCAN_VALU)
    d_ct, d_out = run_scan(shape, d_dbt, 3, 2)
    check_modgemm("rowsel", (d_db,), {2: (d_ct, d_out)}, N, MED_Q, [(0, P)], "rowsel medium 3 GiB B=1 VALU")
    del d_db, d_dbt, d_ct, d_out
    release()


@pytest.fixture(scope="module")
def large():
    shape, d_db, d_dbt = build_db(4, 1024, 1024)
    yield shape, d_db, d_dbt
    del d_db, d_dbt
    release()


def test_large_b1_every_output(large):
    shape, d_db, d_dbt = large
    d_ct, d_out = run_scan(shape, d_dbt, 4, 2)
    check_modgemm("rowsel", (d_db,), {2: (d_ct, d_out)}, N, MED_Q, [(0, P)], "rowsel large 48 GiB B=1")
    del d_ct, d_out
    release()


@pytest.fixture(scope="module")
def large_b16(large):
    shape, d_db, d_dbt = large
    d_ct, d_out = run_scan(shape, d_dbt, 4, 32)
    yield d_ct, d_out
    del d_ct, d_out
    release()


@pytest.mark.parametrize("limb", [0, 1, 2])
def test_large_b16_every_output(large, large_b16, limb):
    """One scan of the B = 16 batch; each RNS limb's 4096 points are checked
    by one test (about half a minute of oracle work each)."""
    shape, d_db, d_dbt = large
    d_ct, d_out = large_b16
    check_modgemm("rowsel", (d_db,), {32: (d_ct, d_out)}, N, MED_Q, [(limb * N, (limb + 1) * N)],
                  f"rowsel large 48 GiB B=16 limb {limb}")
