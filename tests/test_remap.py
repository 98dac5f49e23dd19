"""The workgroup-to-XCD maps of the scans (internal.hpp) are permutations.

A scan kernel derives its tile from the remapped workgroup id, so a map that
repeats or skips an id would compute a tile twice and leave another unwritten.
This compiles a host program against the library's header (no GPU needed) and
checks xcd_remap and every scan_remap chunk size used by the kernels on grid
sizes with and without a whole number of chunk rounds."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "he_database_scan_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"

PROGRAM = r"""
#include <cstdio>
#include <vector>
#include "internal.hpp"
using namespace pirscan;
template <uint32_t C>
static bool check(uint32_t num) {
  std::vector<char> seen(num, 0);
  for (uint32_t h = 0; h < num; ++h) {
    const uint32_t v = scan_remap<C>(h, num);
    if (v >= num || seen[v]) return false;
    seen[v] = 1;
  }
  return true;
}
int main() {
  const uint32_t sizes[] = {1, 7, 8, 9, 63, 64, 100, 511, 512, 513, 4096, 12345, 65536, 196608, 196611};
  int bad = 0;
  for (uint32_t n : sizes) {
    if (!check<0>(n)) { std::printf("xcd_remap not a permutation at %u\n", n); ++bad; }
    if (!check<1>(n)) { std::printf("identity failed at %u\n", n); ++bad; }
    if (!check<8>(n)) { std::printf("chunk 8 not a permutation at %u\n", n); ++bad; }
    if (!check<64>(n)) { std::printf("chunk 64 not a permutation at %u\n", n); ++bad; }
    if (!check<512>(n)) { std::printf("chunk 512 not a permutation at %u\n", n); ++bad; }
  }
  // chunk C: hardware ids h and h + 8 land C logical ids apart within a round
  if (scan_remap<64>(0, 1024) != 0 || scan_remap<64>(1, 1024) != 64 || scan_remap<64>(8, 1024) != 1) {
    std::printf("chunk 64 layout\n");
    ++bad;
  }
  std::printf(bad ? "FAIL\n" : "OK\n");
  return bad != 0;
}
"""


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_workgroup_maps_are_permutations(tmp_path):
    src = tmp_path / "remap.hip"
    src.write_text(PROGRAM)
    exe = tmp_path / "remap"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-I", CSRC, "-o", str(exe), str(src)],
                   check=True, capture_output=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True)
    assert res.returncode == 0 and res.stdout.strip().endswith("OK"), res.stdout
