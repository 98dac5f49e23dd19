"""Every gfx950 kernel the package builds has a body that ends the wave.

Undefined behaviour in device code (for instance a 32-bit shift by 32) lets
the compiler treat a kernel as unreachable and emit it with no instructions,
so that its waves run on into whatever code follows.  This test compiles each
HIP source to gfx950 assembly (no GPU needed) and checks that every kernel
symbol has instructions and an s_endpgm before the end of its function."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = [os.path.join(ROOT, "he_database_scan_amd", "csrc", f)
           for f in ("rowsel.hip", "rowsel_mfma.hip", "scalar.hip", "ntt.hip", "readprobe.hip")] + \
          [os.path.join(ROOT, "synth", "synth.hip")]
HIPCC = "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
@pytest.mark.parametrize("src", SOURCES, ids=os.path.basename)
def test_every_kernel_has_a_terminated_body(src, tmp_path):
    out = tmp_path / "dev.s"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
                    "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form", "--cuda-device-only",
                    "-S", "-o", str(out), src],
                   check=True, capture_output=True)
    asm = out.read_text()
    kernels = re.findall(r"^\s+\.amdhsa_kernel\s+(\S+)", asm, re.M)
    assert kernels, "no kernels found"
    for name in kernels:
        m = re.search(r"^" + re.escape(name) + r":.*?$(.*?)^\.Lfunc_end", asm, re.M | re.S)
        assert m, f"{name}: function body not found"
        body = m.group(1)
        insts = re.findall(r"^\s+[a-z][a-z0-9_]*\b", body, re.M)
        assert len(insts) >= 4, f"{name}: empty body"
        assert "s_endpgm" in body, f"{name}: no s_endpgm"
