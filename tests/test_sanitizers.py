"""CPU builds with AddressSanitizer and UndefinedBehaviorSanitizer
(tests/c/Makefile): the oracle run over every function on small and edge
shapes, and libpirscan's host layer (validation, size queries, overlap and
overflow checks) driven through its C ABI without a GPU.  Any out-of-bounds
access, leak or undefined operation stops the run with a non-zero status."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "_build", "sanitize")


def build(target):
    subprocess.run(["make", "-s", "-C", os.path.join(ROOT, "tests", "c"), os.path.join(BUILD, target)], check=True)
    return os.path.join(BUILD, target)


def run(exe, leaks=True):
    env = dict(os.environ, ASAN_OPTIONS=f"detect_leaks={int(leaks)}:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    p = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert p.returncode == 0, p.stdout + p.stderr
    return p.stdout


def test_oracle_under_asan_ubsan():
    assert "ok" in run(build("oracle_sanitize"))


def test_host_layer_under_asan_ubsan():
    assert "ok" in run(build("abi_sanitize"))
