"""The C-ABI libraries (no GPU needed): libpirscan.so loads and exports
exactly the functions include/pirscan.h declares; libpirscan_bench.so exports
those and include/pirscan_bench.h's; both reject bad arguments before
touching the device."""
import ctypes
import os
import re

import pytest

from he_database_scan_amd import pirscan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pirscan.h")
BENCH_HEADER = os.path.join(ROOT, "include", "pirscan_bench.h")


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pirscan_[a-z0-9_]+)\s*\(", text)))


def exported_functions(path):
    """Names of the functions a shared library exports (its dynamic symbol
    table), read with the ELF tools' nm."""
    import subprocess

    out = subprocess.run(["nm", "-D", "--defined-only", path], check=True, capture_output=True, text=True).stdout
    return sorted(ln.split()[-1] for ln in out.splitlines() if ln.split()[-2:-1] == ["T"])


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("pirscan_layout_db", "pirscan_rowsel_modgemm", "pirscan_rowsel_workspace_bytes",
                 "pirscan_scalar_gemm_u32", "pirscan_scalar_layout_db", "pirscan_scalar_layout_db_bytes",
                 "pirscan_scalar_tiled_workspace_bytes", "pirscan_scalar_gemm_u32_tiled",
                 "pirscan_scalar_workspace_bytes", "pirscan_layout_db_bytes", "pirscan_strerror",
                 "pirscan_exppack_layout_h", "pirscan_exppack_layout_h_bytes",
                 "pirscan_exppack_workspace_bytes", "pirscan_exppack_modgemm",
                 "pirscan_ntt_plan_bytes", "pirscan_ntt_plan_init", "pirscan_ntt_forward",
                 "pirscan_ntt_inverse", "pirscan_ntt_rns_forward",
                 "pirscan_version", "pirscan_last_device_error"):
        assert want in names
    assert declared_functions(BENCH_HEADER) == ["pirscan_bench_read", "pirscan_kernel_timer_begin",
                                                "pirscan_kernel_timer_end"]
    assert not set(names) & set(declared_functions(BENCH_HEADER))


def test_libraries_export_exactly_their_headers():
    """The product library exports the scan surface only (no benchmark hooks,
    no internal C++ symbols); the benchmark build adds pirscan_bench.h."""
    assert exported_functions(pirscan.LIB_PATH) == declared_functions()
    assert exported_functions(pirscan.BENCH_LIB_PATH) == sorted(declared_functions() +
                                                                declared_functions(BENCH_HEADER))
    L = ctypes.CDLL(pirscan.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name
    assert not hasattr(L, "pirscan_kernel_timer_begin")


def test_struct_layouts_match_the_header():
    # N, R, q[8], D0, D1, scan / N, R, q[8], Dr, n, scan / N, R, q[8], psi[8]
    assert ctypes.sizeof(pirscan.RowselShape) == 4 * 13
    assert ctypes.sizeof(pirscan.ExppackShape) == 4 * 13
    assert ctypes.sizeof(pirscan.NttShape) == 4 * 18
    assert pirscan.RowselShape.scan.offset == 48 and pirscan.ExppackShape.scan.offset == 48


def test_version_and_strerror():
    assert pirscan.version() == 20000
    assert pirscan.bench_library().version() == 20000
    assert pirscan.strerror(0) == "ok"
    assert "invalid" in pirscan.strerror(-1)
    assert "gfx950" in pirscan.strerror(-3)


Q3 = [536813569, 536690689, 536641537]


def test_layout_bytes_and_invalid_shapes():
    s = pirscan.RowselShape.make(4096, Q3, 1024, 1024)
    assert pirscan.layout_db_bytes(s) == 51539607552  # 48 GiB: the packed limbs are exactly the words
    # packed (every q < 2^31, D0 <= 16384): per point ceil(D1/16) column tiles
    # (rounded up to a multiple of 16 from 16 tiles on) x ceil(D0/64) steps x 4 KiB
    assert pirscan.layout_db_bytes(pirscan.RowselShape.make(16, Q3, 65, 17)) == 48 * 2 * 2 * 4096
    assert pirscan.layout_db_bytes(pirscan.RowselShape.make(16, Q3, 65, 240)) == 48 * 15 * 2 * 4096
    assert pirscan.layout_db_bytes(pirscan.RowselShape.make(16, Q3, 65, 300)) == 48 * 32 * 2 * 4096
    assert pirscan.layout_db_bytes(pirscan.RowselShape.make(4, [7], 1, 1)) == 4 * 4096
    # word layout for the VALU scan: a modulus >= 2^31, or D0 > 16384
    assert pirscan.layout_db_bytes(pirscan.RowselShape.make(16, [2147483659], 65, 17)) == 4 * 16 * 65 * 17
    assert pirscan.layout_db_bytes(pirscan.RowselShape.make(4, Q3, 16385, 3)) == 4 * 12 * 16385 * 3
    bad = [pirscan.RowselShape.make(0, Q3, 4, 4), pirscan.RowselShape.make(4, Q3, 0, 4),
           pirscan.RowselShape.make(4, Q3, 4, 0), pirscan.RowselShape.make(4, [1], 4, 4),
           pirscan.RowselShape.make(4, [0, 7], 4, 4)]
    for b in bad:
        assert pirscan.layout_db_bytes(b) == 0
    b = pirscan.RowselShape.make(4, Q3, 4, 4)
    b.R = 9
    assert pirscan.layout_db_bytes(b) == 0
    # the VALU scan on request: the word layout whatever the moduli
    v = pirscan.RowselShape.make(16, Q3, 65, 17, scan=pirscan.SCAN_VALU)
    assert pirscan.layout_db_bytes(v) == 4 * 48 * 65 * 17
    assert pirscan.layout_db_bytes(pirscan.RowselShape.make(4096, Q3, 1024, 1024, scan=pirscan.SCAN_VALU)) == \
        51539607552
    assert pirscan.layout_db_bytes(pirscan.RowselShape.make(16, Q3, 65, 17, scan=2)) == 0   # unknown kind


def test_page_size_identities():
    """Sizes the pages print fix the layout conventions: a ciphertext is m=2
    polynomials x R limbs x N points of 4 bytes (VIPIR 96 KiB / 48 KiB); GPIR's
    a-polynomial is 4N points x 32 bit."""
    sizes = {}
    for line in open(os.path.join(ROOT, "tests", "golden", "page_sizes.txt")):
        if line.strip() and not line.startswith("#"):
            name, val = line.split()[:2]
            sizes[name] = int(val)
    N = 4096
    ct_shape = pirscan.RowselShape.make(N, Q3, 1, 1)      # one DB point set: P = 3N
    assert 2 * ct_shape.P * 4 == sizes["rlwe_ct_rns3_n4096"]   # ct [m=2][D0=1][P]
    assert ct_shape.P * 4 == sizes["poly_rns3_n4096"]
    gp = pirscan.RowselShape.make(N, [536813569] * 4, 1, 1)  # GPIR's 4N points
    assert gp.P * 4 == sizes["gpir_a_poly_4n_n4096"]
    assert 2 * gp.P * 4 == sizes["gpir_ct_4n_n4096"]
    assert (1 << 16) * 4 == sizes["scalar_query_d0_65536"]


def test_rowsel_workspace_sizes():
    s = pirscan.RowselShape.make(4096, Q3, 1024, 1024)
    P = 12288
    # MFMA path: A fragments of the largest pass + output staging.  Up to 16 rows
    # the fragments hold only the live rows (m x 4 limbs x 4 k-groups x 16 bytes
    # per 64-k step: the bytes of ct); beyond, two whole 16-row tiles (8 KiB per step)
    limbs2 = P * 16 * 2 * 4096
    assert pirscan.rowsel_workspace_bytes(s, 2) == P * 16 * 256 * 2 + 4 * P * 2 * 1024
    assert pirscan.rowsel_workspace_bytes(s, 15) == P * 16 * 256 * 15 + 4 * P * 15 * 1024
    assert pirscan.rowsel_workspace_bytes(s, 32) == limbs2 + 4 * P * 32 * 1024
    assert pirscan.rowsel_workspace_bytes(s, 40) == limbs2 + 4 * P * 40 * 1024   # passes of 32 rows
    big_q = pirscan.RowselShape.make(16, [2147483659], 64, 64)  # a modulus >= 2^31: VALU path
    assert pirscan.rowsel_workspace_bytes(big_q, 32) == 4 * 16 * 32 * 64
    assert pirscan.rowsel_workspace_bytes(pirscan.RowselShape.make(16, Q3, 20000, 64), 32) == 4 * 48 * 32 * 64
    assert pirscan.rowsel_workspace_bytes(pirscan.RowselShape.make(1, [7], 1, 1), 1) == 256 + 256
    assert pirscan.rowsel_workspace_bytes(s, 0) == 0
    # the VALU scan on request: the output staging only
    v = pirscan.RowselShape.make(4096, Q3, 1024, 1024, scan=pirscan.SCAN_VALU)
    assert pirscan.rowsel_workspace_bytes(v, 2) == 4 * P * 2 * 1024
    assert pirscan.rowsel_workspace_bytes(v, 32) == 4 * P * 32 * 1024
    # m up to 2^31 (passes of 32 rows stay inside 32 bits); beyond, invalid
    one = pirscan.RowselShape.make(1, [7], 1, 1)
    assert pirscan.rowsel_workspace_bytes(one, 1 << 31) > 0
    assert pirscan.rowsel_workspace_bytes(one, (1 << 31) + 1) == 0
    assert pirscan.rowsel_workspace_bytes(one, 0xFFFFFFF0) == 0


def test_scalar_tiled_sizes_and_validation():
    # groups of 16 row tiles of 16 rows x 64-byte steps of 1 KiB, zero-padded
    assert pirscan.scalar_layout_db_bytes(262144, 262144) == 1 << 36
    assert pirscan.scalar_layout_db_bytes(17, 65) == 16 * 2 * 1024
    assert pirscan.scalar_layout_db_bytes(257, 64) == 2 * 16 * 1024
    assert pirscan.scalar_layout_db_bytes(1, 1) == 16 * 1024
    assert pirscan.scalar_layout_db_bytes(0, 5) == 0 and pirscan.scalar_layout_db_bytes(5, 0) == 0
    # B > 1: the MFMA plan's digit planes of up to 64 columns and split-K
    # partials; B = 1: 4 digit bytes per k (and one 64-k step of zeros) and
    # one partial sum per row for each k-block of 128 steps (8192 k)
    assert pirscan.scalar_tiled_workspace_bytes(262144, 262144, 32) == 262144 * 128
    assert pirscan.scalar_tiled_workspace_bytes(262144, 262144, 1) == (262144 + 64) * 4 + 32 * 262144 * 4
    assert pirscan.scalar_tiled_workspace_bytes(32768, 32768, 1) == (32768 + 64) * 4 + 4 * 32768 * 4
    assert pirscan.scalar_tiled_workspace_bytes(4096, 8192, 1) == (8192 + 64) * 4   # one k-block: no partials
    assert pirscan.scalar_tiled_workspace_bytes(0, 16, 1) == 0
    # more than 64 columns: passes of up to four 128-column groups (2048 digit
    # columns); the hint shape runs unsplit, the second fold in 4 k-blocks with
    # 512-column partials
    assert pirscan.scalar_tiled_workspace_bytes(1 << 20, 1 << 16, 1280) == (1 << 16) * 2048
    assert pirscan.scalar_tiled_workspace_bytes(32768, 1 << 17, 1281) == (1 << 17) * 2048 + 4 * 32768 * 512 * 4
    # one group and a partial one (more than 64 columns left: 256 digit
    # columns, 200-column partials), or one group and a narrow remainder (64 or
    # fewer); 4096 rows split K into 16 k-blocks of 256
    assert pirscan.scalar_tiled_workspace_bytes(4096, 4096, 200) == 4096 * 4 * 256 + 16 * 4096 * 200 * 4
    assert pirscan.scalar_tiled_workspace_bytes(4096, 4096, 150) == 4096 * 4 * 128 + 16 * 4096 * 128 * 4
    L = pirscan.lib()
    A = 1 << 40   # never dereferenced: every call below fails validation first
    vp = ctypes.c_void_p
    # misaligned tiled DB, too small a workspace, overlaps
    assert L.pirscan_scalar_layout_db(vp(A), vp(A + (1 << 30) + 8), 64, 64, None) == pirscan.EINVAL
    assert L.pirscan_scalar_layout_db(vp(A), vp(A + 1024), 64, 64, None) == pirscan.EINVAL
    need = pirscan.scalar_tiled_workspace_bytes(64, 64, 2)
    f = L.pirscan_scalar_gemm_u32_tiled
    assert f(vp(A), vp(A + 8192), vp(A + 16384), 64, 64, 2, vp(A + 32768), need - 1, None) == pirscan.EINVAL
    assert f(vp(A + 8), vp(A + 8192), vp(A + 16384), 64, 64, 2, vp(A + 32768), need, None) == pirscan.EINVAL
    assert f(vp(A), vp(A + 8192), vp(A), 64, 64, 2, vp(A + 32768), need, None) == pirscan.EINVAL


def test_scalar_workspace_sizes():
    # B=1: 4 digit bytes per k (k padded to 4096) + split-K partials
    assert pirscan.scalar_workspace_bytes(32768, 32768, 1) == 32768 * 4 + 8 * 32768 * 4
    assert pirscan.scalar_workspace_bytes(10, 4096, 1) == 4096 * 4          # one k-block: no partials
    # B=8 (one MFMA pass, 16 padded digit columns x 4 planes); K splits into as
    # many blocks as it takes to reach 512 tiles of 256 rows: 128 row tiles -> 4
    assert pirscan.scalar_workspace_bytes(32768, 32768, 8) == 32768 * 64 + 4 * 32768 * 8 * 4
    # enough row tiles: one k-block, no partial sums (the 64 GiB B=32 shape)
    assert pirscan.scalar_workspace_bytes(262144, 262144, 32) == 262144 * 128
    # B=1280: passes of 64 columns, digit planes for one pass
    assert pirscan.scalar_workspace_bytes(1 << 20, 1 << 16, 1280) == (1 << 16) * 256
    assert pirscan.scalar_workspace_bytes(0, 16, 1) == 0
    assert pirscan.scalar_workspace_bytes(5, 17, 1) == 0                    # generic path


def _call_rowsel(shape, m, ct, db, out, ws=0, ws_bytes=0):
    L = pirscan.lib()
    return L.pirscan_rowsel_modgemm(ctypes.byref(shape) if shape is not None else None, m,
                                    ctypes.c_void_p(ct), ctypes.c_void_p(db), ctypes.c_void_p(out),
                                    ctypes.c_void_p(ws), ws_bytes, None)


def test_rowsel_rejects_bad_arguments_without_a_device():
    s = pirscan.RowselShape.make(8, Q3, 4, 4)
    A, B, C, W = 1 << 20, 1 << 30, 1 << 40, 1 << 44  # fake, never dereferenced
    assert _call_rowsel(s, 2, A, B, C) == pirscan.EINVAL                         # no workspace
    small = pirscan.rowsel_workspace_bytes(s, 2)
    assert _call_rowsel(s, 2, A, B, C, W, small - 1) == pirscan.EINVAL
    assert _call_rowsel(None, 2, A, B, C) == pirscan.EINVAL
    assert _call_rowsel(s, 0, A, B, C) == pirscan.EINVAL
    assert _call_rowsel(s, 0xFFFFFFF0, A, B, C) == pirscan.EINVAL              # m past 2^31
    assert _call_rowsel(s, 2, 0, B, C) == pirscan.EINVAL
    assert _call_rowsel(s, 2, A, 0, C) == pirscan.EINVAL
    assert _call_rowsel(s, 2, A, B, 0) == pirscan.EINVAL
    assert _call_rowsel(s, 2, A, B, A + 4) == pirscan.EINVAL      # out overlaps ct
    assert _call_rowsel(s, 2, A, B, B + 64) == pirscan.EINVAL     # out overlaps db
    bad = pirscan.RowselShape.make(8, [1], 4, 4)
    assert _call_rowsel(bad, 2, A, B, C) == pirscan.EINVAL
    # the batched (MFMA) path needs its workspace
    big = pirscan.RowselShape.make(8, Q3, 64, 32)
    need = pirscan.rowsel_workspace_bytes(big, 32)
    W = 1 << 44
    assert need > 0
    assert _call_rowsel(big, 32, A, B, C) == pirscan.EINVAL                     # no workspace
    assert _call_rowsel(big, 32, A, B, C, W, need - 1) == pirscan.EINVAL        # too small
    assert _call_rowsel(big, 32, A, B, C, W + 8, need) == pirscan.EINVAL        # misaligned
    assert _call_rowsel(big, 32, A, B, C, C + 64, need) == pirscan.EINVAL       # overlaps out
    L = pirscan.lib()
    assert L.pirscan_layout_db(ctypes.byref(s), ctypes.c_void_p(A), ctypes.c_void_p(A + 16), None) == pirscan.EINVAL


def test_exppack_sizes():
    # VIPIR section 3.6: N = 2^12, #RNS = 3, Dr = 2^8, n = 1280 -> H is 15 GiB
    s = pirscan.ExppackShape.make(4096, Q3, 256, 1280)
    assert pirscan.exppack_layout_h_bytes(s) == 15 * (1 << 30)
    P = 12288
    limbs2 = P * 20 * 2 * 4096                                    # 20 k-steps of 64, 2 row tiles
    assert pirscan.exppack_workspace_bytes(s, 1) == P * 20 * 256 * 2 + 4 * P * 2 * 256     # m = 2
    assert pirscan.exppack_workspace_bytes(s, 7) == P * 20 * 256 * 14 + 4 * P * 14 * 256   # m = 14
    assert pirscan.exppack_workspace_bytes(s, 16) == limbs2 + 4 * P * 32 * 256
    big = pirscan.ExppackShape.make(4096, [4294967291], 256, 1280)              # VALU: output staging
    assert pirscan.exppack_workspace_bytes(big, 1) == 4 * 4096 * 2 * 256
    assert pirscan.exppack_layout_h_bytes(big) == 4 * 4096 * 256 * 1280
    assert pirscan.exppack_workspace_bytes(s, 0) == 0
    assert pirscan.exppack_workspace_bytes(s, (1 << 30) + 1) == 0            # 2B past 2^31
    sv = pirscan.ExppackShape.make(4096, Q3, 256, 1280, scan=pirscan.SCAN_VALU)
    assert pirscan.exppack_layout_h_bytes(sv) == 15 * (1 << 30)
    assert pirscan.exppack_workspace_bytes(sv, 16) == 4 * P * 32 * 256
    assert pirscan.exppack_layout_h_bytes(pirscan.ExppackShape.make(4096, Q3, 256, 1280, scan=7)) == 0
    for bad in (pirscan.ExppackShape.make(0, Q3, 4, 4), pirscan.ExppackShape.make(4, Q3, 0, 4),
                pirscan.ExppackShape.make(4, Q3, 4, 0), pirscan.ExppackShape.make(4, [1], 4, 4)):
        assert pirscan.exppack_layout_h_bytes(bad) == 0
        assert pirscan.exppack_workspace_bytes(bad, 16) == 0


def test_exppack_rejects_bad_arguments_without_a_device():
    L = pirscan.lib()
    A, H, G, O, W = 1 << 20, 1 << 30, 1 << 36, 1 << 40, 1 << 44
    f = lambda shp, B, c, h, g, o, w=0, wb=0: L.pirscan_exppack_modgemm(
        ctypes.byref(shp) if shp is not None else None, B, ctypes.c_void_p(c), ctypes.c_void_p(h),
        ctypes.c_void_p(g), ctypes.c_void_p(o), ctypes.c_void_p(w), wb, None)
    s = pirscan.ExppackShape.make(8, Q3, 4, 40)
    assert f(None, 1, A, H, G, O) == pirscan.EINVAL
    assert f(s, 0, A, H, G, O) == pirscan.EINVAL
    assert f(s, 1, 0, H, G, O) == pirscan.EINVAL
    assert f(s, 1, A, 0, G, O) == pirscan.EINVAL
    assert f(s, 1, A, H, G, 0) == pirscan.EINVAL
    assert f(s, 1, A, H, G, A + 4) == pirscan.EINVAL            # out overlaps C
    assert f(s, 1, A, H, G, H + 64) == pirscan.EINVAL           # out overlaps H
    assert f(s, 1, A, H, G, G + 8) == pirscan.EINVAL            # out overlaps G
    need = pirscan.exppack_workspace_bytes(s, 8)
    assert need > 0
    assert f(s, 1, A, H, G, O) == pirscan.EINVAL                # every path needs a workspace
    assert f(s, 8, A, H, G, O) == pirscan.EINVAL
    assert f(s, 8, A, H, G, O, W, need - 1) == pirscan.EINVAL
    assert f(s, 8, A, H, G, O, W + 4, need) == pirscan.EINVAL   # misaligned
    assert f(s, 8, A, H, G, O, G, need) == pirscan.EINVAL       # workspace overlaps G
    assert f(s, 1 << 31, A, H, G, O) == pirscan.EINVAL          # 2B overflows
    assert L.pirscan_exppack_layout_h(ctypes.byref(s), ctypes.c_void_p(A), ctypes.c_void_p(A + 16),
                                      None) == pirscan.EINVAL


def test_scalar_rejects_bad_arguments_without_a_device():
    L = pirscan.lib()
    A, B, C, W = 1 << 20, 1 << 30, 1 << 40, 1 << 44
    f = lambda db, q, o, M, K, Bq, w, wb: L.pirscan_scalar_gemm_u32(
        ctypes.c_void_p(db), ctypes.c_void_p(q), ctypes.c_void_p(o), M, K, Bq, ctypes.c_void_p(w), wb, None)
    need = pirscan.scalar_workspace_bytes(64, 8192, 1)
    assert f(0, B, C, 64, 8192, 1, W, need) == pirscan.EINVAL
    assert f(A, B, C, 0, 8192, 1, W, need) == pirscan.EINVAL
    assert f(A, B, C, 64, 8192, 0, W, need) == pirscan.EINVAL
    assert f(A, B, C, 64, 8192, 1, W, need - 1) == pirscan.EINVAL     # workspace too small
    assert f(A, B, C, 64, 8192, 1, 0, need) == pirscan.EINVAL          # no workspace
    assert f(A, B, C, 64, 8192, 1, W + 4, need) == pirscan.EINVAL      # misaligned workspace
    assert f(A, B, A + 8, 64, 8192, 1, W, need) == pirscan.EINVAL      # out overlaps db
    assert f(A, B, C, 64, 8192, 1, B + 16, need) == pirscan.EINVAL     # workspace overlaps query
    assert f(A, B, C, 1 << 40, 1 << 40, 1, W, need) == pirscan.EINVAL  # size overflow


def test_binding_fails_loudly_without_library():
    with pytest.raises(RuntimeError):
        pirscan.Library("/nonexistent/libpirscan.so").version()
    # the benchmark hooks exist in the benchmark build only
    with pytest.raises(RuntimeError):
        pirscan.Library(pirscan.LIB_PATH).kernel_timer_begin(1)


def test_kernel_timer_argument_checks():
    L = pirscan.bench_library().lib()
    assert L.pirscan_kernel_timer_begin(0) == pirscan.EINVAL
    assert L.pirscan_kernel_timer_begin((1 << 20) + 1) == pirscan.EINVAL
    n = ctypes.c_uint32(7)
    assert L.pirscan_kernel_timer_end(None, 0, ctypes.byref(n)) == pirscan.EINVAL   # not begun


def test_bench_read_argument_checks():
    """The read-stream reference validates before touching a device."""
    L = pirscan.bench_library().lib()
    vp = ctypes.c_void_p
    buf, sink = vp(1 << 20), vp(1 << 21)   # never dereferenced: every call below is rejected first
    assert L.pirscan_bench_read(None, 4096, sink, None) == pirscan.EINVAL
    assert L.pirscan_bench_read(buf, 4096, None, None) == pirscan.EINVAL
    assert L.pirscan_bench_read(buf, 0, sink, None) == pirscan.EINVAL
    assert L.pirscan_bench_read(buf, 4100, sink, None) == pirscan.EINVAL
    assert L.pirscan_bench_read(vp((1 << 20) + 4), 4096, sink, None) == pirscan.EINVAL


# primitive 2N-th roots of unity (N = 4096) for the three 29-bit primes: each
# satisfies psi^N == -1 (mod q), checked here with Python's pow
PSI3 = [327210582, 176946644, 321217896]


def test_ntt_shape_validation_without_a_device():
    for q, w in zip(Q3, PSI3):
        assert pow(w, 4096, q) == q - 1
    s = pirscan.NttShape.make(4096, Q3, PSI3)
    assert pirscan.ntt_plan_bytes(s) == 16 * 3 * 4096
    import oracle

    big_q = oracle.ntt_primes(31, 8192, 1)[0]  # a valid NTT prime above 2^30
    big_psi = oracle.psi(big_q, 4096)
    assert big_q > (1 << 30) and pow(big_psi, 4096, big_q) == big_q - 1
    comp = 8193 * 8193                       # == 1 mod 8192, composite, < 2^30
    assert comp % 8192 == 1 and comp < (1 << 30)
    bad = [pirscan.NttShape.make(4096, Q3, [PSI3[0], PSI3[1], pow(PSI3[2], 2, Q3[2])]),  # psi^N = 1
           pirscan.NttShape.make(4096, Q3, [0, PSI3[1], PSI3[2]]),
           pirscan.NttShape.make(4096, [Q3[0], Q3[1], Q3[2] + 1], PSI3),                  # even modulus
           pirscan.NttShape.make(4096, [comp], [1]),                                        # composite
           pirscan.NttShape.make(4096, [1073738753], [536638208]),                          # 1 mod 512 only
           pirscan.NttShape.make(4096, [big_q], [big_psi]),                                 # >= 2^30
           pirscan.NttShape.make(3000, Q3, PSI3), pirscan.NttShape.make(8, Q3, PSI3),
           pirscan.NttShape.make(16384, Q3, PSI3)]
    for b in bad:
        assert pirscan.ntt_plan_bytes(b) == 0
    b = pirscan.NttShape.make(4096, Q3, PSI3)
    b.R = 0
    assert pirscan.ntt_plan_bytes(b) == 0
    b.R = 9
    assert pirscan.ntt_plan_bytes(b) == 0


def test_ntt_rejects_bad_arguments_without_a_device():
    L = pirscan.lib()
    s = pirscan.NttShape.make(4096, Q3, PSI3)
    A, O, PL = 1 << 30, 1 << 40, 1 << 44
    row = 3 * 4096 * 4                        # bytes of one polynomial (3 limbs)
    fwd = lambda i, o, c, plan=PL: L.pirscan_ntt_forward(ctypes.byref(s), ctypes.c_void_p(plan),
                                                         ctypes.c_void_p(i), ctypes.c_void_p(o), c, None)
    rns = lambda i, o, c, plan=PL: L.pirscan_ntt_rns_forward(ctypes.byref(s), ctypes.c_void_p(plan),
                                                             ctypes.c_void_p(i), ctypes.c_void_p(o), c, None)
    assert fwd(A, O, 0) == pirscan.EINVAL                 # zero polynomials
    assert fwd(0, O, 1) == pirscan.EINVAL
    assert fwd(A, 0, 1) == pirscan.EINVAL
    assert fwd(A, O, 1, plan=0) == pirscan.EINVAL
    assert fwd(A, O, 1, plan=PL + 8) == pirscan.EINVAL    # misaligned plan
    assert fwd(A, A + 4, 2) == pirscan.EINVAL             # partial overlap
    assert fwd(A, A + row, 2) == pirscan.EINVAL           # rows shifted by one: still overlapping
    assert fwd(A, O, 1, plan=O + 64) == pirscan.EINVAL    # plan inside out
    assert rns(A, A, 1) == pirscan.EINVAL                 # the fused form is never in place
    assert fwd(A, O, 1 << 62) == pirscan.EINVAL           # size overflow
    assert L.pirscan_ntt_plan_init(ctypes.byref(s), ctypes.c_void_p(PL), 16 * 3 * 4096 - 1, None) == \
        pirscan.EINVAL                                     # short plan
    assert L.pirscan_ntt_plan_init(ctypes.byref(s), ctypes.c_void_p(0), 1 << 20, None) == pirscan.EINVAL


def test_noalloc_entry_point_limits_without_a_device():
    """The no-allocation scalar product refuses, before touching a device,
    problems whose scratch exceeds its built-in buffer, and bad arguments."""
    L = pirscan.lib()
    vp = ctypes.c_void_p
    A, Q, O = vp(1 << 40), vp(1 << 44), vp(1 << 45)   # never dereferenced
    f = L.pirscan_scalar_gemm_u32_noalloc
    assert pirscan.scalar_workspace_bytes(1 << 19, 1 << 18, 1) > pirscan.NOALLOC_SCRATCH_BYTES
    assert f(A, Q, O, 1 << 19, 1 << 18, 1, None) == pirscan.ESCRATCH
    assert f(None, Q, O, 64, 4096, 1, None) == pirscan.EINVAL
    assert f(A, Q, O, 0, 4096, 1, None) == pirscan.EINVAL
    assert f(A, Q, vp((1 << 40) + 8), 64, 4096, 1, None) == pirscan.EINVAL   # out overlaps db
    assert "scratch" in pirscan.strerror(pirscan.ESCRATCH)
