/* Drives libpirscan's host layer -- argument validation, size queries,
 * overlap and overflow checks -- in a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer on the host code.  Runs without a GPU: every
 * call either fails validation before any device work (PIRSCAN_EINVAL /
 * PIRSCAN_ESCRATCH, fake pointers never dereferenced) or stops at the
 * device check (PIRSCAN_EDEVICE when no device is present). */
#include <stdint.h>
#include <stdio.h>

#include "pirscan.h"

#define FAKE(x) ((void*)(uintptr_t)(x))

static int bad = 0;
static void expect(int cond, const char* what) {
  if (!cond) {
    printf("FAIL %s\n", what);
    bad = 1;
  }
}

int main(void) {
  const uint32_t q3[3] = {536813569u, 536690689u, 536641537u};
  pirscan_rowsel_shape s = {4096, 3, {0}, 1024, 1024, PIRSCAN_SCAN_AUTO};
  for (int r = 0; r < 3; ++r) s.q[r] = q3[r];
  expect(pirscan_layout_db_bytes(&s) == 51539607552ull, "48 GiB layout bytes");
  s.scan = PIRSCAN_SCAN_VALU;
  expect(pirscan_layout_db_bytes(&s) == 51539607552ull, "48 GiB word layout");
  expect(pirscan_rowsel_workspace_bytes(&s, 32) == 4ull * 12288 * 32 * 1024, "VALU workspace");
  s.scan = 9;
  expect(pirscan_layout_db_bytes(&s) == 0, "unknown scan kind");
  s.scan = PIRSCAN_SCAN_AUTO;
  expect(pirscan_rowsel_workspace_bytes(&s, 0) == 0, "m = 0");
  expect(pirscan_rowsel_workspace_bytes(&s, 0xFFFFFFF0u) == 0, "m past 2^31");
  pirscan_rowsel_shape huge = {0xFFFFFFFFu, 8, {0}, 0xFFFFFFFFu, 0xFFFFFFFFu, 0};
  for (int r = 0; r < 8; ++r) huge.q[r] = 7;
  expect(pirscan_layout_db_bytes(&huge) == 0, "size overflow");
  expect(pirscan_layout_db_bytes(NULL) == 0, "null shape");
  /* bad arguments: rejected before touching the device */
  const size_t ws = pirscan_rowsel_workspace_bytes(&s, 2);
  expect(pirscan_rowsel_modgemm(&s, 2, FAKE(1ull << 20), FAKE(1ull << 30), FAKE(1ull << 20), FAKE(1ull << 44), ws,
                                NULL) == PIRSCAN_EINVAL, "out overlaps ct");
  expect(pirscan_rowsel_modgemm(&s, 2, FAKE(1ull << 20), FAKE(1ull << 36), FAKE(1ull << 42), FAKE(1ull << 44),
                                ws - 1, NULL) == PIRSCAN_EINVAL, "short workspace");
  expect(pirscan_layout_db(&s, FAKE(1ull << 20), FAKE((1ull << 20) + 16), NULL) == PIRSCAN_EINVAL, "layout overlap");
  pirscan_exppack_shape e = {4096, 3, {0}, 256, 1280, PIRSCAN_SCAN_AUTO};
  for (int r = 0; r < 3; ++r) e.q[r] = q3[r];
  expect(pirscan_exppack_layout_h_bytes(&e) == 15ull << 30, "15 GiB hint");
  expect(pirscan_exppack_workspace_bytes(&e, (1u << 30) + 1) == 0, "2B past 2^31");
  expect(pirscan_exppack_modgemm(&e, 1, FAKE(1ull << 20), FAKE(1ull << 36), FAKE(1ull << 38), FAKE(1ull << 20),
                                 FAKE(1ull << 44), 1u << 30, NULL) == PIRSCAN_EINVAL, "exppack overlap");
  /* scalar: sizes, validation, the no-allocation limit */
  expect(pirscan_scalar_workspace_bytes(262144, 262144, 32) == 262144ull * 128, "scalar B=32 workspace");
  expect(pirscan_scalar_tiled_workspace_bytes(0, 16, 1) == 0, "zero rows");
  expect(pirscan_scalar_layout_db_bytes(1ull << 40, 1ull << 40) == 0, "scalar size overflow");
  expect(pirscan_scalar_gemm_u32(FAKE(1ull << 20), FAKE(1ull << 30), FAKE((1ull << 20) + 8), 64, 8192, 1,
                                 FAKE(1ull << 44), 1 << 20, NULL) == PIRSCAN_EINVAL, "scalar out overlaps db");
  expect(pirscan_scalar_gemm_u32_noalloc(FAKE(1ull << 40), FAKE(1ull << 44), FAKE(1ull << 45), 1ull << 19,
                                         1ull << 18, 1, NULL) == PIRSCAN_ESCRATCH, "no-allocation limit");
  expect(pirscan_scalar_gemm_u32_tiled(FAKE((1ull << 20) + 8), FAKE(1ull << 30), FAKE(1ull << 40), 64, 64, 2,
                                       FAKE(1ull << 44), 1 << 20, NULL) == PIRSCAN_EINVAL, "misaligned tiled DB");
  /* NTT shapes */
  pirscan_ntt_shape n = {4096, 3, {0}, {327210582u, 176946644u, 321217896u, 0, 0, 0, 0, 0}};
  for (int r = 0; r < 3; ++r) n.q[r] = q3[r];
  expect(pirscan_ntt_plan_bytes(&n) == 16ull * 3 * 4096, "plan bytes");
  n.psi[0] = 1;
  expect(pirscan_ntt_plan_bytes(&n) == 0, "bad psi");
  expect(pirscan_ntt_forward(&n, FAKE(1ull << 44), FAKE(1ull << 30), FAKE(1ull << 40), 1, NULL) == PIRSCAN_EINVAL,
         "invalid NTT shape");
  /* a valid call reaches the device check: no device here, or a device */
  const int st = pirscan_scalar_gemm_u32(FAKE(1ull << 20), FAKE(1ull << 30), FAKE(1ull << 40), 64, 64, 5, NULL, 0,
                                         NULL);  /* K = 64: the MFMA plan needs a workspace -> EINVAL */
  expect(st == PIRSCAN_EINVAL, "missing workspace");
  for (int c = 1; c >= -5; --c) (void)pirscan_strerror(c);
  expect(pirscan_version() == PIRSCAN_VERSION, "version");
  printf(bad ? "host layer sanitizer run: FAILED\n" : "host layer sanitizer run: ok\n");
  return bad;
}
