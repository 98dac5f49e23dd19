/* Runs every oracle function on small and edge shapes, for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer (the sanitizers report any
 * out-of-bounds access, leak or undefined operation and stop the run).  The
 * values are checked only loosely here -- the pins in tests/test_oracle_*.py
 * check them -- except for a few closed forms stated beside each call. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "oracle.h"

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) { /* xorshift64*: a throwaway input generator */
  state ^= state >> 12;
  state ^= state << 25;
  state ^= state >> 27;
  return (uint32_t)((state * 0x2545F4914F6CDD1Dull) >> 32);
}

static uint32_t *residues(size_t n, const uint32_t *q, uint32_t N, uint32_t P) {
  uint32_t *a = malloc(sizeof(uint32_t) * (n ? n : 1));
  for (size_t i = 0; i < n; ++i) a[i] = next_u32() % q[(i % P) / N];
  return a;
}

static int fail(const char *what) {
  printf("FAIL %s\n", what);
  return 1;
}

int main(void) {
  int bad = 0;
  /* RowSel over several shapes and thread counts, including one point and D0 = 1 */
  const uint32_t shapes[][5] = {{1, 1, 1, 1, 1}, {4, 2, 3, 17, 5}, {8, 3, 2, 65, 9}, {3, 1, 34, 7, 3}};
  const uint32_t q3[3] = {536813569u, 4294967291u, 2u};
  for (size_t s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s) {
    const uint32_t N = shapes[s][0], R = shapes[s][1], m = shapes[s][2], D0 = shapes[s][3], D1 = shapes[s][4];
    const uint32_t P = N * R;
    uint32_t *ct = residues((size_t)m * D0 * P, q3, N, P), *db = residues((size_t)D0 * D1 * P, q3, N, P);
    uint32_t *out = malloc(sizeof(uint32_t) * m * D1 * P);
    for (int th = 0; th <= 5; th += 5)
      if (oracle_rowsel(ct, db, out, N, R, q3, m, D0, D1, th) != 0) bad |= fail("rowsel");
    /* all (q-1): every output is D0 mod q */
    for (size_t i = 0; i < (size_t)m * D0 * P; ++i) ct[i] = q3[(i % P) / N] - 1;
    for (size_t i = 0; i < (size_t)D0 * D1 * P; ++i) db[i] = q3[(i % P) / N] - 1;
    oracle_rowsel(ct, db, out, N, R, q3, m, D0, D1, 3);
    for (size_t i = 0; i < (size_t)m * D1 * P; ++i)
      if (out[i] != D0 % q3[(i % P) / N]) bad |= fail("rowsel closed form");
    /* ExpPack with the same operands: Dr = D1 rows, n = D0, B = max(1, m / 2) */
    const uint32_t B = m / 2 ? m / 2 : 1;
    uint32_t *H = residues((size_t)D1 * D0 * P, q3, N, P), *C = residues((size_t)D0 * 2 * B * P, q3, N, P);
    uint32_t *G = residues((size_t)D1 * B * P, q3, N, P), *o2 = malloc(sizeof(uint32_t) * D1 * 2 * B * P);
    if (oracle_exppack(H, C, G, o2, N, R, q3, D1, D0, B, 4) != 0) bad |= fail("exppack");
    if (oracle_exppack(H, C, NULL, o2, N, R, q3, D1, D0, B, 1) != 0) bad |= fail("exppack no G");
    free(ct), free(db), free(out), free(H), free(C), free(G), free(o2);
  }
  /* scalar product: B = 1 (register sum) and B > 1, rows fewer than threads */
  for (uint32_t B = 1; B <= 5; B += 4) {
    const uint64_t M = 3, K = 37;
    int8_t *db = malloc(M * K);
    uint32_t *Q = malloc(sizeof(uint32_t) * K * B), *out = malloc(sizeof(uint32_t) * M * B);
    for (uint64_t i = 0; i < M * K; ++i) db[i] = (int8_t)-128;
    for (uint64_t i = 0; i < K * B; ++i) Q[i] = 0xFFFFFFFFu;
    if (oracle_scalar(db, Q, out, M, K, B, 8) != 0) bad |= fail("scalar");
    for (uint64_t i = 0; i < M * B; ++i)
      if (out[i] != (uint32_t)(128 * K)) bad |= fail("scalar closed form");
    free(db), free(Q), free(out);
  }
  /* digit split and number theory */
  int8_t d[4];
  const uint32_t words[] = {0u, 0x80u, 0xFFu, 0x80808080u, 0x7F7F7F7Fu, 0xFFFFFFFFu, 0x12345678u};
  for (size_t i = 0; i < sizeof(words) / sizeof(words[0]); ++i) oracle_signed_digits(words[i], d);
  int8_t ds[4 * 7];
  oracle_signed_digits_batch(words, ds, 7);
  uint32_t primes[3];
  if (oracle_ntt_primes(29, 8192, 3, primes) != 3 || primes[0] != 536813569u) bad |= fail("primes");
  if (oracle_ntt_primes(32, 2, 2, primes) != 2) bad |= fail("primes near 2^32");
  for (uint32_t n = 0; n < 200; ++n) (void)oracle_is_prime_u32(n);
  (void)oracle_is_prime_u32(4294967291u);
  (void)oracle_primitive_root(4294967291u);
  /* NTT: single, batched, RNS-decomposed, inverse, schoolbook product */
  const uint32_t N = 16, qn[2] = {7681u, 12289u};
  uint32_t psi[2];
  for (int r = 0; r < 2; ++r) psi[r] = oracle_psi(qn[r], N);
  uint32_t a[16], A[16], back[16], c[16];
  for (uint32_t i = 0; i < N; ++i) a[i] = next_u32() % qn[0];
  oracle_ntt(a, A, N, qn[0], psi[0]);
  oracle_intt(A, back, N, qn[0], psi[0]);
  for (uint32_t i = 0; i < N; ++i)
    if (back[i] != a[i]) bad |= fail("intt(ntt)");
  oracle_negacyclic_mul(a, a, c, N, qn[0]);
  uint32_t coef[3 * 16], res[3 * 2 * 16], inv[3 * 2 * 16];
  for (int i = 0; i < 3 * 16; ++i) coef[i] = next_u32();
  if (oracle_ntt_rns(coef, res, 3, N, 2, qn, psi, 2) != 0) bad |= fail("ntt_rns");
  if (oracle_ntt_batch(res, inv, 3, N, 2, qn, psi, 1, 7) != 0) bad |= fail("ntt_batch inverse");
  if (oracle_ntt_batch(inv, res, 3, N, 2, qn, psi, 0, 1) != 0) bad |= fail("ntt_batch forward");
  printf(bad ? "oracle sanitizer run: FAILED\n" : "oracle sanitizer run: ok\n");
  return bad;
}
