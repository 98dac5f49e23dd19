/*
 * oracle.c -- plain CPU definitions of the PIR database-multiplication scan.
 * TEST INFRASTRUCTURE ONLY: see oracle.h for who may use it and for the
 * passages of the pages each function restates.
 *
 * Style rule for this file: each function is the definition written out as
 * loops.  Every output is its own exact sum, taken over the summed index in
 * the pages' order (k, i) and reduced once; only the order in which the
 * independent outputs are visited is chosen, so that the contiguous index of
 * each array runs innermost.  Threads split only the outermost independent
 * index (points for RowSel and ExpPack, rows for the scalar product); they
 * never change the order or the exactness of any sum.
 */
#include "oracle.h"

#include <pthread.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef unsigned __int128 u128;

int oracle_default_threads(void) {
  long n = sysconf(_SC_NPROCESSORS_ONLN);
  if (n < 1) n = 1;
  if (n > 256) n = 256;
  return (int)n;
}

static int clamp_threads(int nthreads, uint64_t work_items) {
  if (nthreads <= 0) nthreads = oracle_default_threads();
  if ((uint64_t)nthreads > work_items) nthreads = (int)(work_items ? work_items : 1);
  return nthreads;
}

/* Runs worker(job t) on thread t (job 0 on the calling thread) and joins
 * them; -1 if a thread could not start or a worker reported failure. */
static int run_workers(pthread_t *th, int nthreads, void *(*worker)(void *), void *jobs, size_t job_size) {
  char *base = (char *)jobs;
  int rc = 0, started = 1;
  for (int t = 1; t < nthreads; ++t) {
    if (pthread_create(&th[t], NULL, worker, base + (size_t)t * job_size) != 0) { rc = -1; break; }
    ++started;
  }
  if (worker(base) != NULL) rc = -1;
  for (int t = 1; t < started; ++t) {
    void *ret = NULL;
    pthread_join(th[t], &ret);
    if (ret != NULL) rc = -1;
  }
  return rc;
}

/* ------------------------------------------------------------------------ */
/* RowSel                                                                   */
/* ------------------------------------------------------------------------ */

typedef struct {
  const uint32_t *ct, *db;
  uint32_t *out;
  uint32_t N, m, D0, D1;
  uint64_t P;
  const uint32_t *q;
  uint64_t p_begin, p_end;
} rowsel_job;

static void *rowsel_worker(void *arg) {
  const rowsel_job *j = (const rowsel_job *)arg;
  const uint64_t P = j->P, np = j->p_end - j->p_begin;
  /* One exact 128-bit sum per output.  The free indices run n outermost and
   * p innermost (the contiguous index of the p-major arrays), so every DB word
   * is read once; each sum still takes k = 0 .. D0-1 in order. */
  u128 *acc = (u128 *)malloc(sizeof(u128) * ((uint64_t)j->m * np + 1));
  if (!acc) return (void *)1;
  for (uint32_t n = 0; n < j->D1; ++n) {
    for (uint64_t t = 0; t < (uint64_t)j->m * np; ++t) acc[t] = 0;
    for (uint32_t k = 0; k < j->D0; ++k) {
      const uint32_t *b = j->db + ((uint64_t)k * j->D1 + n) * P + j->p_begin;
      for (uint32_t mi = 0; mi < j->m; ++mi) {
        const uint32_t *a = j->ct + ((uint64_t)mi * j->D0 + k) * P + j->p_begin;
        u128 *s = acc + (uint64_t)mi * np;
        for (uint64_t t = 0; t < np; ++t) s[t] += (u128)((uint64_t)a[t] * b[t]);
      }
    }
    for (uint32_t mi = 0; mi < j->m; ++mi) {
      uint32_t *o = j->out + ((uint64_t)mi * j->D1 + n) * P;
      for (uint64_t t = 0; t < np; ++t) {
        const uint64_t p = j->p_begin + t;
        o[p] = (uint32_t)(acc[(uint64_t)mi * np + t] % j->q[p / j->N]);
      }
    }
  }
  free(acc);
  return NULL;
}

int oracle_rowsel(const uint32_t *ct, const uint32_t *db, uint32_t *out,
                  uint32_t N, uint32_t R, const uint32_t *q,
                  uint32_t m, uint32_t D0, uint32_t D1, int nthreads) {
  if (!ct || !db || !out || !q || N == 0 || R == 0) return -1;
  for (uint32_t r = 0; r < R; ++r)
    if (q[r] == 0) return -1;
  const uint64_t P = (uint64_t)R * N;
  nthreads = clamp_threads(nthreads, P);
  pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
  rowsel_job *jobs = (rowsel_job *)calloc((size_t)nthreads, sizeof(rowsel_job));
  if (!th || !jobs) { free(th); free(jobs); return -1; }
  for (int t = 0; t < nthreads; ++t) {
    rowsel_job *j = &jobs[t];
    j->ct = ct; j->db = db; j->out = out;
    j->N = N; j->m = m; j->D0 = D0; j->D1 = D1; j->P = P; j->q = q;
    j->p_begin = P * (uint64_t)t / (uint64_t)nthreads;
    j->p_end = P * (uint64_t)(t + 1) / (uint64_t)nthreads;
  }
  int rc = run_workers(th, nthreads, rowsel_worker, jobs, sizeof(rowsel_job));
  free(th);
  free(jobs);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* ExpPack packing GEMM H*C + (0|G)                                          */
/* ------------------------------------------------------------------------ */

typedef struct {
  const uint32_t *H, *C, *G;
  uint32_t *out;
  uint32_t N, Dr, n, B;
  uint64_t P;
  const uint32_t *q;
  uint64_t p_begin, p_end;
} exppack_job;

static void *exppack_worker(void *arg) {
  const exppack_job *j = (const exppack_job *)arg;
  const uint64_t P = j->P, cols = 2ull * j->B, np = j->p_end - j->p_begin;
  /* One exact 128-bit sum per output.  The free indices run r outermost and
   * p innermost (the contiguous index of the p-major arrays), so every hint
   * word is read once; each sum still takes i = 0 .. n-1 in order. */
  u128 *acc = (u128 *)malloc(sizeof(u128) * (cols * np + 1));
  if (!acc) return (void *)1;
  for (uint32_t r = 0; r < j->Dr; ++r) {
    for (uint64_t t = 0; t < cols * np; ++t) acc[t] = 0;
    for (uint32_t i = 0; i < j->n; ++i) {
      const uint32_t *h = j->H + ((uint64_t)r * j->n + i) * P + j->p_begin;
      for (uint64_t c = 0; c < cols; ++c) {
        const uint32_t *x = j->C + ((uint64_t)i * cols + c) * P + j->p_begin;
        u128 *s = acc + c * np;
        for (uint64_t t = 0; t < np; ++t) s[t] += (u128)((uint64_t)h[t] * x[t]);
      }
    }
    for (uint64_t c = 0; c < cols; ++c) {
      uint32_t *o = j->out + ((uint64_t)r * cols + c) * P;
      for (uint64_t t = 0; t < np; ++t) {
        const uint64_t p = j->p_begin + t;
        u128 v = acc[c * np + t];
        /* (0 | G): the second column of client c/2 carries G */
        if (j->G && (c & 1)) v += j->G[((uint64_t)r * j->B + c / 2) * P + p];
        o[p] = (uint32_t)(v % j->q[p / j->N]);
      }
    }
  }
  free(acc);
  return NULL;
}

int oracle_exppack(const uint32_t *H, const uint32_t *C, const uint32_t *G,
                   uint32_t *out, uint32_t N, uint32_t R, const uint32_t *q,
                   uint32_t Dr, uint32_t n, uint32_t B, int nthreads) {
  if (!H || !C || !out || !q || N == 0 || R == 0) return -1;
  for (uint32_t r = 0; r < R; ++r)
    if (q[r] == 0) return -1;
  const uint64_t P = (uint64_t)R * N;
  nthreads = clamp_threads(nthreads, P);
  pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
  exppack_job *jobs = (exppack_job *)calloc((size_t)nthreads, sizeof(exppack_job));
  if (!th || !jobs) { free(th); free(jobs); return -1; }
  for (int t = 0; t < nthreads; ++t) {
    exppack_job *j = &jobs[t];
    j->H = H; j->C = C; j->G = G; j->out = out;
    j->N = N; j->Dr = Dr; j->n = n; j->B = B; j->P = P; j->q = q;
    j->p_begin = P * (uint64_t)t / (uint64_t)nthreads;
    j->p_end = P * (uint64_t)(t + 1) / (uint64_t)nthreads;
  }
  int rc = run_workers(th, nthreads, exppack_worker, jobs, sizeof(exppack_job));
  free(th);
  free(jobs);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Scalar-HE product mod 2^32                                               */
/* ------------------------------------------------------------------------ */

typedef struct {
  const int8_t *db;
  const uint32_t *Q;
  uint32_t *out;
  uint64_t K;
  uint32_t B;
  uint64_t i_begin, i_end;
} scalar_job;

static void *scalar_worker(void *arg) {
  const scalar_job *j = (const scalar_job *)arg;
  /* One uint32 sum per output, wrapping mod 2^32.  For each row the free index
   * b runs innermost (the contiguous index of Q); each sum still takes
   * k = 0 .. K-1 in order. */
  uint32_t *acc = (uint32_t *)malloc(sizeof(uint32_t) * ((uint64_t)j->B + 1));
  if (!acc) return (void *)1;
  for (uint64_t i = j->i_begin; i < j->i_end; ++i) {
    if (j->B == 1) { /* a single column: the sum stays in a register */
      uint32_t s = 0;
      for (uint64_t k = 0; k < j->K; ++k) s += (uint32_t)(int32_t)j->db[i * j->K + k] * j->Q[k];
      j->out[i] = s;
      continue;
    }
    for (uint32_t b = 0; b < j->B; ++b) acc[b] = 0;
    for (uint64_t k = 0; k < j->K; ++k) {
      const uint32_t d = (uint32_t)(int32_t)j->db[i * j->K + k]; /* sign-extend */
      const uint32_t *qk = j->Q + k * j->B;
      for (uint32_t b = 0; b < j->B; ++b) acc[b] += d * qk[b];  /* wraps mod 2^32 */
    }
    for (uint32_t b = 0; b < j->B; ++b) j->out[i * j->B + b] = acc[b];
  }
  free(acc);
  return NULL;
}

int oracle_scalar(const int8_t *db, const uint32_t *Q, uint32_t *out,
                  uint64_t M, uint64_t K, uint32_t B, int nthreads) {
  if (!db || !Q || !out) return -1;
  nthreads = clamp_threads(nthreads, M);
  pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
  scalar_job *jobs = (scalar_job *)calloc((size_t)nthreads, sizeof(scalar_job));
  if (!th || !jobs) { free(th); free(jobs); return -1; }
  for (int t = 0; t < nthreads; ++t) {
    scalar_job *j = &jobs[t];
    j->db = db; j->Q = Q; j->out = out; j->K = K; j->B = B;
    j->i_begin = M * (uint64_t)t / (uint64_t)nthreads;
    j->i_end = M * (uint64_t)(t + 1) / (uint64_t)nthreads;
  }
  int rc = run_workers(th, nthreads, scalar_worker, jobs, sizeof(scalar_job));
  free(th);
  free(jobs);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Signed-digit split                                                       */
/* ------------------------------------------------------------------------ */

void oracle_signed_digits(uint32_t x, int8_t s[4]) {
  uint32_t carry = 0;
  for (int j = 0; j < 4; ++j) {
    const uint32_t t = ((x >> (8 * j)) & 0xFFu) + carry; /* 0 .. 256 */
    if (t >= 128) {
      s[j] = (int8_t)((int32_t)t - 256);
      carry = 1;
    } else {
      s[j] = (int8_t)t;
      carry = 0;
    }
  }
  /* the final carry is 2^32, which vanishes modulo 2^32 */
}

void oracle_signed_digits_batch(const uint32_t *x, int8_t *s, uint64_t n) {
  for (uint64_t i = 0; i < n; ++i) oracle_signed_digits(x[i], s + 4 * i);
}

/* ------------------------------------------------------------------------ */
/* Number theory (used by the tests that pin the oracle)                    */
/* ------------------------------------------------------------------------ */

static uint32_t mulmod(uint32_t a, uint32_t b, uint32_t q) {
  return (uint32_t)(((uint64_t)a * b) % q);
}

uint32_t oracle_powmod(uint32_t a, uint64_t e, uint32_t q) {
  uint32_t r = 1 % q, base = a % q;
  while (e) {
    if (e & 1) r = mulmod(r, base, q);
    base = mulmod(base, base, q);
    e >>= 1;
  }
  return r;
}

static int mr_witness(uint32_t n, uint32_t a) {
  /* returns 1 if a proves n composite */
  uint32_t d = n - 1;
  int s = 0;
  while ((d & 1) == 0) { d >>= 1; ++s; }
  uint32_t x = oracle_powmod(a % n, d, n);
  if (x == 1 || x == n - 1) return 0;
  for (int r = 1; r < s; ++r) {
    x = mulmod(x, x, n);
    if (x == n - 1) return 0;
  }
  return 1;
}

int oracle_is_prime_u32(uint32_t n) {
  if (n < 2) return 0;
  static const uint32_t small[] = {2, 3, 5, 7, 11, 13, 17, 19, 23, 29, 31, 37, 41, 43, 47, 53, 59, 61};
  for (size_t i = 0; i < sizeof(small) / sizeof(small[0]); ++i) {
    if (n == small[i]) return 1;
    if (n % small[i] == 0) return 0;
  }
  static const uint32_t bases[] = {2, 7, 61};
  for (size_t i = 0; i < 3; ++i)
    if (mr_witness(n, bases[i])) return 0;
  return 1;
}

int oracle_ntt_primes(uint32_t bits, uint32_t two_n, int count, uint32_t *out) {
  if (bits < 2 || bits > 32 || two_n == 0) return 0;
  const uint64_t limit = (uint64_t)1 << bits; /* q < limit */
  /* largest candidate q = t*two_n + 1 < limit */
  uint64_t t = (limit - 2) / two_n;
  int found = 0;
  for (; found < count; --t) {
    const uint64_t cand = t * two_n + 1;
    if (cand < 2) break;
    if (oracle_is_prime_u32((uint32_t)cand)) out[found++] = (uint32_t)cand;
    if (t == 0) break;
  }
  return found;
}

uint32_t oracle_primitive_root(uint32_t q) {
  /* distinct prime factors of q-1 by trial division */
  uint32_t f[32];
  int nf = 0;
  uint32_t r = q - 1;
  for (uint32_t d = 2; (uint64_t)d * d <= r; ++d) {
    if (r % d == 0) {
      f[nf++] = d;
      while (r % d == 0) r /= d;
    }
  }
  if (r > 1) f[nf++] = r;
  for (uint32_t g = 2; g < q; ++g) {
    int ok = 1;
    for (int i = 0; i < nf && ok; ++i)
      if (oracle_powmod(g, (q - 1) / f[i], q) == 1) ok = 0;
    if (ok) return g;
  }
  return 0;
}

uint32_t oracle_psi(uint32_t q, uint32_t N) {
  const uint32_t g = oracle_primitive_root(q);
  return oracle_powmod(g, (q - 1) / (2ull * N), q);
}

void oracle_ntt(const uint32_t *a, uint32_t *A, uint32_t N, uint32_t q,
                uint32_t psi) {
  for (uint32_t j = 0; j < N; ++j) {
    const uint32_t w = oracle_powmod(psi, 2ull * j + 1, q); /* psi^(2j+1) */
    uint64_t acc = 0;
    uint32_t wi = 1; /* w^i */
    for (uint32_t i = 0; i < N; ++i) {
      acc = (acc + mulmod(a[i] % q, wi, q)) % q;
      wi = mulmod(wi, w, q);
    }
    A[j] = (uint32_t)acc;
  }
}

void oracle_intt(const uint32_t *A, uint32_t *a, uint32_t N, uint32_t q,
                 uint32_t psi) {
  const uint32_t psi_inv = oracle_powmod(psi, q - 2, q);
  const uint32_t n_inv = oracle_powmod(N % q, q - 2, q);
  for (uint32_t i = 0; i < N; ++i) {
    /* e_j = psi^-((2j+1) i): e_0 = psi^-i, e_{j+1} = e_j * psi^-2i */
    const uint32_t step = oracle_powmod(psi_inv, 2ull * i, q);
    uint32_t e = oracle_powmod(psi_inv, i, q);
    uint64_t acc = 0;
    for (uint32_t j = 0; j < N; ++j) {
      acc = (acc + mulmod(A[j] % q, e, q)) % q;
      e = mulmod(e, step, q);
    }
    a[i] = mulmod((uint32_t)acc, n_inv, q);
  }
}

/* ---- batched transforms over RNS polynomials ---------------------------- */

typedef struct {
  const uint32_t *in;
  uint32_t *out;
  uint32_t N, R;
  const uint32_t *q, *psi;
  int mode; /* 0 forward, 1 inverse, 2 RNS decomposition + forward */
  uint64_t begin, end; /* limb-polynomial range [begin, end) of count*R */
} ntt_job;

static void *ntt_worker(void *arg) {
  const ntt_job *j = (const ntt_job *)arg;
  uint32_t *tmp = (uint32_t *)malloc(sizeof(uint32_t) * j->N);
  if (!tmp) return NULL;
  for (uint64_t lp = j->begin; lp < j->end; ++lp) {
    const uint64_t c = lp / j->R;
    const uint32_t r = (uint32_t)(lp % j->R);
    uint32_t *dst = j->out + lp * j->N; /* out [count][R][N] */
    if (j->mode == 2) {
      /* limb r of the coefficient vector: each integer coefficient mod q[r] */
      const uint32_t *coef = j->in + c * j->N; /* in [count][N] */
      for (uint32_t i = 0; i < j->N; ++i) tmp[i] = coef[i] % j->q[r];
      oracle_ntt(tmp, dst, j->N, j->q[r], j->psi[r]);
    } else if (j->mode == 1) {
      oracle_intt(j->in + lp * j->N, dst, j->N, j->q[r], j->psi[r]);
    } else {
      oracle_ntt(j->in + lp * j->N, dst, j->N, j->q[r], j->psi[r]);
    }
  }
  free(tmp);
  return NULL;
}

static int ntt_batch_run(const uint32_t *in, uint32_t *out, uint64_t count, uint32_t N,
                         uint32_t R, const uint32_t *q, const uint32_t *psi, int mode,
                         int nthreads) {
  if (!in || !out || !q || !psi || N == 0 || R == 0) return -1;
  for (uint32_t r = 0; r < R; ++r)
    if (q[r] < 2) return -1;
  const uint64_t items = count * R;
  if (items == 0) return 0;
  nthreads = clamp_threads(nthreads, items);
  pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
  ntt_job *jobs = (ntt_job *)calloc((size_t)nthreads, sizeof(ntt_job));
  if (!th || !jobs) { free(th); free(jobs); return -1; }
  for (int t = 0; t < nthreads; ++t) {
    ntt_job *j = &jobs[t];
    j->in = in; j->out = out; j->N = N; j->R = R; j->q = q; j->psi = psi; j->mode = mode;
    j->begin = items * (uint64_t)t / (uint64_t)nthreads;
    j->end = items * (uint64_t)(t + 1) / (uint64_t)nthreads;
  }
  for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, ntt_worker, &jobs[t]);
  ntt_worker(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
  free(th);
  free(jobs);
  return 0;
}

int oracle_ntt_batch(const uint32_t *in, uint32_t *out, uint64_t count, uint32_t N,
                     uint32_t R, const uint32_t *q, const uint32_t *psi, int inverse,
                     int nthreads) {
  return ntt_batch_run(in, out, count, N, R, q, psi, inverse ? 1 : 0, nthreads);
}

int oracle_ntt_rns(const uint32_t *coeffs, uint32_t *out, uint64_t count, uint32_t N,
                   uint32_t R, const uint32_t *q, const uint32_t *psi, int nthreads) {
  return ntt_batch_run(coeffs, out, count, N, R, q, psi, 2, nthreads);
}

void oracle_negacyclic_mul(const uint32_t *a, const uint32_t *b, uint32_t *c,
                           uint32_t N, uint32_t q) {
  for (uint32_t t = 0; t < N; ++t) c[t] = 0;
  for (uint32_t i = 0; i < N; ++i) {
    for (uint32_t j = 0; j < N; ++j) {
      const uint32_t prod = mulmod(a[i] % q, b[j] % q, q);
      const uint32_t t = i + j;
      if (t < N) {
        c[t] = (uint32_t)(((uint64_t)c[t] + prod) % q);
      } else { /* X^N = -1 */
        c[t - N] = (uint32_t)(((uint64_t)c[t - N] + q - prod) % q);
      }
    }
  }
}
