/*
 * oracle.h -- plain, slow, obviously-correct CPU definitions of the PIR
 * database-multiplication scan.  TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the package smoke check and the CPU-baseline leg of the
 * benchmark may load this library.  The product path (libpirscan) never links,
 * loads or calls it, and this code shares nothing with the GPU path: no
 * headers, helpers, tables or constant generators.
 *
 * Sources (the pages these definitions restate):
 *   [VIPIR] "VIPIR: a general GPU framework for integrated private information
 *           retrieval protocols" (CSDN translation), sections 2.3, 2.5, 4, 4.1,
 *           4.2, 5.
 *   [GPIR]  "GPIR: Enabling Practical Private Information Retrieval with GPUs",
 *           the OnionPIRv2 background paragraphs (DB as a D0 x D1 grid of
 *           NTT-domain polynomials) and the paragraph that states RowSel as
 *           point-wise GEMMs M_out[p,m,n] = sum_k M_in0[p,m,k] * M_in1[p,k,n].
 *
 * Every function is a direct transcription of a definition: no blocking, no
 * lazy reduction, no digit splitting.  All arithmetic is exact integer.
 */
#ifndef PIR_ORACLE_H
#define PIR_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Number of worker threads used when a caller passes nthreads <= 0. */
int oracle_default_threads(void);

/*
 * RowSel [GPIR RowSel formulation; VIPIR section 4, the (#RNS*N)-parallel
 * INT32 modular GEMM; VIPIR section 2.3, one RNS row per prime]:
 *
 *   out[mi][n][p] = ( sum_{k<D0} ct[mi][k][p] * db[k][n][p] ) mod q[p / N]
 *
 * for mi < m, n < D1, p < P = R*N.  Layouts are p-major (the P points of each
 * polynomial contiguous): ct [m][D0][P], db [D0][D1][P], out [m][D1][P].
 * The sum is accumulated exactly in unsigned 128-bit integers and reduced
 * once at the end, so the result is the canonical representative in
 * [0, q[r]).  Inputs may be any uint32 (no precondition is needed here).
 * Returns 0, or -1 on a zero modulus / null pointer.
 */
int oracle_rowsel(const uint32_t *ct, const uint32_t *db, uint32_t *out,
                  uint32_t N, uint32_t R, const uint32_t *q,
                  uint32_t m, uint32_t D0, uint32_t D1, int nthreads);

/*
 * Scalar-HE database product [VIPIR section 2.5, the D1 x B x D0 INT8-INT32
 * GEMM of batched SimplePIR; section 4, "mod 2^32 is free"]:
 *
 *   out[i][b] = sum_{k<K} sext32(db[i][k]) * Q[k][b]   (mod 2^32)
 *
 * db is int8 row-major [M][K] (two's complement, sign-extended before the
 * product), Q is uint32 [K][B], out is uint32 [M][B].  Computed in uint32
 * wrapping arithmetic, which is exact modulo 2^32.
 */
int oracle_scalar(const int8_t *db, const uint32_t *Q, uint32_t *out,
                  uint64_t M, uint64_t K, uint32_t B, int nthreads);

/*
 * ExpPack packing GEMM [VIPIR section 3.5.2: after the NTT the packing step
 * H*C + (0|G) is a (#RNS*N)-parallel ceil(D1/N) x 2B x n INT32 GEMM with a
 * modular reduction; section 3.6 gives its sizes]:
 *
 *   out[r][j][p] = ( sum_{i<n} H[r][i][p] * C[i][j][p] + Z[r][j][p] ) mod q[p / N]
 *   Z[r][2b][p] = 0,  Z[r][2b+1][p] = G[r][b][p]
 *
 * for r < Dr (= ceil(D1/N) output ciphertexts), j < 2B, p < P = R*N.  H is the
 * Dr x n hint matrix, C the n x 2B matrix of expanded special ciphertexts
 * (client b owns columns 2b, 2b+1), G the Dr x B body matrix; every matrix is
 * row-major with p-major polynomial entries: H [Dr][n][P], C [n][2B][P],
 * G [Dr][B][P], out [Dr][2B][P].  G may be NULL (Z = 0).  Exact unsigned
 * 128-bit accumulation, one final reduction: out is canonical in [0, q[r]).
 */
int oracle_exppack(const uint32_t *H, const uint32_t *C, const uint32_t *G,
                   uint32_t *out, uint32_t N, uint32_t R, const uint32_t *q,
                   uint32_t Dr, uint32_t n, uint32_t B, int nthreads);

/*
 * Signed-digit split of a 32-bit word [VIPIR section 4.1 splits the INT32
 * operand into four INT8 matrices; the signed reading is the one an
 * int8 x int8 datapath accepts]: digits s[0..3] in [-128, 127] with
 * sum_j s[j] * 2^(8j) == x (mod 2^32), produced byte by byte with a carry.
 */
void oracle_signed_digits(uint32_t x, int8_t s[4]);
/* Batch form: s has 4*n entries, s[4*i + j] is digit j of x[i]. */
void oracle_signed_digits_batch(const uint32_t *x, int8_t *s, uint64_t n);

/* ---- number-theory support used only to pin the oracle ------------------ */

/* 1 if n is prime.  Deterministic Miller-Rabin with bases {2, 7, 61}, which
 * is exact for every n < 4,759,123,141 and hence for every 32-bit n. */
int oracle_is_prime_u32(uint32_t n);

/* The `count` largest primes q < 2^bits with q == 1 (mod two_n), in
 * decreasing order, written to out.  Returns how many were found. */
int oracle_ntt_primes(uint32_t bits, uint32_t two_n, int count, uint32_t *out);

/* Smallest generator g of the multiplicative group mod prime q. */
uint32_t oracle_primitive_root(uint32_t q);

/* psi = g^((q-1)/(2N)) for the smallest generator g: a primitive 2N-th root
 * of unity mod q (requires 2N | q-1). */
uint32_t oracle_psi(uint32_t q, uint32_t N);

uint32_t oracle_powmod(uint32_t a, uint64_t e, uint32_t q);

/*
 * Negacyclic NTT by direct evaluation [VIPIR section 2.3: after the NTT a
 * polynomial product in Z_q[X]/(X^N+1) becomes a point-wise product]:
 *   A[j] = sum_i a[i] * psi^((2j+1) i)  mod q,  j < N   (natural order)
 * i.e. evaluation of a at the N odd powers of psi, the roots of X^N + 1.
 */
void oracle_ntt(const uint32_t *a, uint32_t *A, uint32_t N, uint32_t q,
                uint32_t psi);
/* Inverse: a[i] = N^-1 * sum_j A[j] * psi^-((2j+1) i)  mod q, for prime q
 * (psi^-1 and N^-1 are taken as powers q-2, by Fermat). */
void oracle_intt(const uint32_t *A, uint32_t *a, uint32_t N, uint32_t q,
                 uint32_t psi);

/*
 * Batched transforms over RNS polynomials [VIPIR section 2.3: a polynomial of
 * R_q is an #RNS x N matrix, one row of residues per prime q_r, and the NTT
 * transforms every row; GPIR: the NTT-domain points of a polynomial are
 * stored contiguously].  in and out are [count][R][N]: limb r of polynomial
 * c is the N words at (c*R + r)*N, transformed with q[r] and psi[r] by
 * oracle_ntt (inverse == 0) or oracle_intt (inverse != 0).  Threads split the
 * count*R independent limb-polynomials.  Returns 0, or -1 on a null pointer,
 * zero N or R, or a modulus < 2.
 */
int oracle_ntt_batch(const uint32_t *in, uint32_t *out, uint64_t count, uint32_t N,
                     uint32_t R, const uint32_t *q, const uint32_t *psi, int inverse,
                     int nthreads);

/*
 * RNS decomposition followed by the NTT [VIPIR section 3.5.2: each length-N
 * vector of a first-step output is read as a polynomial whose coefficients
 * are its integer entries, then transformed; section 4.3 fuses the RNS
 * decomposition into the NTT]:
 *   out[c][r][:] = NTT_{q[r], psi[r]}( coeffs[c][i] mod q[r], i < N )
 * coeffs is [count][N] uint32, each entry the integer in [0, 2^32) it
 * denotes; out is [count][R][N].  Returns as oracle_ntt_batch.
 */
int oracle_ntt_rns(const uint32_t *coeffs, uint32_t *out, uint64_t count, uint32_t N,
                   uint32_t R, const uint32_t *q, const uint32_t *psi, int nthreads);

/* Schoolbook product in Z_q[X]/(X^N + 1): c = a * b, with X^N = -1. */
void oracle_negacyclic_mul(const uint32_t *a, const uint32_t *b, uint32_t *c,
                           uint32_t N, uint32_t q);

#ifdef __cplusplus
}
#endif
#endif
