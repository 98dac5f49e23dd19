/*
 * pirscan.h -- C ABI of libpirscan, the PIR server's database-multiplication
 * scan on AMD Instinct MI355X (gfx950).
 *
 * Two forms of the scan that every PIR query forces over the whole database:
 *
 *  RowSel (GPIR: "Enabling Practical Private Information Retrieval with GPUs",
 *  the paragraph that formulates RowSel as M_out[p,m,n] =
 *  sum_k M_in0[p,m,k] * M_in1[p,k,n] with extents 4N, 2, D1, D0; VIPIR
 *  section 4, the (#RNS*N)-parallel INT32 modular GEMM mod q_i; VIPIR
 *  section 2.3, one RNS row per prime q_i < 2^32):
 *
 *      out[mi][n][p] = ( sum_{k<D0} ct[mi][k][p] * db[k][n][p] ) mod q[p / N]
 *
 *  Scalar-HE / Regev (VIPIR section 2.5, the D1 x B x D0 INT8-INT32 GEMM of
 *  batched SimplePIR; VIPIR section 4, where reduction mod 2^32 is free):
 *
 *      out[i][b] = sum_{k<K} sext32(db[i][k]) * query[k][b]   (mod 2^32)
 *
 * Conventions shared by every entry point:
 *  - Buffers are DEVICE pointers unless stated.  The caller allocates and owns
 *    all of them (including workspaces); the library never allocates, frees or
 *    synchronises on the hot path and keeps no pointer after returning.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is enqueued asynchronously on it; buffers must stay valid until the
 *    stream reaches that work.  The return value reports argument validation
 *    and launch only.
 *  - Status codes: PIRSCAN_OK (0) or a negative PIRSCAN_E* value.  No C++
 *    exception crosses this ABI.  Calls are thread-safe; the only global
 *    state is a lazily initialised, per-thread last HIP error.
 *  - All arithmetic is integer; results are exact (bit-identical to the
 *    definitions above).
 */
#ifndef PIRSCAN_H
#define PIRSCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PIRSCAN_VERSION 10000 /* 1.0.0 */
#define PIRSCAN_MAX_R 8

enum {
  PIRSCAN_OK = 0,
  PIRSCAN_EINVAL = -1,       /* bad argument: null pointer, zero extent, modulus
                                outside [2, 2^32), R > PIRSCAN_MAX_R, m == 0,
                                output overlapping an input, workspace too small,
                                size overflow */
  PIRSCAN_EDEVICE = -2,      /* a HIP call failed; see pirscan_last_device_error */
  PIRSCAN_EUNSUPPORTED = -3  /* current device is not gfx950 */
};

/*
 * Shape of one RowSel problem.  P = R*N points; point p belongs to RNS limb
 * r = p / N and is reduced modulo q[r] (VIPIR section 2.3: a polynomial is an
 * #RNS x N INT32 matrix, one row per prime).  D0 is the reduction extent k
 * (the DB rows a query selects among), D1 the number of DB columns n (output
 * ciphertexts).  Read by value during the call.
 */
typedef struct {
  uint32_t N;                  /* points per RNS limb (polynomial degree) */
  uint32_t R;                  /* RNS limbs, 1..PIRSCAN_MAX_R */
  uint32_t q[PIRSCAN_MAX_R];   /* moduli, each in [2, 2^32); q[r] for r >= R ignored */
  uint32_t D0;                 /* k extent */
  uint32_t D1;                 /* n extent */
} pirscan_rowsel_shape;

/* Bytes of the tiled RowSel database produced by pirscan_layout_db:
 * exactly 4 * P * D0 * D1 (no padding).  0 if the shape is invalid. */
size_t pirscan_layout_db_bytes(const pirscan_rowsel_shape* s);

/*
 * One-time relayout of a RowSel database (the DB is static, so the transpose
 * that GPIR applies around RowSel and VIPIR section 4.2 inserts around its
 * modular GEMM is paid once, offline, and never per query).
 *   db_pmajor : [D0][D1][P] uint32, p-major (the HE-library/NTT layout in which
 *               each polynomial's P points are contiguous; GPIR layout
 *               paragraph).  Entries must be < q[p / N].
 *   db_tiled  : pirscan_layout_db_bytes(s) bytes, written in the library's
 *               internal layout (opaque; consumed by pirscan_rowsel_modgemm).
 * Must not overlap.  Pure permutation of words; no arithmetic.
 */
int pirscan_layout_db(const pirscan_rowsel_shape* s, const uint32_t* db_pmajor,
                      uint32_t* db_tiled, void* stream);

/*
 * Workspace bytes pirscan_rowsel_modgemm needs for (shape, m): 0 when the
 * batch runs on the VALU path (m < 16, a modulus >= 2^31, or D0 > 16384),
 * else room for the per-query relayout of ct and of the output used by the
 * int8-MFMA path (GPIR: batching makes RowSel a dense contraction).  0 also
 * on an invalid shape.
 */
size_t pirscan_rowsel_workspace_bytes(const pirscan_rowsel_shape* s, uint32_t m);

/*
 * RowSel scan: out[mi][n][p] = (sum_k ct[mi][k][p] * db[k][n][p]) mod q[p/N].
 *   m         : ciphertext polynomials in the query batch (m = 2B for B BFV
 *               ciphertexts of two polynomials each), m >= 1.
 *   ct        : [m][D0][P] uint32, p-major, entries < q[p/N].
 *   db_tiled  : output of pirscan_layout_db for the same shape.
 *   out       : [m][D1][P] uint32, p-major, canonical residues in [0, q[p/N]).
 *   workspace : >= pirscan_rowsel_workspace_bytes(s, m) bytes of device
 *               memory, 16-byte aligned, owned by the caller (may be NULL with
 *               workspace_bytes 0 when that size is 0); contents ignored on
 *               entry and unspecified on return.
 * Entries >= q are a precondition violation (not checked; the result is then
 * unspecified but memory-safe).  `out` and `workspace` must not overlap ct,
 * db_tiled or each other.
 */
int pirscan_rowsel_modgemm(const pirscan_rowsel_shape* s, uint32_t m,
                           const uint32_t* ct, const uint32_t* db_tiled,
                           uint32_t* out, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Workspace bytes pirscan_scalar_gemm_u32 needs for (M, K, B): the signed
 * digit planes of the query plus split-K partial sums.  0 on invalid sizes. */
size_t pirscan_scalar_workspace_bytes(uint64_t M, uint64_t K, uint32_t B);

/*
 * Scalar-HE database product mod 2^32.
 *   db        : [M][K] int8, row-major, two's complement (sign-extended before
 *               the product).
 *   query     : [K][B] uint32, row-major (B queries as columns; VIPIR section
 *               4.5 treats the query batch as a D0 x B matrix).
 *   out       : [M][B] uint32, row-major, = db * query mod 2^32.
 *   workspace : >= pirscan_scalar_workspace_bytes(M, K, B) bytes of device
 *               memory, 16-byte aligned, owned by the caller, contents
 *               ignored on entry and unspecified on return.
 * Each query word is split on the device into four signed int8 digits (the
 * INT8 decomposition of VIPIR section 4.1 in signed form); B == 1 runs a
 * packed int8 dot-product GEMV, B > 1 runs int8 MFMA over the digit planes.
 * `out` and `workspace` must not overlap db, query or each other.
 */
int pirscan_scalar_gemm_u32(const int8_t* db, const uint32_t* query, uint32_t* out,
                            uint64_t M, uint64_t K, uint32_t B,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Human-readable text for a status code (static storage). */
const char* pirscan_strerror(int status);

/* PIRSCAN_VERSION of the loaded library. */
int pirscan_version(void);

/* The hipError_t (as int) behind the calling thread's last PIRSCAN_EDEVICE. */
int pirscan_last_device_error(void);

#ifdef __cplusplus
}
#endif
#endif /* PIRSCAN_H */
