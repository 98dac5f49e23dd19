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
 *  ExpPack packing GEMM (VIPIR section 3.5.2: H*C + (0|G) after the NTT is a
 *  (#RNS*N)-parallel ceil(D1/N) x 2B x n INT32 GEMM with modular reduction):
 *
 *      out[r][j][p] = ( sum_{i<n} H[r][i][p] * C[i][j][p] + Z[r][j][p] ) mod q[p / N]
 *      Z[r][2b+1][p] = G[r][b][p],  Z[r][2b][p] = 0
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
 *    exception crosses this ABI.  Calls are thread-safe.  The library's own
 *    state is the calling thread's last HIP error and, per device, a cache
 *    of whether the device is a gfx950 and of its compute-unit count and
 *    kernel occupancy (filled on first use; nothing else persists between
 *    calls).
 *  - All arithmetic is integer; results are exact (bit-identical to the
 *    definitions above).
 *  - Inputs that are residues (RowSel / ExpPack operands, NTT inputs) must be
 *    below their modulus; this is not checked on the hot path.  With the
 *    environment variable PIRSCAN_VALIDATE_INPUTS=1 (read at each call) the
 *    entry points that take such inputs first check every one on the device
 *    and return PIRSCAN_EINVAL if one is out of range -- a debugging aid
 *    that synchronises the caller's stream.
 */
#ifndef PIRSCAN_H
#define PIRSCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PIRSCAN_VERSION 20000 /* 2.0.0 */
#define PIRSCAN_MAX_R 8

enum {
  PIRSCAN_OK = 0,
  PIRSCAN_EINVAL = -1,       /* bad argument: null pointer, zero extent, modulus
                                outside [2, 2^32), R > PIRSCAN_MAX_R, m out of
                                range, unknown scan kind, output overlapping an
                                input, workspace too small, size overflow */
  PIRSCAN_EDEVICE = -2,      /* a HIP call failed; see pirscan_last_device_error */
  PIRSCAN_EUNSUPPORTED = -3, /* current device is not gfx950 */
  PIRSCAN_ESCRATCH = -4      /* the problem needs more scratch memory than the
                                built-in buffer of the no-allocation entry point
                                (PIRSCAN_NOALLOC_SCRATCH_BYTES) holds */
};

/*
 * Which scan kernel a RowSel / ExpPack shape uses (the `scan` member of the
 * shapes below).  Both give the same, exact result; they differ in speed and
 * in the stored layout of the static operand, so the choice is part of the
 * shape and must be the same for the one-time layout and every later scan.
 *  PIRSCAN_SCAN_AUTO: the int8 matrix-core scan over centred signed limbs
 *    (VIPIR section 4.1's INT8 decomposition) when every q[r] < 2^31 and the
 *    reduction extent is <= 16384, else the VALU scan.
 *  PIRSCAN_SCAN_VALU: always the VALU scan -- 32x32 -> 64-bit products with
 *    lazy 64-bit accumulation and one reduction per output (VIPIR section
 *    4.2) -- on a word-for-word transposed layout.
 */
#define PIRSCAN_SCAN_AUTO 0u
#define PIRSCAN_SCAN_VALU 1u

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
  uint32_t scan;               /* PIRSCAN_SCAN_AUTO (0) or PIRSCAN_SCAN_VALU */
} pirscan_rowsel_shape;

/* Bytes of the tiled RowSel database produced by pirscan_layout_db, or 0 if
 * the shape is invalid.  For the int8 matrix-core scan (PIRSCAN_SCAN_AUTO
 * with every q[r] < 2^31 and D0 <= 16384): per point, ceil(D1/16) column
 * tiles (rounded up to a multiple of 16 from 16 tiles on) x ceil(D0/64)
 * k-steps x 4 KiB (exactly 4 * P * D0 * D1 when 256 | D1 and 64 | D0, or
 * D1 = 16 * T with T < 16).  For the VALU scan the words are stored
 * transposed, 4 * P * D0 * D1. */
size_t pirscan_layout_db_bytes(const pirscan_rowsel_shape* s);

/*
 * One-time relayout of a RowSel database (the DB is static, so the transpose
 * that GPIR applies around RowSel and VIPIR section 4.2 inserts around its
 * modular GEMM is paid once, offline, and never per query).
 *   db_pmajor : [D0][D1][P] uint32, p-major (the HE-library/NTT layout in which
 *               each polynomial's P points are contiguous; GPIR layout
 *               paragraph).  Entries must be < q[p / N].
 *   db_tiled  : pirscan_layout_db_bytes(s) bytes, 16-byte aligned, written in
 *               the library's internal layout (opaque; consumed by
 *               pirscan_rowsel_modgemm with the same shape).  For the matrix-
 *               core scan every residue is centred (x - q when x > q/2) and
 *               split into four signed 8-bit limbs (VIPIR section 4.1's INT8
 *               decomposition), stored in the order of the scan's fragments.
 * Must not overlap.  EINVAL for a misaligned db_tiled on the matrix-core
 * layout.
 */
int pirscan_layout_db(const pirscan_rowsel_shape* s, const uint32_t* db_pmajor,
                      uint32_t* db_tiled, void* stream);

/*
 * Workspace bytes pirscan_rowsel_modgemm needs for (shape, m), 0 only on an
 * invalid shape or m outside [1, 2^31]: the per-point staging of the output
 * (4 * P * m * D1 bytes) and, on the matrix-core scan (GPIR: batching makes
 * RowSel a dense contraction, and at batch 1 the scan streams the same
 * bytes), the per-query limb split of ct: 16 * m bytes per point and 64-k
 * step for m <= 16, else 8 KiB (passes of 32 rows).  Each part is rounded up
 * to 256 bytes.
 */
size_t pirscan_rowsel_workspace_bytes(const pirscan_rowsel_shape* s, uint32_t m);

/*
 * RowSel scan: out[mi][n][p] = (sum_k ct[mi][k][p] * db[k][n][p]) mod q[p/N].
 *   m         : ciphertext polynomials in the query batch (m = 2B for B BFV
 *               ciphertexts of two polynomials each), 1 <= m <= 2^31.
 *   ct        : [m][D0][P] uint32, p-major, entries < q[p/N].
 *   db_tiled  : output of pirscan_layout_db for the same shape.
 *   out       : [m][D1][P] uint32, p-major, canonical residues in [0, q[p/N]).
 *   workspace : >= pirscan_rowsel_workspace_bytes(s, m) bytes of device
 *               memory, 16-byte aligned, owned by the caller; contents ignored
 *               on entry and unspecified on return.
 * Entries >= q are a precondition violation (not checked; the result is then
 * unspecified but memory-safe).  `out` and `workspace` must not overlap ct,
 * db_tiled or each other.
 */
int pirscan_rowsel_modgemm(const pirscan_rowsel_shape* s, uint32_t m,
                           const uint32_t* ct, const uint32_t* db_tiled,
                           uint32_t* out, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * Shape of one ExpPack packing GEMM (VIPIR section 3.5.2; section 3.6 sizes it
 * at N = 2^12, #RNS = 3, Dr = 2^8, n = 1280).  P = R*N points as for RowSel.
 * Read by value during the call.
 */
typedef struct {
  uint32_t N;                  /* points per RNS limb (polynomial degree) */
  uint32_t R;                  /* RNS limbs, 1..PIRSCAN_MAX_R */
  uint32_t q[PIRSCAN_MAX_R];   /* moduli, each in [2, 2^32); q[r] for r >= R ignored */
  uint32_t Dr;                 /* output ciphertexts, ceil(D1 / N): rows of H and G */
  uint32_t n;                  /* LWE dimension: columns of H, rows of C */
  uint32_t scan;               /* PIRSCAN_SCAN_AUTO (0) or PIRSCAN_SCAN_VALU (reduction extent n) */
} pirscan_exppack_shape;

/* Bytes of the tiled hint produced by pirscan_exppack_layout_h, or 0 if the
 * shape is invalid: as pirscan_layout_db_bytes with D0 = n and D1 = Dr
 * (exactly 4 * P * Dr * n = 15 GiB at section 3.6's sizes). */
size_t pirscan_exppack_layout_h_bytes(const pirscan_exppack_shape* s);

/*
 * One-time relayout of the NTT-domain hint H (VIPIR section 3.6: H is
 * computed offline and is, after the database, the largest object the
 * packing streams; section 4.2 transposes between the polynomial-major NTT
 * layout and the GEMM layout).
 *   h_pmajor : [Dr][n][P] uint32, p-major, entries < q[p / N].
 *   h_tiled  : pirscan_exppack_layout_h_bytes(s) bytes, 16-byte aligned,
 *              opaque layout consumed by pirscan_exppack_modgemm (the limb
 *              split of pirscan_layout_db when every q < 2^31 and n <= 16384,
 *              else a word transpose).
 * Must not overlap.
 */
int pirscan_exppack_layout_h(const pirscan_exppack_shape* s, const uint32_t* h_pmajor,
                             uint32_t* h_tiled, void* stream);

/*
 * Workspace bytes pirscan_exppack_modgemm needs for (shape, B): as
 * pirscan_rowsel_workspace_bytes with m = 2B, D0 = n and D1 = Dr.  0 only on
 * an invalid shape or B outside [1, 2^30].
 */
size_t pirscan_exppack_workspace_bytes(const pirscan_exppack_shape* s, uint32_t B);

/*
 * ExpPack packing GEMM for B clients:
 *   out[r][j][p] = (sum_i H[r][i][p] * C[i][j][p] + Z[r][j][p]) mod q[p/N],
 *   Z[r][2b+1][p] = G[r][b][p], Z[r][2b][p] = 0.
 *   B         : clients, 1 <= B <= 2^30; client b owns columns 2b and 2b+1 of
 *               C and out (the two polynomials of its ciphertexts).
 *   C         : [n][2B][P] uint32, p-major, entries < q[p/N]: the expanded
 *               special ciphertexts (n x 2B matrix of polynomials).
 *   h_tiled   : output of pirscan_exppack_layout_h for the same shape.
 *   G         : [Dr][B][P] uint32, p-major, entries < q[p/N] (the NTT of the
 *               first-step outputs), or NULL for G = 0.
 *   out       : [Dr][2B][P] uint32, p-major, canonical residues in [0, q[p/N]):
 *               Dr packed ciphertexts per client.
 *   workspace : >= pirscan_exppack_workspace_bytes(s, B) bytes, 16-byte
 *               aligned, caller-owned; contents ignored on entry.
 * Entries >= q are a precondition violation (unchecked; memory-safe).  `out`
 * and `workspace` must not overlap C, h_tiled, G or each other.
 */
int pirscan_exppack_modgemm(const pirscan_exppack_shape* s, uint32_t B, const uint32_t* C,
                            const uint32_t* h_tiled, const uint32_t* G, uint32_t* out,
                            void* workspace, size_t workspace_bytes, void* stream);

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

/*
 * pirscan_scalar_gemm_u32 without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the digit planes and split-K
 * partial sums live in a scratch buffer built into the library, one per GPU,
 * of PIRSCAN_NOALLOC_SCRATCH_BYTES, which each GPU the library runs on holds
 * until the process ends.  Same arguments, layouts and result as
 * pirscan_scalar_gemm_u32; the call allocates nothing.
 *   Returns PIRSCAN_ESCRATCH when pirscan_scalar_workspace_bytes(M, K, B)
 *   exceeds PIRSCAN_NOALLOC_SCRATCH_BYTES (every B at M = K = 2^18, the
 *   64 GiB database, fits), before touching the device.
 *   Every call on one GPU shares that GPU's buffer: calls that overlap in
 *   time on one GPU (on different streams, or from different threads without
 *   ordering between their streams) race and give undefined results.  Calls
 *   ordered on one stream are safe; nothing in the buffer has to start at any
 *   particular value.
 */
#define PIRSCAN_NOALLOC_SCRATCH_BYTES ((size_t)72 << 20)
int pirscan_scalar_gemm_u32_noalloc(const int8_t* db, const uint32_t* query, uint32_t* out,
                                    uint64_t M, uint64_t K, uint32_t B, void* stream);

/*
 * Tiled scalar database.  The DB is static (VIPIR section 2.5: the server
 * holds it and every query multiplies it), so it can be laid out once in the
 * order the scans read it: 16-row tiles x 64-byte k steps, 1 KiB per
 * (tile, step), in groups of 16 tiles whose fragments follow each other step
 * after step -- a workgroup then streams one contiguous range instead of
 * 64-byte pieces of 256 different rows.
 * pirscan_scalar_layout_db_bytes: ceil(M/256) * 16 * ceil(K/64) * 1024 (zero
 * bytes pad M to 256 and K to 64), 0 on invalid sizes.
 * pirscan_scalar_layout_db: db [M][K] int8 row-major (any alignment) ->
 * db_tiled (device memory of that many bytes, 16-byte aligned, opaque, must
 * not overlap db).  Pure permutation of bytes plus zero padding.
 */
size_t pirscan_scalar_layout_db_bytes(uint64_t M, uint64_t K);
int pirscan_scalar_layout_db(const int8_t* db, void* db_tiled, uint64_t M, uint64_t K, void* stream);
/* Workspace bytes pirscan_scalar_gemm_u32_tiled needs for (M, K, B): the
 * signed digit planes of the widest pass (up to 64 query columns; when B > 64,
 * up to four groups of 128) plus split-K partial sums.  0 on invalid sizes. */
size_t pirscan_scalar_tiled_workspace_bytes(uint64_t M, uint64_t K, uint32_t B);
/*
 * The scalar-HE product on the tiled DB: the same result as
 * pirscan_scalar_gemm_u32 (out[i][b] = sum_k sext32(db[i][k]) * query[k][b]
 * mod 2^32): B = 1 with packed int8 dot products (v_dot4) against the four
 * digit planes, B > 1 on int8 MFMA over them.
 *   db_tiled  : output of pirscan_scalar_layout_db for the same M, K.
 *   query, out: as for pirscan_scalar_gemm_u32.
 *   workspace : >= pirscan_scalar_tiled_workspace_bytes(M, K, B) bytes,
 *               16-byte aligned, caller-owned; contents ignored on entry.
 * `out` and `workspace` must not overlap db_tiled, query or each other.
 */
int pirscan_scalar_gemm_u32_tiled(const void* db_tiled, const uint32_t* query, uint32_t* out,
                                  uint64_t M, uint64_t K, uint32_t B,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Negacyclic NTT over RNS polynomials -- the transform on either side of the
 * scans: it takes first-step outputs and the hint into the point-wise domain
 * that ExpPack's GEMM consumes (VIPIR section 3.5.2), the plaintext DB into
 * the NTT-domain points that RowSel scans (GPIR, the OnionPIRv2 background
 * paragraphs), and results back out.  VIPIR section 2.3: a polynomial of
 * Z_q[X]/(X^N + 1), q = q_0 ... q_{R-1}, is an R x N matrix of residues, and
 * the NTT turns polynomial products into point-wise products mod q_r.  For
 * limb r with psi = psi[r]:
 *
 *      forward:  A[j] = sum_{i<N} a[i] * psi^((2j+1) i)          mod q[r]
 *      inverse:  a[i] = N^-1 * sum_{j<N} A[j] * psi^-((2j+1) i)  mod q[r]
 *
 * for j, i < N, both in natural order, canonical results in [0, q[r]).
 * Layout: [count][R][N] uint32 -- polynomial c's limb r is the N words at
 * (c*R + r)*N, i.e. each polynomial's P = R*N points contiguous (the p-major
 * layout RowSel's ct / DB and ExpPack's H, C, G use).  VIPIR section 4.3 runs
 * an N = 2^12 NTT as one kernel and fuses the RNS decomposition into it;
 * here every transform is one kernel and pirscan_ntt_rns_forward fuses the
 * decomposition.
 */
typedef struct {
  uint32_t N;                    /* degree: a power of two in [16, 8192] */
  uint32_t R;                    /* RNS limbs, 1..PIRSCAN_MAX_R */
  uint32_t q[PIRSCAN_MAX_R];     /* primes, q[r] < 2^30, q[r] == 1 (mod 2N) */
  uint32_t psi[PIRSCAN_MAX_R];   /* psi[r]: a primitive 2N-th root of unity mod q[r],
                                    i.e. psi^N == q[r] - 1 (mod q[r]) */
} pirscan_ntt_shape;

/* Bytes of the twiddle plan for the shape (16 * R * N), or 0 if the shape is
 * invalid: N not a power of two in [16, 8192], R out of range, some q[r] not
 * a prime below 2^30 with q[r] == 1 (mod 2N), or psi[r]^N != -1 (mod q[r]). */
size_t pirscan_ntt_plan_bytes(const pirscan_ntt_shape* s);

/*
 * Fills `plan` (device memory, >= pirscan_ntt_plan_bytes(s) bytes, 16-byte
 * aligned, owned by the caller) with the shape's twiddle factors, on `stream`.
 * A plan serves every later transform of the same shape (forward, inverse,
 * RNS) and is read-only to them.  EINVAL on an invalid shape or a short or
 * misaligned plan.
 */
int pirscan_ntt_plan_init(const pirscan_ntt_shape* s, void* plan, size_t plan_bytes, void* stream);

/*
 * Forward / inverse transform of `count` polynomials (count >= 1):
 *   in  : [count][R][N] uint32 residues, entries < q[r] (precondition, not
 *         checked; violations give unspecified but memory-safe results).
 *   out : [count][R][N] uint32, canonical.  out == in (in place) is allowed;
 *         any other overlap of in, out or plan is EINVAL.
 *   plan: from pirscan_ntt_plan_init with the same shape.
 */
int pirscan_ntt_forward(const pirscan_ntt_shape* s, const void* plan, const uint32_t* in, uint32_t* out,
                        uint64_t count, void* stream);
int pirscan_ntt_inverse(const pirscan_ntt_shape* s, const void* plan, const uint32_t* in, uint32_t* out,
                        uint64_t count, void* stream);

/*
 * RNS decomposition fused with the forward transform (VIPIR section 3.5.2
 * reads each length-N vector of integer first-step outputs as a polynomial's
 * coefficients; section 4.3 fuses the decomposition into the NTT):
 *   out[c][r][:] = forward transform of ( coeffs[c][i] mod q[r], i < N )
 *   coeffs : [count][N] uint32, each entry the integer in [0, 2^32) it denotes.
 *   out    : [count][R][N] uint32, canonical.  Must not overlap coeffs or plan.
 * The coefficients are read from HBM once for all R limbs.
 */
int pirscan_ntt_rns_forward(const pirscan_ntt_shape* s, const void* plan, const uint32_t* coeffs,
                            uint32_t* out, uint64_t count, void* stream);

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
