// scalar.hip -- the scalar-HE (Regev/LWE) database product on gfx950:
//
//     out[i][b] = sum_k sext32(db[i][k]) * query[k][b]   (mod 2^32)
//
// (VIPIR section 2.5: the batched SimplePIR online step is one D1 x B x D0
// INT8-INT32 GEMM; section 4: with a 2^32 ciphertext modulus the reduction is
// free.)
//
// Every query word is split into four signed int8 digits s_j in [-128, 127]
// with sum_j s_j 2^(8j) == word (mod 2^32) (VIPIR section 4.1 splits the INT32
// operand into four INT8 matrices and recombines with shifts; the signed form
// fits the signed int8 x int8 datapaths of gfx950).  The split is unique, and
// the whole digit vector of a word w is the byte-wise view of
// (w + 0x80808080) ^ 0x80808080: adding 128 to every byte position with full
// carries moves each digit into [0, 255], flipping each byte's top bit moves
// it back to [-128, 127].
//
//  * B == 1 (S2): HBM-bound GEMV.  Each wavefront keeps the digits of one
//    4096-wide k-block in registers and streams 64 DB rows of that block with
//    128-bit loads, one v_dot4 (4 int8 products) per DB dword per digit plane.
//    Split-K partial sums (one per row and k-block) are added mod 2^32.
//  * B  > 1 (S3): int8 MFMA (v_mfma_i32_16x16x64_i8).  DB rows are the A
//    operand, the 4*B digit columns the B operand; the int32 accumulators
//    wrap modulo 2^32, which is exact for a result taken mod 2^32.  The
//    epilogue recombines the four digit planes with shifts, mod 2^32.
#include <hip/hip_runtime.h>

#include <atomic>
#include <type_traits>

#include "internal.hpp"

namespace pirscan {
namespace {

constexpr int kThreads = 256;
constexpr uint64_t kScalarGroupTiles = 16;  // row tiles per contiguous group of the tiled DB
constexpr int kGemvJ = 4;                          // 16-byte loads per lane per row
constexpr uint64_t kGemvKBlock = 64 * 16 * kGemvJ;  // 4096
constexpr int kGemvRowsPerWave = 64;
constexpr int kGemvRowBatch = 4;
// The B > 1 path splits K only as far as it must for the tiles to fill the
// GPU (a tile is 256 rows of one k-block): int8 MFMA accumulation wraps
// modulo 2^32 in two's complement (measured on gfx950 with sums well past
// 2^31), so a k-block of any length gives the exact digit-plane sums mod
// 2^32, which is all the recombination below needs.
constexpr uint64_t kMfmaTargetTiles = 512;
constexpr uint32_t kMfmaMaxCols = 64;  // query columns per MFMA pass (4 digit planes each)

typedef int v4i __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// The GEMV streams each DB row segment once with non-temporal 128-bit loads
// (measured faster than cached loads for pure streaming on gfx950).  The MFMA
// kernel reads every 128-byte row line as two 64-byte halves issued back to
// back; plain cached loads let the second half hit the line the first one
// brought in (measured faster than non-temporal loads there).
__device__ __forceinline__ uint4 load_db16(const int8_t* p) {
  const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ v4i load_db16_v4i(const int8_t* p) {
  return *reinterpret_cast<const v4i*>(p);
}

__device__ __forceinline__ uint32_t signed_digits_word(uint32_t w) {
  return (w + 0x80808080u) ^ 0x80808080u;
}

// ---------------------------------------------------------------------------
// S1, GEMV layout: for every group g of 4 consecutive k, 4 dwords (one per
// digit plane j); byte t of dword j is digit j of query[4g + t].  Zero past K.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void split_gemv_kernel(const uint32_t* __restrict__ query,
                                                              uint32_t* __restrict__ dig,
                                                              uint64_t K, uint64_t groups, uint32_t ldq,
                                                              uint32_t col) {
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t g = (uint64_t)blockIdx.x * kThreads + threadIdx.x; g < groups; g += stride) {
    uint32_t d[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint64_t k = 4 * g + t;
      d[t] = k < K ? signed_digits_word(query[k * ldq + col]) : 0u;
    }
    // plane j gathers byte j of the four words
    uint32_t p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      p[j] = ((d[0] >> (8 * j)) & 0xFFu) | (((d[1] >> (8 * j)) & 0xFFu) << 8) |
             (((d[2] >> (8 * j)) & 0xFFu) << 16) | (((d[3] >> (8 * j)) & 0xFFu) << 24);
    uint4 o;
    o.x = p[0]; o.y = p[1]; o.z = p[2]; o.w = p[3];
    reinterpret_cast<uint4*>(dig)[g] = o;
  }
}

// ---------------------------------------------------------------------------
// S2: GEMV.  Workgroup = 4 wavefronts x 64 rows of one k-block.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t xor_sum_tail(uint32_t v, int from) {
  for (int off = from; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__global__ __launch_bounds__(kThreads) void gemv_kernel(const int8_t* __restrict__ db,
                                                        const uint32_t* __restrict__ dig,
                                                        uint32_t* __restrict__ dst, uint64_t M,
                                                        uint64_t K, uint64_t nkb) {
  const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t wg = xcd_remap(blockIdx.x, gridDim.x);
  const uint64_t kb = wg % nkb, rb = wg / nkb;
  const uint64_t row0 = (rb * (kThreads / 64) + wave) * kGemvRowsPerWave;
  if (row0 >= M) return;  // no barriers below
  const uint64_t rows = (M - row0) < (uint64_t)kGemvRowsPerWave ? (M - row0) : kGemvRowsPerWave;

  // digits of this lane's 16*J k values: [t][u][j]
  uint32_t dg[kGemvJ][4][4];
  bool chunk_on[kGemvJ];
#pragma unroll
  for (int t = 0; t < kGemvJ; ++t) {
    const uint64_t kc = kb * kGemvKBlock + (uint64_t)(t * 64 + lane) * 16;
    chunk_on[t] = kc < K;
    const uint4* src = reinterpret_cast<const uint4*>(dig + kc);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint4 v = src[u];
      dg[t][u][0] = v.x; dg[t][u][1] = v.y; dg[t][u][2] = v.z; dg[t][u][3] = v.w;
    }
  }

  const int8_t* base = db + row0 * K + kb * kGemvKBlock + (uint64_t)lane * 16;
  uint32_t result = 0;
  for (uint64_t r = 0; r < rows; r += kGemvRowBatch) {
    uint32_t s[kGemvRowBatch];
    uint4 v[kGemvRowBatch][kGemvJ];
#pragma unroll
    for (int rr = 0; rr < kGemvRowBatch; ++rr) {
      const bool row_on = r + rr < rows;
#pragma unroll
      for (int t = 0; t < kGemvJ; ++t) {
        v[rr][t] = (row_on && chunk_on[t])
                       ? load_db16(base + (r + rr) * K + t * 1024)
                       : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int rr = 0; rr < kGemvRowBatch; ++rr) {
      int acc[4] = {0, 0, 0, 0};
#pragma unroll
      for (int t = 0; t < kGemvJ; ++t) {
        const uint32_t w[4] = {v[rr][t].x, v[rr][t].y, v[rr][t].z, v[rr][t].w};
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[j] = __builtin_amdgcn_sdot4((int)w[u], (int)dg[t][u][j], acc[j], false);
      }
      s[rr] = (uint32_t)acc[0] + ((uint32_t)acc[1] << 8) + ((uint32_t)acc[2] << 16) +
              ((uint32_t)acc[3] << 24);
    }
    // Reduce 4 rows over 64 lanes with 7 cross-lane adds: two merge steps
    // leave row (2*bit4 + bit5) of the lane's index in each lane, then a
    // 16-lane butterfly finishes every row.
    const bool hi32 = lane & 32, hi16 = lane & 16;
    const uint32_t a01 = (hi32 ? s[1] : s[0]) + __shfl_xor(hi32 ? s[0] : s[1], 32, 64);
    const uint32_t a23 = (hi32 ? s[3] : s[2]) + __shfl_xor(hi32 ? s[2] : s[3], 32, 64);
    uint32_t t = (hi16 ? a23 : a01) + __shfl_xor(hi16 ? a01 : a23, 16, 64);
    t = xor_sum_tail(t, 8);
    const uint32_t sum0 = __shfl(t, 0, 64), sum1 = __shfl(t, 32, 64);
    const uint32_t sum2 = __shfl(t, 16, 64), sum3 = __shfl(t, 48, 64);
    const uint64_t lr = lane;
    if (lr == r) result = sum0;
    if (lr == r + 1) result = sum1;
    if (lr == r + 2) result = sum2;
    if (lr == r + 3) result = sum3;
  }
  if (lane < rows) dst[kb * M + row0 + lane] = result;
}

// ---------------------------------------------------------------------------
// S1, MFMA layout: for every 16-k group and digit column c = j*bpad + b, 16
// bytes (digit j of query[k][b] for the 16 k of the group).  Zero for k >= K
// and for padding columns b >= bgroup.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void split_mfma_kernel(const uint32_t* __restrict__ query,
                                                              uint8_t* __restrict__ dig,
                                                              uint64_t K, uint64_t k16_groups,
                                                              uint32_t bpad, uint32_t bgroup,
                                                              uint32_t ldq, uint32_t col0) {
  const uint64_t total = k16_groups * bpad;
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t e = (uint64_t)blockIdx.x * kThreads + threadIdx.x; e < total; e += stride) {
    const uint64_t g = e / bpad;
    const uint32_t b = (uint32_t)(e % bpad);
    uint32_t plane[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int w = 0; w < 4; ++w) plane[j][w] = 0;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const uint64_t k = g * 16 + t;
      const uint32_t d = (k < K && b < bgroup) ? signed_digits_word(query[k * ldq + col0 + b]) : 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) plane[j][t / 4] |= ((d >> (8 * j)) & 0xFFu) << (8 * (t % 4));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint4 o;
      o.x = plane[j][0]; o.y = plane[j][1]; o.z = plane[j][2]; o.w = plane[j][3];
      reinterpret_cast<uint4*>(dig)[g * 4 * bpad + (uint64_t)j * bpad + b] = o;
    }
  }
}

// S1, wide-pass layout: the same digits in MFMA B-fragment order, one 1 KiB
// fragment per (64-k step s, plane j, 16-column tile ct): lane (li, lg) holds
// digit j of query[64s + 16lg + 0..15][col0 + 16ct + li], at 16-byte index
// ((s * 4 + j) * (bpad / 16) + ct) * 64 + 16 lg + li.  Zero past K and bgroup.
__global__ __launch_bounds__(kThreads) void split_wide_kernel(const uint32_t* __restrict__ query,
                                                              uint4* __restrict__ dig, uint64_t K,
                                                              uint64_t k16_groups, uint32_t bpad, uint32_t bgroup,
                                                              uint32_t ldq, uint32_t col0) {
  const uint64_t total = k16_groups * bpad;
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  const uint32_t ctiles = bpad / 16;
  for (uint64_t e = (uint64_t)blockIdx.x * kThreads + threadIdx.x; e < total; e += stride) {
    const uint64_t g = e / bpad;
    const uint32_t b = (uint32_t)(e % bpad);
    uint32_t plane[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int w = 0; w < 4; ++w) plane[j][w] = 0;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const uint64_t k = g * 16 + t;
      const uint32_t d = (k < K && b < bgroup) ? signed_digits_word(query[k * ldq + col0 + b]) : 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) plane[j][t / 4] |= ((d >> (8 * j)) & 0xFFu) << (8 * (t % 4));
    }
    const uint64_t s = g / 4, lg = g % 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint4 o;
      o.x = plane[j][0]; o.y = plane[j][1]; o.z = plane[j][2]; o.w = plane[j][3];
      dig[((s * 4 + j) * ctiles + b / 16) * 64 + lg * 16 + b % 16] = o;
    }
  }
}

// ---------------------------------------------------------------------------
// S3: int8 MFMA GEMM.  A tile = 8 wavefronts x kMfmaRowTiles2*16 rows of one
// k-block; NT = 16-column tiles = 4 * bpad / 16.  The kernel is persistent:
// one workgroup per CU walks a list of tiles.  The tiles are split into 8
// contiguous ranges, one per XCD, and the workgroups of an XCD take the tiles
// of its range round-robin, so they start together on the same k-block and
// read the same digit chunks at nearly the same time: each chunk is fetched
// into that XCD's L2 once and reused by all its workgroups.
//  * Digit fragments (the B operand, shared by all rows) are staged once per
//    workgroup into LDS in chunks of 256 k, double-buffered: the next chunk is
//    loaded into registers at the start of a chunk and written to LDS at its
//    end, one barrier per chunk.
//  * DB rows (the A operand, each byte used by exactly one wavefront) stream
//    straight into registers through a ring of kMfmaDepth 64-k steps: the
//    slot consumed by a step is refilled with the step kMfmaDepth ahead, so
//    ~kMfmaDepth * 2 KiB per wavefront are in flight without extra registers.
// ---------------------------------------------------------------------------
#ifndef PIRSCAN_SCALAR_MFMA_DEPTH
#define PIRSCAN_SCALAR_MFMA_DEPTH 8
#endif
#ifndef PIRSCAN_SCALAR_MFMA_CHUNK
#define PIRSCAN_SCALAR_MFMA_CHUNK 4
#endif
#ifndef PIRSCAN_SCALAR_MFMA_ROWTILES
#define PIRSCAN_SCALAR_MFMA_ROWTILES 2
#endif
#ifndef PIRSCAN_SCALAR_BAHEAD
#define PIRSCAN_SCALAR_BAHEAD 4  // digit fragments read ahead of their MFMAs (0: as the compiler schedules)
#endif
constexpr int kBAhead = PIRSCAN_SCALAR_BAHEAD;

constexpr int kMfmaWaves = 8;
constexpr int kMfmaRowTiles2 = PIRSCAN_SCALAR_MFMA_ROWTILES;  // 16-row tiles per wavefront
constexpr int kMfmaDepth = PIRSCAN_SCALAR_MFMA_DEPTH;        // A ring depth in 64-k steps
constexpr int kMfmaChunkSteps = PIRSCAN_SCALAR_MFMA_CHUNK;   // B chunk = 4 steps = 256 k
static_assert(kMfmaDepth % kMfmaChunkSteps == 0, "the ring turns in whole B chunks");
constexpr uint64_t kMfmaChunkK = 64 * kMfmaChunkSteps;

template <int NT>
struct MfmaShape {
  // A ring depth: 8 steps, or 4 for the widest passes, whose 16 column tiles
  // of accumulators leave fewer registers for the ring
  static constexpr int DEPTH = NT >= 16 ? 4 : kMfmaDepth;
  static_assert(DEPTH % kMfmaChunkSteps == 0, "the ring turns in whole B chunks");
  static constexpr int HT = NT / 4;                        // column tiles per digit plane
  static constexpr int DCOLS = 16 * NT;                    // 4 * bpad digit columns
  static constexpr int CHUNK_BYTES = kMfmaChunkK * DCOLS;  // 32 KiB at bpad = 32
  static constexpr int PIECES = CHUNK_BYTES / 16 / (64 * kMfmaWaves);  // 16-byte pieces per thread
  static_assert(PIECES >= 1 && CHUNK_BYTES % (16 * 64 * kMfmaWaves) == 0, "chunk tiling");
};

// One tile (kb, rb).  Starts and ends with every wave past a barrier, so the
// LDS buffers are free on entry and on exit.  PACKED: the DB is in the tiled
// layout of pirscan_scalar_layout_db (16-row tiles x 64-k steps of 1 KiB
// A fragments, `ptiles` x `psteps` of them, zero-padded), otherwise row-major.
template <int NT, bool PACKED>
__device__ __forceinline__ void mfma_tile(const int8_t* __restrict__ db, const uint8_t* dig,
                                          uint32_t* __restrict__ dst, uint64_t M, uint64_t K,
                                          uint64_t kblock, uint64_t nkb, uint32_t bgroup, uint64_t ldd,
                                          uint32_t dcol0, uint64_t kb, uint64_t rb, uint64_t ptiles,
                                          uint64_t psteps, uint8_t (*bsm)[MfmaShape<NT>::CHUNK_BYTES]) {
  constexpr int HT = MfmaShape<NT>::HT;
  constexpr int DCOLS = MfmaShape<NT>::DCOLS;
  constexpr int CHUNK_BYTES = MfmaShape<NT>::CHUNK_BYTES;
  constexpr int PIECES = MfmaShape<NT>::PIECES;
  constexpr int DEPTH = MfmaShape<NT>::DEPTH;

  const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t row0 = (rb * kMfmaWaves + wave) * (16 * kMfmaRowTiles2);
  const uint32_t li = lane % 16, lg = lane / 16;
  const uint64_t kbeg = kb * kblock;
  const uint32_t nsteps = (uint32_t)(kblock / 64);
  const uint32_t nchunks = nsteps / kMfmaChunkSteps;

  // A rows past M and k past K are read from clamped (valid) addresses: rows
  // past M are never stored, and k past K meets zero digits.
  const int8_t* arow[kMfmaRowTiles2];
  const v4i* atile[kMfmaRowTiles2];
#pragma unroll
  for (int rt = 0; rt < kMfmaRowTiles2; ++rt) {
    if constexpr (PACKED) {
      uint64_t t = (row0 + rt * 16) / 16;
      t = t < ptiles ? t : ptiles - 1;
      atile[rt] = reinterpret_cast<const v4i*>(db) +
                  ((t / kScalarGroupTiles) * psteps * kScalarGroupTiles + t % kScalarGroupTiles) * 64 + lane;
    } else {
      const uint64_t row = row0 + rt * 16 + li;
      arow[rt] = db + (row < M ? row : M - 1) * K;
    }
  }
  const uint64_t klast = K - 16;  // last valid 16-byte chunk of a row (K % 16 == 0)
  // A fragment of row tile rt at 64-k step `step` of this k-block
  auto load_a = [&](int rt, uint32_t step) -> v4i {
    if constexpr (PACKED) {
      uint64_t sg = kbeg / 64 + step;
      sg = sg < psteps ? sg : psteps - 1;
      return __builtin_nontemporal_load(atile[rt] + sg * (64 * kScalarGroupTiles));
    } else {
      uint64_t ko = kbeg + (uint64_t)step * 64 + 16 * lg;
      ko = ko < klast ? ko : klast;
      return load_db16_v4i(arow[rt] + ko);
    }
  };

  // chunk c of this k-block is CHUNK_BYTES contiguous bytes of the digit array
  // (dig is not __restrict__: the compiler barrier below must be able to
  // order these loads, which restrict would let the compiler ignore.)
  const u32x4* bsrc = reinterpret_cast<const u32x4*>(dig + (kbeg / 16) * (uint64_t)DCOLS * 16) + tid;
  u32x4* bdst0 = reinterpret_cast<u32x4*>(bsm[0]) + tid;
  u32x4* bdst1 = reinterpret_cast<u32x4*>(bsm[1]) + tid;

  v4i acc[kMfmaRowTiles2][NT];
#pragma unroll
  for (int rt = 0; rt < kMfmaRowTiles2; ++rt)
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) acc[rt][ct] = v4i{0, 0, 0, 0};

  // prologue: A ring for steps 0..depth-1, B chunk 0 into LDS
  v4i a[DEPTH][kMfmaRowTiles2];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d)
#pragma unroll
    for (int rt = 0; rt < kMfmaRowTiles2; ++rt) a[d][rt] = load_a(rt, d);
  {
    u32x4 breg[PIECES];
#pragma unroll
    for (int i = 0; i < PIECES; ++i) breg[i] = bsrc[i * (64 * kMfmaWaves)];
#pragma unroll
    for (int i = 0; i < PIECES; ++i) bdst0[i * (64 * kMfmaWaves)] = breg[i];
  }
  __syncthreads();

  constexpr int kChunksPerTurn = DEPTH / kMfmaChunkSteps;  // one turn of the A ring
  for (uint32_t c = 0; c < nchunks; c += kChunksPerTurn) {
    // a whole ring turn per iteration so that every ring slot index is static
#pragma unroll
    for (int half = 0; half < kChunksPerTurn; ++half) {
      const uint32_t cc = c + half;
      if (cc < nchunks) {
        // next chunk (or this one again at the end: same bytes, harmless)
        const uint32_t cn = cc + 1 < nchunks ? cc + 1 : cc;
        u32x4 breg[PIECES];
#pragma unroll
        for (int i = 0; i < PIECES; ++i)
          breg[i] = bsrc[(uint64_t)cn * (CHUNK_BYTES / 16) + i * (64 * kMfmaWaves)];
        // Issue the chunk loads here, a whole chunk before their LDS store:
        // the empty asm is a compiler memory barrier that stops the loads from
        // being merged with that store (into a copy at the end of the chunk),
        // and the scheduling barrier stops the scheduler from sinking them.
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        const v4i* bl = reinterpret_cast<const v4i*>(bsm[cc & 1]);
        // digit fragment i = s * NT + ct of the chunk; with kBAhead > 0 the
        // fragments are read kBAhead ahead of their MFMAs, through the chunk
        constexpr int kNB = kMfmaChunkSteps * NT;
        constexpr int kBA = kBAhead < kNB ? kBAhead : kNB;
        auto bfrag = [&](int i) -> v4i { return bl[((i / NT) * 4 + lg) * DCOLS + (i % NT) * 16 + li]; };
        v4i bq[kBA > 0 ? kBA : 1];
#pragma unroll
        for (int i = 0; i < kBA; ++i) bq[i] = bfrag(i);
#pragma unroll
        for (int s = 0; s < kMfmaChunkSteps; ++s) {
          const uint32_t step = cc * kMfmaChunkSteps + s;
          const int slot = (half * kMfmaChunkSteps + s) % DEPTH;
#pragma unroll
          for (int ct = 0; ct < NT; ++ct) {
            const int i = s * NT + ct;
            const v4i bf = kBA > 0 ? bq[i % (kBA > 0 ? kBA : 1)] : bfrag(i);
#pragma unroll
            for (int rt = 0; rt < kMfmaRowTiles2; ++rt)
              acc[rt][ct] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[slot][rt], bf, acc[rt][ct], 0, 0, 0);
            if (kBA > 0 && i + kBA < kNB) {
              bq[i % (kBA > 0 ? kBA : 1)] = bfrag(i + kBA);
              // pin the read here, kBA fragments ahead of its MFMAs: left
              // alone the scheduler sinks it next to its use
              __builtin_amdgcn_sched_barrier(0);
            }
          }
          if (s & 1) {
            // Refill the slots of steps s-1 and s together: the two 64-byte
            // halves of each 128-byte row line are requested back to back, so
            // the line is fetched from HBM once.  Past the last step the
            // refill re-reads the last step (valid, unused): keeping it
            // unconditional keeps the chunk one basic block, so the compiler
            // cannot sink the digit-chunk loads down to their LDS store.
            uint32_t nxt = step - 1 + DEPTH;
            nxt = nxt < nsteps ? nxt : nsteps - 2;
#pragma unroll
            for (int rt = 0; rt < kMfmaRowTiles2; ++rt) {
              a[slot - 1][rt] = load_a(rt, nxt);
              a[slot][rt] = load_a(rt, nxt + 1);
            }
            // keep the refill here: the scheduler would otherwise sink it
            // next to its use (to save registers) and undo the prefetch
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        // The other buffer was last read in chunk cc-1, which every wave
        // finished before the previous barrier.
        u32x4* bdst = (cc & 1) ? bdst0 : bdst1;
#pragma unroll
        for (int i = 0; i < PIECES; ++i) bdst[i * (64 * kMfmaWaves)] = breg[i];
        __syncthreads();
      }
    }
  }

  // D element i of lane l is (row 4*(l/16) + i, column l%16) of the tile.
#pragma unroll
  for (int rt = 0; rt < kMfmaRowTiles2; ++rt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint64_t row = row0 + rt * 16 + 4 * lg + i;
      if (row >= M) continue;
#pragma unroll
      for (int h = 0; h < HT; ++h) {
        const uint32_t b = h * 16 + li;
        if (b >= bgroup) continue;
        uint32_t v = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) v += (uint32_t)acc[rt][j * HT + h][i] << (8 * j);
        if (nkb == 1) dst[row * ldd + dcol0 + b] = v;
        else dst[(kb * M + row) * bgroup + b] = v;
      }
    }
  }
}

template <int NT, bool PACKED>
__global__ __launch_bounds__(64 * kMfmaWaves) void mfma_kernel(const int8_t* __restrict__ db,
                                                               const uint8_t* dig,
                                                               uint32_t* __restrict__ dst, uint64_t M,
                                                               uint64_t K, uint64_t kblock, uint64_t nkb,
                                                               uint64_t row_blocks, uint32_t bgroup,
                                                               uint64_t ldd, uint32_t dcol0, uint64_t ptiles,
                                                               uint64_t psteps) {
  __shared__ __attribute__((aligned(16))) uint8_t bsm[2][MfmaShape<NT>::CHUNK_BYTES];
  constexpr uint32_t kXcds = 8;
  const uint32_t hw = blockIdx.x, G = gridDim.x;  // G >= kXcds (host guarantees)
  const uint32_t xcd = hw % kXcds, j = hw / kXcds;
  const uint32_t per_xcd = (G - xcd + kXcds - 1) / kXcds;  // workgroups with this residue
  const uint64_t tiles = nkb * row_blocks;
  const uint64_t lo = tiles * xcd / kXcds, hi = tiles * (xcd + 1) / kXcds;
  for (uint64_t t = lo + j; t < hi; t += per_xcd)
    mfma_tile<NT, PACKED>(db, dig, dst, M, K, kblock, nkb, bgroup, ldd, dcol0, t / row_blocks, t % row_blocks,
                          ptiles, psteps, bsm);
}

// ---------------------------------------------------------------------------
// S3, wide passes (more than 64 query columns, tiled DB): tiles of 128 query
// columns, and one launch takes up to kWideGroups such column groups, so a
// batch of n columns streams the DB from HBM about ceil(n / 512) times
// instead of ceil(n / 64).  A tile = 128 rows (8 row tiles, half a tile group
// of the tiled layout) x 512 digit columns (4 planes x 128 columns) of one
// k-block, 8 wavefronts: wave w accumulates all 8 row tiles against planes
// 0..3 of query columns 16w..16w+15 of its group (one column tile per plane),
// 32 accumulator tiles.  The column groups of one row block are neighbouring
// tiles, run side by side on one XCD: the first to read a DB fragment brings
// it into that XCD's L2 for the others.  (The clock the chip holds during
// these passes falls with their HBM and L2 traffic; the HBM reads saved
// this way raise it.)
//  * DB fragments (the A operand, used by all 8 waves) come into a six-step
//    LDS ring once per workgroup with direct global-to-LDS loads, one 1 KiB
//    fragment per wave per step, four steps ahead.
//  * Digit fragments (the B operand, 1 KiB each in fragment order, each used
//    by one wave) stream from global memory straight into a three-step
//    register ring, two steps ahead (all workgroups of an XCD walk k together,
//    so they come from L2).
// Persistent over tiles like mfma_kernel, with the same XCD-local ranges.
// ---------------------------------------------------------------------------
constexpr int kWideWaves = 8;
constexpr uint32_t kWideCols = 128;            // query columns per wide pass (= bpad)
constexpr int kWideRowTiles = 8;               // row tiles per wave (all of the tile's)
constexpr int kWidePlanes = 4;                 // column tiles per wave: one per digit plane
constexpr uint64_t kWideRows = kWideRowTiles * 16;  // rows per tile: 128
constexpr int kWideARing = 6;                  // A ring depth (LDS) in 64-k steps: loads 4 steps ahead
constexpr int kWideBRing = 3;                  // B ring depth (registers): loads 2 steps ahead
#ifndef PIRSCAN_WIDE_GROUPS
#define PIRSCAN_WIDE_GROUPS 4
#endif
constexpr uint32_t kWideGroups = PIRSCAN_WIDE_GROUPS;  // 128-column groups per wide launch

__device__ __forceinline__ void wide_tile(const v4i* __restrict__ dbp, const v4i* dig, uint32_t* __restrict__ dst,
                                          uint64_t M, uint64_t kblock, uint64_t nkb, uint32_t bgroup, uint64_t ldd,
                                          uint32_t dcol0, uint64_t kb, uint64_t rb, uint32_t g, uint32_t ctiles,
                                          uint64_t psteps, v4i (*aring)[kWideWaves * 64]) {
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t li = lane % 16, lg = lane / 16;
  const uint64_t s_first = kb * kblock / 64;  // first 64-k step of this k-block
  const uint32_t nsteps = (uint32_t)(kblock / 64);
  // this workgroup's 8 row tiles: tiles 8rb .. 8rb+7, inside tile group rb / 2
  const uint64_t t0 = rb * 8;
  const v4i* abase = dbp + ((t0 / kScalarGroupTiles) * psteps * kScalarGroupTiles + t0 % kScalarGroupTiles + wave) * 64 +
                     lane;
  // digits in B-fragment order (split_wide_kernel, ctiles column tiles per
  // plane): this wave's fragment (step, plane j) is column tile 8g + w, 1 KiB
  // of contiguous lanes
  const v4i* bbase = dig + (uint64_t)(kWideCols / 16 * g + wave) * 64 + lane;

  v4i acc[kWideRowTiles][kWidePlanes];
#pragma unroll
  for (int rt = 0; rt < kWideRowTiles; ++rt)
#pragma unroll
    for (int j = 0; j < kWidePlanes; ++j) acc[rt][j] = v4i{0, 0, 0, 0};

  // step s's DB fragments -> LDS ring slot s % kWideARing; wave w moves
  // fragment w.  The ring runs four steps ahead, so the last steps load
  // fragments past this k-block that no MFMA reads; past the DB's last step
  // the address is clamped to stay inside the buffer.
  auto issue_a = [&](uint32_t s) {
    uint64_t sg = s_first + s;
    sg = sg < psteps ? sg : psteps - 1;
    __builtin_amdgcn_global_load_lds((const void*)(abase + sg * (64 * kScalarGroupTiles)),
                                     LDS_PTR(aring[s % kWideARing] + wave * 64), 16, 0, 0);
  };
  v4i bb[kWideBRing][kWidePlanes];
  auto load_b = [&](int slot, uint32_t s) {
    const uint32_t ss = s < nsteps ? s : nsteps - 1;  // past the end: a harmless reload
    const v4i* bs = bbase + (s_first + ss) * (4ull * ctiles * 64);
#pragma unroll
    for (int j = 0; j < kWidePlanes; ++j) bb[slot][j] = bs[(uint64_t)j * ctiles * 64];
  };
  // One step.  Per step B(s+2) (4 loads), then A(s+4) (1) are issued.  At
  // the wait of step s the loads issued after B(s) are A(s+2), B(s+1) and
  // A(s+3), six in all, so vmcnt(6) leaves A(s) (issued before B(s)) and B(s)
  // landed.  The barrier publishes every wave's share of A(s) and tells each
  // wave that all others are done with step s-2's slot, which A(s+4)
  // overwrites; B(s+2) goes to register slot (s+2) % 3, last read by step
  // s-1's MFMAs.
  auto step = [&](auto slot_tag, uint32_t s) {
    constexpr int slot = decltype(slot_tag)::value;
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(kWidePlanes + 2));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    const v4i* as = aring[s % kWideARing] + lane;
    v4i af[kWideRowTiles];
#pragma unroll
    for (int rt = 0; rt < kWideRowTiles; ++rt) af[rt] = as[rt * 64];
    __builtin_amdgcn_sched_barrier(0);
    load_b((slot + 2) % kWideBRing, s + 2);
    issue_a(s + 4);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int rt = 0; rt < kWideRowTiles; ++rt)
#pragma unroll
      for (int j = 0; j < kWidePlanes; ++j)
        acc[rt][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[rt], bb[slot][j], acc[rt][j], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  issue_a(0);
  issue_a(1);
  load_b(0, 0);
  issue_a(2);
  load_b(1, 1);
  issue_a(3);
  uint32_t s = 0;
  for (; s + 2 < nsteps; s += 3) {
    step(std::integral_constant<int, 0>{}, s);
    step(std::integral_constant<int, 1>{}, s + 1);
    step(std::integral_constant<int, 2>{}, s + 2);
  }
  if (s < nsteps) step(std::integral_constant<int, 0>{}, s);
  if (s + 1 < nsteps) step(std::integral_constant<int, 1>{}, s + 1);
  __builtin_amdgcn_s_waitcnt(0);  // no ring load may outlive this tile's use of the LDS
  __syncthreads();                // the next tile's prologue overwrites the ring

  // D element i of lane l is (row 4*(l/16) + i, column l%16) of a tile;
  // this wave's column tile j is plane j of query columns 128g + 16w + 0..15
  const uint32_t b = kWideCols * g + 16 * wave + li;
  if (b >= bgroup) return;
#pragma unroll
  for (int rt = 0; rt < kWideRowTiles; ++rt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint64_t row = rb * kWideRows + rt * 16 + 4 * lg + i;
      if (row >= M) continue;
      uint32_t v = 0;
#pragma unroll
      for (int j = 0; j < kWidePlanes; ++j) v += (uint32_t)acc[rt][j][i] << (8 * j);
      if (nkb == 1) dst[row * ldd + dcol0 + b] = v;
      else dst[(kb * M + row) * bgroup + b] = v;
    }
  }
}

__global__ __launch_bounds__(64 * kWideWaves) void mfma_wide_kernel(const v4i* __restrict__ dbp, const v4i* dig,
                                                                     uint32_t* __restrict__ dst, uint64_t M,
                                                                     uint64_t kblock, uint64_t nkb,
                                                                     uint64_t row_blocks, uint32_t bgroup,
                                                                     uint64_t ldd, uint32_t dcol0, uint64_t psteps,
                                                                     uint32_t groups) {
  __shared__ v4i aring[kWideARing][kWideWaves * 64];
  constexpr uint32_t kXcds = 8;
  const uint32_t hw = blockIdx.x, G = gridDim.x;  // G >= kXcds (host guarantees)
  const uint32_t xcd = hw % kXcds, j = hw / kXcds;
  const uint32_t per_xcd = (G - xcd + kXcds - 1) / kXcds;
  // tile t: column group t % groups (fastest, so that the workgroups of one
  // row block's groups run side by side on one XCD and read its DB
  // fragments from HBM once), then row block, then k-block
  const uint64_t tiles = nkb * row_blocks * groups;
  const uint64_t lo = tiles * xcd / kXcds, hi = tiles * (xcd + 1) / kXcds;
  for (uint64_t t = lo + j; t < hi; t += per_xcd) {
    const uint64_t r = t / groups;
    wide_tile(dbp, dig, dst, M, kblock, nkb, bgroup, ldd, dcol0, r / row_blocks, r % row_blocks,
              (uint32_t)(t % groups), 8 * groups, psteps, aring);
  }
}

// ---------------------------------------------------------------------------
// Split-K reduction: out[row*ldo + col0 + b] = sum_kb part[(kb*M + row)*cols + b]
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void reduce_kernel(const uint32_t* __restrict__ part,
                                                          uint32_t* __restrict__ out, uint64_t M,
                                                          uint32_t cols, uint64_t nkb, uint64_t ldo,
                                                          uint32_t col0) {
  const uint64_t total = M * cols;
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t e = (uint64_t)blockIdx.x * kThreads + threadIdx.x; e < total; e += stride) {
    uint32_t s = 0;
    for (uint64_t kb = 0; kb < nkb; ++kb) s += part[kb * total + e];
    const uint64_t row = e / cols;
    const uint32_t b = (uint32_t)(e % cols);
    out[row * ldo + col0 + b] = s;
  }
}

// ---------------------------------------------------------------------------
// Any shape / alignment: one thread per output, byte loads.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void generic_kernel(const int8_t* __restrict__ db,
                                                           const uint32_t* __restrict__ query,
                                                           uint32_t* __restrict__ out, uint64_t M,
                                                           uint64_t K, uint32_t B) {
  const uint64_t total = M * B;
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t e = (uint64_t)blockIdx.x * kThreads + threadIdx.x; e < total; e += stride) {
    const uint64_t row = e / B;
    const uint32_t b = (uint32_t)(e % B);
    uint32_t s = 0;
    for (uint64_t k = 0; k < K; ++k) s += (uint32_t)(int32_t)db[row * K + k] * query[k * B + b];
    out[e] = s;
  }
}

uint32_t grid_for(uint64_t items, uint64_t cap = 1u << 20) {
  uint64_t g = (items + kThreads - 1) / kThreads;
  if (g > cap) g = cap;
  return (uint32_t)(g ? g : 1);
}

uint64_t ceil_div(uint64_t a, uint64_t b) { return (a + b - 1) / b; }
uint64_t align_up(uint64_t a, uint64_t b) { return ceil_div(a, b) * b; }

// Workgroups of kernel KERNEL (THREADS threads each) the current device
// holds at once (compute units x occupancy), queried once per device and kept.
template <auto KERNEL, int THREADS>
hipError_t resident_workgroups(uint64_t* out) {
  static std::atomic<uint64_t> cache[kMaxDevices];  // 0: not yet queried
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool cached = dev >= 0 && dev < kMaxDevices;
  if (cached) {
    const uint64_t v = cache[dev].load(std::memory_order_relaxed);
    if (v) {
      *out = v;
      return hipSuccess;
    }
  }
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, KERNEL, THREADS, 0);
  if (e != hipSuccess) return e;
  const uint64_t v = (uint64_t)(cus > 0 ? cus : 1) * (uint64_t)(per_cu > 0 ? per_cu : 1);
  if (cached) cache[dev].store(v, std::memory_order_relaxed);
  *out = v;
  return hipSuccess;
}

template <int NT, bool PACKED>
hipError_t launch_mfma(const int8_t* db, const uint8_t* dig, uint32_t* dst, uint64_t M, uint64_t K,
                       const ScalarPlan& pl, uint32_t bgroup, uint64_t ldd, uint32_t dcol0,
                       hipStream_t stream) {
  const uint64_t rows_per_wg = kMfmaWaves * 16 * kMfmaRowTiles2;
  const uint64_t row_blocks = ceil_div(M, rows_per_wg);
  if (pl.kblock % kMfmaChunkK != 0) return hipErrorInvalidValue;
  // persistent: as many workgroups as are co-resident, at least one per XCD
  uint64_t grid = 0;
  const hipError_t e = resident_workgroups<mfma_kernel<NT, PACKED>, 64 * kMfmaWaves>(&grid);
  if (e != hipSuccess) return e;
  if (grid > row_blocks * pl.nkb) grid = row_blocks * pl.nkb;
  if (grid < 8) grid = 8;
  hipLaunchKernelGGL((mfma_kernel<NT, PACKED>), dim3((uint32_t)grid), dim3(64 * kMfmaWaves), 0, stream, db,
                     dig, dst, M, K, pl.kblock, pl.nkb, row_blocks, bgroup, ldd, dcol0,
                     ceil_div(M, 16 * kScalarGroupTiles) * kScalarGroupTiles, ceil_div(K, 64));
  return hipGetLastError();
}

hipError_t launch_mfma_wide(const int8_t* db, const uint8_t* dig, uint32_t* dst, uint64_t M, uint64_t K,
                            const ScalarPlan& pl, uint32_t bgroup, uint32_t groups, uint64_t ldd, uint32_t dcol0,
                            hipStream_t stream) {
  const uint64_t row_blocks = ceil_div(M, kWideRows);
  if (pl.kblock % 64 != 0) return hipErrorInvalidValue;
  uint64_t grid = 0;
  const hipError_t e = resident_workgroups<mfma_wide_kernel, 64 * kWideWaves>(&grid);
  if (e != hipSuccess) return e;
  if (grid > row_blocks * pl.nkb * groups) grid = row_blocks * pl.nkb * groups;
  if (grid < 8) grid = 8;
  hipLaunchKernelGGL(mfma_wide_kernel, dim3((uint32_t)grid), dim3(64 * kWideWaves), 0, stream,
                     reinterpret_cast<const v4i*>(db), reinterpret_cast<const v4i*>(dig), dst, M, pl.kblock, pl.nkb,
                     row_blocks, bgroup, ldd, dcol0, ceil_div(K, 64), groups);
  return hipGetLastError();
}

// B == 1 on the tiled DB: GEMV with packed int8 dot products.  A wavefront
// owns TG row tiles (16 TG rows) of one k-block; per 64-k step it loads the
// TG 1 KiB fragments (lane (li, lg): row li, k = 64s + 16lg + 0..15) one step
// ahead, and the 64 bytes of digits of its 16 k (the GEMV digit layout: per
// 4-k group, one dword per plane), the same address for the 16 lanes of a
// k-group.  Each DB dword meets its 4 digit dwords in 4 v_dot4_i32_i8 (int32
// wrap-around = mod 2^32); the planes are recombined with shifts and the 4
// k-groups of a row summed across lanes at the end.
#ifndef PIRSCAN_TGEMV_TILES
#define PIRSCAN_TGEMV_TILES 4
#endif
#ifndef PIRSCAN_TGEMV_WAVES
#define PIRSCAN_TGEMV_WAVES 4096
#endif
#ifndef PIRSCAN_TGEMV_RING
#define PIRSCAN_TGEMV_RING 2
#endif
#ifndef PIRSCAN_TGEMV_WINDOW_STEPS
#define PIRSCAN_TGEMV_WINDOW_STEPS 128  // k-block per workgroup (0: one resident long share per wave)
#endif
constexpr int kTiledGemvTiles = PIRSCAN_TGEMV_TILES;
constexpr int kTiledGemvRing = PIRSCAN_TGEMV_RING;
constexpr uint64_t kTiledGemvTargetWaves = PIRSCAN_TGEMV_WAVES;  // 4 per SIMD
__global__ __launch_bounds__(kThreads) void gemv_tiled_kernel(const u32x4* __restrict__ dbp,
                                                              const u32x4* __restrict__ dig,
                                                              uint32_t* __restrict__ dst, uint64_t M,
                                                              uint64_t ptiles, uint64_t psteps,
                                                              uint64_t kblock_steps, uint64_t nkb,
                                                              uint64_t items) {
  constexpr int TG = kTiledGemvTiles;
  const uint32_t lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t li = lane % 16, lg = lane / 16;
  uint64_t kb, tg;
  if constexpr (PIRSCAN_TGEMV_WINDOW_STEPS > 0) {
    static_assert(4 * kTiledGemvTiles == kScalarGroupTiles, "a workgroup is one tile group");
    // workgroup = the 16 row tiles of one group x one k-block, in address
    // order: the k-blocks in flight form one window moving through the DB
    const uint64_t wg = blockIdx.x;
    kb = wg % nkb;
    tg = (wg / nkb) * 4 + wave;
    if (tg * nkb >= items) return;  // no barriers in this kernel
  } else {
    const uint64_t item = (uint64_t)xcd_remap(blockIdx.x, gridDim.x) * 4 + wave;
    if (item >= items) return;  // no barriers in this kernel
    kb = item % nkb;
    tg = item / nkb;
  }
  const uint64_t s0 = kb * kblock_steps;
  const uint64_t nst = (s0 + kblock_steps < psteps ? s0 + kblock_steps : psteps) - s0;  // >= 1
  const u32x4* frag[TG];
#pragma unroll
  for (int t = 0; t < TG; ++t) {
    uint64_t tile = tg * TG + t;
    tile = tile < ptiles ? tile : ptiles - 1;
    frag[t] = dbp + ((tile / kScalarGroupTiles * psteps + s0) * kScalarGroupTiles + tile % kScalarGroupTiles) * 64 +
              lane;
  }
  const u32x4* dg = dig + s0 * 16 + 4 * lg;  // per step: 16 groups of 4 k, 4 of them this lane's

  int acc[TG][4];
#pragma unroll
  for (int t = 0; t < TG; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[t][j] = 0;
  // ring of kRingG steps, loads kRingG - 1 steps ahead; the step count is
  // rounded up to whole ring turns, the extra steps reading a reloaded DB
  // fragment against the zero digits past the array's last real step
  constexpr int R = kTiledGemvRing;
  u32x4 a[R][TG], d[R][4];
  const u32x4* dzero = dig + psteps * 16 + 4 * lg;
  auto load = [&](int slot, uint64_t s) {
    const uint64_t ss = s < nst ? s : nst - 1;
#pragma unroll
    for (int t = 0; t < TG; ++t) a[slot][t] = __builtin_nontemporal_load(frag[t] + ss * (64 * kScalarGroupTiles));
    const u32x4* ds = s < nst ? dg + s * 16 : dzero;
#pragma unroll
    for (int u = 0; u < 4; ++u) d[slot][u] = ds[u];
  };
#pragma unroll
  for (int r = 0; r < R - 1; ++r) load(r, r);
  for (uint64_t s = 0; s < nst; s += R) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      load((r + R - 1) % R, s + r + R - 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < TG; ++t) {
        const uint32_t w[4] = {a[r][t].x, a[r][t].y, a[r][t].z, a[r][t].w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t dj[4] = {d[r][u].x, d[r][u].y, d[r][u].z, d[r][u].w};
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[t][j] = __builtin_amdgcn_sdot4((int)w[u], (int)dj[j], acc[t][j], false);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

#pragma unroll
  for (int t = 0; t < TG; ++t) {
    uint32_t v = (uint32_t)acc[t][0] + ((uint32_t)acc[t][1] << 8) + ((uint32_t)acc[t][2] << 16) +
                 ((uint32_t)acc[t][3] << 24);
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    const uint64_t row = (tg * TG + t) * 16 + li;
    if (lg == 0 && row < M) dst[kb * M + row] = v;
  }
}

// Columns of the next wide launch with `left` (> kMfmaMaxCols) columns to
// go, and its 128-column groups: whole groups up to kWideGroups, plus a
// partial group when more than kMfmaMaxCols of it remain (a smaller
// remainder takes a narrow pass).
uint32_t wide_launch(uint32_t left, uint32_t* groups) {
  const uint32_t full = left / kWideCols, rem = left % kWideCols;
  if (full >= kWideGroups) {
    *groups = kWideGroups;
    return kWideGroups * kWideCols;
  }
  *groups = full + (rem > kMfmaMaxCols ? 1u : 0u);
  return rem > kMfmaMaxCols ? left : full * kWideCols;
}

// The MFMA passes: digit split, scan, split-K reduction.  Passes take up to
// kMfmaMaxCols query columns, or on the tiled DB, while more than
// kMfmaMaxCols columns remain (the plan's `wide`), up to kWideGroups groups
// of kWideCols (wide_launch).
template <bool PACKED>
hipError_t run_mfma_passes(const int8_t* db, const uint32_t* query, uint32_t* out, uint64_t M, uint64_t K,
                           uint32_t B, const ScalarPlan& pl, uint8_t* dig, uint32_t* part, hipStream_t stream) {
  hipError_t e;
  uint32_t bg = 0;
  for (uint32_t c0 = 0; c0 < B; c0 += bg) {
    const uint32_t left = B - c0;
    const bool wide = PACKED && pl.wide && left > kMfmaMaxCols;
    uint32_t groups = 1;
    bg = wide ? wide_launch(left, &groups) : (left < kMfmaMaxCols ? left : kMfmaMaxCols);
    const uint32_t bpad = wide ? groups * kWideCols : (uint32_t)align_up(bg, 16);
    const uint64_t k16 = pl.kpad / 16;
    if (wide)
      hipLaunchKernelGGL(split_wide_kernel, dim3(grid_for(k16 * bpad)), dim3(kThreads), 0, stream, query,
                         reinterpret_cast<uint4*>(dig), K, k16, bpad, bg, B, c0);
    else
      hipLaunchKernelGGL(split_mfma_kernel, dim3(grid_for(k16 * bpad)), dim3(kThreads), 0, stream, query,
                         dig, K, k16, bpad, bg, B, c0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    uint32_t* dst = pl.nkb > 1 ? part : out;
    timer_mark_start(stream);  // first pass only
    if (wide) {
      e = launch_mfma_wide(db, dig, dst, M, K, pl, bg, groups, B, c0, stream);
    } else {
      switch (bpad) {
        case 16: e = launch_mfma<4, PACKED>(db, dig, dst, M, K, pl, bg, B, c0, stream); break;
        case 32: e = launch_mfma<8, PACKED>(db, dig, dst, M, K, pl, bg, B, c0, stream); break;
        case 48: e = launch_mfma<12, PACKED>(db, dig, dst, M, K, pl, bg, B, c0, stream); break;
        default: e = launch_mfma<16, PACKED>(db, dig, dst, M, K, pl, bg, B, c0, stream); break;
      }
    }
    if (e != hipSuccess) return e;
    if (c0 + bg >= B) timer_mark_stop(stream);  // last pass: before its reduction
    if (pl.nkb > 1) {
      hipLaunchKernelGGL(reduce_kernel, dim3(grid_for(M * bg)), dim3(kThreads), 0, stream, part, out, M,
                         bg, pl.nkb, (uint64_t)B, c0);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

// MFMA plan: up to kMfmaMaxCols columns per pass (kWideCols with `wide`,
// the tiled DB, when B > kMfmaMaxCols), K split only as far as the tiles
// must be to fill the GPU.  The workspace holds the digit planes and partial
// sums of the widest pass.
void mfma_plan(uint64_t M, uint64_t K, uint32_t B, bool wide_ok, ScalarPlan* p) {
  p->mfma = true;
  p->wide = wide_ok && B > kMfmaMaxCols;
  if (p->wide) {  // the first launch is the widest
    uint32_t groups = 1;
    p->bgroup = wide_launch(B, &groups);
    p->bpad = groups * kWideCols;
  } else {
    p->bgroup = B < kMfmaMaxCols ? B : kMfmaMaxCols;
    p->bpad = (uint32_t)align_up(p->bgroup, 16);
  }
  const uint64_t row_blocks = ceil_div(M, (uint64_t)kMfmaWaves * 16 * kMfmaRowTiles2);
  uint64_t nkb = ceil_div(kMfmaTargetTiles, row_blocks);
  const uint64_t chunks = ceil_div(K, kMfmaChunkK);
  if (nkb > chunks) nkb = chunks;
  p->kblock = align_up(ceil_div(K, nkb), kMfmaChunkK);
  p->nkb = ceil_div(K, p->kblock);
  p->kpad = p->nkb * p->kblock;
  p->digit_bytes = p->kpad * 4 * p->bpad;
  p->part_bytes = p->nkb > 1 ? p->nkb * M * p->bgroup * 4 : 0;
  p->total_bytes = align_up(p->digit_bytes, 256) + p->part_bytes;
}

// Tiled scalar DB: 16-byte lane (li, lg) of (row tile T, 64-k step s) holds
// db[16T + li][64s + 16lg + 0..15], zero past M and K; one thread per lane.
// Fragment order [T / 16][s][T % 16][lane]: a group of 16 row tiles (the
// tiles of one workgroup) is one contiguous run, step after step.
template <bool VEC>
__global__ __launch_bounds__(kThreads) void pack_scalar_kernel(const int8_t* __restrict__ db,
                                                               uint4* __restrict__ dst, uint64_t M,
                                                               uint64_t K, uint64_t steps, uint64_t total) {
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t e = (uint64_t)blockIdx.x * kThreads + threadIdx.x; e < total; e += stride) {
    const uint32_t lane = (uint32_t)(e % 64);
    const uint64_t f = e / 64, tl = f % kScalarGroupTiles, gs = f / kScalarGroupTiles;
    const uint64_t s = gs % steps, t = (gs / steps) * kScalarGroupTiles + tl;
    const uint64_t row = t * 16 + lane % 16, k0 = s * 64 + (lane / 16) * 16;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row < M && k0 < K) {
      const int8_t* src = db + row * K + k0;
      if (VEC) {  // K % 16 == 0: the 16 bytes are all inside the row
        v = *reinterpret_cast<const uint4*>(src);
      } else {
        uint32_t w[4] = {0, 0, 0, 0};
        for (uint32_t i = 0; i < 16 && k0 + i < K; ++i) w[i / 4] |= (uint32_t)(uint8_t)src[i] << (8 * (i % 4));
        v = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
    dst[e] = v;
  }
}

}  // namespace

bool scalar_plan(uint64_t M, uint64_t K, uint32_t B, uintptr_t db_addr, ScalarPlan* p) {
  *p = ScalarPlan{};
  if (M == 0 || K == 0 || B == 0) return false;
  if (B > (1u << 20)) return false;
  const unsigned __int128 lim = (unsigned __int128)1 << 62;
  if ((unsigned __int128)M * K > lim || (unsigned __int128)M * B * 4 > lim ||
      (unsigned __int128)K * B * 4 > lim)
    return false;
  p->fast = (K % 16 == 0) && (db_addr % 16 == 0);
  if (!p->fast) return true;  // generic kernel, no workspace
  if (B == 1) {
    p->mfma = false;
    p->bgroup = 1;
    p->bpad = 1;
    p->kblock = kGemvKBlock;
    p->nkb = ceil_div(K, p->kblock);
    p->kpad = p->nkb * p->kblock;
    p->digit_bytes = p->kpad * 4;  // 4 digit planes x 1 byte per k
    p->part_bytes = p->nkb > 1 ? p->nkb * M * 4 : 0;
    p->total_bytes = align_up(p->digit_bytes, 256) + p->part_bytes;
  } else {
    mfma_plan(M, K, B, false, p);
  }
  return true;
}

hipError_t launch_scalar(const int8_t* db, const uint32_t* query, uint32_t* out, uint64_t M,
                         uint64_t K, uint32_t B, const ScalarPlan& pl, void* workspace,
                         hipStream_t stream) {
  if (!pl.fast) {
    timer_mark_start(stream);
    hipLaunchKernelGGL(generic_kernel, dim3(grid_for(M * B)), dim3(kThreads), 0, stream, db, query,
                       out, M, K, B);
    timer_mark_stop(stream);
    return hipGetLastError();
  }
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint32_t* part = reinterpret_cast<uint32_t*>(ws + align_up(pl.digit_bytes, 256));
  hipError_t e;
  if (!pl.mfma) {
    uint32_t* dig = reinterpret_cast<uint32_t*>(ws);
    const uint64_t groups = pl.kpad / 4;
    hipLaunchKernelGGL(split_gemv_kernel, dim3(grid_for(groups)), dim3(kThreads), 0, stream, query,
                       dig, K, groups, 1u, 0u);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const uint64_t row_blocks = ceil_div(M, (kThreads / 64) * kGemvRowsPerWave);
    const uint64_t grid = row_blocks * pl.nkb;
    if (grid > 0x7FFFFFFFull) return hipErrorInvalidValue;
    uint32_t* dst = pl.nkb > 1 ? part : out;
    timer_mark_start(stream);
    hipLaunchKernelGGL(gemv_kernel, dim3((uint32_t)grid), dim3(kThreads), 0, stream, db, dig, dst, M,
                       K, pl.nkb);
    timer_mark_stop(stream);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (pl.nkb > 1) {
      hipLaunchKernelGGL(reduce_kernel, dim3(grid_for(M)), dim3(kThreads), 0, stream, part, out, M, 1u,
                         pl.nkb, 1ull, 0u);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
  }
  return run_mfma_passes<false>(db, query, out, M, K, B, pl, ws, part, stream);
}

bool scalar_tiled_plan(uint64_t M, uint64_t K, uint32_t B, ScalarPlan* p) {
  *p = ScalarPlan{};
  if (M == 0 || K == 0 || B == 0 || B > (1u << 20)) return false;
  const unsigned __int128 lim = (unsigned __int128)1 << 62;
  if ((unsigned __int128)M * K > lim || (unsigned __int128)M * B * 4 > lim ||
      (unsigned __int128)K * B * 4 > lim)
    return false;
  p->fast = true;
  if (B > 1) {
    mfma_plan(M, K, B, true, p);
    return true;
  }
  // B == 1: GEMV over wavefronts of kTiledGemvTiles row tiles, K split into
  // whole 64-k steps until there are enough wavefronts to fill the GPU
  p->mfma = false;
  p->bgroup = 1;
  p->bpad = 1;
  const uint64_t psteps = ceil_div(K, 64);
  const uint64_t waves = ceil_div(ceil_div(M, 16), kTiledGemvTiles);
  uint64_t nkb = PIRSCAN_TGEMV_WINDOW_STEPS > 0 ? ceil_div(psteps, PIRSCAN_TGEMV_WINDOW_STEPS)
                                                : ceil_div(kTiledGemvTargetWaves, waves);
  if (nkb > psteps) nkb = psteps;
  p->kblock = ceil_div(psteps, nkb) * 64;
  p->nkb = ceil_div(psteps * 64, p->kblock);
  p->kpad = (psteps + 1) * 64;  // one step of zero digits past the last (the ring's padding steps)
  p->digit_bytes = p->kpad * 4;
  p->part_bytes = p->nkb > 1 ? p->nkb * M * 4 : 0;
  p->total_bytes = align_up(p->digit_bytes, 256) + p->part_bytes;
  return true;
}

uint64_t scalar_layout_bytes(uint64_t M, uint64_t K) {
  return ceil_div(M, 16 * kScalarGroupTiles) * kScalarGroupTiles * ceil_div(K, 64) * 1024;
}

hipError_t launch_scalar_layout(const int8_t* db, void* dst, uint64_t M, uint64_t K, hipStream_t stream) {
  const uint64_t total = scalar_layout_bytes(M, K) / 16;
  const bool vec = K % 16 == 0 && reinterpret_cast<uintptr_t>(db) % 16 == 0;
  if (vec)
    hipLaunchKernelGGL((pack_scalar_kernel<true>), dim3(grid_for(total)), dim3(kThreads), 0, stream, db,
                       static_cast<uint4*>(dst), M, K, ceil_div(K, 64), total);
  else
    hipLaunchKernelGGL((pack_scalar_kernel<false>), dim3(grid_for(total)), dim3(kThreads), 0, stream, db,
                       static_cast<uint4*>(dst), M, K, ceil_div(K, 64), total);
  return hipGetLastError();
}

hipError_t launch_scalar_tiled(const void* db_tiled, const uint32_t* query, uint32_t* out, uint64_t M,
                               uint64_t K, uint32_t B, const ScalarPlan& pl, void* workspace,
                               hipStream_t stream) {
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint32_t* part = reinterpret_cast<uint32_t*>(ws + align_up(pl.digit_bytes, 256));
  if (pl.mfma)
    return run_mfma_passes<true>(static_cast<const int8_t*>(db_tiled), query, out, M, K, B, pl, ws, part, stream);
  hipError_t e;
  const uint64_t groups = pl.kpad / 4;
  hipLaunchKernelGGL(split_gemv_kernel, dim3(grid_for(groups)), dim3(kThreads), 0, stream, query,
                     reinterpret_cast<uint32_t*>(ws), K, groups, 1u, 0u);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const uint64_t ptiles = ceil_div(M, 16 * kScalarGroupTiles) * kScalarGroupTiles, psteps = ceil_div(K, 64);
  const uint64_t items = ceil_div(ptiles, kTiledGemvTiles) * pl.nkb, grid = ceil_div(items, 4);
  if (grid > 0x7FFFFFFFull) return hipErrorInvalidValue;
  uint32_t* dst = pl.nkb > 1 ? part : out;
  timer_mark_start(stream);
  hipLaunchKernelGGL(gemv_tiled_kernel, dim3((uint32_t)grid), dim3(kThreads), 0, stream,
                     static_cast<const u32x4*>(db_tiled), reinterpret_cast<const u32x4*>(ws), dst, M, ptiles, psteps,
                     pl.kblock / 64, pl.nkb, items);
  timer_mark_stop(stream);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (pl.nkb > 1) {
    hipLaunchKernelGGL(reduce_kernel, dim3(grid_for(M)), dim3(kThreads), 0, stream, part, out, M, 1u, pl.nkb,
                       1ull, 0u);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace pirscan
