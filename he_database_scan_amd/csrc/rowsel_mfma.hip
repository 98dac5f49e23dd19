// rowsel_mfma.hip -- RowSel and ExpPack on int8 MFMA over centred signed
// limbs (gfx950), for every batch size.
//
// The per-point product C[mi][n] = sum_k A[mi][k] * B[k][n] (A = ct, B = DB,
// all values < q) runs on v_mfma_i32_16x16x64_i8 (VIPIR section 4.1 emulates
// a wide integer product with INT8 tensor-core GEMMs on split operands,
// section 4.2 discusses the modular GEMM's reduction; GPIR: "Enabling
// Practical Private Information Retrieval with GPUs" observes that batching
// raises RowSel's arithmetic intensity).  At batch 1 the matrix cores are
// mostly idle, but the scan is HBM-bound at every batch and the MFMA form
// needs no per-word ALU work, so one kernel serves all m.
//
// Every value x < q is centred, v = x - q if x > q/2 (so |v| <= q/2 < 2^30
// for q < 2^31), and written in four signed 8-bit limbs v = sum_i v_i 2^(8i),
// v_i in [-128, 127] (the bytes of (v + 0x80808080) ^ 0x80808080).  Then
//
//   sum_k a_k b_k = sum_{d=0..6} 2^(8d) S_d,  S_d = sum_{i+j=d} sum_k a_{k,i} b_{k,j}
//
// exactly; each S_d is an int32 accumulation of at most four limb GEMMs with
// |S_d| <= 4 * D0 * 2^14, which fits for D0 <= 16384.  The epilogue folds the
// seven diagonals into one residue: sum_d (S_d + 2^31) (2^(8d) mod q) plus a
// precomputed correction for the offsets, with the same hi*(2^32 mod q) + lo
// fold as the VALU scan, and one Barrett reduction.
//
// Data movement:
//  * The DB (or ExpPack's hint) is packed once, at layout time, into MFMA
//    B-fragment order: per point, per 16-column tile t and 64-k step s, four
//    1 KiB fragments (one per limb), lane (li, lg) holding limb j of the 16
//    consecutive k 64s + 16lg + 0..15 of column 16t + li.  A tile's steps are
//    contiguous, so a wavefront streams its columns as 1 KiB vector loads with
//    no ALU work per word.
//  * The query side (ct, or ExpPack's C) is packed per call the same way into
//    A fragments [p][s][row tile][limb][lane] in the workspace.  The four
//    wavefronts of a workgroup scan the same point, so each step's A
//    fragments come into LDS once per workgroup (direct global-to-LDS loads,
//    a three-step ring) and every wave reads them from there.
//  * Results are written per point, [p][mi][n], and a transpose pass
//    produces the p-major output (adding ExpPack's body term G where the
//    launch carries one).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "internal.hpp"

namespace pirscan {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kRing = 3;         // A-fragment ring depth in steps
#ifndef PIRSCAN_SMALL_ROWS
#define PIRSCAN_SMALL_ROWS 4
#endif
#ifndef PIRSCAN_SMALL_NTW
#define PIRSCAN_SMALL_NTW 1
#endif
#ifndef PIRSCAN_DIRECT_DEPTH
#define PIRSCAN_DIRECT_DEPTH 3  // steps in the one-tile direct kernel's register ring (2 or 3)
#endif
constexpr uint32_t kDirectRows = 16;  // passes of at most this many rows: the direct kernel
constexpr uint32_t kFrag = 256;  // v4i per step and 16-row (or 16-column) tile: 4 limbs x 64 lanes

// Centred signed-limb digits of a residue x < q (the byte vector of the
// centred value's four signed 8-bit digits): with v = x - q when x > q/2,
// digits = (v + 0x80808080) ^ 0x80808080.  The two possible offsets are
// precomputed (bias_lo = 0x80808080, bias_hi = 0x80808080 - q), so a word
// costs one compare, one select, one add and one xor.
__device__ __forceinline__ uint32_t centred_digits(uint32_t x, uint32_t half, uint32_t bias_lo,
                                                   uint32_t bias_hi) {
  return (x + (x > half ? bias_hi : bias_lo)) ^ 0x80808080u;
}

// Four words -> four dwords, dword j holding byte j of words a, b, c, d (in
// that order): a 4x4 byte transpose in two rounds of byte permutes
// (v_perm_b32 picks bytes 0-3 from its second operand, 4-7 from its first).
__device__ __forceinline__ void bytes_transpose4(uint32_t a, uint32_t b, uint32_t c, uint32_t d,
                                                 uint32_t o[4]) {
  const uint32_t ab01 = __builtin_amdgcn_perm(b, a, 0x05010400u);  // a0 b0 a1 b1
  const uint32_t ab23 = __builtin_amdgcn_perm(b, a, 0x07030602u);  // a2 b2 a3 b3
  const uint32_t cd01 = __builtin_amdgcn_perm(d, c, 0x05010400u);  // c0 d0 c1 d1
  const uint32_t cd23 = __builtin_amdgcn_perm(d, c, 0x07030602u);  // c2 d2 c3 d3
  o[0] = __builtin_amdgcn_perm(cd01, ab01, 0x05040100u);           // a0 b0 c0 d0
  o[1] = __builtin_amdgcn_perm(cd01, ab01, 0x07060302u);           // a1 b1 c1 d1
  o[2] = __builtin_amdgcn_perm(cd23, ab23, 0x05040100u);           // a2 b2 c2 d2
  o[3] = __builtin_amdgcn_perm(cd23, ab23, 0x07060302u);           // a3 b3 c3 d3
}

// 16 digit words (k = 0..15 of one row or column) -> 4 limb fragments.
__device__ __forceinline__ void limb_fragments(const uint32_t w[16], v4i f[4]) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    uint32_t o[4];
    bytes_transpose4(w[4 * u], w[4 * u + 1], w[4 * u + 2], w[4 * u + 3], o);
#pragma unroll
    for (int j = 0; j < 4; ++j) f[j][u] = (int)o[j];
  }
}

// ---------------------------------------------------------------------------
// Limb packing: a p-major operand -> MFMA fragments.
// Source word (row, k, p) at src[row * s_row + k * s_k + p] for rows
// row_base .. rows-1 and k < K; fragment lane (li, lg) of (p, t, s, j) at
// dst[p * d_p + (t / tgroup) * d_g + (t % tgroup) * d_t + s * d_s +
// (4 j + lg) * lpg + li] for li < lpg,
// holding limb j of row row_base + 16t + li at k = 64s + 16lg + 0..15 (with
// lpg = 16 that is j * 64 + lane, whole 1 KiB fragments).  Rows past `rows`
// and k past K give zero bytes.
// ---------------------------------------------------------------------------

// One workgroup per (32 points, tile t, `sub` consecutive (step s, k-group
// lg) pairs): 16 row slots x 16 k are read as 256 runs of 32 points (128
// contiguous bytes each) into LDS, then each thread forms the fragment lanes
// of points p: 16 words -> centred signed limbs -> 4 x 16 bytes.  With
// lpg = 16 a slot is a row of the tile and sub = 1; a small batch's compact
// packing (lpg < 16 live rows) gives slot = j * lpg2 + row (lpg2 = lpg
// rounded up to a power of two) to sub = 16 / lpg2 pairs, so every slot
// holds live rows.  Pair index u * sub + j is lg + 4s.  Needs P % 4 == 0, a
// 16-byte aligned source and strides that are multiples of 4 words.
// LDS word of (slot r, point p): r*32 + ((p + 4*(r/16)) mod 32), which keeps
// both the 16-byte row stores and the per-thread column reads at two-way
// bank conflicts at most.
constexpr int kPackPoints = 32;
__host__ __device__ __forceinline__ uint32_t pack_lpg2(uint32_t lpg) {
  uint32_t v = 1;
  while (v < lpg) v <<= 1;
  return v;  // lpg in [1, 16]
}

__global__ __launch_bounds__(kThreads) void pack_limbs4_kernel(PackDesc d, uint64_t pblocks, uint64_t total) {
  __shared__ uint32_t tile[256 * kPackPoints];
  const uint32_t tid = threadIdx.x;
  const uint32_t lpg2 = pack_lpg2(d.lpg), sub = 16 / lpg2, pairs = 4 * d.S;
  for (uint64_t id = blockIdx.x; id < total; id += gridDim.x) {
    const uint64_t pb = id % pblocks;
    const uint64_t rest = id / pblocks;
    const uint32_t t = (uint32_t)(rest % d.tiles);
    const uint32_t u = (uint32_t)(rest / d.tiles);
    const uint64_t p0 = pb * kPackPoints;
    __syncthreads();  // the previous item's reads of `tile` are done
#pragma unroll
    for (int pass = 0; pass < 8; ++pass) {
      const uint32_t r = pass * 32 + tid / 8, c4 = (tid % 8) * 4;
      const uint32_t slot = r / 16, rr = slot % lpg2, pr = u * sub + slot / lpg2;
      const uint64_t row = (uint64_t)d.row_base + t * 16 + rr;
      const uint32_t k = (pr / 4) * 64 + (pr % 4) * 16 + r % 16;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (rr < d.lpg && pr < pairs && row < d.rows && k < d.K && p0 + c4 < d.P)
        v = *reinterpret_cast<const uint4*>(d.src + row * d.s_row + (uint64_t)k * d.s_k + p0 + c4);
      *reinterpret_cast<uint4*>(&tile[r * kPackPoints + ((c4 + 4 * (r / 16)) % kPackPoints)]) = v;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t li = tid % 16, pp = h * 16 + tid / 16;  // li: the slot
      const uint32_t rr = li % lpg2, pr = u * sub + li / lpg2;
      const uint64_t p = p0 + pp;
      if (p >= d.P || rr >= d.lpg || pr >= pairs) continue;
      const uint32_t s = pr / 4, lg = pr % 4;
      const uint32_t q = d.q[p / d.N], half = q / 2;
      uint32_t w[16];
#pragma unroll
      for (int i = 0; i < 16; ++i)
        w[i] = centred_digits(tile[(li * 16 + i) * kPackPoints + ((pp + 4 * li) % kPackPoints)], half,
                              0x80808080u, 0x80808080u - q);  // x = 0 gives digit bytes 0
      v4i f[4];
      limb_fragments(w, f);
      v4i* dst = static_cast<v4i*>(d.dst) + p * d.d_p + (t / d.tgroup) * d.d_g + (t % d.tgroup) * d.d_t +
                 s * d.d_s + lg * d.lpg + rr;
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[j * 4 * d.lpg] = f[j];
    }
  }
}

// Any P, strides and alignment: one thread per fragment lane, 16 strided loads.
__global__ __launch_bounds__(kThreads) void pack_limbs_kernel(PackDesc d, uint64_t total) {
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t e = (uint64_t)blockIdx.x * kThreads + threadIdx.x; e < total; e += stride) {
    const uint32_t lane = (uint32_t)(e % 64);
    uint64_t rest = e / 64;
    const uint32_t s = (uint32_t)(rest % d.S);
    rest /= d.S;
    const uint32_t t = (uint32_t)(rest % d.tiles);
    const uint64_t p = rest / d.tiles;
    const uint32_t li = lane % 16, lg = lane / 16;
    if (li >= d.lpg) continue;
    const uint64_t row = (uint64_t)d.row_base + t * 16 + li;
    const uint32_t q = d.q[p / d.N], half = q / 2;
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t k = s * 64 + lg * 16 + i;
      const uint32_t x = (row < d.rows && k < d.K) ? d.src[row * d.s_row + (uint64_t)k * d.s_k + p] : 0u;
      w[i] = centred_digits(x, half, 0x80808080u, 0x80808080u - q);
    }
    v4i f[4];
    limb_fragments(w, f);
    v4i* dst = static_cast<v4i*>(d.dst) + p * d.d_p + (t / d.tgroup) * d.d_g + (t % d.tgroup) * d.d_t +
               s * d.d_s + lg * d.lpg + li;
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[j * 4 * d.lpg] = f[j];
  }
}

// ---------------------------------------------------------------------------
// The scan.
// ---------------------------------------------------------------------------

#ifndef PIRSCAN_DIRECT_XCD_CHUNK
#define PIRSCAN_DIRECT_XCD_CHUNK 64  // workgroups per XCD chunk, up-to-16-row scan (4 points)
#endif
#ifndef PIRSCAN_RING_XCD_CHUNK
#define PIRSCAN_RING_XCD_CHUNK 8  // workgroups per XCD chunk, 17-32-row scan (1 point at D1 = 1024)
#endif
// (scan_remap: measured at 48 GiB, one contiguous eighth of the grid per XCD
// is 7-9% slower than chunks of 8-64 workgroups dealt round the XCDs, at
// every batch size.)
// The packed DB keeps column tiles in groups whose fragments follow each
// other step after step: per point [t / G][s][t % G][limb][lane], so the
// tiles a workgroup scans form one contiguous run.  G = 16 (T padded to a
// multiple of 16; measured best against 1, 4 and 8), or T itself below 16.
__host__ __device__ __forceinline__ uint32_t tile_group(uint32_t T) { return T < 16 ? T : 16; }
__host__ __device__ __forceinline__ uint32_t padded_tiles(uint32_t T) {
  const uint32_t G = tile_group(T);
  return (T + G - 1) / G * G;
}
// Offset (in 16-byte units) of fragment (point p, column tile t, step 0, limb 0).
__device__ __forceinline__ uint64_t db_tile_offset(uint64_t p, uint32_t t, uint32_t S, uint32_t T) {
  const uint32_t G = tile_group(T);
  return (p * padded_tiles(T) + (uint64_t)(t / G) * G) * S * kFrag + (uint64_t)(t % G) * kFrag;
}

struct MfmaEpilogue {
  uint32_t w[kMaxLimbs][7];  // 2^(8d) mod q
  uint32_t corr[kMaxLimbs];  // -(2^31 * sum_d w_d) mod q: undoes the +2^31 offsets
};

#ifndef PIRSCAN_NT_STORE
#define PIRSCAN_NT_STORE 1
#endif
#ifndef PIRSCAN_STAGE_STORE
#define PIRSCAN_STAGE_STORE 1  // outputs leave through LDS as whole-row 16-byte stores
#endif

// Residue of accumulator element e of (row tile mt, column tile b): the
// seven diagonals folded with hi * (2^32 mod q) + lo, then one Barrett step.
template <int MT, int NTW>
__device__ __forceinline__ uint32_t fold_residue(const MfmaEpilogue& ep, const v4i (&acc)[7][MT][NTW], int mt,
                                                 int b, int e, uint32_t limb, uint64_t c32, uint64_t mu,
                                                 uint32_t q) {
  uint64_t x = ep.corr[limb];
#pragma unroll
  for (int dd = 0; dd < 7; ++dd) {
    x = (x >> 32) * c32 + (uint32_t)x;  // <= (2^32-1)(c32+1) < 2^63
    x += (uint64_t)((uint32_t)acc[dd][mt][b][e] + 0x80000000u) * ep.w[limb][dd];
  }
  uint64_t r = x - __umul64hi(x, mu) * q;
  if (r >= q) r -= q;
  return (uint32_t)r;
}

// Epilogue of a wave: folds the seven diagonals of each accumulator element
// into its residue and stores rows < m - m_base, columns < D1 of the wave's
// tiles to out_t[p][m][D1]; lane (li, lg) holds rows mt * 16 + 4 * lg + e,
// column li of the 16 x 16 tile.
template <int MT, int NTW>
__device__ __forceinline__ void store_outputs(const RowselLaunch& a, const MfmaEpilogue& ep,
                                              const v4i (&acc)[7][MT][NTW], uint32_t* __restrict__ out_t,
                                              uint64_t p, uint32_t g, uint32_t limb, uint32_t m_base, uint32_t lg,
                                              uint32_t li) {
  const uint64_t c32 = a.lc.c[limb], mu = a.lc.mu[limb];
  const uint32_t q = a.lc.q[limb];
  const uint32_t mrows = a.m - m_base;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t row = mt * 16 + 4 * lg + e;
      if (row >= mrows) continue;
#pragma unroll
      for (int b = 0; b < NTW; ++b) {
        const uint32_t c = (g * NTW + b) * 16 + li;
        if (c >= a.D1) continue;
        const uint32_t r = fold_residue<MT, NTW>(ep, acc, mt, b, e, limb, c32, mu, q);
        uint32_t* dst = out_t + ((uint64_t)p * a.m + m_base + row) * a.D1 + c;
        if (PIRSCAN_NT_STORE) __builtin_nontemporal_store(r, dst);
        else *dst = r;
      }
    }
  }
}

// The same residues written to an LDS block stage[row][col0 + b * 16 + li]
// (row stride ld words), for a later store of whole rows.
template <int MT, int NTW>
__device__ __forceinline__ void stage_outputs(const RowselLaunch& a, const MfmaEpilogue& ep,
                                              const v4i (&acc)[7][MT][NTW], uint32_t* stage, uint32_t ld,
                                              uint32_t col0, uint32_t limb, uint32_t mrows, uint32_t lg,
                                              uint32_t li) {
  const uint64_t c32 = a.lc.c[limb], mu = a.lc.mu[limb];
  const uint32_t q = a.lc.q[limb];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t row = mt * 16 + 4 * lg + e;
      if (row >= mrows) continue;
#pragma unroll
      for (int b = 0; b < NTW; ++b)
        stage[row * ld + col0 + b * 16 + li] = fold_residue<MT, NTW>(ep, acc, mt, b, e, limb, c32, mu, q);
    }
  }
}

// Rows 0 .. mrows-1 of an LDS block of `width` columns (a multiple of 4, row
// stride ld, a multiple of 4) to out_t[p][m_base + row][c0 ..]: `threads`
// consecutive threads (thread index `tid`) cover the block as 16-byte
// stores, width / 4 per row, so each store instruction writes whole rows.
// Needs D1 % 4 == 0 and c0 % 4 == 0 (16-byte aligned rows).
__device__ __forceinline__ void store_staged(const uint32_t* stage, uint32_t ld, uint32_t width, uint32_t mrows,
                                             uint32_t* __restrict__ out_t, uint64_t p, uint32_t m,
                                             uint32_t m_base, uint32_t D1, uint32_t c0, uint32_t tid,
                                             uint32_t threads) {
  const uint32_t lpr = width / 4, rpp = threads / lpr;
  for (uint32_t r0 = 0; r0 < mrows; r0 += rpp) {
    const uint32_t row = r0 + tid / lpr, c4 = (tid % lpr) * 4;
    if (row < mrows && tid < rpp * lpr && c0 + c4 < D1) {
      const v4i v = *reinterpret_cast<const v4i*>(stage + row * ld + c4);
      v4i* dst = reinterpret_cast<v4i*>(out_t + ((uint64_t)p * m + m_base + row) * D1 + c0 + c4);
      if (PIRSCAN_NT_STORE) __builtin_nontemporal_store(v, dst);
      else *dst = v;
    }
  }
}


// Workgroup = 4 wavefronts on one point p; wave w scans column tiles
// (4g' + w) * NTW .. + NTW-1 (g' = the workgroup's quad of tile groups) over
// every 64-k step, for MT row tiles of 16 (rows m_base ..).  Per step a wave
// consumes NTW x 4 KiB of packed DB from HBM (register double buffer, one
// step ahead) and MT x 4 KiB of A fragments from the shared LDS ring, and
// issues 16 * MT * NTW MFMAs.  Waves past the last tile group run the same
// loads, barriers and MFMAs on clamped tiles and store nothing.  Each live
// wave's residues leave through its own LDS block as whole 128-byte rows.
template <int MT, int NTW>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(MT == 2 ? 2 : 3)))
void rowsel_packed_kernel(RowselLaunch a, MfmaEpilogue ep, const v4i* __restrict__ limbs,
                          const v4i* __restrict__ dbp, uint32_t* __restrict__ out_t, uint32_t m_base,
                          uint32_t S, uint32_t T, uint32_t ngroups, uint32_t gq) {
  constexpr int kAFrags = MT * 4;  // A fragments per step (row tile x limb)
  __shared__ v4i aring[kRing][kAFrags * 64];
  constexpr uint32_t kStageLd = NTW * 16 + 4;  // a wave's output block: MT * 16 rows x NTW * 16 columns
  __shared__ uint32_t ostage[PIRSCAN_STAGE_STORE ? 4 : 1][PIRSCAN_STAGE_STORE ? MT * 16 * kStageLd : 1];
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t li = lane % 16, lg = lane / 16;
  const uint32_t wg = scan_remap<PIRSCAN_RING_XCD_CHUNK>(blockIdx.x, gridDim.x);  // grid = P * gq exactly
  const uint64_t p = wg / gq;
  const uint32_t g = (wg % gq) * 4 + wave;
  const bool live = g < ngroups;
  const uint32_t limb = (uint32_t)(p / a.N);

  // this wave's column tiles (clamped for dead waves and the last group)
  const uint64_t gstride = (uint64_t)tile_group(T) * kFrag;  // one step of a tile group
  const v4i* bcol[NTW];
#pragma unroll
  for (int b = 0; b < NTW; ++b) {
    const uint32_t t = g * NTW + b < T ? g * NTW + b : T - 1;
    bcol[b] = dbp + db_tile_offset(p, t, S, T) + lane;
  }
  const v4i* ap = limbs + (p * S) * (uint64_t)(MT * kFrag) + lane;

  v4i acc[7][MT][NTW];
#pragma unroll
  for (int dd = 0; dd < 7; ++dd)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int b = 0; b < NTW; ++b) acc[dd][mt][b] = v4i{0, 0, 0, 0};

  v4i bb[2][NTW][4];
  auto load_b = [&](int slot, uint32_t s) {
    const uint32_t ss = s < S ? s : S - 1;  // past the end: a harmless reload of the last step
#pragma unroll
    for (int b = 0; b < NTW; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j) bb[slot][b][j] = __builtin_nontemporal_load(bcol[b] + ss * gstride + j * 64);
  };
  // step s's A fragments -> ring slot s % kRing; wave w moves fragments w, w+4
  auto issue_a = [&](uint32_t s) {
    const uint32_t ss = s < S ? s : S - 1;
    v4i* slot = aring[s % kRing];
#pragma unroll
    for (int h = 0; h < MT; ++h) {
      const uint32_t f = wave + 4 * h;
      __builtin_amdgcn_global_load_lds((const void*)(ap + (ss * kAFrags + f) * 64), LDS_PTR(slot + f * 64), 16,
                                       0, 0);
    }
  };
  // One step.  Issue order per step: B(s+1), then A(s+2); so at the wait of
  // step s only A(s+1)'s MT loads may still be in flight, and B(s), A(s) have
  // landed (A(s) was issued two steps back).  The barrier makes every wave's
  // share of A(s) visible and tells each wave that all others have finished
  // reading slot (s-1) % kRing, which A(s+2) then overwrites.  Scheduling
  // barriers keep the order: ring reads, next loads, then the MFMAs (which
  // would otherwise pull the next step's loads behind them).
  auto step = [&](auto slot_tag, uint32_t s) {
    constexpr int slot = decltype(slot_tag)::value;
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(MT));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    const v4i* as = aring[s % kRing] + lane;
    v4i af[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) af[mt][j] = as[(mt * 4 + j) * 64];
    __builtin_amdgcn_sched_barrier(0);
    load_b(slot ^ 1, s + 1);
    issue_a(s + kRing - 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int b = 0; b < NTW; ++b)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i + j][mt][b] =
                __builtin_amdgcn_mfma_i32_16x16x64_i8(af[mt][i], bb[slot][b][j], acc[i + j][mt][b], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  load_b(0, 0);
#pragma unroll
  for (int r = 0; r < kRing - 1; ++r) issue_a(r);
  uint32_t s = 0;
  for (; s + 1 < S; s += 2) {
    step(std::integral_constant<int, 0>{}, s);
    step(std::integral_constant<int, 1>{}, s + 1);
  }
  if (s < S) step(std::integral_constant<int, 0>{}, s);
  __builtin_amdgcn_s_waitcnt(0);  // no ring load may outlive the workgroup's LDS

  if (!live) return;
  if (PIRSCAN_STAGE_STORE && a.D1 % 4 == 0) {
    // through a wave-private LDS block, so each store writes whole 128-byte rows
    uint32_t* st = ostage[PIRSCAN_STAGE_STORE ? wave : 0];
    stage_outputs<MT, NTW>(a, ep, acc, st, kStageLd, 0, limb, a.m - m_base, lg, li);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    store_staged(st, kStageLd, NTW * 16, a.m - m_base < MT * 16 ? a.m - m_base : MT * 16, out_t, p, a.m, m_base,
                 a.D1, g * NTW * 16, lane, 64);
    return;
  }
  store_outputs<MT, NTW>(a, ep, acc, out_t, p, g, limb, m_base, lg, li);
}

// Small batches (one pass of at most 16 rows): no LDS ring, and a barrier
// only in the epilogue.  Each wave (point p, column tiles g*NTW ..
// g*NTW+NTW-1) loads its own A fragments with the DB fragments, kDepth - 1
// steps ahead (a register ring).  The A side is packed
// compactly, lanes_per_group = mrows (only the live rows of each k-group), so
// it costs the bytes of ct itself; lanes of rows past mrows read their group's
// row-0 lane instead (same line, no branch).  Their output rows are copies of
// row 0's and are never stored (MFMA rows are independent).
template <int NTW>
__global__ __launch_bounds__(kThreads) void rowsel_packed_direct_kernel(RowselLaunch a, MfmaEpilogue ep,
                                                                        const v4i* __restrict__ limbs,
                                                                        const v4i* __restrict__ dbp,
                                                                        uint32_t* __restrict__ out_t,
                                                                        uint32_t m_base, uint32_t S, uint32_t T,
                                                                        uint32_t ngroups, uint64_t items) {
  constexpr uint32_t kStageLd = 64 * NTW + 4;  // the workgroup's output block: up to 16 rows x 64 NTW columns
  __shared__ uint32_t dstage[PIRSCAN_STAGE_STORE ? 16 * kStageLd : 1];
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t li = lane % 16, lg = lane / 16;
  const uint64_t item = (uint64_t)scan_remap<PIRSCAN_DIRECT_XCD_CHUNK>(blockIdx.x, gridDim.x) * 4 + wave;
  // a workgroup returns here whole or not at all whenever the staged store
  // below (the kernel's only barrier) is taken: then items % 4 == 0
  if (item >= items) return;
  const uint64_t p = item / ngroups;
  const uint32_t g = (uint32_t)(item % ngroups);
  const uint32_t limb = (uint32_t)(p / a.N);
  const uint32_t mrows = a.m - m_base;  // 1..16: the compact A's lanes per k-group
  const uint32_t astep = 16 * mrows;    // A fragments of one step: 4 limbs x 4 groups x mrows

  const uint64_t gstride = (uint64_t)tile_group(T) * kFrag;  // one step of a tile group
  const v4i* bcol[NTW];
#pragma unroll
  for (int b = 0; b < NTW; ++b) {
    const uint32_t t = g * NTW + b < T ? g * NTW + b : T - 1;
    bcol[b] = dbp + db_tile_offset(p, t, S, T) + lane;
  }
  const v4i* ap = limbs + p * S * astep + lg * mrows + (li < mrows ? li : 0);

  v4i acc[7][1][NTW];
#pragma unroll
  for (int dd = 0; dd < 7; ++dd)
#pragma unroll
    for (int b = 0; b < NTW; ++b) acc[dd][0][b] = v4i{0, 0, 0, 0};
  // a register ring of kDepth steps: step s + kDepth - 1 is loaded while s is multiplied
  constexpr int kDepth = NTW == 1 ? PIRSCAN_DIRECT_DEPTH : 2;
  v4i aa[kDepth][4], bb[kDepth][NTW][4];
  auto load = [&](int slot, uint32_t s) {
    const uint32_t ss = s < S ? s : S - 1;  // past the end: a harmless reload of the last step
#pragma unroll
    for (int j = 0; j < 4; ++j) aa[slot][j] = ap[ss * astep + j * 4 * mrows];
#pragma unroll
    for (int b = 0; b < NTW; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j) bb[slot][b][j] = __builtin_nontemporal_load(bcol[b] + ss * gstride + j * 64);
  };
  auto step = [&](auto slot_tag, uint32_t s) {
    constexpr int slot = decltype(slot_tag)::value;
    load((slot + kDepth - 1) % kDepth, s + kDepth - 1);
    __builtin_amdgcn_sched_barrier(0);  // keep the later steps' loads ahead of this step's MFMAs
#pragma unroll
    for (int b = 0; b < NTW; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i + j][0][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aa[slot][i], bb[slot][b][j], acc[i + j][0][b], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  using Slot0 = std::integral_constant<int, 0>;
  using Slot1 = std::integral_constant<int, 1>;
  using Slot2 = std::integral_constant<int, 2>;
  if constexpr (kDepth == 2) {
    load(0, 0);
    uint32_t s = 0;
    for (; s + 1 < S; s += 2) {
      step(Slot0{}, s);
      step(Slot1{}, s + 1);
    }
    if (s < S) step(Slot0{}, s);
  } else {
    static_assert(kDepth == 3, "the direct kernel's ring holds 2 or 3 steps");
    load(0, 0);
    load(1, 1);
    uint32_t s = 0;
    for (; s + 2 < S; s += 3) {
      step(Slot0{}, s);
      step(Slot1{}, s + 1);
      step(Slot2{}, s + 2);
    }
    if (s < S) step(Slot0{}, s);
    if (s + 1 < S) step(Slot1{}, s + 1);
  }
  if (PIRSCAN_STAGE_STORE && ngroups % 4 == 0 && a.D1 % 4 == 0) {
    // every wave of the workgroup is live and on point p, tiles g - wave ..
    // g - wave + 3: their rows meet in LDS and leave as whole-row stores
    stage_outputs<1, NTW>(a, ep, acc, dstage, kStageLd, wave * NTW * 16, limb, mrows, lg, li);
    __syncthreads();
    store_staged(dstage, kStageLd, 64 * NTW, mrows, out_t, p, a.m, m_base, a.D1, (g - wave) * NTW * 16,
                 threadIdx.x, kThreads);
    return;
  }
  store_outputs<1, NTW>(a, ep, acc, out_t, p, g, limb, m_base, lg, li);
}

uint64_t align256(uint64_t x) { return (x + 255) / 256 * 256; }
uint32_t steps_of(uint32_t D0) { return (D0 + 63) / 64; }
uint32_t tiles_of(uint32_t D1) { return (D1 + 15) / 16; }

struct PackedWs {
  uint64_t limbs, out_t, total;  // byte offsets / size
};

// A fragments of the largest pass: the direct kernel's compact m x 4 limbs x
// 4 groups per step (m <= 16), else two whole 16-row tiles.
PackedWs packed_workspace(uint64_t P, uint32_t m, uint32_t D0, uint32_t D1) {
  const uint64_t a_step = m <= kDirectRows ? 16ull * m : 2ull * kFrag;  // v4i per point and step
  PackedWs w{};
  w.limbs = 0;
  w.out_t = align256((uint64_t)P * steps_of(D0) * a_step * 16);
  w.total = w.out_t + align256(4ull * P * m * D1);
  return w;
}

template <int MT, int NTW>
hipError_t launch_scan(const RowselLaunch& a, const MfmaEpilogue& ep, const v4i* limbs, const v4i* dbp,
                       uint32_t* out_t, uint32_t m_base, hipStream_t stream) {
  const uint32_t S = steps_of(a.D0), T = tiles_of(a.D1);
  const uint32_t ngroups = (T + NTW - 1) / NTW, gq = (ngroups + 3) / 4;
  const uint64_t grid = a.P * gq;
  if (grid == 0 || grid > 0x7FFFFFFFull) return hipErrorInvalidValue;
  hipLaunchKernelGGL((rowsel_packed_kernel<MT, NTW>), dim3((uint32_t)grid), dim3(kThreads), 0, stream, a, ep,
                     limbs, dbp, out_t, m_base, S, T, ngroups, gq);
  return hipGetLastError();
}

template <int NTW>
hipError_t launch_scan_direct(const RowselLaunch& a, const MfmaEpilogue& ep, const v4i* limbs, const v4i* dbp,
                              uint32_t* out_t, uint32_t m_base, hipStream_t stream) {
  const uint32_t S = steps_of(a.D0), T = tiles_of(a.D1);
  const uint32_t ngroups = (T + NTW - 1) / NTW;
  const uint64_t items = a.P * ngroups, grid = (items + 3) / 4;
  if (grid == 0 || grid > 0x7FFFFFFFull) return hipErrorInvalidValue;
  hipLaunchKernelGGL((rowsel_packed_direct_kernel<NTW>), dim3((uint32_t)grid), dim3(kThreads), 0, stream, a, ep,
                     limbs, dbp, out_t, m_base, S, T, ngroups, items);
  return hipGetLastError();
}

}  // namespace

bool rowsel_packed_ok(const uint32_t* q, uint32_t R, uint32_t D0) {
  if (D0 > kPackedMaxD0) return false;
  for (uint32_t r = 0; r < R; ++r)
    if (q[r] >= (1u << 31)) return false;
  return true;
}

uint64_t packed_layout_bytes(uint64_t P, uint32_t D0, uint32_t D1) {
  return P * padded_tiles(tiles_of(D1)) * steps_of(D0) * (uint64_t)kFrag * 16;
}

hipError_t launch_pack(const PackDesc& d, hipStream_t stream) {
  auto a16 = [](const void* ptr) { return reinterpret_cast<uintptr_t>(ptr) % 16 == 0; };
  if (d.P % 4 == 0 && d.s_row % 4 == 0 && d.s_k % 4 == 0 && a16(d.src)) {
    const uint64_t pblocks = (d.P + kPackPoints - 1) / kPackPoints;
    const uint32_t sub = 16 / pack_lpg2(d.lpg);
    const uint64_t total = pblocks * d.tiles * ((4ull * d.S + sub - 1) / sub);
    const uint64_t grid = total < (1ull << 20) ? total : (1ull << 20);
    hipLaunchKernelGGL(pack_limbs4_kernel, dim3((uint32_t)grid), dim3(kThreads), 0, stream, d, pblocks, total);
  } else {
    const uint64_t total = d.P * d.tiles * d.S * 64;
    uint64_t grid = (total + kThreads - 1) / kThreads;
    if (grid > (1u << 20)) grid = 1u << 20;
    hipLaunchKernelGGL(pack_limbs_kernel, dim3((uint32_t)grid), dim3(kThreads), 0, stream, d, total);
  }
  return hipGetLastError();
}

hipError_t launch_pack_operand(const uint32_t* src, void* dst, uint64_t P, uint32_t N, const uint32_t* q,
                               uint32_t R, uint32_t rows, uint32_t K, uint64_t s_row, uint64_t s_k,
                               hipStream_t stream) {
  PackDesc d{};
  d.src = src;
  d.dst = dst;
  d.P = P;
  d.N = N;
  d.rows = rows;
  d.row_base = 0;
  d.K = K;
  d.s_row = s_row;
  d.s_k = s_k;
  d.tiles = tiles_of(rows);
  d.S = steps_of(K);
  d.lpg = 16;
  d.tgroup = tile_group(d.tiles);
  d.d_t = kFrag;
  d.d_s = (uint64_t)d.tgroup * kFrag;
  d.d_g = (uint64_t)d.S * d.d_s;
  d.d_p = (uint64_t)padded_tiles(d.tiles) * d.S * kFrag;
  for (uint32_t r = 0; r < R; ++r) d.q[r] = q[r];
  return launch_pack(d, stream);
}

size_t rowsel_packed_workspace_bytes(uint64_t P, uint32_t m, uint32_t D0, uint32_t D1) {
  return (size_t)packed_workspace(P, m, D0, D1).total;
}

hipError_t launch_rowsel_packed(const RowselLaunch& a, uint32_t R, void* workspace, hipStream_t stream) {
  const PackedWs ws = packed_workspace(a.P, a.m, a.D0, a.D1);
  uint8_t* base = static_cast<uint8_t*>(workspace);
  v4i* limbs = reinterpret_cast<v4i*>(base + ws.limbs);
  uint32_t* out_t = reinterpret_cast<uint32_t*>(base + ws.out_t);
  const v4i* dbp = reinterpret_cast<const v4i*>(a.dbt);
  const uint32_t S = steps_of(a.D0);

  MfmaEpilogue ep{};
  for (uint32_t r = 0; r < R; ++r) {
    const uint64_t q = a.lc.q[r];
    uint64_t sum = 0;
    for (int d = 0; d < 7; ++d) {
      ep.w[r][d] = (uint32_t)((((unsigned __int128)1) << (8 * d)) % q);
      sum += ep.w[r][d];
    }
    const uint64_t off = (uint64_t)(((unsigned __int128)(1ull << 31) * sum) % q);
    ep.corr[r] = (uint32_t)((q - off) % q);
  }

  hipError_t e = hipSuccess;
  for (uint64_t mb = 0; mb < a.m; mb += 32) {
    const uint32_t m_base = (uint32_t)mb;
    const uint32_t rows = a.m - m_base < 32 ? a.m - m_base : 32;
    const bool direct = rows <= kDirectRows;
    // ct rows m_base .. m_base + rows -> A fragments [p][s][row tile][limb][group][lane]:
    // whole 16-lane groups for the ring kernel, only the live rows for the direct one
    PackDesc d{};
    d.src = a.ct;
    d.dst = limbs;
    d.P = a.P;
    d.N = a.N;
    d.rows = a.m;
    d.row_base = m_base;
    d.K = a.D0;
    d.s_row = a.ct_sm;
    d.s_k = a.ct_sk;
    d.tiles = direct ? 1 : 2;
    d.lpg = direct ? rows : 16;
    d.S = S;
    d.tgroup = d.tiles;  // one group: [p][s][tile][limb][group][lane]
    d.d_t = 16ull * d.lpg;
    d.d_s = d.tiles * d.d_t;
    d.d_g = 0;
    d.d_p = (uint64_t)S * d.d_s;
    for (uint32_t r = 0; r < R; ++r) d.q[r] = a.lc.q[r];
    if ((e = launch_pack(d, stream)) != hipSuccess) return e;
    timer_mark_start(stream);  // first pass only
    // one column tile per wave while the A stream is small next to the DB's
    // (rows <= 4: at most a quarter), four beyond, which divides it by four
    if (direct && rows <= PIRSCAN_SMALL_ROWS) e = launch_scan_direct<PIRSCAN_SMALL_NTW>(a, ep, limbs, dbp, out_t, m_base, stream);
    else if (direct) e = launch_scan_direct<4>(a, ep, limbs, dbp, out_t, m_base, stream);
    else e = launch_scan<2, 2>(a, ep, limbs, dbp, out_t, m_base, stream);
    if (e != hipSuccess) return e;
  }
  timer_mark_stop(stream);
  // out_t [P][m][D1] -> out(mi, n, p), adding ExpPack's body term on the way
  return launch_out_relayout(a, out_t, stream);
}

}  // namespace pirscan
