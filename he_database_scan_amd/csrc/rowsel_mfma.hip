// rowsel_mfma.hip -- batched RowSel on int8 MFMA (gfx950).
//
// For a batch of m >= 16 ciphertext polynomials the per-point product
// C[mi][n] = sum_k A[mi][k] * B[k][n] (A = ct, B = DB, all values < q) is a
// dense contraction, so it runs on v_mfma_i32_16x16x64_i8 instead of the
// 32x32->64-bit VALU multiply (GPIR: "Enabling Practical Private Information
// Retrieval with GPUs" observes that batching raises RowSel's arithmetic
// intensity; VIPIR section 4.1 emulates a wide integer product with INT8
// tensor-core GEMMs on split operands and section 4.2 discusses the modular
// GEMM's reduction overhead).
//
// Every value x < q is first centred, v = x - q if x > q/2 (so |v| <= q/2 <
// 2^30 when q < 2^31), then written in four signed 8-bit limbs
// v = sum_i v_i 2^(8i), v_i in [-128, 127] (the bytes of
// (v + 0x80808080) ^ 0x80808080).  Then
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
//  * ct is relaid per query (two small passes into the caller's workspace):
//    a strided transpose to [p][mi][k] (from RowSel's [mi][k][p] or ExpPack's
//    C [k][mi][p]) and a limb split into MFMA A-fragment order, so
//    each wavefront loads its A fragments as 16-byte vectors.
//  * The DB stays in the scan layout [p][k][n].  Lane (li, lg) of a B fragment
//    needs 16 consecutive k of its column; the two column tiles of a wave take
//    the even and the odd columns of a 32-column block, so the lane's two
//    columns are adjacent and each k comes in one 64-bit load (an instruction
//    covers 128-byte runs of 4 k-rows), addressed by 32-bit offsets from the
//    point's wave-uniform base.  The words are centred and split into the four
//    limb fragments in registers (4 ALU ops per word, and a byte transpose of
//    8 byte-permutes per 4 words).
//  * Results are written per point, [p][mi][n] (contiguous 64-byte runs), and
//    a transpose pass produces the p-major output (adding ExpPack's body term
//    G where the launch carries one).
#include <hip/hip_runtime.h>

#include "internal.hpp"

namespace pirscan {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;

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

// ct_t [P][m][D0] -> A fragments [p][s][mt][limb][lane] (16 bytes each) for
// rows m_base .. m_base + 16*MT of this pass; zero past m and past D0.
__global__ __launch_bounds__(kThreads) void rowsel_limbs_kernel(const uint32_t* __restrict__ ct_t,
                                                                v4i* __restrict__ limbs, uint64_t P,
                                                                uint32_t m, uint32_t D0, uint32_t m_base,
                                                                uint32_t MT, uint32_t S, uint32_t N,
                                                                LimbConsts lc) {
  const uint64_t total = P * S * MT * 64;
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t e = (uint64_t)blockIdx.x * kThreads + threadIdx.x; e < total; e += stride) {
    const uint32_t lane = (uint32_t)(e % 64);
    uint64_t rest = e / 64;
    const uint32_t mt = (uint32_t)(rest % MT);
    rest /= MT;
    const uint32_t s = (uint32_t)(rest % S);
    const uint64_t p = rest / S;
    const uint32_t li = lane % 16, lg = lane / 16;
    const uint32_t mi = m_base + mt * 16 + li;
    const uint32_t q = lc.q[p / N], half = q / 2;
    uint32_t w[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const uint32_t k = s * 64 + lg * 16 + t;
      const uint32_t x = (mi < m && k < D0) ? ct_t[(p * m + mi) * D0 + k] : 0u;
      w[t] = centred_digits(x, half, 0x80808080u, 0x80808080u - q);  // x = 0 gives digit bytes 0
    }
    v4i f[4];
    limb_fragments(w, f);
#pragma unroll
    for (int j = 0; j < 4; ++j) limbs[((((p * S + s) * MT + mt) * 4 + j) * 64) + lane] = f[j];
  }
}

// ct(mi, k, p) -> A fragments [p][s][mt][limb][lane] in one pass, for rows
// m_base .. m_base + 16*MT: one workgroup per (32 points, step s, row tile
// mt, k-group lg).  The 16 rows x 16 k of the tile are read as 256 runs of
// 32 points (128 contiguous bytes each) into LDS, then each thread forms the
// fragment lanes (li, lg) of points p: 16 words (k = 64 s + 16 lg + t) ->
// centred signed limbs -> 4 x 16 bytes, written as 256-byte runs per point
// and limb.  Rows past m and k past D0 are zero.  Needs P % 4 == 0 and a
// 16-byte aligned ct with strides that are multiples of 4 words.
// LDS word of (row r, point p): r*32 + ((p + 4*(r/16)) mod 32), which keeps
// both the 16-byte row stores and the per-thread column reads at two-way
// bank conflicts at most.
constexpr int kPrepPoints = 32;
__global__ __launch_bounds__(kThreads) void rowsel_prep_kernel(RowselLaunch a, v4i* __restrict__ limbs,
                                                               uint32_t m_base, uint32_t MT, uint32_t S,
                                                               uint32_t pblocks) {
  __shared__ uint32_t tile[256 * kPrepPoints];
  const uint32_t tid = threadIdx.x;
  uint32_t id = blockIdx.x;
  const uint32_t pb = id % pblocks;
  id /= pblocks;
  const uint32_t lg = id % 4;
  id /= 4;
  const uint32_t mt = id % MT;
  const uint32_t s = id / MT;
  const uint64_t p0 = (uint64_t)pb * kPrepPoints;
  // load: row r = li*16 + t (mi = m_base + 16 mt + li, k = 64 s + 16 lg + t), 8 threads x 16 B per row
#pragma unroll
  for (int pass = 0; pass < 8; ++pass) {
    const uint32_t r = pass * 32 + tid / 8, c4 = (tid % 8) * 4;
    const uint32_t mi = m_base + mt * 16 + r / 16, k = s * 64 + lg * 16 + r % 16;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (mi < a.m && k < a.D0 && p0 + c4 < a.P)
      v = *reinterpret_cast<const uint4*>(a.ct + mi * a.ct_sm + (uint64_t)k * a.ct_sk + p0 + c4);
    *reinterpret_cast<uint4*>(&tile[r * kPrepPoints + ((c4 + 4 * (r / 16)) % kPrepPoints)]) = v;
  }
  __syncthreads();
  // form: thread -> (li = tid % 16, point pair), two points per thread
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t li = tid % 16, pp = h * 16 + tid / 16;
    const uint64_t p = p0 + pp;
    if (p >= a.P) continue;
    const uint32_t q = a.lc.q[p / a.N], half = q / 2;
    uint32_t w[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const uint32_t r = li * 16 + t;
      w[t] = centred_digits(tile[r * kPrepPoints + ((pp + 4 * li) % kPrepPoints)], half, 0x80808080u,
                            0x80808080u - q);
    }
    v4i f[4];
    limb_fragments(w, f);
    v4i* dst = limbs + (((p * S + s) * MT + mt) * 4) * 64 + li + 16 * lg;
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[j * 64] = f[j];
  }
}

struct MfmaEpilogue {
  uint32_t w[kMaxLimbs][7];  // 2^(8d) mod q
  uint32_t corr[kMaxLimbs];  // -(2^31 * sum_d w_d) mod q: undoes the +2^31 offsets
};

// DB words of one 64-k step into w[nt][t]: 16 consecutive k (from kb) of the
// lane's column in each tile.  CLAMP: the last step, where rows past D0 are
// replaced by row D0-1 (the A limbs are zero there, so any valid row serves).
// PAIR: the lane's two columns are adjacent, so both come in one 64-bit load.
// Offsets are 32-bit words from the point's (wave-uniform) base.
template <int NTW, bool PAIR, bool CLAMP>
__device__ __forceinline__ void load_b_step(const uint32_t* dbp, const uint32_t (&col)[NTW], uint32_t kb,
                                            uint32_t D0, uint32_t D1, uint32_t (&w)[NTW][16]) {
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    uint32_t k = kb + t;
    if constexpr (CLAMP) k = k < D0 ? k : D0 - 1;
    const uint32_t off = k * D1 + col[0];
    if constexpr (PAIR) {
      const uint2 v = *reinterpret_cast<const uint2*>(dbp + off);
      w[0][t] = v.x;
      w[1][t] = v.y;
    } else {
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) w[nt][t] = dbp[off + (col[nt] - col[0])];
    }
  }
}

// One wavefront = one point and NTW column tiles of 16; MT row tiles of 16.
// PAIR: tile 0 takes the even and tile 1 the odd columns of a 32-column
// block (D1 even), so a lane's two columns are one 64-bit word pair.
template <int MT, int NTW, bool PAIR>
__global__ __launch_bounds__(kThreads) void rowsel_mfma_kernel(RowselLaunch a, MfmaEpilogue ep,
                                                               const v4i* __restrict__ limbs,
                                                               uint32_t* __restrict__ out_t,
                                                               uint32_t m_base, uint32_t nblk,
                                                               uint64_t items, uint32_t S) {
  static_assert(!PAIR || NTW == 2, "paired columns need two tiles");
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t li = lane % 16, lg = lane / 16;
  const uint32_t wg = xcd_remap(blockIdx.x, gridDim.x);
  const uint64_t item = (uint64_t)wg * (kThreads / 64) + wave;
  if (item >= items) return;  // no barriers in this kernel
  const uint64_t p = item / nblk;
  const uint32_t n0 = (uint32_t)(item % nblk) * NTW * 16;
  const uint32_t limb = (uint32_t)(p / a.N);
  const uint32_t q = a.lc.q[limb], half = q / 2, bias_hi = 0x80808080u - q;
  const uint32_t D0 = a.D0, D1 = a.D1;

  // the column of this lane in tile nt, clamped (results past D1 are not stored)
  uint32_t col[NTW], cout[NTW];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const uint32_t c = PAIR ? n0 + 2 * li + nt : n0 + nt * 16 + li;
    cout[nt] = c;
    if constexpr (PAIR) col[nt] = (n0 + 2 * li + 1) < D1 ? c : D1 - 2 + nt;  // D1 is even here
    else col[nt] = c < D1 ? c : D1 - 1;
  }
  const uint32_t* dbp = a.dbt + p * (uint64_t)D0 * D1;  // D0*D1 < 2^31 words on this path

  v4i acc[7][MT][NTW];
#pragma unroll
  for (int d = 0; d < 7; ++d)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) acc[d][mt][nt] = v4i{0, 0, 0, 0};

  const v4i* lp = limbs + (p * S) * MT * 4 * 64 + lane;
  for (uint32_t s = 0; s < S; ++s) {
    v4i af[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) af[mt][j] = lp[(((uint64_t)s * MT + mt) * 4 + j) * 64];
    uint32_t w[NTW][16];
    const uint32_t kb = s * 64 + lg * 16;
    if ((s + 1) * 64 <= D0) load_b_step<NTW, PAIR, false>(dbp, col, kb, D0, D1, w);
    else load_b_step<NTW, PAIR, true>(dbp, col, kb, D0, D1, w);
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
#pragma unroll
      for (int t = 0; t < 16; ++t) w[nt][t] = centred_digits(w[nt][t], half, 0x80808080u, bias_hi);
      v4i bf[4];
      limb_fragments(w[nt], bf);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i + j][mt][nt] =
                __builtin_amdgcn_mfma_i32_16x16x64_i8(af[mt][i], bf[j], acc[i + j][mt][nt], 0, 0, 0);
    }
  }

  // Epilogue.  D element e of lane l is (row 4*(l/16) + e, column l%16 of the tile).
  const uint64_t c32 = a.lc.c[limb], mu = a.lc.mu[limb];
  const uint32_t mrows = a.m - m_base;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t row = mt * 16 + 4 * lg + e;
      if (row >= mrows) continue;
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const uint32_t c = cout[nt];
        if (c >= D1) continue;
        uint64_t x = ep.corr[limb];
#pragma unroll
        for (int d = 0; d < 7; ++d) {
          x = (x >> 32) * c32 + (uint32_t)x;  // <= (2^32-1)(c32+1) < 2^63
          x += (uint64_t)((uint32_t)acc[d][mt][nt][e] + 0x80000000u) * ep.w[limb][d];
        }
        uint64_t r = x - __umul64hi(x, mu) * q;
        if (r >= q) r -= q;
        out_t[((uint64_t)p * a.m + m_base + row) * D1 + c] = (uint32_t)r;
      }
    }
  }
}

uint64_t align256(uint64_t x) { return (x + 255) / 256 * 256; }

struct MfmaWs {
  uint64_t ct_t, limbs, out_t, total;  // byte offsets / size
};

MfmaWs mfma_workspace(uint64_t P, uint32_t m, uint32_t D0, uint32_t D1) {
  const uint64_t S = (D0 + 63) / 64;
  const uint32_t mt_max = m >= 32 ? 2 : (m + 15) / 16;
  MfmaWs w{};
  w.ct_t = 0;
  w.limbs = align256(4ull * P * m * D0);
  w.out_t = w.limbs + align256(P * S * mt_max * 4 * 64 * 16);
  w.total = w.out_t + align256(4ull * P * m * D1);
  return w;
}

template <int MT, int NTW>
hipError_t launch_mfma_pass(const RowselLaunch& a, const MfmaEpilogue& ep, const v4i* limbs,
                            uint32_t* out_t, uint32_t m_base, uint32_t S, hipStream_t stream) {
  const uint32_t nblk = (a.D1 + NTW * 16 - 1) / (NTW * 16);
  const uint64_t items = a.P * nblk;
  const uint64_t grid = (items + 3) / 4;
  if (grid == 0 || grid > 0x7FFFFFFFull) return hipErrorInvalidValue;
  // adjacent column pairs need an even row length (8-byte aligned pairs)
  if (a.D1 % 2 == 0)
    hipLaunchKernelGGL((rowsel_mfma_kernel<MT, NTW, true>), dim3((uint32_t)grid), dim3(kThreads), 0, stream,
                       a, ep, limbs, out_t, m_base, nblk, items, S);
  else
    hipLaunchKernelGGL((rowsel_mfma_kernel<MT, NTW, false>), dim3((uint32_t)grid), dim3(kThreads), 0,
                       stream, a, ep, limbs, out_t, m_base, nblk, items, S);
  return hipGetLastError();
}

uint32_t grid_for(uint64_t items) {
  uint64_t g = (items + kThreads - 1) / kThreads;
  if (g > (1u << 20)) g = 1u << 20;
  return (uint32_t)(g ? g : 1);
}

}  // namespace

bool rowsel_mfma_eligible(const RowselLaunch& a, uint32_t R) {
  if (a.m < kRowselMfmaMinRows || a.D0 > 16384) return false;
  if ((uint64_t)a.D0 * a.D1 >= (1ull << 31)) return false;  // 32-bit word offsets within a point
  for (uint32_t r = 0; r < R; ++r)
    if (a.lc.q[r] >= (1u << 31)) return false;
  return true;
}

size_t rowsel_mfma_workspace_bytes(uint64_t P, uint32_t m, uint32_t D0, uint32_t D1) {
  return (size_t)mfma_workspace(P, m, D0, D1).total;
}

hipError_t launch_rowsel_mfma(const RowselLaunch& a, uint32_t R, void* workspace, hipStream_t stream) {
  const MfmaWs ws = mfma_workspace(a.P, a.m, a.D0, a.D1);
  uint8_t* base = static_cast<uint8_t*>(workspace);
  uint32_t* ct_t = reinterpret_cast<uint32_t*>(base + ws.ct_t);
  v4i* limbs = reinterpret_cast<v4i*>(base + ws.limbs);
  uint32_t* out_t = reinterpret_cast<uint32_t*>(base + ws.out_t);
  const uint32_t S = (a.D0 + 63) / 64;

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

  // ct -> A fragments in one pass where the 16-byte point runs are aligned
  const bool fused = a.P % 4 == 0 && a.ct_sm % 4 == 0 && a.ct_sk % 4 == 0 &&
                     reinterpret_cast<uintptr_t>(a.ct) % 16 == 0;
  hipError_t e = hipSuccess;
  if (fused) {
    const uint64_t pblocks = (a.P + kPrepPoints - 1) / kPrepPoints;
    for (uint32_t m_base = 0; m_base < a.m; m_base += 32) {
      const uint32_t MT = a.m - m_base > 16 ? 2 : 1;
      const uint64_t grid = pblocks * 4 * MT * S;
      if (grid > 0x7FFFFFFFull) return hipErrorInvalidValue;
      hipLaunchKernelGGL(rowsel_prep_kernel, dim3((uint32_t)grid), dim3(kThreads), 0, stream, a, limbs,
                         m_base, MT, S, (uint32_t)pblocks);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      timer_mark_start(stream);  // first pass only
      if (MT == 2) e = launch_mfma_pass<2, 2>(a, ep, limbs, out_t, m_base, S, stream);
      else e = launch_mfma_pass<1, 2>(a, ep, limbs, out_t, m_base, S, stream);
      if (e != hipSuccess) return e;
    }
    timer_mark_stop(stream);
    return launch_out_relayout(a, out_t, stream);
  }

  // otherwise: ct(mi, k, p) -> ct_t [P][m][D0], then the limb split
  TransposeDesc tc{};
  tc.src = a.ct;
  tc.dst = ct_t;
  tc.batch = a.m;
  tc.rows = a.D0;
  tc.cols = a.P;
  tc.s_batch = a.ct_sm;
  tc.s_row = a.ct_sk;
  tc.d_batch = a.D0;
  tc.d_row = (uint64_t)a.m * a.D0;
  e = launch_transpose(tc, stream);
  if (e != hipSuccess) return e;
  for (uint32_t m_base = 0; m_base < a.m; m_base += 32) {
    const uint32_t rows = a.m - m_base;
    const uint32_t MT = rows > 16 ? 2 : 1;
    hipLaunchKernelGGL(rowsel_limbs_kernel, dim3(grid_for(a.P * S * MT * 64)), dim3(kThreads), 0, stream,
                       ct_t, limbs, a.P, a.m, a.D0, m_base, MT, S, a.N, a.lc);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    timer_mark_start(stream);  // first pass only
    if (MT == 2) e = launch_mfma_pass<2, 2>(a, ep, limbs, out_t, m_base, S, stream);
    else e = launch_mfma_pass<1, 2>(a, ep, limbs, out_t, m_base, S, stream);
    if (e != hipSuccess) return e;
  }
  timer_mark_stop(stream);
  // out_t [P][m][D1] -> out(mi, n, p), adding ExpPack's body term on the way
  return launch_out_relayout(a, out_t, stream);
}

}  // namespace pirscan
