// rowsel.hip -- RowSel in the NTT/RNS domain on gfx950.
//
// Computes, for every point p of P = R*N independent point-wise GEMMs
// (GPIR: "Enabling Practical Private Information Retrieval with GPUs", the
// RowSel formulation M_out[p,m,n] = sum_k M_in0[p,m,k] * M_in1[p,k,n]):
//
//     out[mi][n][p] = ( sum_k ct[mi][k][p] * db[k][n][p] ) mod q_{p/N}
//
// The same kernel runs VIPIR's ExpPack packing GEMM (section 3.5.2,
// H*C + (0|G)) with the operands' roles swapped: ct = C^T, db = H^T, strided
// ct / out addressing, and the body term G added by the output relayout.
//
// Design (MI355X-first, HBM-bound at small m):
//  * The DB is static, so it is relaid once (transpose_kernel) from the
//    p-major HE layout [k][n][p] to [p][k][n]: for a fixed point every k-row
//    of D1 words is contiguous and a wavefront streams it with 128-bit loads.
//    (GPIR moves RowSel to a transposed layout; VIPIR section 4.2 transposes
//    around its modular GEMM.  Here that transpose is paid once, offline.)
//  * One wavefront owns one point and a slice of 64*NPL columns.  The query
//    ciphertext values ct[.][k][p] are the same for the whole wave, so each
//    workgroup stages them into LDS once per k-chunk and every lane reads
//    them as an LDS broadcast (the per-query relayout of the ct operand).
//  * Products are 32x32->64-bit (v_mad_u64_u32) accumulated lazily in 64 bits
//    (VIPIR section 4.2: primes below 2^29 and 64-bit accumulators defer the
//    reduction over up to 32 multiply-adds).  Every `fold` products the
//    accumulator is folded, hi*2^32 + lo -> hi*(2^32 mod q) + lo, which is one
//    more v_mad_u64_u32, keeps the value congruent mod q and bounds it so the
//    next `fold` products cannot overflow (the bound is computed per prime on
//    the host).  One Barrett reduction per output gives the canonical residue.
//  * Residues are staged per point ([p][mi][n], 128-bit stores into the
//    caller's workspace) and a tiled transpose writes the p-major output: a
//    direct p-major store is one scattered 4-byte write per residue, which
//    HBM serves as a partial-line write and which cost ~13% of the scan.
#include <hip/hip_runtime.h>

#include "internal.hpp"

namespace pirscan {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kLdsWords = 8192;  // 32 KiB of staged ct per workgroup

// ---------------------------------------------------------------------------
// Batched word transposes via 64x64 LDS tiles: R1's one-time DB relayout
// [X][P] -> [P][X], the ExpPack hint relayout, and the per-query ct / output
// relayouts of the batched MFMA path (which fuse ExpPack's body term).
// ---------------------------------------------------------------------------
constexpr int kTile = 64;

template <bool kAdd>
__global__ __launch_bounds__(kThreads) void transpose_kernel(TransposeDesc t, uint64_t tiles_c,
                                                             uint64_t tiles_rc, uint64_t tiles) {
  __shared__ uint32_t tile[kTile][kTile + 1];
  const int tx = threadIdx.x % kTile, ty = threadIdx.x / kTile;
  for (uint64_t id = blockIdx.x; id < tiles; id += gridDim.x) {
    const uint64_t b = id / tiles_rc, rc = id % tiles_rc;
    const uint64_t c0 = (rc % tiles_c) * kTile, r0 = (rc / tiles_c) * kTile;
    const uint32_t* src = t.src + b * t.s_batch;
    for (int i = ty; i < kTile; i += kThreads / kTile) {
      const uint64_t r = r0 + i, c = c0 + tx;
      tile[i][tx] = (r < t.rows && c < t.cols) ? src[r * t.s_row + c] : 0u;
    }
    __syncthreads();
    uint32_t* dst = t.dst + b * t.d_batch;
    for (int i = ty; i < kTile; i += kThreads / kTile) {
      const uint64_t c = c0 + i, r = r0 + tx;
      if (c < t.cols && r < t.rows) {
        uint32_t v = tile[tx][i];
        if constexpr (kAdd) {
          if (b & 1) {  // (0 | G): the body term goes to each client's second column
            const uint64_t q = t.lc.q[r / t.N];
            uint64_t x = (uint64_t)v + t.add[(b >> 1) * t.add_b + c * t.add_c + r];
            if (x >= q) x -= q;
            v = (uint32_t)x;
          }
        }
        dst[c * t.d_row + r] = v;
      }
    }
    __syncthreads();
  }
}

// The same transpose with 16-byte accesses on both sides, for the common case
// where every extent, stride and base pointer is a multiple of 4 words: a
// thread reads 4 consecutive columns of a source row and writes 4
// consecutive rows of a destination row, so a wavefront moves 1 KiB per
// global instruction instead of 256 bytes.  The tile stays 64 x 64 words
// (padded rows keep the LDS column reads at two-way bank conflicts).
typedef uint32_t u32x4t __attribute__((ext_vector_type(4)));

template <bool kAdd>
__global__ __launch_bounds__(kThreads) void transpose4_kernel(TransposeDesc t, uint64_t tiles_c,
                                                              uint64_t tiles_rc, uint64_t tiles) {
  __shared__ uint32_t tile[kTile][kTile + 1];
  const int c4 = (threadIdx.x % 16) * 4, ty = threadIdx.x / 16;  // 16 threads per 64-word row
  for (uint64_t id = blockIdx.x; id < tiles; id += gridDim.x) {
    const uint64_t b = id / tiles_rc, rc = id % tiles_rc;
    const uint64_t c0 = (rc % tiles_c) * kTile, r0 = (rc / tiles_c) * kTile;
    const uint32_t* src = t.src + b * t.s_batch;
#pragma unroll
    for (int i = ty; i < kTile; i += kThreads / 16) {
      const uint64_t r = r0 + i, c = c0 + c4;
      u32x4t v = {0u, 0u, 0u, 0u};
      if (r < t.rows && c < t.cols) v = *reinterpret_cast<const u32x4t*>(src + r * t.s_row + c);
      tile[i][c4] = v.x;
      tile[i][c4 + 1] = v.y;
      tile[i][c4 + 2] = v.z;
      tile[i][c4 + 3] = v.w;
    }
    __syncthreads();
    uint32_t* dst = t.dst + b * t.d_batch;
#pragma unroll
    for (int i = ty; i < kTile; i += kThreads / 16) {
      const uint64_t c = c0 + i, r = r0 + c4;
      if (c < t.cols && r < t.rows) {
        u32x4t v = {tile[c4][i], tile[c4 + 1][i], tile[c4 + 2][i], tile[c4 + 3][i]};
        if constexpr (kAdd) {
          if (b & 1) {  // (0 | G): the body term goes to each client's second column
            const u32x4t g = *reinterpret_cast<const u32x4t*>(t.add + (b >> 1) * t.add_b + c * t.add_c + r);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const uint64_t q = t.lc.q[(r + j) / t.N];
              uint64_t x = (uint64_t)v[j] + g[j];
              if (x >= q) x -= q;
              v[j] = (uint32_t)x;
            }
          }
        }
        *reinterpret_cast<u32x4t*>(dst + c * t.d_row + r) = v;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// R2-R4: the scan.
// ---------------------------------------------------------------------------
// DB columns of one lane.  The DB is streamed exactly once per scan, so its
// loads are non-temporal: they do not displace the staged ct lines and the
// output lines that the workgroups on an XCD share in L2 (non-temporal 128-bit
// reads also sustain a higher HBM read rate on gfx950 than cached ones).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// NT: non-temporal loads, used when each DB word is loaded by exactly one
// lane.  With several row groups per wavefront (G > 1) the same words are
// loaded by G lanes of one instruction, and only cached loads let the later
// lanes hit the line the first one brought in (non-temporal ones re-fetch it
// from HBM).
template <bool NT>
__device__ __forceinline__ u32x4 ld4(const uint32_t* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  else return *reinterpret_cast<const u32x4*>(p);
}
template <bool NT>
__device__ __forceinline__ uint32_t ld1(const uint32_t* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

template <int NPL, bool NT>
struct Vec;
template <bool NT>
struct Vec<8, NT> {
  uint32_t v[8];
  __device__ __forceinline__ void load(const uint32_t* p) {
    const u32x4 t0 = ld4<NT>(p), t1 = ld4<NT>(p + 4);
    v[0] = t0.x; v[1] = t0.y; v[2] = t0.z; v[3] = t0.w;
    v[4] = t1.x; v[5] = t1.y; v[6] = t1.z; v[7] = t1.w;
  }
};
template <bool NT>
struct Vec<4, NT> {
  uint32_t v[4];
  __device__ __forceinline__ void load(const uint32_t* p) {
    const u32x4 t = ld4<NT>(p);
    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
  }
};
template <bool NT>
struct Vec<1, NT> {
  uint32_t v[1];
  __device__ __forceinline__ void load(const uint32_t* p) { v[0] = ld1<NT>(p); }
};

// acc[i][j] += ct value of row i (from LDS) * DB word j of k-row kk.
template <int MR, int RPL, int NPL, bool NT>
__device__ __forceinline__ void mac_row(uint64_t (&acc)[RPL][NPL], const uint32_t* L, uint32_t kk,
                                        const Vec<NPL, NT>& d) {
  uint32_t cv[RPL];
  if constexpr (RPL == 1) {
    cv[0] = L[kk * MR];
  } else if constexpr (RPL == 2) {
    const uint2 t = *reinterpret_cast<const uint2*>(L + kk * MR);
    cv[0] = t.x;
    cv[1] = t.y;
  } else {
#pragma unroll
    for (int i = 0; i < RPL; i += 4) {
      const uint4 t = *reinterpret_cast<const uint4*>(L + kk * MR + i);
      cv[i] = t.x;
      cv[i + 1] = t.y;
      cv[i + 2] = t.z;
      cv[i + 3] = t.w;
    }
  }
#pragma unroll
  for (int i = 0; i < RPL; ++i)
#pragma unroll
    for (int j = 0; j < NPL; ++j) acc[i][j] += (uint64_t)cv[i] * d.v[j];
}

// fold: hi*2^32 + lo == hi*(2^32 mod q) + lo  (mod q)
template <int RPL, int NPL>
__device__ __forceinline__ void fold_acc(uint64_t (&acc)[RPL][NPL], uint64_t cfold) {
#pragma unroll
  for (int i = 0; i < RPL; ++i)
#pragma unroll
    for (int j = 0; j < NPL; ++j) acc[i][j] = (acc[i][j] >> 32) * cfold + (uint32_t)acc[i][j];
}

// MR:  ct rows handled per pass (m padded up to MR with zero rows).
// G:   row groups per wavefront.  Lane l works on rows [g*MR/G, (g+1)*MR/G)
//      of the pass, g = l / (64/G), and on NPL columns; so each ct value read
//      from LDS feeds NPL products and each DB word feeds MR/G products.  With
//      G = 1 the ct values are wave-uniform LDS broadcasts; for large MR,
//      G > 1 cuts the LDS traffic per product by G at the same product count
//      per wavefront (LDS bandwidth, not the multiplier, would otherwise bound
//      the scan).
// NPL: DB columns per lane (256/128/32-bit loads).
// UNR: k-rows kept in flight per lane (must divide the fold period).
template <int MR, int G, int NPL, int UNR>
__global__ __launch_bounds__(kThreads) void rowsel_kernel(RowselLaunch a, uint32_t m_base,
                                                          uint32_t nslices, uint64_t items) {
  constexpr int KC = kLdsWords / (kWaves * MR);  // k-rows per staged chunk
  constexpr int RPL = MR / G;                    // rows per lane
  constexpr int LPG = 64 / G;                    // lanes per row group
  constexpr bool NT = G == 1;
  static_assert(MR % G == 0 && 64 % G == 0 && (RPL == 1 || RPL % 2 == 0), "row split");
  __shared__ __attribute__((aligned(16))) uint32_t lds[kLdsWords];  // [point][KC][MR]

  const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t grp = lane / LPG, col = lane % LPG;
  const uint32_t wg = xcd_remap(blockIdx.x, gridDim.x);
  const uint64_t item0 = (uint64_t)wg * kWaves;
  const uint64_t item_last = (item0 + kWaves < items ? item0 + kWaves : items) - 1;
  const uint64_t p_lo = item0 / nslices;
  const uint32_t npts = (uint32_t)(item_last / nslices - p_lo + 1);
  const uint64_t item = item0 + wave;
  const bool wave_on = item < items;
  const uint64_t p = wave_on ? item / nslices : p_lo;
  const uint32_t pl = (uint32_t)(p - p_lo);
  const uint32_t slice = wave_on ? (uint32_t)(item % nslices) : 0u;
  const uint32_t n0 = (slice * LPG + col) * NPL;
  const bool lane_on = wave_on && n0 < a.D1;
  const uint32_t limb = (uint32_t)(p / a.N);
  const uint64_t cfold = a.lc.c[limb];
  const uint32_t mrows = (a.m - m_base) < (uint32_t)MR ? (a.m - m_base) : (uint32_t)MR;

  uint64_t acc[RPL][NPL];
#pragma unroll
  for (int i = 0; i < RPL; ++i)
#pragma unroll
    for (int j = 0; j < NPL; ++j) acc[i][j] = 0;

  const uint32_t* dbp = a.dbt + (p * a.D0) * (uint64_t)a.D1 + n0;

  for (uint32_t k0 = 0; k0 < a.D0; k0 += KC) {
    const uint32_t kc = (a.D0 - k0) < (uint32_t)KC ? (a.D0 - k0) : (uint32_t)KC;
    __syncthreads();  // the previous chunk is fully consumed
    // Stage ct(m_base+mi, k0+kk, p_lo+pt) -> lds[(pt*KC + kk)*MR + mi]; the
    // point index is fastest so global reads are runs along p.
    const uint32_t total = npts * kc * MR;
    for (uint32_t e = threadIdx.x; e < total; e += kThreads) {
      const uint32_t pt = e % npts, rest = e / npts;
      const uint32_t mi = rest % MR, kk = rest / MR;
      uint32_t v = 0;
      if (mi < mrows) v = a.ct[(uint64_t)(m_base + mi) * a.ct_sm + (uint64_t)(k0 + kk) * a.ct_sk + p_lo + pt];
      lds[(pt * KC + kk) * MR + mi] = v;
    }
    __syncthreads();
    if (lane_on) {
      const uint32_t* L = lds + pl * (KC * MR) + grp * RPL;
      const uint32_t* rowp = dbp + (uint64_t)k0 * a.D1;
      const uint32_t fmask = a.fold - 1;  // the fold period is a power of two
      uint32_t kk = 0;
      if constexpr (UNR > 1) {
        // A rolling ring of UNR rows: slot u is refilled with the row UNR
        // ahead as soon as it has been consumed, so UNR row loads stay in
        // flight while the products run.  UNR divides the fold period, so
        // every fold falls on a group boundary.
        if (kc >= (uint32_t)UNR) {
          Vec<NPL, NT> d[UNR];
#pragma unroll
          for (int u = 0; u < UNR; ++u) d[u].load(rowp + (uint64_t)u * a.D1);
          for (; kk + 2 * UNR <= kc; kk += UNR) {
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
              mac_row<MR, RPL, NPL, NT>(acc, L, kk + u, d[u]);
              d[u].load(rowp + (uint64_t)(kk + UNR + u) * a.D1);
              // keep the refills in slot order: loads complete in issue order,
              // so the next slot then waits only for its own row
              __builtin_amdgcn_sched_barrier(0);
            }
            if (((kk + UNR) & fmask) == 0) fold_acc(acc, cfold);
          }
#pragma unroll
          for (int u = 0; u < UNR; ++u) mac_row<MR, RPL, NPL, NT>(acc, L, kk + u, d[u]);
          kk += UNR;
          if ((kk & fmask) == 0) fold_acc(acc, cfold);
        }
      }
      for (; kk < kc; ++kk) {
        Vec<NPL, NT> d;
        d.load(rowp + (uint64_t)kk * a.D1);
        mac_row<MR, RPL, NPL, NT>(acc, L, kk, d);
        if (((kk + 1) & fmask) == 0) fold_acc(acc, cfold);
      }
      fold_acc(acc, cfold);  // bounded again for the next chunk and the reduction
    }
  }

  if (lane_on) {
    const uint64_t q = a.lc.q[limb];
    const uint64_t mu = a.lc.mu[limb];
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const uint32_t mi = m_base + grp * RPL + i;
      if (grp * RPL + i < mrows) {
        uint32_t r[NPL];
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
          // Barrett with mu = floor((2^64-1)/q): the estimate is at most one
          // short of the quotient.
          const uint64_t x = acc[i][j];
          uint64_t t = x - __umul64hi(x, mu) * q;
          if (t >= q) t -= q;
          r[j] = (uint32_t)t;
        }
        // Per-point staging: the lane's NPL columns are contiguous, so the
        // store is one 128-bit write per 4 columns (a p-major store would be
        // a scattered 4-byte write per residue).
        uint32_t* dst = a.out_t + ((uint64_t)p * a.m + mi) * a.D1 + n0;
        if constexpr (NPL % 4 == 0) {
#pragma unroll
          for (int j = 0; j < NPL; j += 4)
            *reinterpret_cast<uint4*>(dst + j) = make_uint4(r[j], r[j + 1], r[j + 2], r[j + 3]);
        } else {
#pragma unroll
          for (int j = 0; j < NPL; ++j) dst[j] = r[j];
        }
      }
    }
  }
}

template <int MR, int G, int NPL, int UNR>
hipError_t launch_one(const RowselLaunch& a, uint32_t m_base, hipStream_t stream) {
  const uint32_t cols_per_wave = (64u / G) * NPL;
  const uint32_t nslices = (a.D1 + cols_per_wave - 1) / cols_per_wave;
  const uint64_t items = a.P * nslices;
  const uint64_t grid = (items + kWaves - 1) / kWaves;
  if (grid == 0 || grid > 0x7FFFFFFFull) return hipErrorInvalidValue;
  hipLaunchKernelGGL((rowsel_kernel<MR, G, NPL, UNR>), dim3((uint32_t)grid), dim3(kThreads), 0, stream,
                     a, m_base, nslices, items);
  return hipGetLastError();
}

// Picks the widest column vector the shape allows, then the unroll the fold
// period allows.
template <int MR, int G, int NPL_MAX>
hipError_t launch_mr(const RowselLaunch& a, uint32_t m_base, hipStream_t stream) {
  constexpr int U = (MR / G) * NPL_MAX <= 16 ? 8 : 4;
  const bool wide = (a.D1 % NPL_MAX) == 0 &&
                    (reinterpret_cast<uintptr_t>(a.dbt) % (4u * (NPL_MAX > 4 ? 4 : NPL_MAX))) == 0;
  if ((a.fold % U) != 0) return launch_one<MR, G, 1, 1>(a, m_base, stream);
  if (wide) return launch_one<MR, G, NPL_MAX, U>(a, m_base, stream);
  return launch_one<MR, G, 1, U>(a, m_base, stream);
}

}  // namespace

uint32_t rowsel_fold_period(uint32_t q) {
  // After a fold the accumulator is at most (2^32-1)*c + (2^32-1) with
  // c = 2^32 mod q; `fold` further products of at most (q-1)^2 must keep it
  // below 2^64.  Capped at 32 and rounded down to a power of two.
  const unsigned __int128 two64m1 = ~(uint64_t)0;
  const uint64_t c = (uint64_t)((((unsigned __int128)1) << 32) % q);
  const unsigned __int128 rmax = (unsigned __int128)0xFFFFFFFFu * c + 0xFFFFFFFFu;
  const unsigned __int128 pmax = (unsigned __int128)(q - 1) * (q - 1);
  uint64_t f = 32;
  if (pmax > 0) {
    const unsigned __int128 room = two64m1 - rmax;  // rmax < 2^64 for every q < 2^32
    const unsigned __int128 lim = room / pmax;
    if (lim < f) f = (uint64_t)lim;
  }
  uint32_t p2 = 1;
  while (p2 * 2 <= f) p2 *= 2;
  return p2;  // >= 1 for every 2 <= q < 2^32
}

hipError_t launch_transpose(const TransposeDesc& t, hipStream_t stream) {
  if (t.batch == 0 || t.rows == 0 || t.cols == 0) return hipSuccess;
  const uint64_t tiles_c = (t.cols + kTile - 1) / kTile, tiles_r = (t.rows + kTile - 1) / kTile;
  const uint64_t tiles_rc = tiles_c * tiles_r, tiles = tiles_rc * t.batch;
  const uint64_t grid = tiles < (1ull << 20) ? tiles : (1ull << 20);
  auto a16 = [](const void* ptr) { return reinterpret_cast<uintptr_t>(ptr) % 16 == 0; };
  const bool vec4 = t.rows % 4 == 0 && t.cols % 4 == 0 && t.s_row % 4 == 0 && t.s_batch % 4 == 0 &&
                    t.d_row % 4 == 0 && t.d_batch % 4 == 0 && a16(t.src) && a16(t.dst) &&
                    (!t.add || (t.add_b % 4 == 0 && t.add_c % 4 == 0 && a16(t.add)));
  if (vec4) {
    if (t.add)
      hipLaunchKernelGGL(transpose4_kernel<true>, dim3((uint32_t)grid), dim3(kThreads), 0, stream, t,
                         tiles_c, tiles_rc, tiles);
    else
      hipLaunchKernelGGL(transpose4_kernel<false>, dim3((uint32_t)grid), dim3(kThreads), 0, stream, t,
                         tiles_c, tiles_rc, tiles);
  } else if (t.add) {
    hipLaunchKernelGGL(transpose_kernel<true>, dim3((uint32_t)grid), dim3(kThreads), 0, stream, t,
                       tiles_c, tiles_rc, tiles);
  } else {
    hipLaunchKernelGGL(transpose_kernel<false>, dim3((uint32_t)grid), dim3(kThreads), 0, stream, t,
                       tiles_c, tiles_rc, tiles);
  }
  return hipGetLastError();
}

hipError_t launch_layout_db(const uint32_t* src, uint32_t* dst, uint64_t X, uint64_t P,
                            hipStream_t stream) {
  TransposeDesc t{};
  t.src = src;
  t.dst = dst;
  t.batch = 1;
  t.rows = X;
  t.cols = P;
  t.s_row = P;
  t.d_row = X;
  return launch_transpose(t, stream);
}

size_t rowsel_valu_workspace_bytes(uint64_t P, uint32_t m, uint32_t D1) {
  return (size_t)((4ull * P * m * D1 + 255) / 256 * 256);
}

hipError_t launch_out_relayout(const RowselLaunch& a, const uint32_t* out_t, hipStream_t stream) {
  TransposeDesc to{};
  to.src = out_t;
  to.dst = a.out;
  to.batch = a.m;
  to.rows = a.P;
  to.cols = a.D1;
  to.s_batch = a.D1;
  to.s_row = (uint64_t)a.m * a.D1;
  to.d_batch = a.out_sm;
  to.d_row = a.out_sn;
  to.add = a.add;
  to.add_b = a.add_sb;
  to.add_c = a.add_sn;
  to.N = a.N;
  to.lc = a.lc;
  return launch_transpose(to, stream);
}

hipError_t launch_rowsel(const RowselLaunch& a0, void* workspace, hipStream_t stream) {
  RowselLaunch a = a0;
  a.out_t = static_cast<uint32_t*>(workspace);
  timer_mark_start(stream);
  for (uint64_t mb = 0; mb < a.m; mb += 32) {
    const uint32_t m_base = (uint32_t)mb;
    const uint32_t rows = a.m - m_base;
    hipError_t e;
    if (rows <= 2) e = launch_mr<2, 1, 4>(a, m_base, stream);
    else if (rows <= 4) e = launch_mr<4, 1, 4>(a, m_base, stream);
    else if (rows <= 8) e = launch_mr<8, 2, 4>(a, m_base, stream);
    else if (rows <= 16) e = launch_mr<16, 2, 8>(a, m_base, stream);
    else e = launch_mr<32, 2, 4>(a, m_base, stream);
    if (e != hipSuccess) return e;
  }
  timer_mark_stop(stream);
  return launch_out_relayout(a, a.out_t, stream);
}

}  // namespace pirscan
