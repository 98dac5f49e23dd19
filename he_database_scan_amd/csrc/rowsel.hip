// rowsel.hip -- RowSel in the NTT/RNS domain on gfx950.
//
// Computes, for every point p of P = R*N independent point-wise GEMMs
// (GPIR: "Enabling Practical Private Information Retrieval with GPUs", the
// RowSel formulation M_out[p,m,n] = sum_k M_in0[p,m,k] * M_in1[p,k,n]):
//
//     out[mi][n][p] = ( sum_k ct[mi][k][p] * db[k][n][p] ) mod q_{p/N}
//
// Design (MI355X-first, HBM-bound at small m):
//  * The DB is static, so it is relaid once (layout_db_kernel) from the
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
#include <hip/hip_runtime.h>

#include "internal.hpp"

namespace pirscan {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kLdsWords = 8192;  // 32 KiB of staged ct per workgroup

// ---------------------------------------------------------------------------
// R1: one-time DB relayout [X][P] -> [P][X], X = D0*D1, via 64x64 LDS tiles.
// ---------------------------------------------------------------------------
constexpr int kTile = 64;

__global__ __launch_bounds__(kThreads) void layout_db_kernel(const uint32_t* __restrict__ src,
                                                             uint32_t* __restrict__ dst,
                                                             uint64_t X, uint64_t P,
                                                             uint64_t tiles_x, uint64_t tiles) {
  __shared__ uint32_t tile[kTile][kTile + 1];
  const int tx = threadIdx.x % kTile, ty = threadIdx.x / kTile;
  for (uint64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
    const uint64_t x0 = (t % tiles_x) * kTile, p0 = (t / tiles_x) * kTile;
    for (int r = ty; r < kTile; r += kThreads / kTile) {
      const uint64_t x = x0 + r, p = p0 + tx;
      tile[r][tx] = (x < X && p < P) ? src[x * P + p] : 0u;
    }
    __syncthreads();
    for (int r = ty; r < kTile; r += kThreads / kTile) {
      const uint64_t p = p0 + r, x = x0 + tx;
      if (p < P && x < X) dst[p * X + x] = tile[tx][r];
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

// MR:  ct rows handled per pass (m padded up to MR with zero rows).
// G:   row groups per wavefront.  Lane l works on rows [g*MR/G, (g+1)*MR/G)
//      of the pass, g = l / (64/G), and on NPL columns; so each ct value read
//      from LDS feeds NPL products and each DB word feeds MR/G products.  With
//      G = 1 the ct values are wave-uniform LDS broadcasts; for large MR,
//      G > 1 cuts the LDS traffic per product by G at the same product count
//      per wavefront (LDS bandwidth, not the multiplier, would otherwise bound
//      the scan).
// NPL: DB columns per lane (256/128/32-bit loads).
// UNR: k-rows whose loads are issued back to back (must divide the fold).
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
    // Stage ct[m_base+mi][k0+kk][p_lo+pt] -> lds[(pt*KC + kk)*MR + mi]; the
    // point index is fastest so global reads are runs along p.
    const uint32_t total = npts * kc * MR;
    for (uint32_t e = threadIdx.x; e < total; e += kThreads) {
      const uint32_t pt = e % npts, rest = e / npts;
      const uint32_t mi = rest % MR, kk = rest / MR;
      uint32_t v = 0;
      if (mi < mrows) v = a.ct[((uint64_t)(m_base + mi) * a.D0 + k0 + kk) * a.P + p_lo + pt];
      lds[(pt * KC + kk) * MR + mi] = v;
    }
    __syncthreads();
    if (lane_on) {
      const uint32_t* L = lds + pl * (KC * MR) + grp * RPL;
      for (uint32_t s0 = 0; s0 < kc; s0 += a.fold) {
        const uint32_t s1 = (s0 + a.fold < kc) ? s0 + a.fold : kc;
        uint32_t kk = s0;
        if constexpr (UNR > 1) {
          for (; kk + UNR <= s1; kk += UNR) {
            Vec<NPL, NT> d[UNR];
#pragma unroll
            for (int u = 0; u < UNR; ++u) d[u].load(dbp + (uint64_t)(k0 + kk + u) * a.D1);
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
              uint32_t cv[RPL];
              if constexpr (RPL == 1) {
                cv[0] = L[(kk + u) * MR];
              } else if constexpr (RPL == 2) {
                const uint2 t = *reinterpret_cast<const uint2*>(L + (kk + u) * MR);
                cv[0] = t.x; cv[1] = t.y;
              } else {
#pragma unroll
                for (int i = 0; i < RPL; i += 4) {
                  const uint4 t = *reinterpret_cast<const uint4*>(L + (kk + u) * MR + i);
                  cv[i] = t.x; cv[i + 1] = t.y; cv[i + 2] = t.z; cv[i + 3] = t.w;
                }
              }
#pragma unroll
              for (int i = 0; i < RPL; ++i)
#pragma unroll
                for (int j = 0; j < NPL; ++j) acc[i][j] += (uint64_t)cv[i] * d[u].v[j];
            }
          }
        }
        for (; kk < s1; ++kk) {
          Vec<NPL, NT> d;
          d.load(dbp + (uint64_t)(k0 + kk) * a.D1);
#pragma unroll
          for (int i = 0; i < RPL; ++i) {
            const uint64_t cvi = L[kk * MR + i];
#pragma unroll
            for (int j = 0; j < NPL; ++j) acc[i][j] += cvi * d.v[j];
          }
        }
        // fold: hi*2^32 + lo == hi*(2^32 mod q) + lo  (mod q)
#pragma unroll
        for (int i = 0; i < RPL; ++i)
#pragma unroll
          for (int j = 0; j < NPL; ++j)
            acc[i][j] = (acc[i][j] >> 32) * cfold + (uint32_t)acc[i][j];
      }
    }
  }

  if (lane_on) {
    const uint64_t q = a.lc.q[limb];
    const uint64_t mu = a.lc.mu[limb];
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const uint32_t mi = grp * RPL + i;
      if (mi < mrows) {
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
          // Barrett with mu = floor((2^64-1)/q): the estimate is at most one short.
          const uint64_t x = acc[i][j];
          uint64_t r = x - __umul64hi(x, mu) * q;
          if (r >= q) r -= q;
          a.out[((uint64_t)(m_base + mi) * a.D1 + n0 + j) * a.P + p] = (uint32_t)r;
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

hipError_t launch_layout_db(const uint32_t* src, uint32_t* dst, uint64_t X, uint64_t P,
                            hipStream_t stream) {
  const uint64_t tiles_x = (X + kTile - 1) / kTile, tiles_p = (P + kTile - 1) / kTile;
  const uint64_t tiles = tiles_x * tiles_p;
  const uint64_t grid = tiles < (1ull << 20) ? tiles : (1ull << 20);
  hipLaunchKernelGGL(layout_db_kernel, dim3((uint32_t)grid), dim3(kThreads), 0, stream, src, dst, X,
                     P, tiles_x, tiles);
  return hipGetLastError();
}

hipError_t launch_rowsel(const RowselLaunch& a, hipStream_t stream) {
  for (uint32_t m_base = 0; m_base < a.m; m_base += 32) {
    const uint32_t rows = a.m - m_base;
    hipError_t e;
    if (rows <= 2) e = launch_mr<2, 1, 4>(a, m_base, stream);
    else if (rows <= 4) e = launch_mr<4, 1, 4>(a, m_base, stream);
    else if (rows <= 8) e = launch_mr<8, 2, 4>(a, m_base, stream);
    else if (rows <= 16) e = launch_mr<16, 2, 8>(a, m_base, stream);
    else e = launch_mr<32, 2, 4>(a, m_base, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace pirscan
