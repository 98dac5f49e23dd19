// ntt.hip -- negacyclic NTT / INTT over RNS polynomials on gfx950, and the
// RNS decomposition fused with the forward NTT.
//
// A polynomial of R_q = Z_q[X]/(X^N + 1) with q = q_0 ... q_{R-1} is an R x N
// matrix of residues, one row per prime (VIPIR section 2.3); the NTT of a row
// evaluates it at the N odd powers of a primitive 2N-th root of unity psi,
//     A[j] = sum_i a[i] psi^((2j+1) i)  mod q_r      (natural order in j),
// which turns products in R_q into point-wise products.  VIPIR section 4.3
// runs an N = 2^12 NTT as one kernel whose working set stays on chip and
// fuses the RNS decomposition of integer inputs into it; so does this file:
// one workgroup owns one polynomial row (N/16 threads, 16 residues each) and
// never leaves the chip between its load and its store.
//
// Algorithm.  Forward: Cooley-Tukey butterflies on natural-order input with
// twiddles psi^bitrev(k) (a bit-reversed power table), which leaves A in
// bit-reversed order; the last on-chip exchange writes it back in natural
// order.  Inverse: the input is scattered to bit-reversed positions on chip,
// then Gentleman-Sande butterflies with psi^-bitrev(k) and a final scaling by
// N^-1 give natural order.  Stage b (the butterfly partner differs in index
// bit b) uses twiddle index 2^(n-1-b) + (j >> (b+1)) in both directions.
//
// Mapping.  The n = log2 N index bits are taken four at a time: in a round a
// thread holds the 16 elements whose index differs only in bits [lo, lo+4),
// so four radix-2 stages run in registers; between rounds the workgroup
// exchanges the polynomial through LDS (one word of padding per 16 keeps the
// stride-16 accesses of the low-bit round conflict-free).  Global loads and
// stores are the coalesced mapping j = tid + (N/16) e.
//
// Arithmetic (q < 2^30).  Shoup's multiplication by a fixed w with
// w' = floor(w 2^32 / q): y w mod q = y w - mulhi(y, w') q in [0, 2q) for any
// 32-bit y.  Butterflies keep residues lazily in [0, 4q) (forward) or
// [0, 2q) (inverse) and the output is made canonical, [0, q), once at the end.
// With every q <= 2^29 (8q fits in 32 bits) the bounds are looser, which
// saves conditional subtractions:
//  * forward: a butterfly on inputs below b gives outputs below b + 2q (the
//    Shoup product is below 2q), so from inputs below 2q three stages run
//    with no reduction (to 8q); after that every other stage first brings X
//    below 4q (outputs below 6q) and the stage between lets it grow to 8q;
//  * inverse: the sum path doubles per stage, so the first two stages (from
//    canonical inputs: below 2q, then 4q) skip its reduction and later ones
//    reduce it below 4q; the difference path is offset by the bound of Y
//    before its Shoup product.
// The inverse's last stage (a single twiddle) multiplies both outputs by
// N^-1 (its twiddle premultiplied), so no separate scaling pass follows.
// VIPIR uses Montgomery multiplication inside its NTT; with twiddles that are
// known ahead of time, Shoup's precomputed quotient needs the same three
// 32-bit multiplies and no domain conversion.
#include <hip/hip_runtime.h>

#include "internal.hpp"

namespace pirscan {
namespace {

constexpr int kElems = 16;  // residues per thread

__host__ __device__ constexpr int pad_index(int j) { return j + (j >> 4); }

__device__ __forceinline__ uint32_t mul_shoup(uint32_t y, uint32_t w, uint32_t wq, uint32_t q) {
  return y * w - __umulhi(y, wq) * q;  // in [0, 2q), == y w (mod q)
}

// -(y w) mod q as a value in (-2q, 0], i.e. the 32-bit word 2^32 - r with
// r = y w - mulhi(y, w') q in [0, 2q): the same three multiplies as
// mul_shoup, with the subtraction reversed so that the forward butterfly
// can form X + r = X - n and X - r + 2q = X + n + 2q in one instruction each.
__device__ __forceinline__ uint32_t mul_shoup_neg(uint32_t y, uint32_t w, uint32_t wq, uint32_t q) {
  return __umulhi(y, wq) * q - y * w;
}

__device__ __forceinline__ uint32_t sub_if_ge(uint32_t x, uint32_t m) {
  const uint32_t d = x - m;
  return d < x ? d : x;  // unsigned min: x - m when x >= m, else x
}

// Element e of thread tid in a round whose 16 elements vary in bits [lo, lo+4).
template <int LO>
__device__ __forceinline__ uint32_t elem_index(uint32_t tid, int e) {
  return (tid & ((1u << LO) - 1)) | ((uint32_t)e << LO) | ((tid >> LO) << (LO + 4));
}

// The low n bits of x reversed, n in [0, 32] (n == 0 gives 0; a shift by 32
// would be undefined).
__device__ __forceinline__ uint32_t bit_reverse(uint32_t x, int n) { return n ? __brev(x) >> (32 - n) : 0u; }

// One round of forward (CT) stages on index bits BHI down to BLO, with the
// thread's elements varying in bits [LO, LO+4).  When the thread's index bits
// all lie below LO (the first round), the twiddle index is wave-uniform.
// Forward stage number s (0 first) reduces X before its butterfly: always
// with q < 2^30 (below 2q), with q <= 2^29 (LAZY) at s = 3, 5, 7, ... (below 4q).
__host__ __device__ constexpr bool fwd_reduces(int s, bool lazy) { return !lazy || (s >= 3 && (s - 3) % 2 == 0); }

template <int LOGN, int LO, int BHI, int BLO, bool LAZY>
__device__ __forceinline__ void fwd_round(uint32_t (&x)[kElems], uint32_t tid, const uint2* __restrict__ tw,
                                          uint32_t q) {
  const uint32_t q2 = 2 * q, red = LAZY ? 4 * q : 2 * q;
#pragma unroll
  for (int b = BHI; b >= BLO; --b) {
    const uint32_t m = 1u << (LOGN - 1 - b);
    const bool reduce = fwd_reduces(LOGN - 1 - b, LAZY);
#pragma unroll
    for (int e = 0; e < kElems; ++e) {
      if ((e >> (b - LO)) & 1) continue;
      const int e2 = e | (1 << (b - LO));
      uint32_t t;
      if constexpr (LO == LOGN - 4) t = m + (uint32_t)(e >> (b - LO + 1));
      else t = m + ((tid >> LO) << (LO + 3 - b)) + (uint32_t)(e >> (b - LO + 1));
      const uint2 w = tw[t];
      const uint32_t X = reduce ? sub_if_ge(x[e], red) : x[e];
      const uint32_t nV = mul_shoup_neg(x[e2], w.x, w.y, q);
      x[e] = X - nV;
      x[e2] = X + nV + q2;
    }
  }
}

// The inverse's last stage (index bit LOGN-1, the single twiddle w1 =
// psi^-(N/2)): both outputs times N^-1, the twiddle premultiplied.
struct InvLast {
  uint32_t ninv, ninv_q;  // N^-1 mod q and its Shoup quotient
  uint32_t w, w_q;        // w1 N^-1 mod q and its Shoup quotient
};

// One round of inverse (GS) stages on index bits BLO up to BHI (stage number
// = bit).  With q < 2^30 inputs are below 2q and every stage reduces the sum
// below 2q; with q <= 2^29 (LAZY) stages 0 and 1 let the sum grow (below 2q,
// then 4q) and later ones reduce it below 4q, the difference offset by Y's
// bound (2q, then 4q).
template <int LOGN, int LO, int BLO, int BHI, bool LAZY>
__device__ __forceinline__ void inv_round(uint32_t (&x)[kElems], uint32_t tid, const uint2* __restrict__ tw,
                                          uint32_t q, const InvLast& last) {
#pragma unroll
  for (int b = BLO; b <= BHI; ++b) {
    const uint32_t h = 1u << (LOGN - 1 - b);
    const bool reduce = !LAZY || b >= 2;
    const uint32_t red = LAZY ? 4 * q : 2 * q;
    const uint32_t off = (LAZY && b >= 2) ? 4 * q : 2 * q;
#pragma unroll
    for (int e = 0; e < kElems; ++e) {
      if ((e >> (b - LO)) & 1) continue;
      const int e2 = e | (1 << (b - LO));
      uint32_t t;
      if constexpr (LO == LOGN - 4) t = h + (uint32_t)(e >> (b - LO + 1));
      else t = h + ((tid >> LO) << (LO + 3 - b)) + (uint32_t)(e >> (b - LO + 1));
      const uint32_t X = x[e], Y = x[e2];
      if (b == LOGN - 1) {  // outputs below 2q
        x[e] = mul_shoup(X + Y, last.ninv, last.ninv_q, q);
        x[e2] = mul_shoup(X - Y + off, last.w, last.w_q, q);
      } else {
        const uint2 w = tw[t];
        x[e] = reduce ? sub_if_ge(X + Y, red) : X + Y;
        x[e2] = mul_shoup(X - Y + off, w.x, w.y, q);
      }
    }
  }
}

// LDS word of element e in the mapping with base LO.  When e's bits do not
// straddle bit 4 (LO == 0 or LO >= 4) the padded index is the padded index
// of element 0 plus a compile-time step, so each access is one base register
// and an immediate offset.
template <int LO>
__device__ __forceinline__ uint32_t* lds_slot(uint32_t* lds, uint32_t base, uint32_t tid, int e) {
  if constexpr (LO == 0) return lds + base + e;                                  // pad(16a + e) = 17a + e
  else if constexpr (LO >= 4) return lds + base + e * ((1 << LO) + (1 << (LO - 4)));
  else return lds + pad_index((int)elem_index<LO>(tid, e));
}

template <int LO>
__device__ __forceinline__ uint32_t lds_base(uint32_t tid) {
  return (uint32_t)pad_index((int)elem_index<LO>(tid, 0));
}

// Register <-> LDS exchange between rounds with element mappings LA -> LB.
template <int LA, int LB>
__device__ __forceinline__ void exchange(uint32_t (&x)[kElems], uint32_t tid, uint32_t* lds) {
  __syncthreads();  // the previous exchange's reads are done
  const uint32_t wb = lds_base<LA>(tid), rb = lds_base<LB>(tid);
#pragma unroll
  for (int e = 0; e < kElems; ++e) *lds_slot<LA>(lds, wb, tid, e) = x[e];
  __syncthreads();
#pragma unroll
  for (int e = 0; e < kElems; ++e) x[e] = *lds_slot<LB>(lds, rb, tid, e);
}

__host__ __device__ constexpr int bit_reverse4(int e) {
  return ((e & 1) << 3) | ((e & 2) << 1) | ((e & 4) >> 1) | ((e & 8) >> 3);
}

// Round r of the forward transform: bits [hi-4, hi) from the top, hi = LOGN - 4r;
// a partial last round (LOGN % 4 bits) maps its elements to bits [0, 4).
template <int LOGN, int R>
struct FwdRound {
  static constexpr int hi = LOGN - 4 * R;
  static constexpr int blo = hi - 4 > 0 ? hi - 4 : 0;
  static constexpr int lo = (hi - blo == 4) ? blo : 0;
};
// Round r of the inverse: bits [4r, min(4r+4, LOGN)); a partial last round
// maps its elements to bits [LOGN-4, LOGN).
template <int LOGN, int R>
struct InvRound {
  static constexpr int blo = 4 * R;
  static constexpr int bhi = (4 * R + 4 < LOGN ? 4 * R + 4 : LOGN) - 1;
  static constexpr int lo = (bhi + 1 - blo == 4) ? blo : LOGN - 4;
};

template <int LOGN, int R, bool LAZY>
__device__ __forceinline__ void fwd_rounds_from(uint32_t (&x)[kElems], uint32_t tid, const uint2* tw, uint32_t q,
                                                uint32_t* lds) {
  if constexpr (FwdRound<LOGN, R>::hi > 0) {
    using C = FwdRound<LOGN, R>;
    if constexpr (R > 0) exchange<FwdRound<LOGN, R - 1>::lo, C::lo>(x, tid, lds);
    fwd_round<LOGN, C::lo, C::hi - 1, C::blo, LAZY>(x, tid, tw, q);
    fwd_rounds_from<LOGN, R + 1, LAZY>(x, tid, tw, q, lds);
  }
}

template <int LOGN, int R, bool LAZY>
__device__ __forceinline__ void inv_rounds_from(uint32_t (&x)[kElems], uint32_t tid, const uint2* tw, uint32_t q,
                                                const InvLast& last, uint32_t* lds) {
  if constexpr (4 * R < LOGN) {
    using C = InvRound<LOGN, R>;
    if constexpr (R > 0) exchange<InvRound<LOGN, R - 1>::lo, C::lo>(x, tid, lds);
    inv_round<LOGN, C::lo, C::blo, C::bhi, LAZY>(x, tid, tw, q, last);
    inv_rounds_from<LOGN, R + 1, LAZY>(x, tid, tw, q, last, lds);
  }
}

template <int LOGN>
constexpr int last_fwd_lo() {
  return FwdRound<LOGN, (LOGN + 3) / 4 - 1>::lo;
}

// Forward transform of x (the coalesced mapping on entry, residues < 2q) and
// store: out[j] = A[j] in natural order, canonical.
template <int LOGN, bool LAZY>
__device__ __forceinline__ uint32_t fwd_canonical(uint32_t v, uint32_t q) {
  if constexpr (LAZY) v = sub_if_ge(v, 4 * q);  // below 8q
  return sub_if_ge(sub_if_ge(v, 2 * q), q);      // below 4q
}

template <int LOGN, bool LAZY>
__device__ __forceinline__ void forward_and_store(uint32_t (&x)[kElems], uint32_t tid, const uint2* tw,
                                                  uint32_t q, uint32_t* lds, uint32_t* __restrict__ dst) {
  constexpr uint32_t T = 1u << (LOGN - 4);
  fwd_rounds_from<LOGN, 0, LAZY>(x, tid, tw, q, lds);
  // canonical, then to natural order: element j holds A[bitrev(j)]
  constexpr int LL = last_fwd_lo<LOGN>();
  __syncthreads();
  if constexpr (LL == 0 && LOGN >= 8) {
    // element j = 16 tid + e goes to bitrev(j) = bitrev4(e) 2^(n-4) + bitrev_{n-4}(tid)
    const uint32_t wb = (uint32_t)pad_index((int)bit_reverse(tid, LOGN - 4));
#pragma unroll
    for (int e = 0; e < kElems; ++e)
      lds[wb + bit_reverse4(e) * ((1 << (LOGN - 4)) + (1 << (LOGN - 8)))] = fwd_canonical<LOGN, LAZY>(x[e], q);
  } else {
#pragma unroll
    for (int e = 0; e < kElems; ++e) {
      const uint32_t v = fwd_canonical<LOGN, LAZY>(x[e], q);
      lds[pad_index((int)bit_reverse(elem_index<LL>(tid, e), LOGN))] = v;
    }
  }
  __syncthreads();
  const uint32_t rb = (uint32_t)pad_index((int)tid);
#pragma unroll
  for (int e = 0; e < kElems; ++e) {
    const uint32_t j = tid + T * (uint32_t)e;
    if constexpr (T >= 16) dst[j] = lds[rb + e * (T + T / 16)];
    else dst[j] = lds[pad_index((int)j)];
  }
}

struct NttArgs {
  const uint32_t* in;
  uint32_t* out;
  const uint2* plan;  // [R][2][N] (w, w'): forward psi^bitrev(k), inverse psi^-bitrev(k)
  uint64_t count;
  uint32_t R;
  uint32_t q[kMaxLimbs];
  uint32_t ninv[kMaxLimbs], ninv_q[kMaxLimbs];  // N^-1 mod q and its Shoup quotient
  uint32_t w1n[kMaxLimbs], w1n_q[kMaxLimbs];    // psi^-(N/2) N^-1 mod q and its Shoup quotient
  uint32_t one_q[kMaxLimbs];                    // floor(2^32 / q): x mod q in [0, 2q) for x < 2^32
};

// Residue transforms: one workgroup per (polynomial, limb) row.  LAZY: every
// q <= 2^29.
template <int LOGN, bool INVERSE, bool LAZY>
__global__ __launch_bounds__(1 << (LOGN - 4)) void ntt_kernel(NttArgs a) {
  constexpr uint32_t N = 1u << LOGN, T = N >> 4;
  __shared__ uint32_t lds[pad_index((int)N)];
  const uint32_t tid = threadIdx.x;
  const uint64_t row = blockIdx.x;  // c * R + r
  const uint32_t r = (uint32_t)(row % a.R);
  const uint32_t q = a.q[r];
  const uint32_t* src = a.in + row * N;
  uint32_t* dst = a.out + row * N;
  uint32_t x[kElems];
  if constexpr (!INVERSE) {
    const uint2* tw = a.plan + (uint64_t)(2 * r) * N;
#pragma unroll
    for (int e = 0; e < kElems; ++e) x[e] = __builtin_nontemporal_load(src + tid + T * (uint32_t)e);
    forward_and_store<LOGN, LAZY>(x, tid, tw, q, lds, dst);
  } else {
    const uint2* tw = a.plan + (uint64_t)(2 * r + 1) * N;
    // scatter the natural-order input to bit-reversed positions
#pragma unroll
    for (int e = 0; e < kElems; ++e) x[e] = __builtin_nontemporal_load(src + tid + T * (uint32_t)e);
    // bitrev(tid + T e) = 16 bitrev_{n-4}(tid) + bitrev4(e): padded, 17 bitrev_{n-4}(tid) + bitrev4(e)
    const uint32_t sb = 17 * bit_reverse(tid, LOGN - 4);
#pragma unroll
    for (int e = 0; e < kElems; ++e) lds[sb + bit_reverse4(e)] = x[e];
    __syncthreads();
    constexpr int L0 = InvRound<LOGN, 0>::lo;
    const uint32_t rb = lds_base<L0>(tid);
#pragma unroll
    for (int e = 0; e < kElems; ++e) x[e] = *lds_slot<L0>(lds, rb, tid, e);
    const InvLast last{a.ninv[r], a.ninv_q[r], a.w1n[r], a.w1n_q[r]};
    inv_rounds_from<LOGN, 0, LAZY>(x, tid, tw, q, last, lds);
    // the last round's mapping is lo = LOGN - 4: element e sits at tid + T e
    static_assert(InvRound<LOGN, (LOGN + 3) / 4 - 1>::lo == LOGN - 4, "inverse ends coalesced");
#pragma unroll
    for (int e = 0; e < kElems; ++e) dst[tid + T * (uint32_t)e] = sub_if_ge(x[e], q);  // scaled: below 2q
  }
}

// RNS decomposition fused with the forward transform: one workgroup per
// polynomial reads its N integer coefficients once and writes all R limbs.
template <int LOGN, bool LAZY>
__global__ __launch_bounds__(1 << (LOGN - 4)) void ntt_rns_kernel(NttArgs a) {
  constexpr uint32_t N = 1u << LOGN, T = N >> 4;
  __shared__ uint32_t lds[pad_index((int)N)];
  const uint32_t tid = threadIdx.x;
  const uint64_t c = blockIdx.x;
  const uint32_t* src = a.in + c * N;
  uint32_t coef[kElems];
#pragma unroll
  for (int e = 0; e < kElems; ++e) coef[e] = __builtin_nontemporal_load(src + tid + T * (uint32_t)e);
  for (uint32_t r = 0; r < a.R; ++r) {
    const uint32_t q = a.q[r], oq = a.one_q[r];
    uint32_t x[kElems];
#pragma unroll
    for (int e = 0; e < kElems; ++e) x[e] = coef[e] - __umulhi(coef[e], oq) * q;  // [0, 2q)
    forward_and_store<LOGN, LAZY>(x, tid, a.plan + (uint64_t)(2 * r) * N, q, lds, a.out + (c * a.R + r) * N);
  }
}

// Plan: for limb r and k < N, (w, floor(w 2^32 / q)) with w = psi^bitrev(k)
// (forward) and psi^-bitrev(k) (inverse), psi^-1 = psi^(2N-1).
__host__ __device__ uint32_t pow_mod(uint32_t b, uint32_t e, uint32_t q) {
  uint64_t r = 1 % q, x = b % q;
  while (e) {
    if (e & 1) r = (r * x) % q;
    x = (x * x) % q;
    e >>= 1;
  }
  return (uint32_t)r;
}

__global__ void ntt_plan_kernel(uint2* __restrict__ plan, uint32_t logn, uint32_t R, NttArgs a,
                                PsiTable psi) {
  const uint32_t N = 1u << logn;
  const uint64_t total = (uint64_t)R * 2 * N;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (uint64_t)gridDim.x * blockDim.x) {
    const uint32_t k = (uint32_t)(i % N);
    const uint32_t dir = (uint32_t)((i / N) % 2);
    const uint32_t r = (uint32_t)(i / (2ull * N));
    const uint32_t q = a.q[r];
    const uint32_t base = dir ? pow_mod(psi.v[r], 2 * N - 1, q) : psi.v[r];
    const uint32_t w = pow_mod(base, bit_reverse(k, (int)logn), q);
    plan[i] = make_uint2(w, (uint32_t)(((uint64_t)w << 32) / q));
  }
}

template <int LOGN, bool LAZY>
hipError_t launch_for(const NttArgs& a, NttMode mode, hipStream_t stream) {
  constexpr uint32_t T = 1u << (LOGN - 4);
  const uint64_t blocks = mode == NttMode::kRnsForward ? a.count : a.count * a.R;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7FFFFFFFull) return hipErrorInvalidValue;
  switch (mode) {
    case NttMode::kForward:
      hipLaunchKernelGGL((ntt_kernel<LOGN, false, LAZY>), dim3((uint32_t)blocks), dim3(T), 0, stream, a);
      break;
    case NttMode::kInverse:
      hipLaunchKernelGGL((ntt_kernel<LOGN, true, LAZY>), dim3((uint32_t)blocks), dim3(T), 0, stream, a);
      break;
    case NttMode::kRnsForward:
      hipLaunchKernelGGL((ntt_rns_kernel<LOGN, LAZY>), dim3((uint32_t)blocks), dim3(T), 0, stream, a);
      break;
  }
  return hipGetLastError();
}

template <int LOGN>
hipError_t launch_for(const NttArgs& a, bool lazy, NttMode mode, hipStream_t stream) {
  return lazy ? launch_for<LOGN, true>(a, mode, stream) : launch_for<LOGN, false>(a, mode, stream);
}

}  // namespace

size_t ntt_plan_bytes(uint32_t N, uint32_t R) { return (size_t)R * 2 * N * sizeof(uint2); }

hipError_t launch_ntt_plan(const NttDesc& d, void* plan, hipStream_t stream) {
  NttArgs a{};
  a.R = d.R;
  for (uint32_t r = 0; r < d.R; ++r) a.q[r] = d.q[r];
  const uint64_t total = (uint64_t)d.R * 2 * d.N;
  const uint32_t grid = (uint32_t)((total + 255) / 256);
  hipLaunchKernelGGL(ntt_plan_kernel, dim3(grid), dim3(256), 0, stream, static_cast<uint2*>(plan), d.logn, d.R,
                     a, d.psi);
  return hipGetLastError();
}

hipError_t launch_ntt(const NttDesc& d, NttMode mode, const void* plan, const uint32_t* in, uint32_t* out,
                      uint64_t count, hipStream_t stream) {
  NttArgs a{};
  a.in = in;
  a.out = out;
  a.plan = static_cast<const uint2*>(plan);
  a.count = count;
  a.R = d.R;
  bool lazy = true;  // every q <= 2^29: 8q fits in 32 bits
  for (uint32_t r = 0; r < d.R; ++r) {
    const uint32_t q = d.q[r];
    a.q[r] = q;
    a.ninv[r] = d.ninv[r];
    a.ninv_q[r] = (uint32_t)(((uint64_t)d.ninv[r] << 32) / q);
    a.one_q[r] = (uint32_t)((1ull << 32) / q);
    // the inverse's last twiddle, psi^-bitrev(1) = (psi^-1)^(N/2) as the plan
    // computes it, times N^-1
    const uint32_t w1 = pow_mod(pow_mod(d.psi.v[r], 2 * d.N - 1, q), d.N / 2, q);
    a.w1n[r] = (uint32_t)((uint64_t)w1 * d.ninv[r] % q);
    a.w1n_q[r] = (uint32_t)(((uint64_t)a.w1n[r] << 32) / q);
    lazy = lazy && q <= (1u << 29);
  }
  timer_mark_start(stream);
  hipError_t e = hipErrorInvalidValue;
  switch (d.logn) {
    case 4: e = launch_for<4>(a, lazy, mode, stream); break;
    case 5: e = launch_for<5>(a, lazy, mode, stream); break;
    case 6: e = launch_for<6>(a, lazy, mode, stream); break;
    case 7: e = launch_for<7>(a, lazy, mode, stream); break;
    case 8: e = launch_for<8>(a, lazy, mode, stream); break;
    case 9: e = launch_for<9>(a, lazy, mode, stream); break;
    case 10: e = launch_for<10>(a, lazy, mode, stream); break;
    case 11: e = launch_for<11>(a, lazy, mode, stream); break;
    case 12: e = launch_for<12>(a, lazy, mode, stream); break;
    case 13: e = launch_for<13>(a, lazy, mode, stream); break;
    default: break;
  }
  timer_mark_stop(stream);
  return e;
}

}  // namespace pirscan
