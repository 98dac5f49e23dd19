// internal.hpp -- launch interfaces between the C-ABI layer (pirscan_api.hip)
// and the gfx950 kernels.  Nothing here is exported.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pirscan {

constexpr int kMaxLimbs = 8;
constexpr int kMaxDevices = 64;  // per-device caches cover device ids below this

// Per-limb constants precomputed on the host for the RowSel kernels.
struct LimbConsts {
  uint32_t q[kMaxLimbs];      // modulus
  uint32_t c[kMaxLimbs];      // 2^32 mod q: folds hi*2^32 + lo into hi*c + lo
  uint64_t mu[kMaxLimbs];     // floor((2^64 - 1) / q): Barrett constant for the final reduction
};

// The point-wise modular GEMM out[mi][n] = sum_k ct[mi][k] * db[k][n] (+ Z)
// mod q_{p/N} over P points.  ct and out are p-major with the given word
// strides (the point stride is 1); the DB is in the scan layout [P][D0][D1].
// RowSel:  ct [m][D0][P] (ct_sm = D0*P, ct_sk = P), out [m][D1][P].
// ExpPack: ct = C^T with C [D0][m][P] (ct_sm = P, ct_sk = m*P), DB = H^T,
//          out [D1][m][P], and Z = the body term: for odd mi,
//          Z[mi][n] = add[(mi >> 1) * add_sb + n * add_sn + p], else 0.
// Both kernels write the residues per point, out_t [P][m][D1] in the caller's
// workspace (contiguous stores), and a tiled transpose produces `out`, adding
// Z on the way.
struct RowselLaunch {
  const uint32_t* ct;
  const uint32_t* dbt;     // [P][D0][D1], or the packed fragments (launch_rowsel_packed)
  uint32_t* out;
  uint32_t* out_t;         // staging [P][m][D1] (workspace)
  const uint32_t* add;     // optional body term (residues < q), null for none
  uint64_t ct_sm, ct_sk;
  uint64_t out_sm, out_sn;
  uint64_t add_sb, add_sn;
  uint64_t P;
  uint32_t N, D0, D1, m;
  uint32_t fold;           // products accumulated between two folds (>= 1)
  uint32_t scan;           // PIRSCAN_SCAN_AUTO or PIRSCAN_SCAN_VALU (which kernel, which DB layout)
  LimbConsts lc;
};

// Batched word transpose: dst[b][c][r] = src[b][r][c] for b < batch,
// r < rows, c < cols, with
//   src(b, r, c) = b * s_batch + r * s_row + c
//   dst(b, c, r) = b * d_batch + c * d_row + r.
// With `add` set (the ExpPack body term) the destination's contiguous index r
// is a point p, and odd batches b get
//   dst += add[(b >> 1) * add_b + c * add_c + r]  mod q_{r / N}.
struct TransposeDesc {
  const uint32_t* src;
  uint32_t* dst;
  uint64_t batch, rows, cols;
  uint64_t s_batch, s_row;
  uint64_t d_batch, d_row;
  const uint32_t* add;
  uint64_t add_b, add_c;
  uint32_t N;
  LimbConsts lc;
};
hipError_t launch_transpose(const TransposeDesc& t, hipStream_t stream);

// R1: [X][P] -> [P][X] word transpose (the RowSel DB layout, X = D0*D1).
hipError_t launch_layout_db(const uint32_t* src, uint32_t* dst, uint64_t X, uint64_t P,
                            hipStream_t stream);

// R2-R4: the modular GEMM scan on the VALU (any m, any q < 2^32).  The
// workspace holds out_t (rowsel_valu_workspace_bytes).
size_t rowsel_valu_workspace_bytes(uint64_t P, uint32_t m, uint32_t D1);
hipError_t launch_rowsel(const RowselLaunch& a, void* workspace, hipStream_t stream);

// out_t [P][m][D1] -> out (strided, p-major), adding the body term if any.
hipError_t launch_out_relayout(const RowselLaunch& a, const uint32_t* out_t, hipStream_t stream);

// RowSel / ExpPack on int8 MFMA over centred signed limbs, any m, with the
// DB operand packed once into B-fragment order.  Usable when every q < 2^31
// and D0 <= kPackedMaxD0 (the int32 limb diagonals cannot overflow); other
// shapes, and shapes that ask for the VALU scan, keep the [P][D0][D1] layout
// and the VALU scan.
constexpr uint32_t kPackedMaxD0 = 16384;
bool rowsel_packed_ok(const uint32_t* q, uint32_t R, uint32_t D0);
// Largest m a RowSel call accepts (ExpPack: 2B), so every row-pass loop and
// its 32-row steps stay far inside 32 bits.
constexpr uint32_t kMaxRows = 1u << 31;
// Bytes of the packed operand: per point ceil(D1/16) column tiles (rounded up
// to a whole group of tiles) x ceil(D0/64) steps x 4 KiB.
uint64_t packed_layout_bytes(uint64_t P, uint32_t D0, uint32_t D1);

// Limb packing of a p-major operand into MFMA fragments.  Source word
// (row, k, p) at src[row * s_row + k * s_k + p] (rows row_base .. rows-1,
// k < K); the 16 bytes of fragment lane (li, lg) of (p, t, s, limb j) at
// dst[p * d_p + (t / tgroup) * d_g + (t % tgroup) * d_t + s * d_s +
// (4 j + lg) * lpg + li] (strides in 16-byte units) for li < lpg, holding limb j of the centred residues of row
// row_base + 16t + li at k = 64s + 16lg + 0..15; zero past rows / K.  With
// lpg = 16 a fragment is 1 KiB of contiguous lanes.
struct PackDesc {
  const uint32_t* src;
  void* dst;
  uint64_t P, s_row, s_k;
  uint64_t d_p, d_g, d_t, d_s;
  uint32_t N, rows, row_base, K, tiles, S;
  uint32_t tgroup;  // tiles per group (t / tgroup selects the group)
  uint32_t lpg;     // lanes stored per k-group (16, or the live rows of a small batch)
  uint32_t q[kMaxLimbs];
};
hipError_t launch_pack(const PackDesc& d, hipStream_t stream);
// The one-time DB / hint packing: rows = the DB's columns (D1), K = D0,
// tile-major fragments [p][t][s][j][lane].
hipError_t launch_pack_operand(const uint32_t* src, void* dst, uint64_t P, uint32_t N, const uint32_t* q,
                               uint32_t R, uint32_t rows, uint32_t K, uint64_t s_row, uint64_t s_k,
                               hipStream_t stream);
// The scan (a.dbt = the packed operand).  Workspace: the A fragments of one
// 32-row pass plus the per-point output staging.
size_t rowsel_packed_workspace_bytes(uint64_t P, uint32_t m, uint32_t D0, uint32_t D1);
hipError_t launch_rowsel_packed(const RowselLaunch& a, uint32_t R, void* workspace, hipStream_t stream);

// Products of (q-1)^2 that fit between folds for modulus q (host helper).
uint32_t rowsel_fold_period(uint32_t q);

// ---- scalar-HE ---------------------------------------------------------

struct ScalarPlan {
  bool fast;          // aligned fast paths (K % 16 == 0, 16-byte aligned db)
  bool mfma;          // B > 1 on int8 MFMA
  bool wide;          // wide passes (groups of 128 columns) while more than 64 remain (tiled DB)
  uint32_t bgroup;    // columns of the widest pass
  uint32_t bpad;      // its digit columns per plane: bgroup rounded up to 16, or whole 128-column groups
  uint64_t kblock;    // split-K block (k per partial sum)
  uint64_t nkb;       // number of k blocks
  uint64_t kpad;      // nkb * kblock
  size_t digit_bytes; // digit planes
  size_t part_bytes;  // split-K partial sums (0 when nkb == 1)
  size_t total_bytes; // workspace requirement
};

bool scalar_plan(uint64_t M, uint64_t K, uint32_t B, uintptr_t db_addr, ScalarPlan* plan);

hipError_t launch_scalar(const int8_t* db, const uint32_t* query, uint32_t* out, uint64_t M,
                         uint64_t K, uint32_t B, const ScalarPlan& plan, void* workspace,
                         hipStream_t stream);

// The tiled scalar DB (pirscan_scalar_layout_db): 16-row tiles x 64-k steps
// of 1 KiB int8 MFMA A fragments, lane (li, lg) = db[16t + li][64s + 16lg ..
// +15], zero past M and K.  Every batch size runs the MFMA scan on it.
uint64_t scalar_layout_bytes(uint64_t M, uint64_t K);
hipError_t launch_scalar_layout(const int8_t* db, void* dst, uint64_t M, uint64_t K, hipStream_t stream);
bool scalar_tiled_plan(uint64_t M, uint64_t K, uint32_t B, ScalarPlan* plan);
hipError_t launch_scalar_tiled(const void* db_tiled, const uint32_t* query, uint32_t* out, uint64_t M,
                               uint64_t K, uint32_t B, const ScalarPlan& plan, void* workspace,
                               hipStream_t stream);

// ---- negacyclic NTT over RNS polynomials ------------------------------

struct PsiTable {
  uint32_t v[kMaxLimbs];  // psi_r: primitive 2N-th root of unity mod q_r
};

// A validated NTT shape: N = 2^logn in [16, 8192], every q < 2^30 prime with
// q == 1 (mod 2N), psi^N == -1 (mod q), ninv = N^-1 mod q.
struct NttDesc {
  uint32_t N, logn, R;
  uint32_t q[kMaxLimbs];
  PsiTable psi;
  uint32_t ninv[kMaxLimbs];
};

enum class NttMode { kForward, kInverse, kRnsForward };

// Twiddle tables: [R][2][N] pairs (w, floor(w 2^32 / q)), forward then inverse.
size_t ntt_plan_bytes(uint32_t N, uint32_t R);
hipError_t launch_ntt_plan(const NttDesc& d, void* plan, hipStream_t stream);
// kForward / kInverse: in, out [count][R][N] residues (in == out allowed).
// kRnsForward: in [count][N] integer coefficients, out [count][R][N].
hipError_t launch_ntt(const NttDesc& d, NttMode mode, const void* plan, const uint32_t* in, uint32_t* out,
                      uint64_t count, hipStream_t stream);

// Benchmark hook (include/pirscan_bench.h, only in the build with
// PIRSCAN_BENCH_HOOKS=1, libpirscan_bench.so): when the calling thread has it
// on, the launchers bracket their main kernel with these two calls, which
// record a HIP event pair on `stream`.  In the product build they are empty.
#ifndef PIRSCAN_BENCH_HOOKS
#define PIRSCAN_BENCH_HOOKS 0
#endif
#if PIRSCAN_BENCH_HOOKS
void timer_mark_start(hipStream_t stream);
void timer_mark_stop(hipStream_t stream);
// Benchmark reference: one non-temporal 16-byte read pass over `bytes` of buf
// (bytes % 16 == 0, buf 16-byte aligned), timed by the kernel-timer hook.
hipError_t launch_read_stream(const void* buf, uint64_t bytes, uint32_t* sink, hipStream_t stream);
#else
inline void timer_mark_start(hipStream_t) {}
inline void timer_mark_stop(hipStream_t) {}
#endif

// The C-ABI layer's device check (PIRSCAN_OK when the current device is a
// gfx950, else a PIRSCAN_E* status) and its mapping of a HIP error to a
// status (recording the error as the thread's last device error).
int api_device_check();
int api_device_status(hipError_t e);

// s_waitcnt immediate: vmcnt = n (< 64), expcnt and lgkmcnt left unconstrained.
constexpr int waitcnt_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// An LDS address for the direct global-to-LDS loads.
#define LDS_PTR(x) ((__attribute__((address_space(3))) void*)(x))

// Maps a hardware workgroup id to a logical tile id so that consecutive
// logical tiles run on the same XCD (gfx950 dispatches workgroups round-robin
// over its 8 XCDs, each with a private L2).
__host__ __device__ __forceinline__ uint32_t xcd_remap(uint32_t pid, uint32_t num) {
  constexpr uint32_t kXcds = 8;
  const uint32_t xcd = pid % kXcds, local = pid / kXcds;
  const uint32_t per = num / kXcds, rem = num % kXcds;
  return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

// Logical workgroup id of hardware id h (gfx950 deals workgroups to its 8
// XCDs round-robin).  C > 1: XCD x takes the C-id chunks x, x + 8, x + 16,
// ... so the eight XCDs stream neighbouring parts of a database at any time
// (ids past the last whole round of 8 chunks keep their hardware order); 1:
// no remap; 0: xcd_remap, each XCD one contiguous eighth of the grid.
template <uint32_t C>
__host__ __device__ __forceinline__ uint32_t scan_remap(uint32_t h, uint32_t num) {
  if constexpr (C == 0) {
    return xcd_remap(h, num);
  } else if constexpr (C == 1) {
    return h;
  } else {
    const uint32_t full = num / (8 * C) * (8 * C);
    if (h >= full) return h;
    const uint32_t x = h % 8, l = h / 8;
    return ((l / C) * 8 + x) * C + l % C;
  }
}

}  // namespace pirscan
