// pirscan_api.hip -- the C ABI of libpirscan: argument validation, device
// check, constant precomputation and kernel dispatch on the caller's stream.
// Every entry point declared in include/pirscan.h is defined here.
#include <hip/hip_runtime.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/pirscan.h"
#include "internal.hpp"

namespace {

thread_local int g_last_hip_error = 0;

// Per-device "is gfx950" cache: 0 unknown, 1 yes, 2 no.
using pirscan::kMaxDevices;
std::atomic<int> g_arch_ok[kMaxDevices];

int device_check() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return PIRSCAN_EDEVICE;
  }
  if (dev < 0 || dev >= kMaxDevices) return PIRSCAN_EUNSUPPORTED;
  int st = g_arch_ok[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) {
      g_last_hip_error = (int)e;
      return PIRSCAN_EDEVICE;
    }
    st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_ok[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? PIRSCAN_OK : PIRSCAN_EUNSUPPORTED;
}

int device_status(hipError_t e) {
  if (e == hipSuccess) return PIRSCAN_OK;
  g_last_hip_error = (int)e;
  return PIRSCAN_EDEVICE;
}

bool overlap(const void* a, uint64_t na, const void* b, uint64_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  if (na == 0 || nb == 0) return false;
  return x < y + nb && y < x + na;
}

// Bytes of the packed operand, with the same overflow bound as the words.
unsigned __int128 packed_bytes_wide(unsigned __int128 P, uint32_t D0, uint32_t D1) {
  return P * ((D1 + 15ull) / 16) * ((D0 + 63ull) / 64) * 4096;
}

// Validates a RowSel shape; on success returns P and the p-major DB word count.
bool rowsel_shape_ok(const pirscan_rowsel_shape* s, uint64_t* P, uint64_t* db_words) {
  if (!s || s->N == 0 || s->R == 0 || s->R > PIRSCAN_MAX_R || s->D0 == 0 || s->D1 == 0) return false;
  if (s->scan != PIRSCAN_SCAN_AUTO && s->scan != PIRSCAN_SCAN_VALU) return false;
  for (uint32_t r = 0; r < s->R; ++r)
    if (s->q[r] < 2) return false;
  const unsigned __int128 p = (unsigned __int128)s->R * s->N;
  const unsigned __int128 words = p * s->D0 * s->D1;
  if (words * 4 > (unsigned __int128)(~(uint64_t)0 >> 1)) return false;
  if (packed_bytes_wide(p, s->D0, s->D1) > (unsigned __int128)(~(uint64_t)0 >> 1)) return false;
  *P = (uint64_t)p;
  *db_words = (uint64_t)words;
  return true;
}

// Per-prime constants and the fold period shared by every modular GEMM.
void fill_limb_consts(const uint32_t* q, uint32_t R, pirscan::RowselLaunch* a) {
  a->fold = 32;
  for (uint32_t r = 0; r < R; ++r) {
    a->lc.q[r] = q[r];
    a->lc.c[r] = (uint32_t)((((uint64_t)1) << 32) % q[r]);
    a->lc.mu[r] = ~(uint64_t)0 / q[r];
    const uint32_t f = pirscan::rowsel_fold_period(q[r]);
    if (f < a->fold) a->fold = f;
  }
}

constexpr unsigned __int128 kMaxBytes = ~(uint64_t)0 >> 1;

// Validates an ExpPack shape and batch (B may be 0 when only the hint size is
// wanted); on success returns P and the word counts of H, C, G and out.
bool exppack_shape_ok(const pirscan_exppack_shape* s, uint32_t B, uint64_t* P, uint64_t* h_words,
                      uint64_t* c_words, uint64_t* g_words, uint64_t* o_words) {
  if (!s || s->N == 0 || s->R == 0 || s->R > PIRSCAN_MAX_R || s->Dr == 0 || s->n == 0) return false;
  if (s->scan != PIRSCAN_SCAN_AUTO && s->scan != PIRSCAN_SCAN_VALU) return false;
  if (B > pirscan::kMaxRows / 2) return false;
  for (uint32_t r = 0; r < s->R; ++r)
    if (s->q[r] < 2) return false;
  const unsigned __int128 p = (unsigned __int128)s->R * s->N;
  const unsigned __int128 h = p * s->Dr * s->n, c = p * s->n * 2 * B, g = p * s->Dr * B,
                          o = p * s->Dr * 2 * B;
  if (h * 4 > kMaxBytes || c * 4 > kMaxBytes || o * 4 > kMaxBytes) return false;
  if (packed_bytes_wide(p, s->n, s->Dr) > kMaxBytes) return false;
  *P = (uint64_t)p;
  *h_words = (uint64_t)h;
  *c_words = (uint64_t)c;
  *g_words = (uint64_t)g;
  *o_words = (uint64_t)o;
  return true;
}

// ExpPack as the point-wise modular GEMM with roles swapped (ct = C^T,
// DB = H^T, D0 = n, D1 = Dr, m = 2B) and G as the body term.
void exppack_launch_desc(const pirscan_exppack_shape* s, uint32_t B, uint64_t P, const uint32_t* C,
                         const uint32_t* h_tiled, const uint32_t* G, uint32_t* out,
                         pirscan::RowselLaunch* a) {
  *a = pirscan::RowselLaunch{};
  const uint64_t cols = 2ull * B;
  a->ct = C;
  a->dbt = h_tiled;
  a->out = out;
  a->add = G;
  a->ct_sm = P;  // C [n][2B][P]: column j of C is row mi = j of C^T
  a->ct_sk = cols * P;
  a->out_sm = P;  // out [Dr][2B][P]
  a->out_sn = cols * P;
  a->add_sb = P;  // G [Dr][B][P]
  a->add_sn = (uint64_t)B * P;
  a->P = P;
  a->N = s->N;
  a->D0 = s->n;
  a->D1 = s->Dr;
  a->m = (uint32_t)cols;
  a->scan = s->scan;
  fill_limb_consts(s->q, s->R, a);
}

// Whether the shape's DB / hint operand is packed for the MFMA scan (scan
// kind AUTO with every q < 2^31 and D0 <= 16384), or kept word-transposed for
// the VALU scan.
bool packed_shape(const uint32_t* q, uint32_t R, uint32_t D0, uint32_t scan) {
  return scan == PIRSCAN_SCAN_AUTO && pirscan::rowsel_packed_ok(q, R, D0);
}

// Bytes of the relaid DB / hint operand (D0 = reduction extent, D1 = columns).
uint64_t operand_layout_bytes(const uint32_t* q, uint32_t R, uint64_t P, uint32_t D0, uint32_t D1,
                              uint32_t scan) {
  if (packed_shape(q, R, D0, scan)) return pirscan::packed_layout_bytes(P, D0, D1);
  return 4ull * P * D0 * D1;
}

// Workspace of the point-wise modular GEMM: the MFMA path's A fragments and
// output staging, or the VALU path's output staging.
size_t modgemm_workspace_bytes(const pirscan::RowselLaunch& a, uint32_t R) {
  if (packed_shape(a.lc.q, R, a.D0, a.scan)) return pirscan::rowsel_packed_workspace_bytes(a.P, a.m, a.D0, a.D1);
  return pirscan::rowsel_valu_workspace_bytes(a.P, a.m, a.D1);
}

struct Span {
  const void* p;
  uint64_t bytes;
};

// Workspace checks shared by RowSel and ExpPack, then dispatch.
int run_modgemm(const pirscan::RowselLaunch& a, uint32_t R, const Span* bufs, int nbufs, void* workspace,
                size_t workspace_bytes, void* stream) {
  const size_t need = modgemm_workspace_bytes(a, R);
  if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) % 16) != 0)
    return PIRSCAN_EINVAL;
  for (int i = 0; i < nbufs; ++i)
    if (overlap(workspace, need, bufs[i].p, bufs[i].bytes)) return PIRSCAN_EINVAL;
  const bool packed = packed_shape(a.lc.q, R, a.D0, a.scan);
  if (packed && (reinterpret_cast<uintptr_t>(a.dbt) % 16) != 0) return PIRSCAN_EINVAL;
  const int dc = device_check();
  if (dc != PIRSCAN_OK) return dc;
  if (packed) return device_status(pirscan::launch_rowsel_packed(a, R, workspace, (hipStream_t)stream));
  return device_status(pirscan::launch_rowsel(a, workspace, (hipStream_t)stream));
}

// Optional input validation (defined below, with its device flag).
bool validation_on();
int check_residues(const uint32_t* x, uint64_t words, uint64_t P, uint32_t N, const uint32_t* q, uint32_t R,
                   hipStream_t stream);

// ---- NTT shape validation (host) -----------------------------------------

uint32_t host_mulmod(uint32_t a, uint32_t b, uint32_t q) { return (uint32_t)(((uint64_t)a * b) % q); }

uint32_t host_powmod(uint32_t b, uint64_t e, uint32_t q) {
  uint32_t r = 1 % q;
  b %= q;
  for (; e; e >>= 1) {
    if (e & 1) r = host_mulmod(r, b, q);
    b = host_mulmod(b, b, q);
  }
  return r;
}

// Deterministic primality for 32-bit n: Miller-Rabin to the bases 2, 7 and 61
// (Jaeschke: no odd composite below 4,759,123,141 is a strong pseudoprime to
// all three).
bool host_is_prime(uint32_t n) {
  if (n < 2) return false;
  for (uint32_t p : {2u, 3u, 5u, 7u, 11u, 13u, 61u}) {
    if (n == p) return true;
    if (n % p == 0) return false;
  }
  uint32_t d = n - 1;
  int s = 0;
  while ((d & 1) == 0) {
    d >>= 1;
    ++s;
  }
  for (uint32_t a : {2u, 7u, 61u}) {
    uint32_t x = host_powmod(a, d, n);
    if (x == 1 || x == n - 1) continue;
    bool composite = true;
    for (int i = 1; i < s && composite; ++i) {
      x = host_mulmod(x, x, n);
      if (x == n - 1) composite = false;
    }
    if (composite) return false;
  }
  return true;
}

// Validates an NTT shape (N a power of two in [16, 8192]; every q prime,
// < 2^30, q == 1 mod 2N; psi^N == -1 mod q) and precomputes N^-1 mod q.
bool ntt_shape_ok(const pirscan_ntt_shape* s, pirscan::NttDesc* d) {
  if (!s || s->R == 0 || s->R > PIRSCAN_MAX_R) return false;
  if (s->N < 16 || s->N > 8192 || (s->N & (s->N - 1)) != 0) return false;
  *d = pirscan::NttDesc{};
  d->N = s->N;
  d->R = s->R;
  while ((1u << d->logn) < s->N) ++d->logn;
  for (uint32_t r = 0; r < s->R; ++r) {
    const uint32_t q = s->q[r], psi = s->psi[r];
    if (q >= (1u << 30) || (q - 1) % (2 * s->N) != 0 || !host_is_prime(q)) return false;
    if (psi == 0 || psi >= q || host_powmod(psi, s->N, q) != q - 1) return false;
    d->q[r] = q;
    d->psi.v[r] = psi;
    d->ninv[r] = host_powmod(s->N, q - 2, q);  // Fermat: q is prime
  }
  return true;
}

// Runs one transform after the checks every transform shares.
int run_ntt(const pirscan_ntt_shape* s, pirscan::NttMode mode, const void* plan, const uint32_t* in,
            uint32_t* out, uint64_t count, void* stream) {
  pirscan::NttDesc d;
  if (!ntt_shape_ok(s, &d) || !plan || !in || !out || count == 0) return PIRSCAN_EINVAL;
  if ((reinterpret_cast<uintptr_t>(plan) % 16) != 0) return PIRSCAN_EINVAL;
  const unsigned __int128 poly = (unsigned __int128)count * d.N;
  const unsigned __int128 ow = poly * d.R;
  const unsigned __int128 iw = mode == pirscan::NttMode::kRnsForward ? poly : ow;
  if (ow * 4 > kMaxBytes || count > 0x7FFFFFFFull / d.R) return PIRSCAN_EINVAL;
  const uint64_t plan_b = pirscan::ntt_plan_bytes(d.N, d.R);
  // in-place is allowed for the residue transforms (every workgroup reads its
  // whole row before writing it); any other overlap is not
  const bool same = static_cast<const void*>(in) == static_cast<const void*>(out);
  if (!(same && mode != pirscan::NttMode::kRnsForward) && overlap(in, (uint64_t)iw * 4, out, (uint64_t)ow * 4))
    return PIRSCAN_EINVAL;
  if (overlap(plan, plan_b, out, (uint64_t)ow * 4)) return PIRSCAN_EINVAL;
  const int dc = device_check();
  if (dc != PIRSCAN_OK) return dc;
  if (mode != pirscan::NttMode::kRnsForward && validation_on()) {
    const int vc = check_residues(in, (uint64_t)ow, (uint64_t)d.R * d.N, d.N, d.q, d.R, (hipStream_t)stream);
    if (vc != PIRSCAN_OK) return vc;
  }
  return device_status(pirscan::launch_ntt(d, mode, plan, in, out, count, (hipStream_t)stream));
}

// ---- optional input validation -------------------------------------------------
//
// With PIRSCAN_VALIDATE_INPUTS=1 in the environment (read at every call), the
// entry points whose inputs are residues check every one against its modulus
// before any other device work and return PIRSCAN_EINVAL if one is not below
// it.  A debugging aid: the check synchronises the caller's stream.

bool validation_on() {
  const char* v = getenv("PIRSCAN_VALIDATE_INPUTS");
  return v && v[0] == '1' && v[1] == 0;
}

struct Moduli {
  uint32_t v[PIRSCAN_MAX_R];
};

// Set to 1 by the check kernel when a word is out of range; one per device.
__device__ uint32_t g_bad_input;
std::atomic<void*> g_bad_input_ptr[kMaxDevices];

__global__ void clear_word_kernel(uint32_t* w) {
  if (threadIdx.x == 0) *w = 0;
}

// Word i of an array whose last axis is the P = R*N points belongs to limb
// (i % P) / N.
__global__ __launch_bounds__(256) void check_residues_kernel(const uint32_t* __restrict__ x, uint64_t words,
                                                             uint64_t P, uint32_t N, Moduli q,
                                                             uint32_t* __restrict__ bad) {
  const uint64_t stride = (uint64_t)gridDim.x * 256;
  bool any = false;
  for (uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x; i < words; i += stride)
    any |= x[i] >= q.v[(i % P) / N];
  if (any) *bad = 1;
}

// Checks words < q[(i % P) / N] for every word of x; PIRSCAN_EINVAL if one is not.
int check_residues(const uint32_t* x, uint64_t words, uint64_t P, uint32_t N, const uint32_t* q, uint32_t R,
                   hipStream_t stream) {
  if (!x || words == 0) return PIRSCAN_OK;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_status(e);
  if (dev < 0 || dev >= kMaxDevices) return PIRSCAN_EUNSUPPORTED;
  void* flag = g_bad_input_ptr[dev].load(std::memory_order_acquire);
  if (!flag) {
    e = hipGetSymbolAddress(&flag, HIP_SYMBOL(g_bad_input));
    if (e != hipSuccess) return device_status(e);
    g_bad_input_ptr[dev].store(flag, std::memory_order_release);
  }
  Moduli m{};
  for (uint32_t r = 0; r < R && r < PIRSCAN_MAX_R; ++r) m.v[r] = q[r];
  uint32_t* f = static_cast<uint32_t*>(flag);
  hipLaunchKernelGGL(clear_word_kernel, dim3(1), dim3(64), 0, stream, f);
  uint64_t grid = (words + 255) / 256;
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(check_residues_kernel, dim3((uint32_t)grid), dim3(256), 0, stream, x, words, P, N, m, f);
  uint32_t host = 0;
  e = hipGetLastError();
  if (e == hipSuccess) e = hipMemcpyAsync(&host, f, sizeof(host), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return device_status(e);
  return host ? PIRSCAN_EINVAL : PIRSCAN_OK;
}

// ---- scratch of the no-allocation entry point --------------------------------

// The scratch buffer of pirscan_scalar_gemm_u32_noalloc.  Each GPU the library
// runs on holds its own copy, at its own address, until the process ends.  In
// host code `scratch` names a host-side stand-in, never the device memory:
// the device address comes from hipGetSymbolAddress, once per device.
__device__ __align__(256) uint8_t scratch[PIRSCAN_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// The current device's address of `scratch`, looked up on the first call on
// that device (with it current) and kept.
int scratch_on_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_status(e);
  if (dev < 0 || dev >= kMaxDevices) return PIRSCAN_EUNSUPPORTED;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return device_status(e);
      if (!p) return PIRSCAN_EDEVICE;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return PIRSCAN_OK;
}

}  // namespace

namespace pirscan {

int api_device_check() { return device_check(); }
int api_device_status(hipError_t e) { return device_status(e); }

}  // namespace pirscan

extern "C" {

size_t pirscan_layout_db_bytes(const pirscan_rowsel_shape* s) {
  uint64_t P = 0, words = 0;
  if (!rowsel_shape_ok(s, &P, &words)) return 0;
  return (size_t)operand_layout_bytes(s->q, s->R, P, s->D0, s->D1, s->scan);
}

int pirscan_layout_db(const pirscan_rowsel_shape* s, const uint32_t* db_pmajor, uint32_t* db_tiled,
                      void* stream) {
  uint64_t P = 0, words = 0;
  if (!rowsel_shape_ok(s, &P, &words) || !db_pmajor || !db_tiled) return PIRSCAN_EINVAL;
  const uint64_t tiled_bytes = operand_layout_bytes(s->q, s->R, P, s->D0, s->D1, s->scan);
  const bool packed = packed_shape(s->q, s->R, s->D0, s->scan);
  if (overlap(db_pmajor, words * 4, db_tiled, tiled_bytes)) return PIRSCAN_EINVAL;
  if (packed && (reinterpret_cast<uintptr_t>(db_tiled) % 16) != 0) return PIRSCAN_EINVAL;
  const int dc = device_check();
  if (dc != PIRSCAN_OK) return dc;
  if (validation_on()) {
    const int vc = check_residues(db_pmajor, words, P, s->N, s->q, s->R, (hipStream_t)stream);
    if (vc != PIRSCAN_OK) return vc;
  }
  if (packed)  // [D0][D1][P]: column n is fragment row n (stride P), k has stride D1*P
    return device_status(pirscan::launch_pack_operand(db_pmajor, db_tiled, P, s->N, s->q, s->R, s->D1, s->D0, P,
                                                      (uint64_t)s->D1 * P, (hipStream_t)stream));
  return device_status(pirscan::launch_layout_db(db_pmajor, db_tiled, (uint64_t)s->D0 * s->D1, P,
                                                 (hipStream_t)stream));
}

// Fills the launch description (pointers may be null when only sizes are
// wanted).  Returns false on an invalid shape or m.
static bool rowsel_launch_desc(const pirscan_rowsel_shape* s, uint32_t m, const uint32_t* ct,
                               const uint32_t* db_tiled, uint32_t* out, pirscan::RowselLaunch* a,
                               uint64_t* db_words, uint64_t* ct_words, uint64_t* out_words) {
  uint64_t P = 0;
  if (!rowsel_shape_ok(s, &P, db_words) || m == 0 || m > pirscan::kMaxRows) return false;
  const unsigned __int128 cw = (unsigned __int128)m * s->D0 * P;
  const unsigned __int128 ow = (unsigned __int128)m * s->D1 * P;
  if (cw * 4 > (unsigned __int128)(~(uint64_t)0 >> 1) || ow * 4 > (unsigned __int128)(~(uint64_t)0 >> 1))
    return false;
  *ct_words = (uint64_t)cw;
  *out_words = (uint64_t)ow;
  *a = pirscan::RowselLaunch{};
  a->ct = ct;
  a->dbt = db_tiled;
  a->out = out;
  a->ct_sm = (uint64_t)s->D0 * P;  // ct [m][D0][P]
  a->ct_sk = P;
  a->out_sm = (uint64_t)s->D1 * P;  // out [m][D1][P]
  a->out_sn = P;
  a->P = P;
  a->N = s->N;
  a->D0 = s->D0;
  a->D1 = s->D1;
  a->m = m;
  a->scan = s->scan;
  fill_limb_consts(s->q, s->R, a);
  return true;
}

size_t pirscan_rowsel_workspace_bytes(const pirscan_rowsel_shape* s, uint32_t m) {
  pirscan::RowselLaunch a;
  uint64_t dbw, ctw, ow;
  if (!rowsel_launch_desc(s, m, nullptr, nullptr, nullptr, &a, &dbw, &ctw, &ow)) return 0;
  return modgemm_workspace_bytes(a, s->R);
}

int pirscan_rowsel_modgemm(const pirscan_rowsel_shape* s, uint32_t m, const uint32_t* ct,
                           const uint32_t* db_tiled, uint32_t* out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  pirscan::RowselLaunch a;
  uint64_t dbw = 0, ctw = 0, ow = 0;
  if (!ct || !db_tiled || !out || !rowsel_launch_desc(s, m, ct, db_tiled, out, &a, &dbw, &ctw, &ow))
    return PIRSCAN_EINVAL;
  const uint64_t db_bytes = operand_layout_bytes(s->q, s->R, a.P, s->D0, s->D1, s->scan);
  if (overlap(out, ow * 4, ct, ctw * 4) || overlap(out, ow * 4, db_tiled, db_bytes)) return PIRSCAN_EINVAL;
  const Span ins[] = {{ct, ctw * 4}, {db_tiled, db_bytes}, {out, ow * 4}};
  if (validation_on()) {
    const int dc = device_check();
    if (dc != PIRSCAN_OK) return dc;
    const int vc = check_residues(ct, ctw, a.P, s->N, s->q, s->R, (hipStream_t)stream);
    if (vc != PIRSCAN_OK) return vc;
  }
  return run_modgemm(a, s->R, ins, 3, workspace, workspace_bytes, stream);
}

size_t pirscan_exppack_layout_h_bytes(const pirscan_exppack_shape* s) {
  uint64_t P, h, c, g, o;
  if (!exppack_shape_ok(s, 0, &P, &h, &c, &g, &o)) return 0;
  return (size_t)operand_layout_bytes(s->q, s->R, P, s->n, s->Dr, s->scan);
}

int pirscan_exppack_layout_h(const pirscan_exppack_shape* s, const uint32_t* h_pmajor,
                             uint32_t* h_tiled, void* stream) {
  uint64_t P, h, c, g, o;
  if (!exppack_shape_ok(s, 0, &P, &h, &c, &g, &o) || !h_pmajor || !h_tiled) return PIRSCAN_EINVAL;
  const uint64_t tiled_bytes = operand_layout_bytes(s->q, s->R, P, s->n, s->Dr, s->scan);
  const bool packed = packed_shape(s->q, s->R, s->n, s->scan);
  if (overlap(h_pmajor, h * 4, h_tiled, tiled_bytes)) return PIRSCAN_EINVAL;
  if (packed && (reinterpret_cast<uintptr_t>(h_tiled) % 16) != 0) return PIRSCAN_EINVAL;
  const int dc = device_check();
  if (dc != PIRSCAN_OK) return dc;
  if (validation_on()) {
    const int vc = check_residues(h_pmajor, h, P, s->N, s->q, s->R, (hipStream_t)stream);
    if (vc != PIRSCAN_OK) return vc;
  }
  // The GEMM's DB operand is H^T: hint column i is the reduction index k and
  // row r the output column.  H [Dr][n][P]: r has stride n*P, i stride P.
  if (packed)
    return device_status(pirscan::launch_pack_operand(h_pmajor, h_tiled, P, s->N, s->q, s->R, s->Dr, s->n,
                                                      (uint64_t)s->n * P, P, (hipStream_t)stream));
  // [Dr][n][P] -> [P][n][Dr]: for each hint column i, a Dr x P transpose.
  pirscan::TransposeDesc t{};
  t.src = h_pmajor;
  t.dst = h_tiled;
  t.batch = s->n;
  t.rows = s->Dr;
  t.cols = P;
  t.s_batch = P;
  t.s_row = (uint64_t)s->n * P;
  t.d_batch = s->Dr;
  t.d_row = (uint64_t)s->n * s->Dr;
  return device_status(pirscan::launch_transpose(t, (hipStream_t)stream));
}

size_t pirscan_exppack_workspace_bytes(const pirscan_exppack_shape* s, uint32_t B) {
  uint64_t P, h, c, g, o;
  if (B == 0 || !exppack_shape_ok(s, B, &P, &h, &c, &g, &o)) return 0;
  pirscan::RowselLaunch a;
  exppack_launch_desc(s, B, P, nullptr, nullptr, nullptr, nullptr, &a);
  return modgemm_workspace_bytes(a, s->R);
}

int pirscan_exppack_modgemm(const pirscan_exppack_shape* s, uint32_t B, const uint32_t* C,
                            const uint32_t* h_tiled, const uint32_t* G, uint32_t* out,
                            void* workspace, size_t workspace_bytes, void* stream) {
  uint64_t P, hw, cw, gw, ow;
  if (B == 0 || !C || !h_tiled || !out || !exppack_shape_ok(s, B, &P, &hw, &cw, &gw, &ow))
    return PIRSCAN_EINVAL;
  const uint64_t gb = G ? gw * 4 : 0;
  const uint64_t hb = operand_layout_bytes(s->q, s->R, P, s->n, s->Dr, s->scan);
  if (overlap(out, ow * 4, C, cw * 4) || overlap(out, ow * 4, h_tiled, hb) || overlap(out, ow * 4, G, gb))
    return PIRSCAN_EINVAL;
  pirscan::RowselLaunch a;
  exppack_launch_desc(s, B, P, C, h_tiled, G, out, &a);
  const Span ins[] = {{C, cw * 4}, {h_tiled, hb}, {G, gb}, {out, ow * 4}};
  if (validation_on()) {
    const int dc = device_check();
    if (dc != PIRSCAN_OK) return dc;
    int vc = check_residues(C, cw, P, s->N, s->q, s->R, (hipStream_t)stream);
    if (vc == PIRSCAN_OK && G) vc = check_residues(G, gw, P, s->N, s->q, s->R, (hipStream_t)stream);
    if (vc != PIRSCAN_OK) return vc;
  }
  return run_modgemm(a, s->R, ins, 4, workspace, workspace_bytes, stream);
}

size_t pirscan_scalar_workspace_bytes(uint64_t M, uint64_t K, uint32_t B) {
  pirscan::ScalarPlan p;
  // Sized for the aligned fast path, which needs the most.
  if (!pirscan::scalar_plan(M, K, B, 0, &p)) return 0;
  return p.fast ? p.total_bytes : 0;
}

int pirscan_scalar_gemm_u32(const int8_t* db, const uint32_t* query, uint32_t* out, uint64_t M,
                            uint64_t K, uint32_t B, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (!db || !query || !out) return PIRSCAN_EINVAL;
  pirscan::ScalarPlan p;
  if (!pirscan::scalar_plan(M, K, B, reinterpret_cast<uintptr_t>(db), &p)) return PIRSCAN_EINVAL;
  const uint64_t db_bytes = M * K, q_bytes = K * B * 4ull, o_bytes = M * B * 4ull;
  if (p.fast && p.total_bytes > 0) {
    if (!workspace || workspace_bytes < p.total_bytes ||
        (reinterpret_cast<uintptr_t>(workspace) % 16) != 0)
      return PIRSCAN_EINVAL;
    if (overlap(workspace, p.total_bytes, db, db_bytes) ||
        overlap(workspace, p.total_bytes, query, q_bytes) ||
        overlap(workspace, p.total_bytes, out, o_bytes))
      return PIRSCAN_EINVAL;
  }
  if (overlap(out, o_bytes, db, db_bytes) || overlap(out, o_bytes, query, q_bytes))
    return PIRSCAN_EINVAL;
  const int dc = device_check();
  if (dc != PIRSCAN_OK) return dc;
  return device_status(
      pirscan::launch_scalar(db, query, out, M, K, B, p, workspace, (hipStream_t)stream));
}

int pirscan_scalar_gemm_u32_noalloc(const int8_t* db, const uint32_t* query, uint32_t* out, uint64_t M,
                                    uint64_t K, uint32_t B, void* stream) {
  if (!db || !query || !out) return PIRSCAN_EINVAL;
  pirscan::ScalarPlan p;
  if (!pirscan::scalar_plan(M, K, B, reinterpret_cast<uintptr_t>(db), &p)) return PIRSCAN_EINVAL;
  const uint64_t db_bytes = M * K, q_bytes = K * B * 4ull, o_bytes = M * B * 4ull;
  if (overlap(out, o_bytes, db, db_bytes) || overlap(out, o_bytes, query, q_bytes)) return PIRSCAN_EINVAL;
  const bool needs_scratch = p.fast && p.total_bytes > 0;
  if (needs_scratch && p.total_bytes > PIRSCAN_NOALLOC_SCRATCH_BYTES) return PIRSCAN_ESCRATCH;
  const int dc = device_check();
  if (dc != PIRSCAN_OK) return dc;
  void* ws = nullptr;
  if (needs_scratch) {
    const int sc = scratch_on_current_device(&ws);
    if (sc != PIRSCAN_OK) return sc;
  }
  return device_status(pirscan::launch_scalar(db, query, out, M, K, B, p, ws, (hipStream_t)stream));
}

size_t pirscan_scalar_layout_db_bytes(uint64_t M, uint64_t K) {
  pirscan::ScalarPlan p;
  if (!pirscan::scalar_tiled_plan(M, K, 1, &p)) return 0;
  return (size_t)pirscan::scalar_layout_bytes(M, K);
}

int pirscan_scalar_layout_db(const int8_t* db, void* db_tiled, uint64_t M, uint64_t K, void* stream) {
  pirscan::ScalarPlan p;
  if (!db || !db_tiled || !pirscan::scalar_tiled_plan(M, K, 1, &p)) return PIRSCAN_EINVAL;
  if ((reinterpret_cast<uintptr_t>(db_tiled) % 16) != 0) return PIRSCAN_EINVAL;
  if (overlap(db, M * K, db_tiled, pirscan::scalar_layout_bytes(M, K))) return PIRSCAN_EINVAL;
  const int dc = device_check();
  if (dc != PIRSCAN_OK) return dc;
  return device_status(pirscan::launch_scalar_layout(db, db_tiled, M, K, (hipStream_t)stream));
}

size_t pirscan_scalar_tiled_workspace_bytes(uint64_t M, uint64_t K, uint32_t B) {
  pirscan::ScalarPlan p;
  if (!pirscan::scalar_tiled_plan(M, K, B, &p)) return 0;
  return p.total_bytes;
}

int pirscan_scalar_gemm_u32_tiled(const void* db_tiled, const uint32_t* query, uint32_t* out, uint64_t M,
                                  uint64_t K, uint32_t B, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  if (!db_tiled || !query || !out || !workspace) return PIRSCAN_EINVAL;
  pirscan::ScalarPlan p;
  if (!pirscan::scalar_tiled_plan(M, K, B, &p)) return PIRSCAN_EINVAL;
  const uint64_t db_bytes = pirscan::scalar_layout_bytes(M, K), q_bytes = K * B * 4ull, o_bytes = M * B * 4ull;
  if ((reinterpret_cast<uintptr_t>(db_tiled) % 16) != 0) return PIRSCAN_EINVAL;
  if (workspace_bytes < p.total_bytes || (reinterpret_cast<uintptr_t>(workspace) % 16) != 0)
    return PIRSCAN_EINVAL;
  if (overlap(workspace, p.total_bytes, db_tiled, db_bytes) || overlap(workspace, p.total_bytes, query, q_bytes) ||
      overlap(workspace, p.total_bytes, out, o_bytes))
    return PIRSCAN_EINVAL;
  if (overlap(out, o_bytes, db_tiled, db_bytes) || overlap(out, o_bytes, query, q_bytes)) return PIRSCAN_EINVAL;
  const int dc = device_check();
  if (dc != PIRSCAN_OK) return dc;
  return device_status(
      pirscan::launch_scalar_tiled(db_tiled, query, out, M, K, B, p, workspace, (hipStream_t)stream));
}

size_t pirscan_ntt_plan_bytes(const pirscan_ntt_shape* s) {
  pirscan::NttDesc d;
  if (!ntt_shape_ok(s, &d)) return 0;
  return pirscan::ntt_plan_bytes(d.N, d.R);
}

int pirscan_ntt_plan_init(const pirscan_ntt_shape* s, void* plan, size_t plan_bytes, void* stream) {
  pirscan::NttDesc d;
  if (!ntt_shape_ok(s, &d) || !plan || (reinterpret_cast<uintptr_t>(plan) % 16) != 0) return PIRSCAN_EINVAL;
  if (plan_bytes < pirscan::ntt_plan_bytes(d.N, d.R)) return PIRSCAN_EINVAL;
  const int dc = device_check();
  if (dc != PIRSCAN_OK) return dc;
  return device_status(pirscan::launch_ntt_plan(d, plan, (hipStream_t)stream));
}

int pirscan_ntt_forward(const pirscan_ntt_shape* s, const void* plan, const uint32_t* in, uint32_t* out,
                        uint64_t count, void* stream) {
  return run_ntt(s, pirscan::NttMode::kForward, plan, in, out, count, stream);
}

int pirscan_ntt_inverse(const pirscan_ntt_shape* s, const void* plan, const uint32_t* in, uint32_t* out,
                        uint64_t count, void* stream) {
  return run_ntt(s, pirscan::NttMode::kInverse, plan, in, out, count, stream);
}

int pirscan_ntt_rns_forward(const pirscan_ntt_shape* s, const void* plan, const uint32_t* coeffs,
                            uint32_t* out, uint64_t count, void* stream) {
  return run_ntt(s, pirscan::NttMode::kRnsForward, plan, coeffs, out, count, stream);
}

const char* pirscan_strerror(int status) {
  switch (status) {
    case PIRSCAN_OK: return "ok";
    case PIRSCAN_EINVAL: return "invalid argument";
    case PIRSCAN_EDEVICE: return "HIP runtime error";
    case PIRSCAN_EUNSUPPORTED: return "unsupported device (gfx950 required)";
    case PIRSCAN_ESCRATCH: return "problem needs more than the no-allocation entry point's scratch buffer";
    default: return "unknown status";
  }
}

int pirscan_version(void) { return PIRSCAN_VERSION; }

int pirscan_last_device_error(void) { return g_last_hip_error; }

}  // extern "C"
