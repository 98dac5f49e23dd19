// pirscan_api.hip -- the C ABI of libpirscan: argument validation, device
// check, constant precomputation and kernel dispatch on the caller's stream.
// Every entry point declared in include/pirscan.h is defined here.
#include <hip/hip_runtime.h>
#include <string.h>

#include <atomic>

#include "../../include/pirscan.h"
#include "internal.hpp"

namespace {

thread_local int g_last_hip_error = 0;

// Per-device "is gfx950" cache: 0 unknown, 1 yes, 2 no.
constexpr int kMaxDevices = 64;
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

// Validates a RowSel shape; on success returns P and the DB word count.
bool rowsel_shape_ok(const pirscan_rowsel_shape* s, uint64_t* P, uint64_t* db_words) {
  if (!s || s->N == 0 || s->R == 0 || s->R > PIRSCAN_MAX_R || s->D0 == 0 || s->D1 == 0) return false;
  for (uint32_t r = 0; r < s->R; ++r)
    if (s->q[r] < 2) return false;
  const unsigned __int128 p = (unsigned __int128)s->R * s->N;
  const unsigned __int128 words = p * s->D0 * s->D1;
  if (words * 4 > (unsigned __int128)(~(uint64_t)0 >> 1)) return false;
  *P = (uint64_t)p;
  *db_words = (uint64_t)words;
  return true;
}

}  // namespace

extern "C" {

size_t pirscan_layout_db_bytes(const pirscan_rowsel_shape* s) {
  uint64_t P = 0, words = 0;
  if (!rowsel_shape_ok(s, &P, &words)) return 0;
  return (size_t)(words * 4);
}

int pirscan_layout_db(const pirscan_rowsel_shape* s, const uint32_t* db_pmajor, uint32_t* db_tiled,
                      void* stream) {
  uint64_t P = 0, words = 0;
  if (!rowsel_shape_ok(s, &P, &words) || !db_pmajor || !db_tiled) return PIRSCAN_EINVAL;
  if (overlap(db_pmajor, words * 4, db_tiled, words * 4)) return PIRSCAN_EINVAL;
  const int dc = device_check();
  if (dc != PIRSCAN_OK) return dc;
  return device_status(pirscan::launch_layout_db(db_pmajor, db_tiled, (uint64_t)s->D0 * s->D1, P,
                                                 (hipStream_t)stream));
}

// Fills the launch description (pointers may be null when only sizes are
// wanted).  Returns false on an invalid shape or m.
static bool rowsel_launch_desc(const pirscan_rowsel_shape* s, uint32_t m, const uint32_t* ct,
                               const uint32_t* db_tiled, uint32_t* out, pirscan::RowselLaunch* a,
                               uint64_t* db_words, uint64_t* ct_words, uint64_t* out_words) {
  uint64_t P = 0;
  if (!rowsel_shape_ok(s, &P, db_words) || m == 0) return false;
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
  a->P = P;
  a->N = s->N;
  a->D0 = s->D0;
  a->D1 = s->D1;
  a->m = m;
  a->fold = 32;
  for (uint32_t r = 0; r < s->R; ++r) {
    const uint32_t q = s->q[r];
    a->lc.q[r] = q;
    a->lc.c[r] = (uint32_t)((((uint64_t)1) << 32) % q);
    a->lc.mu[r] = ~(uint64_t)0 / q;
    const uint32_t f = pirscan::rowsel_fold_period(q);
    if (f < a->fold) a->fold = f;
  }
  return true;
}

size_t pirscan_rowsel_workspace_bytes(const pirscan_rowsel_shape* s, uint32_t m) {
  pirscan::RowselLaunch a;
  uint64_t dbw, ctw, ow;
  if (!rowsel_launch_desc(s, m, nullptr, nullptr, nullptr, &a, &dbw, &ctw, &ow)) return 0;
  if (!pirscan::rowsel_mfma_eligible(a, s->R)) return 0;
  return pirscan::rowsel_mfma_workspace_bytes(a.P, m, s->D0, s->D1);
}

int pirscan_rowsel_modgemm(const pirscan_rowsel_shape* s, uint32_t m, const uint32_t* ct,
                           const uint32_t* db_tiled, uint32_t* out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  pirscan::RowselLaunch a;
  uint64_t dbw = 0, ctw = 0, ow = 0;
  if (!ct || !db_tiled || !out || !rowsel_launch_desc(s, m, ct, db_tiled, out, &a, &dbw, &ctw, &ow))
    return PIRSCAN_EINVAL;
  if (overlap(out, ow * 4, ct, ctw * 4) || overlap(out, ow * 4, db_tiled, dbw * 4)) return PIRSCAN_EINVAL;
  const bool mfma = pirscan::rowsel_mfma_eligible(a, s->R);
  size_t need = 0;
  if (mfma) {
    need = pirscan::rowsel_mfma_workspace_bytes(a.P, m, s->D0, s->D1);
    if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) % 16) != 0)
      return PIRSCAN_EINVAL;
    if (overlap(workspace, need, ct, ctw * 4) || overlap(workspace, need, db_tiled, dbw * 4) ||
        overlap(workspace, need, out, ow * 4))
      return PIRSCAN_EINVAL;
  }
  const int dc = device_check();
  if (dc != PIRSCAN_OK) return dc;
  if (mfma) return device_status(pirscan::launch_rowsel_mfma(a, s->R, workspace, (hipStream_t)stream));
  return device_status(pirscan::launch_rowsel(a, (hipStream_t)stream));
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

const char* pirscan_strerror(int status) {
  switch (status) {
    case PIRSCAN_OK: return "ok";
    case PIRSCAN_EINVAL: return "invalid argument";
    case PIRSCAN_EDEVICE: return "HIP runtime error";
    case PIRSCAN_EUNSUPPORTED: return "unsupported device (gfx950 required)";
    default: return "unknown status";
  }
}

int pirscan_version(void) { return PIRSCAN_VERSION; }

int pirscan_last_device_error(void) { return g_last_hip_error; }

}  // extern "C"
