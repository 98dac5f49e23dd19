// synth.hip -- device filler for the seeded synthetic inputs.
//
// Same generator as synth/__init__.py: the i-th SplitMix64 output from a
// start state computed on the host, value(i) = mix64(state0 + (i+1)*gamma),
// with the finaliser constants of Vigna's public splitmix64.c.  This file
// holds no part of the scan's arithmetic; it only writes input buffers.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ull;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBull;
  z ^= z >> 31;
  return z;
}

__device__ __forceinline__ uint64_t value(uint64_t st, uint64_t i) {
  return mix64(st + (i + 1) * kGamma);
}

struct Moduli {
  uint32_t q[8];
};

__global__ void fill_residues(uint32_t* out, uint64_t count, uint64_t st, uint64_t first,
                              uint32_t P, uint32_t N, Moduli mods) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < count; j += stride) {
    const uint64_t i = first + j;
    const uint32_t r = (uint32_t)((i % P) / N);
    out[j] = (uint32_t)(value(st, i) % mods.q[r]);
  }
}

// Writes bytes [first, first+count) of the int8 stream.  Each thread owns one
// aligned 8-byte word of the stream; edge words are written byte by byte.
__global__ void fill_int8(uint8_t* out, uint64_t count, uint64_t st, uint64_t first) {
  const uint64_t w0 = first / 8, w1 = (first + count + 7) / 8;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t w = w0 + (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; w < w1; w += stride) {
    const uint64_t v = value(st, w);
    const uint64_t b0 = w * 8;
    if (b0 >= first && b0 + 8 <= first + count && ((b0 - first) % 8) == 0 &&
        (((uintptr_t)(out + (b0 - first))) % 8) == 0) {
      *reinterpret_cast<uint64_t*>(out + (b0 - first)) = v;
    } else {
      for (int t = 0; t < 8; ++t) {
        const uint64_t b = b0 + t;
        if (b >= first && b < first + count) out[b - first] = (uint8_t)(v >> (8 * t));
      }
    }
  }
}

__global__ void fill_uint32(uint32_t* out, uint64_t count, uint64_t st, uint64_t first) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < count; j += stride)
    out[j] = (uint32_t)(value(st, first + j) >> 32);
}

unsigned grid_for(uint64_t items) {
  uint64_t g = (items + 255) / 256;
  if (g > 65536) g = 65536;
  if (g == 0) g = 1;
  return (unsigned)g;
}

}  // namespace

extern "C" {

int pirsynth_fill_residues(void* out, uint64_t count, uint64_t state0, uint64_t first_index,
                           uint32_t P, uint32_t N, const uint32_t* q, void* stream) {
  if (!out || !q || P == 0 || N == 0 || P % N != 0 || P / N > 8) return -1;
  if (count == 0) return 0;
  Moduli m{};
  for (uint32_t r = 0; r < P / N; ++r) {
    if (q[r] == 0) return -1;
    m.q[r] = q[r];
  }
  hipLaunchKernelGGL(fill_residues, dim3(grid_for(count)), dim3(256), 0, (hipStream_t)stream,
                     (uint32_t*)out, count, state0, first_index, P, N, m);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

int pirsynth_fill_int8(void* out, uint64_t count, uint64_t state0, uint64_t first_byte, void* stream) {
  if (!out) return -1;
  if (count == 0) return 0;
  hipLaunchKernelGGL(fill_int8, dim3(grid_for(count / 8 + 2)), dim3(256), 0, (hipStream_t)stream,
                     (uint8_t*)out, count, state0, first_byte);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

int pirsynth_fill_uint32(void* out, uint64_t count, uint64_t state0, uint64_t first_index, void* stream) {
  if (!out) return -1;
  if (count == 0) return 0;
  hipLaunchKernelGGL(fill_uint32, dim3(grid_for(count)), dim3(256), 0, (hipStream_t)stream,
                     (uint32_t*)out, count, state0, first_index);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
