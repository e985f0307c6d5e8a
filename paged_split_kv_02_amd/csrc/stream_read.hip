// Plain streaming read over a device buffer: the practical HBM read ceiling that the
// decode step's effective bandwidth is compared against.  Every 16-byte word is read once
// with a non-temporal load (the decode kernels' load); the XOR of the words a workgroup
// read is its only output, so nothing but the buffer itself is streamed.
// (A grid-stride order, each thread's loads a grid apart, measured 5.5 TB/s; contiguous
// ranges per wave stream faster.)
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../../include/attn_decode.h"
#include "../../include/attn_measure.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kSteps = 16;  // 1 KB loads a wave issues before using any (16 KB in flight)

// Wave v of the grid reads its own contiguous range of words (equal shares, whole 64-word
// kilobytes), kSteps kilobytes at a time: load u of lane l takes word base + 64u + l, so
// every load instruction covers one contiguous, aligned kilobyte.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ buf,
                                                               size_t words, u32x4* partial) {
  const int lane = threadIdx.x & 63;
  const size_t nwaves = size_t(gridDim.x) * kWaves;
  const size_t v = size_t(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  const size_t share = (words + nwaves - 1) / nwaves;
  const size_t per = (share + 63) / 64 * 64;
  const size_t lo = v * per < words ? v * per : words;
  const size_t hi = lo + per < words ? lo + per : words;
  u32x4 acc = {0u, 0u, 0u, 0u};
  size_t i = lo;
  for (; i + 64 * kSteps <= hi; i += 64 * kSteps) {
    u32x4 x[kSteps];
#pragma unroll
    for (int u = 0; u < kSteps; ++u) x[u] = __builtin_nontemporal_load(buf + i + 64 * u + lane);
#pragma unroll
    for (int u = 0; u < kSteps; ++u) acc ^= x[u];
  }
  for (i += lane; i < hi; i += 64) acc ^= __builtin_nontemporal_load(buf + i);

  // XOR over the workgroup: within each wave by lane exchanges, then across the waves.
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1)
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] ^= unsigned(__shfl_xor(int(acc[k]), m, 64));
  __shared__ u32x4 waves[kWaves];
  if ((threadIdx.x & 63) == 0) waves[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    u32x4 x = waves[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) x ^= waves[w];
    partial[blockIdx.x] = x;
  }
}

}  // namespace

extern "C" int attn_stream_read(const void* buf, size_t bytes, uint32_t* partial, void* stream) {
  if (!buf || !partial || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(buf) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(partial) % 16 != 0)
    return ATTN_E_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  hipLaunchKernelGGL(stream_read_kernel, dim3(ATTN_STREAM_READ_GROUPS), dim3(kThreads), 0, s,
                     static_cast<const u32x4*>(buf), bytes / 16, reinterpret_cast<u32x4*>(partial));
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}
