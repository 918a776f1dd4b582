// HBM read probe (measurement aid, see oscar_probe.h): reads a buffer once,
// sequentially or as chunks in a given order, with 16-byte loads, and folds
// the words into one value per work-group so that no load is elided.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "oscar_kv.h"
#include "oscar_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__device__ __forceinline__ uint32_t fold(const u32x4& v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }

// XOR of the wave's 64 values, stored by its first lane to sink[wave of the grid]
__device__ __forceinline__ void store_wave(uint32_t acc, uint32_t* sink) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) acc ^= (uint32_t)__shfl_xor((int)acc, d);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)] = acc;
}

// Sequential sweep: work-group b reads its own contiguous slice of the
// buffer (n16 / grid elements, rounded up to whole 4 KB steps), its 256
// threads 16 bytes apart, kUnroll consecutive 4 KB steps issued before any
// is used (each work-group walks its slice in address order).
__global__ __launch_bounds__(kThreads) void probe_seq_kernel(const u32x4* __restrict__ buf,
                                                             size_t n16, uint32_t* __restrict__ sink) {
  const size_t per = ((n16 + gridDim.x - 1) / gridDim.x + kThreads - 1) / kThreads * kThreads;
  const size_t b0 = (size_t)blockIdx.x * per;
  const size_t b1 = b0 + per < n16 ? b0 + per : n16;
  size_t i = b0 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kUnroll - 1) * kThreads < b1; i += kUnroll * kThreads) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = buf[i + u * kThreads];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= fold(v[u]);
  }
  for (; i < b1; i += kThreads) acc ^= fold(buf[i]);
  store_wave(acc, sink);
}

// Chunk gather: wave w of the grid takes chunk ids w, w + W, ... (W = grid
// waves); a chunk of k KB is k loads of 1 KB per wave (16 bytes per lane),
// all issued before any is used.
__global__ __launch_bounds__(kThreads) void probe_chunk_kernel(const uint8_t* __restrict__ buf,
                                                               int64_t n_valid, const int32_t* __restrict__ ids,
                                                               int n_chunks, int chunk_kb,
                                                               uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int W = gridDim.x * (kThreads / 64);
  const int w = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  uint32_t acc = 0;
  for (int k = w; k < n_chunks; k += W) {
    const int32_t c = ids[k];
    if (c < 0 || c >= n_valid) continue;
    const u32x4* p = (const u32x4*)(buf + (size_t)c * chunk_kb * 1024) + lane;
    for (int b = 0; b < chunk_kb; b += 16) {
      const int m = chunk_kb - b < 16 ? chunk_kb - b : 16;
      u32x4 v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (u < m) v[u] = p[(b + u) * 64];
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (u < m) acc ^= fold(v[u]);
    }
  }
  store_wave(acc, sink);
}

}  // namespace

extern "C" int oscar_read_probe(const void* buf, size_t bytes, const int32_t* chunk_ids,
                                int32_t n_chunks, int32_t chunk_bytes, uint32_t* sink, int32_t grid,
                                int32_t sink_words, void* stream) {
  if (!buf || !sink) return OSCAR_ERR_NULL;
  if (((uintptr_t)buf & 15) != 0 || ((uintptr_t)sink & 3) != 0) return OSCAR_ERR_ARG;
  if (bytes == 0 || bytes % 1024 != 0) return OSCAR_ERR_ARG;
  if (grid < 1 || grid > (1 << 20) || (int64_t)grid * (kThreads / 64) > sink_words)
    return OSCAR_ERR_ARG;
  if (chunk_ids) {
    if (n_chunks < 0 || chunk_bytes < 1024 || chunk_bytes % 1024 != 0) return OSCAR_ERR_ARG;
    if (((uintptr_t)chunk_ids & 3) != 0) return OSCAR_ERR_ARG;
  }
  static int known[64] = {0};   // per device: 0 unknown, 1 gfx950, -1 other
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return OSCAR_ERR_HIP;
  if (dev < 0 || dev >= 64) return OSCAR_ERR_DEVICE;
  if (known[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return OSCAR_ERR_HIP;
    known[dev] = __builtin_strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
  }
  if (known[dev] != 1) return OSCAR_ERR_DEVICE;
  hipStream_t s = (hipStream_t)stream;
  if (chunk_ids) {
    if (n_chunks == 0) return OSCAR_OK;
    hipLaunchKernelGGL(probe_chunk_kernel, dim3(grid), dim3(kThreads), 0, s, (const uint8_t*)buf,
                       (int64_t)(bytes / (size_t)chunk_bytes), chunk_ids, n_chunks,
                       chunk_bytes / 1024, sink);
  } else {
    hipLaunchKernelGGL(probe_seq_kernel, dim3(grid), dim3(kThreads), 0, s, (const u32x4*)buf,
                       bytes / 16, sink);
  }
  return hipGetLastError() == hipSuccess ? OSCAR_OK : OSCAR_ERR_HIP;
}
