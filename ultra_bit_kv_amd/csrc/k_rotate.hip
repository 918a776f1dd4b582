// Fixed per-head rotation x' = x . R of post-RoPE rows, rounded once to bf16
// (the arithmetic is in rotate_common.h).
//
// One launch rotates up to three row sets (keys, values, queries): grid.y
// enumerates (set, head), grid.z the two 64-column halves of the output.
// Dense: wave w of a work-group owns 16 output columns and keeps their slice of R
// (one value per k-quad per lane) in registers; the work-group walks TB
// blocks of 16 tokens, staging each block's input rows in LDS.  Structured
// kinds: one work-group transforms whole rows (fwht_block), grid.z = 1.
#include "rotate_common.h"

namespace oscar {

template <int TB>
__global__ __launch_bounds__(256) void rotate_kernel(RotateJobs jobs, int n_tok) {
  __shared__ uint16_t xs[16][kD + 8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // grid.y enumerates (job, head); the job is selected with constant indices
  // so its fields stay in scalar registers
  int y = blockIdx.y;
  RotateJob jd = jobs.job[0];
  if (jobs.n > 1 && y >= jobs.job[0].heads) {
    y -= jobs.job[0].heads;
    jd = jobs.job[1];
    if (jobs.n > 2 && y >= jobs.job[1].heads) {
      y -= jobs.job[1].heads;
      jd = jobs.job[2];
    }
  }
  const int h = y;
  if (jobs.kind) {   // structured rotation: whole rows per work-group (grid.z = 1)
    auto out8 = [&](int tok, int c0, const uint16_t (&bits)[8]) {
      u32x4_r w;
#pragma unroll
      for (int q = 0; q < 4; ++q) w[q] = (uint32_t)bits[2 * q] | ((uint32_t)bits[2 * q + 1] << 16);
      const size_t o = ((size_t)tok * jd.heads + h) * kD + c0;
      *(u32x4_r*)(jd.dst_a + o) = w;
      if (jd.dst_b) *(u32x4_r*)(jd.dst_b + o) = w;
    };
    for (int b = 0; b < TB; ++b) {
      const int t0 = (blockIdx.x * TB + b) * 16;
      if (t0 >= n_tok) break;   // uniform
      fwht_block<256>(jd.src, jd.heads, h, t0, n_tok, jobs.kind, xs, out8);
    }
    return;
  }
  const int j = 64 * blockIdx.z + 16 * wave + (lane & 15);   // output column of this lane
  float rb[kD / 4];
  load_r_slice(jd.r + (size_t)(h / jd.g) * kD * kD, j, rb);
  auto out = [&](int tok, int col, uint16_t bits) {
    const size_t o = ((size_t)tok * jd.heads + h) * kD + col;
    jd.dst_a[o] = bits;
    if (jd.dst_b) jd.dst_b[o] = bits;
  };
  for (int b = 0; b < TB; ++b) {
    const int t0 = (blockIdx.x * TB + b) * 16;
    if (t0 >= n_tok) break;   // uniform
    rotate_block<256>(jd.src, jd.heads, h, t0, n_tok, j, rb, xs, out);
  }
}

hipError_t launch_rotate(const RotateJobs& jobs, int n_tok, hipStream_t stream) {
  if (n_tok <= 0 || jobs.n <= 0) return hipSuccess;
  int rows = 0;
  for (int k = 0; k < jobs.n; ++k) rows += jobs.job[k].heads;
  const int blocks = (n_tok + 15) / 16;
  const int zc = jobs.kind ? 1 : 2;   // dense: two 64-column halves
  if (blocks <= 64) {   // small calls (decode steps): one 16-token block per work-group
    hipLaunchKernelGGL(rotate_kernel<1>, dim3(blocks, rows, zc), dim3(256), 0, stream, jobs, n_tok);
  } else {              // prefill: each work-group reuses its R slice over 8 blocks
    hipLaunchKernelGGL(rotate_kernel<8>, dim3((blocks + 7) / 8, rows, zc), dim3(256), 0, stream,
                       jobs, n_tok);
  }
  return hipGetLastError();
}

}  // namespace oscar
