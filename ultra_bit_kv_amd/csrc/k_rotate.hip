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

// Dense rotation over TB 16-token blocks per work-group, double-buffered:
// the rows of block b + 1 go to the other LDS buffer (loaded during block
// b - 1) after block b's products, so one barrier per block and no wait for
// global loads before a block's matrix work.  LDS holds each row by k mod 4:
// xt[row][kq][kb] = x[row][4 kb + kq], so lane (i, kq) reads its 32 A
// operands (row i, k = 4 kb + kq) with four 16-byte loads.  The products
// and their order are those of rotate_block: the same fp64 FMA chain.
template <int TB>
__global__ __launch_bounds__(256) void rotate_dense_kernel(RotateJobs jobs, int n_tok) {
  constexpr int kRowW = 4 * 32 + 8;   // bf16 per staged row (padded: rows start 4 banks apart)
  __shared__ __align__(16) uint16_t xt[2][16][kRowW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, kq = lane >> 4;
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
  const int j = 64 * blockIdx.z + 16 * wave + (lane & 15);   // output column of this lane
  float rb[kD / 4];
  load_r_slice(jd.r + (size_t)(h / jd.g) * kD * kD, j, rb);
  // staging: thread (row, c8) takes elements 8 c8 .. 8 c8 + 7 of one row
  const int srow = tid >> 4, c8 = tid & 15;
  auto load_chunk = [&](int b) {
    const int tok = (blockIdx.x * TB + b) * 16 + srow;
    u32x4_r w = {0u, 0u, 0u, 0u};
    if (tok < n_tok) w = *(const u32x4_r*)(jd.src + ((size_t)tok * jd.heads + h) * kD + 8 * c8);
    return w;
  };
  auto deposit = [&](int buf, const u32x4_r& w) {
    // k = 8 c8 + kq (low half) and 8 c8 + 4 + kq (high half): kb = 2 c8, 2 c8 + 1
    const uint32_t q0 = __builtin_amdgcn_perm(w[2], w[0], 0x05040100u);
    const uint32_t q1 = __builtin_amdgcn_perm(w[2], w[0], 0x07060302u);
    const uint32_t q2 = __builtin_amdgcn_perm(w[3], w[1], 0x05040100u);
    const uint32_t q3 = __builtin_amdgcn_perm(w[3], w[1], 0x07060302u);
    __builtin_memcpy(&xt[buf][srow][0 * 32 + 2 * c8], &q0, 4);
    __builtin_memcpy(&xt[buf][srow][1 * 32 + 2 * c8], &q1, 4);
    __builtin_memcpy(&xt[buf][srow][2 * 32 + 2 * c8], &q2, 4);
    __builtin_memcpy(&xt[buf][srow][3 * 32 + 2 * c8], &q3, 4);
  };
  auto out = [&](int tok, int col, uint16_t bits) {
    const size_t o = ((size_t)tok * jd.heads + h) * kD + col;
    jd.dst_a[o] = bits;
    if (jd.dst_b) jd.dst_b[o] = bits;
  };
  deposit(0, load_chunk(0));
  u32x4_r pre = load_chunk(1);
  __syncthreads();
  for (int b = 0; b < TB; ++b) {
    const int t0 = (blockIdx.x * TB + b) * 16;
    if (t0 >= n_tok) break;   // uniform
    u32x4_r aw[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) __builtin_memcpy(&aw[u], &xt[b & 1][lane & 15][32 * kq + 8 * u], 16);
    __builtin_amdgcn_sched_barrier(0);   // (all four reads before the first product)
    double4_t acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int kb = 0; kb < kD / 4; ++kb) {
      const uint32_t w = aw[kb >> 3][(kb >> 1) & 3];
      const double a = (double)__uint_as_float((kb & 1) ? (w & 0xFFFF0000u) : (w << 16));
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a, (double)rb[kb], acc, 0, 0, 0);
    }
    // the next block's rows first: their wait must not also cover this
    // block's stores (stores count in the same counter)
    if (b + 1 < TB) {
      deposit((b + 1) & 1, pre);
      if (b + 2 < TB) pre = load_chunk(b + 2);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int tok = t0 + kq + 4 * v;
      if (tok < n_tok) out(tok, j, f64_to_bf16_rne(acc[v]));
    }
    __syncthreads();   // block b + 1 in, block b read by every wave
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
  } else if (jobs.kind) {   // prefill, structured: 8 blocks per work-group
    hipLaunchKernelGGL(rotate_kernel<8>, dim3((blocks + 7) / 8, rows, zc), dim3(256), 0, stream,
                       jobs, n_tok);
  } else {   // prefill, dense: each work-group reuses its R slice over 8 blocks
    hipLaunchKernelGGL(rotate_dense_kernel<8>, dim3((blocks + 7) / 8, rows, zc), dim3(256), 0,
                       stream, jobs, n_tok);
  }
  return hipGetLastError();
}

}  // namespace oscar
