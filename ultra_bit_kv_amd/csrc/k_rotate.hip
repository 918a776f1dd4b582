// Fixed per-head rotation x' = x . R of post-RoPE rows, rounded once to bf16.
//
// OSCAR summary page, section 4 and appendix B: rows are rotated by the fixed
// per-layer, per-head rotation before they are written to the cache; WUSH-KV
// notes, "method step details": the key transform is applied after RoPE to
// every new key and every new query (queries use their KV head's R_K).
//
// Each product x_i * R_ij (bf16 significand x fp32 significand) is exact in
// fp64 and the 128-term sum is accumulated in fp64, so the final bf16 rounding
// is the rounding of the exact dot product (barring a tie closer than the fp64
// accumulation error, ~1e-14 relative).
//
// One launch rotates up to three row sets (keys, values, queries): grid.y
// enumerates (set, head).  R of the head is staged in LDS with one round of
// coalesced loads; a thread owns one output column j and TT/2 tokens.
#include "device_common.h"

namespace oscar {

template <int TT>
__global__ __launch_bounds__(256) void rotate_kernel(RotateJobs jobs, int n_tok) {
  __shared__ double xs[TT][kD + 1];
  __shared__ float rs[kD][kD];
  const int tid = threadIdx.x;
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
  const int t0 = blockIdx.x * TT;
  // All global loads are issued before the first wait: R (16 x 16 B per
  // thread) and the TT input rows (TT * 256 B, 16 B per thread).
  static_assert(TT * kD == 8 * 256, "one 8-element chunk of the input rows per thread");
  const float4* rh = (const float4*)(jd.r + (size_t)(h / jd.g) * kD * kD);
  float4 rr[kD * kD / 4 / 256];
#pragma unroll
  for (int k = 0; k < kD * kD / 4 / 256; ++k) rr[k] = rh[tid + 256 * k];
  const int xt = tid / 16, xc = 8 * (tid % 16);
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  u32x4_t xw = {0u, 0u, 0u, 0u};
  if (t0 + xt < n_tok) xw = *(const u32x4_t*)(jd.src + ((size_t)(t0 + xt) * jd.heads + h) * kD + xc);
#pragma unroll
  for (int k = 0; k < kD * kD / 4 / 256; ++k) *(float4*)(&rs[0][0] + 4 * (tid + 256 * k)) = rr[k];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    xs[xt][xc + 2 * e] = (double)bf16_bits_to_f32(xw[e] & 0xFFFFu);
    xs[xt][xc + 2 * e + 1] = (double)bf16_bits_to_f32(xw[e] >> 16);
  }
  __syncthreads();

  constexpr int TPT = TT / 2;         // tokens per thread
  const int j = tid % kD;             // output column
  const int tb = (tid / kD) * TPT;
  double acc[TPT];
#pragma unroll
  for (int t = 0; t < TPT; ++t) acc[t] = 0.0;
#pragma unroll 4
  for (int k = 0; k < kD; ++k) {
    const double rk = (double)rs[k][j];
#pragma unroll
    for (int t = 0; t < TPT; ++t) acc[t] = __builtin_fma(xs[tb + t][k], rk, acc[t]);
  }
#pragma unroll
  for (int t = 0; t < TPT; ++t) {
    const int tok = t0 + tb + t;
    if (tok < n_tok) {
      const uint16_t out = f64_to_bf16_rne(acc[t]);
      const size_t o = ((size_t)tok * jd.heads + h) * kD + j;
      jd.dst_a[o] = out;
      if (jd.dst_b) jd.dst_b[o] = out;
    }
  }
}

hipError_t launch_rotate(const RotateJobs& jobs, int n_tok, hipStream_t stream) {
  if (n_tok <= 0 || jobs.n <= 0) return hipSuccess;
  int rows = 0;
  for (int k = 0; k < jobs.n; ++k) rows += jobs.job[k].heads;
  dim3 grid((n_tok + 15) / 16, rows);
  hipLaunchKernelGGL(rotate_kernel<16>, grid, dim3(256), 0, stream, jobs, n_tok);
  return hipGetLastError();
}

}  // namespace oscar
