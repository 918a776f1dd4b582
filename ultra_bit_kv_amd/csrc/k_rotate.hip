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
  int y = blockIdx.y, jb = 0;
  while (jb < jobs.n - 1 && y >= jobs.job[jb].heads) {
    y -= jobs.job[jb].heads;
    ++jb;
  }
  const RotateJob& jd = jobs.job[jb];
  const int h = y;
  const int t0 = blockIdx.x * TT;
  const float4* rh = (const float4*)(jd.r + (size_t)(h / jd.g) * kD * kD);
  for (int e = tid; e < kD * kD / 4; e += 256) *(float4*)(&rs[0][0] + 4 * e) = rh[e];
  for (int e = tid; e < TT * kD; e += 256) {
    const int t = e / kD, c = e % kD;
    double v = 0.0;
    if (t0 + t < n_tok) v = (double)bf16_bits_to_f32(jd.src[((size_t)(t0 + t) * jd.heads + h) * kD + c]);
    xs[t][c] = v;
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
