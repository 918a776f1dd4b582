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
#include "device_common.h"

namespace oscar {

constexpr int kRotTok = 16;   // tokens per work-group

__global__ __launch_bounds__(256) void rotate_kernel(const uint16_t* __restrict__ src, int n_tok,
                                                     int heads, int g, const float* __restrict__ r,
                                                     uint16_t* __restrict__ dst_a,
                                                     uint16_t* __restrict__ dst_b) {
  __shared__ double xs[kRotTok][kD + 1];
  const int tid = threadIdx.x;
  const int h = blockIdx.y;
  const int t0 = blockIdx.x * kRotTok;
  const float* rh = r + (size_t)(h / g) * kD * kD;

  for (int e = tid; e < kRotTok * kD; e += 256) {
    const int t = e / kD, c = e % kD;
    double v = 0.0;
    if (t0 + t < n_tok) v = (double)bf16_bits_to_f32(src[((size_t)(t0 + t) * heads + h) * kD + c]);
    xs[t][c] = v;
  }
  __syncthreads();

  const int j = tid % kD;             // output column
  const int tb = (tid / kD) * 8;      // first of this thread's 8 tokens
  double acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = 0.0;
#pragma unroll 4
  for (int k = 0; k < kD; ++k) {
    const double rk = (double)rh[k * kD + j];
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] = __builtin_fma(xs[tb + t][k], rk, acc[t]);
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int tok = t0 + tb + t;
    if (tok < n_tok) {
      const uint16_t y = f64_to_bf16_rne(acc[t]);
      const size_t o = ((size_t)tok * heads + h) * kD + j;
      dst_a[o] = y;
      if (dst_b) dst_b[o] = y;
    }
  }
}

hipError_t launch_rotate(const uint16_t* src, int n_tok, int heads, int g, const float* r,
                         uint16_t* dst_a, uint16_t* dst_b, hipStream_t stream) {
  if (n_tok <= 0) return hipSuccess;
  dim3 grid((n_tok + kRotTok - 1) / kRotTok, heads);
  hipLaunchKernelGGL(rotate_kernel, grid, dim3(256), 0, stream, src, n_tok, heads, g, r, dst_a,
                     dst_b);
  return hipGetLastError();
}

}  // namespace oscar
