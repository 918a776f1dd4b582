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
// The sums run on the fp64 matrix cores: v_mfma_f64_16x16x4f64 computes each
// output as a chain of fused multiply-adds in ascending k starting from the
// accumulator, so 32 chained instructions give exactly the sequential fp64
// FMA chain over k = 0..127 for a 16-token x 16-column tile.  Lane l supplies
// A[i = l % 16][k = l / 16], B[k = l / 16][j = l % 16] and receives
// D[i = l / 16 + 4 v][j = l % 16], v = 0..3 (checked on gfx950).
//
// One launch rotates up to three row sets (keys, values, queries): grid.y
// enumerates (set, head), grid.z the two 64-column halves of the output.
// Wave w of a work-group owns 16 output columns and keeps their slice of R
// (one value per k-quad per lane) in registers; the work-group walks TB
// blocks of 16 tokens, staging each block's input rows in LDS.
#include "device_common.h"

namespace oscar {

typedef double double4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_r __attribute__((ext_vector_type(4)));

template <int TB>
__global__ __launch_bounds__(256) void rotate_kernel(RotateJobs jobs, int n_tok) {
  __shared__ uint16_t xs[16][kD + 8];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
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
  const int j = 64 * blockIdx.z + 16 * wave + (lane & 15);   // output column of this lane
  const int kq = lane >> 4;                                    // k offset inside a k-quad

  // R[4 kb + kq][j] for kb = 0..31: this lane's share of the B operands
  const float* R = jd.r + (size_t)(h / jd.g) * kD * kD;
  float rb[kD / 4];
#pragma unroll
  for (int kb = 0; kb < kD / 4; ++kb) rb[kb] = R[(size_t)(4 * kb + kq) * kD + j];

  const int xrow = tid / 16, xc = 8 * (tid % 16);   // staging: 16 rows x 16 chunks of 8 values
  for (int b = 0; b < TB; ++b) {
    const int t0 = (blockIdx.x * TB + b) * 16;
    if (t0 >= n_tok) break;   // uniform
    u32x4_r xw = {0u, 0u, 0u, 0u};
    if (t0 + xrow < n_tok)
      xw = *(const u32x4_r*)(jd.src + ((size_t)(t0 + xrow) * jd.heads + h) * kD + xc);
    *(u32x4_r*)(&xs[xrow][xc]) = xw;
    __syncthreads();

    double4_t acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int kb = 0; kb < kD / 4; ++kb) {
      const double a = (double)bf16_bits_to_f32(xs[lane & 15][4 * kb + kq]);
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a, (double)rb[kb], acc, 0, 0, 0);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int tok = t0 + kq + 4 * v;
      if (tok < n_tok) {
        const uint16_t out = f64_to_bf16_rne(acc[v]);
        const size_t o = ((size_t)tok * jd.heads + h) * kD + j;
        jd.dst_a[o] = out;
        if (jd.dst_b) jd.dst_b[o] = out;
      }
    }
    __syncthreads();   // the next block overwrites xs
  }
}

hipError_t launch_rotate(const RotateJobs& jobs, int n_tok, hipStream_t stream) {
  if (n_tok <= 0 || jobs.n <= 0) return hipSuccess;
  int rows = 0;
  for (int k = 0; k < jobs.n; ++k) rows += jobs.job[k].heads;
  const int blocks = (n_tok + 15) / 16;
  if (blocks <= 64) {   // small calls (decode steps): one 16-token block per work-group
    hipLaunchKernelGGL(rotate_kernel<1>, dim3(blocks, rows, 2), dim3(256), 0, stream, jobs, n_tok);
  } else {              // prefill: each work-group reuses its R slice over 8 blocks
    hipLaunchKernelGGL(rotate_kernel<8>, dim3((blocks + 7) / 8, rows, 2), dim3(256), 0, stream,
                       jobs, n_tok);
  }
  return hipGetLastError();
}

}  // namespace oscar
