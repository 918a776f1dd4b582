// One 16-token block of rows of one head through a fixed rotation on the
// fp64 matrix cores, shared by the rotation launch and the one-token append
// launch.
//
// OSCAR summary page, section 4 and appendix B: rows are rotated by the fixed
// per-layer, per-head rotation before they are written to the cache; WUSH-KV
// notes, "method step details": the key transform is applied after RoPE to
// every new key and every new query (queries use their KV head's R_K).
//
// Each product x_i * R_ij (bf16 significand x fp32 significand) is exact in
// fp64 and the 128-term sum is accumulated in fp64, so the final bf16 rounding
// is the rounding of the exact dot product (barring a tie closer than the fp64
// accumulation error, ~1e-14 relative).  v_mfma_f64_16x16x4f64 computes each
// output as a chain of fused multiply-adds in ascending k starting from the
// accumulator, so 32 chained instructions give exactly the sequential fp64
// FMA chain over k = 0..127 for a 16-token x 16-column tile.  Lane l supplies
// A[i = l % 16][k = l / 16], B[k = l / 16][j = l % 16] and receives
// D[i = l / 16 + 4 v][j = l % 16], v = 0..3 (checked on gfx950).
#pragma once
#include "device_common.h"

namespace oscar {

typedef double double4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_r __attribute__((ext_vector_type(4)));

// This lane's share of the B operands: R[4 kb + l / 16][j] for kb = 0..31.
__device__ __forceinline__ void load_r_slice(const float* R, int j, float (&rb)[kD / 4]) {
  const int kq = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int kb = 0; kb < kD / 4; ++kb) rb[kb] = R[(size_t)(4 * kb + kq) * kD + j];
}

// Stages rows t0 .. t0 + 15 of head h of src in xs (rows >= n_tok as zeros),
// 16 chunks of 8 values per row, and waits for the work-group.
template <int NT>
__device__ __forceinline__ void stage_rows(const uint16_t* __restrict__ src, int heads, int h,
                                           int t0, int n_tok, uint16_t (*xs)[kD + 8]) {
#pragma unroll
  for (int e = threadIdx.x; e < 16 * 16; e += NT) {
    const int xrow = e / 16, xc = 8 * (e % 16);
    u32x4_r xw = {0u, 0u, 0u, 0u};
    if (t0 + xrow < n_tok) xw = *(const u32x4_r*)(src + ((size_t)(t0 + xrow) * heads + h) * kD + xc);
    *(u32x4_r*)(&xs[xrow][xc]) = xw;
  }
  __syncthreads();
}

// Rotates rows t0 .. t0 + 15 (those < n_tok) of head h of src
// ([n_tok][heads][128] bf16); a work-group of NT threads stages the rows in
// xs, each wave produces the 16 output columns its lanes' rb slices hold
// (column j of lane l), and out(tok, j, bf16 bits) stores the results.  Ends
// with a barrier (xs may be reused).
template <int NT, class Out>
__device__ __forceinline__ void rotate_block(const uint16_t* __restrict__ src, int heads, int h,
                                             int t0, int n_tok, int j, const float (&rb)[kD / 4],
                                             uint16_t (*xs)[kD + 8], Out out) {
  const int tid = threadIdx.x, lane = tid & 63, kq = lane >> 4;
  stage_rows<NT>(src, heads, h, t0, n_tok, xs);
  double4_t acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int kb = 0; kb < kD / 4; ++kb) {
    const double a = (double)bf16_bits_to_f32(xs[lane & 15][4 * kb + kq]);
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a, (double)rb[kb], acc, 0, 0, 0);
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int tok = t0 + kq + 4 * v;
    if (tok < n_tok) out(tok, j, f64_to_bf16_rne(acc[v]));
  }
  __syncthreads();   // the next block overwrites xs
}

// ---- structured rotation --------------------------------------------------
//
// OScaR notes, step one "Canalized Rotation": the normalized Hadamard matrix
// (entries +-1/sqrt(d), orthogonal) rotates keys and queries; OSCAR summary
// page, section 5 "Rotation Analysis": the composed rotation ends with the
// Hadamard factor and a bit-reversal permutation P_br.  Kind 1 is
// R = H / sqrt(128), kind 2 R = H P_br / sqrt(128), with Sylvester's
// H[i][k] = (-1)^popcount(i & k).
//
// The rotation runs as a fast Walsh-Hadamard transform: 7 butterfly stages
// of fp64 additions.  Every intermediate is a signed sum of the row's bf16
// values, exact in fp64 while the row's magnitudes span less than 2^38, so the
// result is the rounding of (x . H) * fp64(1/sqrt(128)) to bf16.  P_br and H
// commute (H[i][br(k)] = H[br(i)][k]), so kind 2 permutes the input:
// x . H P_br = (x P_br) . H with (x P_br)_k = x_br(k).

constexpr double kInvSqrtD = 0x1.6a09e667f3bcdp-4;   // fp64(sqrt(2)) / 16 = fp64(1 / sqrt(128))

// The value of lane l ^ m (m = 1, 2, 4, 8; within a 16-lane row), as DPP
// moves of the two halves: quad_perm [1,0,3,2] and [2,3,0,1] for m = 1, 2;
// row_ror:8 for m = 8 (row_ror:n gives lane i of a row the value of lane
// i - n mod 16; i - 8 mod 16 = i ^ 8); for m = 4, row_ror:12 (lane i + 4,
// which is i ^ 4 when bit 2 of i is clear) or row_ror:4 (lane i - 4, i ^ 4
// when it is set).
__device__ __forceinline__ double lane_xor(double v, int m) {
  const long long b = __double_as_longlong(v);
  int lo = (int)(b & 0xFFFFFFFFll), hi = (int)(b >> 32);
  if (m == 4) {
    const int lo_up = __builtin_amdgcn_mov_dpp(lo, 0x12C, 0xF, 0xF, false);   // lane i + 4
    const int hi_up = __builtin_amdgcn_mov_dpp(hi, 0x12C, 0xF, 0xF, false);
    const int lo_dn = __builtin_amdgcn_mov_dpp(lo, 0x124, 0xF, 0xF, false);   // lane i - 4
    const int hi_dn = __builtin_amdgcn_mov_dpp(hi, 0x124, 0xF, 0xF, false);
    const bool set = (threadIdx.x & 4) != 0;
    lo = set ? lo_dn : lo_up;
    hi = set ? hi_dn : hi_up;
    return __longlong_as_double(((long long)hi << 32) | (long long)(unsigned)lo);
  }
  const int ctrl = m == 1 ? 0xB1 : (m == 2 ? 0x4E : 0x128);
  if (ctrl == 0xB1) {
    lo = __builtin_amdgcn_mov_dpp(lo, 0xB1, 0xF, 0xF, false);
    hi = __builtin_amdgcn_mov_dpp(hi, 0xB1, 0xF, 0xF, false);
  } else if (ctrl == 0x4E) {
    lo = __builtin_amdgcn_mov_dpp(lo, 0x4E, 0xF, 0xF, false);
    hi = __builtin_amdgcn_mov_dpp(hi, 0x4E, 0xF, 0xF, false);
  } else {
    lo = __builtin_amdgcn_mov_dpp(lo, 0x128, 0xF, 0xF, false);
    hi = __builtin_amdgcn_mov_dpp(hi, 0x128, 0xF, 0xF, false);
  }
  return __longlong_as_double(((long long)hi << 32) | (long long)(unsigned)lo);
}

// Structured rotation of rows t0 .. t0 + 15 (those < n_tok) of head h of src:
// a 16-lane group takes one row, its lane i the 8 elements 8i .. 8i+7 of the
// (permuted) row; the butterflies over index bits 0-2 stay in the lane, those
// over bits 3-6 pair lane i with lane i ^ 1, 2, 4, 8.  out(tok, c0, bits)
// receives the bf16 bits of output channels c0 .. c0 + 7.  Ends with a
// barrier (xs may be reused).
template <int NT, class Out>
__device__ __forceinline__ void fwht_block(const uint16_t* __restrict__ src, int heads, int h,
                                           int t0, int n_tok, int kind, uint16_t (*xs)[kD + 8],
                                           Out out) {
  static_assert(NT % 16 == 0 && 256 % NT == 0, "whole rows per pass");
  stage_rows<NT>(src, heads, h, t0, n_tok, xs);
  const int li = threadIdx.x & 15;
  for (int row = threadIdx.x >> 4; row < 16; row += NT / 16) {
    double x[8];
    if (kind == 2) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = (double)bf16_bits_to_f32(xs[row][bitrev7(8 * li + e)]);
    } else {
      const u32x4_r w = *(const u32x4_r*)(&xs[row][8 * li]);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = (double)bf16_bits_to_f32((w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
    }
#pragma unroll
    for (int m = 1; m < 8; m <<= 1)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (!(e & m)) {
          const double a = x[e], b = x[e | m];
          x[e] = a + b;
          x[e | m] = a - b;
        }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) {
      // the lane with bit m clear keeps a + b, its partner b - a: own value
      // times +-1 plus the partner's, one exact-product fma
      const double sg = (li & m) ? -1.0 : 1.0;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = __builtin_fma(x[e], sg, lane_xor(x[e], m));
    }
    uint16_t bits[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) bits[e] = f64_to_bf16_rne_normal(x[e] * kInvSqrtD);
    if (t0 + row < n_tok) out(t0 + row, 8 * li, bits);
  }
  __syncthreads();   // the next block overwrites xs
}

}  // namespace oscar
