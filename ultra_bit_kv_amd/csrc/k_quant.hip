// Clip-quantize-pack of rows that move to INT2, and window placement of new rows.
//
// OSCAR summary page, section 3 "Scale Determination and Clipping" (affine
// asymmetric INT2, scale and zero point, percentile clipping, per-token
// groups) and section 4 "KV Cache Update" (four 2-bit codes per byte; the
// same clip-quantize step serves prefill rows and rows demoted from the
// recent window).  WUSH-KV notes, "method step details": quantize the
// S_flush-aligned segments beyond the S_sink / S_keep windows and advance
// S_quant; the OSCAR-style quantizer clips at the kappa-quantile.  OScaR
// notes, "integer quantization basics": Q = clamp(round(x / Delta + z), 0, 3).
//
// One work-group quantizes one (quantized position, KV head): wave 0 the key
// row, wave 1 the value row.  The positions of all sequences are numbered
// consecutively (sequence-major); a work-group finds its sequence from a
// prefix sum over the sequences' counts S_quant(after) - S_quant(before).  The order statistics a quantile needs are found
// by ranking (ties broken by channel index, so every rank is held by exactly
// one element); the quantile, step and zero point are computed in fp64 with
// contraction disabled, rounded once to fp16, and codes are decided against
// the exact thresholds zero + (k - 1/2) scale.
#include "rotate_common.h"

namespace oscar {

__device__ __forceinline__ int v_window_index(int t, int c) {
  return 32 * (16 * (t >> 2) + (c >> 3)) + 4 * (c & 7) + (t & 3);
}

__device__ __forceinline__ double lerp_quantile(double a, double b, double f) {
#pragma clang fp contract(off)
  return a + f * (b - a);
}

// Order-preserving 16-bit key of a bf16 value (larger value, larger key);
// -0 is keyed as +0, so a zero order statistic is +0.
__device__ __forceinline__ uint32_t bf16_order_key(uint32_t b) {
  b = b == 0x8000u ? 0u : b;
  return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
}
__device__ __forceinline__ float bf16_of_order_key(uint32_t k) {
  return bf16_bits_to_f32(k & 0x8000u ? k & 0x7FFFu : ~k & 0xFFFFu);
}

// Keys of the order statistics s[i_lo], s[i_lo + 1], s[i_hi], s[i_hi + 1]
// (indices clamped to the group) of this lane's group of 2 LPG channels (LPG
// lanes, two keys per lane).  The per-group search state lives in scalar
// registers: each step compares every key against its group's threshold once
// per search (two ballots) and counts each group's bits of the ballots.
template <int LPG>
__device__ __forceinline__ void group_order_stats(uint32_t key0, uint32_t key1, int lane, int i_lo,
                                                  int i_hi, uint32_t& k_lo, uint32_t& k_lo1,
                                                  uint32_t& k_hi, uint32_t& k_hi1) {
  constexpr int NG = 64 / LPG;
  constexpr unsigned long long kLow = LPG == 64 ? ~0ull : (1ull << LPG) - 1ull;
  const int gi = lane / LPG;
  uint32_t plo[NG], phi[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) plo[g] = phi[g] = 0u;
  auto mine = [&](const uint32_t (&v)[NG]) {
    uint32_t r = v[0];
#pragma unroll
    for (int g = 1; g < NG; ++g) r = gi == g ? v[g] : r;
    return r;
  };
  auto count = [&](unsigned long long b0, unsigned long long b1, int g) -> int {
    return (int)(__popcll((b0 >> (g * LPG)) & kLow) + __popcll((b1 >> (g * LPG)) & kLow));
  };
#pragma unroll
  for (int bit = 15; bit >= 0; --bit) {
    const uint32_t below = (1u << bit) - 1u;
    const uint32_t tl = mine(plo) | below, th = mine(phi) | below;
    const unsigned long long l0 = __ballot(key0 <= tl), l1 = __ballot(key1 <= tl);
    const unsigned long long h0 = __ballot(key0 <= th), h1 = __ballot(key1 <= th);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (count(l0, l1, g) < i_lo + 1) plo[g] |= 1u << bit;
      if (count(h0, h1, g) < i_hi + 1) phi[g] |= 1u << bit;
    }
  }
  // s[i + 1] is s[i] when at least min(i + 1, G - 1) + 1 keys lie at or below
  // it, else the group's smallest key above it
  auto next_key = [&](uint32_t k, int idx) {
    const int want = min(idx + 1, 2 * LPG - 1) + 1;
    const unsigned long long b0 = __ballot(key0 <= k), b1 = __ballot(key1 <= k);
    const int cnt = __popcll((b0 >> (gi * LPG)) & kLow) + __popcll((b1 >> (gi * LPG)) & kLow);
    uint32_t nx = min(key0 > k ? key0 : 0x10000u, key1 > k ? key1 : 0x10000u);
#pragma unroll
    for (int d = 1; d < LPG; d <<= 1) nx = min(nx, (uint32_t)__shfl_xor((int)nx, d));
    return cnt >= want ? k : nx;
  };
  k_lo = mine(plo);
  k_hi = mine(phi);
  k_lo1 = next_key(k_lo, i_lo);
  k_hi1 = next_key(k_hi, i_hi);
}

// The sequence of quantized position `item` of an append (positions of all
// sequences numbered consecutively, sequence-major): its index i, the first
// item of that sequence, its cache row, length before the append and first
// new-token row.  From the host's table when the call has one, else by a
// prefix sum over the device counts S_quant(after) - S_quant(before) that
// the whole wave runs.  False (uniform) when the item lies past them.
__device__ __forceinline__ bool locate_quant_position(const CacheArgs& c, const QuantArgs& clip,
                                                      const SeqArgs& s, int item, int lane, int& i,
                                                      int& before, int& slot, int& lb, int& cu0) {
  auto count_of = [&](int k) {
    const int l0 = s.lens[k];
    const int nn = s.cu_new[k + 1] - s.cu_new[k];
    if (s.slots[k] < 0 || s.slots[k] >= c.max_seqs || l0 < 0 || nn < 0) return 0;
    return s_quant_of(l0 + nn, c.s_sink, c.s_keep, c.s_flush) -
           s_quant_of(l0, c.s_sink, c.s_keep, c.s_flush);
  };
  if (clip.qn > 0) {   // the host's table: the last sequence starting at or before the item
    if (item >= clip.q[clip.qn].before) return false;
    int lo = 0, hi = clip.qn - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (clip.q[mid].before <= item) lo = mid;
      else hi = mid - 1;
    }
    i = lo;
    before = clip.q[lo].before;
    slot = clip.q[lo].slot;
    lb = clip.q[lo].len_before;
    cu0 = clip.q[lo].cu_new;
  } else {
    const int n = s.n_seqs, per = (n + 63) / 64;
    const int k0 = min(lane * per, n), k1 = min(k0 + per, n);
    int run = 0;
    for (int k = k0; k < k1; ++k) run += count_of(k);
    int incl = run;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d);
      if (lane >= d) incl += y;
    }
    const bool hit = item >= incl - run && item < incl;   // exactly one lane, if any
    const unsigned long long hits = __ballot(hit);
    if (hits == 0ull) return false;   // uniform: the device counts do not reach this item
    int seq = -1, off = incl - run;
    if (hit) {
      for (int k = k0; k < k1; ++k) {
        const int q = count_of(k);
        if (seq < 0 && item < off + q) seq = k;
        else if (seq < 0) off += q;
      }
    }
    const int src = __ffsll(hits) - 1;
    i = __shfl(seq, src);
    before = __shfl(off, src);
    slot = s.slots[i];
    lb = s.lens[i];
    cu0 = s.cu_new[i];
  }
  return true;
}

// Quantize position `item` (of all the append's quantized positions) of KV
// head h; run by a work-group of 128 threads, wave 0 on the key row and wave
// 1 on the value row, each on its own (no barrier, no LDS): lane l holds
// channels 2l and 2l + 1.
//
// The clip limits need the order statistics s[i], s[i + 1] of each group
// (type-7 quantiles).  They are found by a bitwise search over the
// order-preserving keys of the bf16 values: from the top bit down, a bit of
// the answer is set when fewer than i + 1 of the group's keys lie at or below
// the prefix with that bit clear (group_order_stats).  The sequence of the
// position comes from the host's table when the call has one.
__device__ __forceinline__ void quantize_item(const CacheArgs& c, const QuantArgs& clip,
                                              const SeqArgs& s,
                                              const uint16_t* __restrict__ stage_k,
                                              const uint16_t* __restrict__ stage_v, int item,
                                              int h) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;   // w: 0 = K, 1 = V
  if (w == 0 && c.key_mode) return;   // OScaR keys: ots_key_block
  int i, before, slot, lb, cu0;
  if (!locate_quant_position(c, clip, s, item, lane, i, before, slot, lb, cu0)) return;
  const int sqb = s_quant_of(lb, c.s_sink, c.s_keep, c.s_flush);
  const int p = sqb + (item - before);
  const int m = (p - c.s_sink) / kPage, t = (p - c.s_sink) % kPage;
  const int phys = m < c.max_pages ? c.block_table[(size_t)slot * c.max_pages + m] : -1;

  // ---- source row: old rows from the recent ring, new rows from staging
  uint32_t pair;
  if (p < lb) {
    const int r = (p - c.s_sink) % c.ring_cap;
    const uint16_t* blk = c.win + (((size_t)slot * c.hkv + h) * c.win_blocks + c.sink_blocks +
                                   r / kPage) * (2 * kPage * kD);
    const int tt = r % kPage;
    if (w == 0) {
      pair = *(const uint32_t*)(blk + tt * kD + 2 * lane);
    } else {
      const uint16_t* vb = blk + kPage * kD;
      pair = (uint32_t)vb[v_window_index(tt, 2 * lane)] |
             ((uint32_t)vb[v_window_index(tt, 2 * lane + 1)] << 16);
    }
  } else {
    const size_t tok = (size_t)cu0 + (p - lb);
    const uint16_t* src = (w == 0 ? stage_k : stage_v) + (tok * c.hkv + h) * kD;
    pair = *(const uint32_t*)(src + 2 * lane);
  }
  if (phys < 0 || phys >= c.num_pages) return;   // uniform: unmapped page, nothing to store
  const float x0 = bf16_bits_to_f32(pair & 0xFFFFu);
  const float x1 = bf16_bits_to_f32(pair >> 16);

  // ---- order statistics of this lane's group (G / 2 adjacent lanes)
  const int G = c.group;
  const int gi = (2 * lane) / G;
  const uint32_t key0 = bf16_order_key(pair & 0xFFFFu), key1 = bf16_order_key(pair >> 16);
  const double kap = (double)(w == 0 ? clip.k[h] : clip.v[h]);
  const double q_hi = kap, q_lo = 1.0 - kap;
  const double h_hi = (double)(G - 1) * q_hi, h_lo = (double)(G - 1) * q_lo;
  const double fl_hi = __builtin_floor(h_hi), fl_lo = __builtin_floor(h_lo);
  const int i_hi = (int)fl_hi, i_lo = (int)fl_lo;
  uint32_t p_lo, p_lo1, p_hi, p_hi1;
  if (G == 128) {
    group_order_stats<64>(key0, key1, lane, i_lo, i_hi, p_lo, p_lo1, p_hi, p_hi1);
  } else if (G == 64) {
    group_order_stats<32>(key0, key1, lane, i_lo, i_hi, p_lo, p_lo1, p_hi, p_hi1);
  } else {
    group_order_stats<16>(key0, key1, lane, i_lo, i_hi, p_lo, p_lo1, p_hi, p_hi1);
  }

  const double lo = lerp_quantile((double)bf16_of_order_key(p_lo), (double)bf16_of_order_key(p_lo1),
                                  h_lo - fl_lo);
  const double hi = lerp_quantile((double)bf16_of_order_key(p_hi), (double)bf16_of_order_key(p_hi1),
                                  h_hi - fl_hi);
  const double delta = (hi - lo) / 3.0;
  const uint32_t s16 = f64_to_f16_rne(delta);
  const uint32_t z16 = f64_to_f16_rne(lo);
  const double sc = f16_bits_to_f64(s16), ze = f16_bits_to_f64(z16);
  const double t1 = ze + 0.5 * sc, t2 = ze + 1.5 * sc, t3 = ze + 2.5 * sc;
  uint32_t q0 = 0, q1 = 0;
  if (sc != 0.0) {
    const double d0 = (double)x0, d1 = (double)x1;
    q0 = (uint32_t)(d0 > t1) + (uint32_t)(d0 >= t2) + (uint32_t)(d0 > t3);
    q1 = (uint32_t)(d1 > t1) + (uint32_t)(d1 >= t2) + (uint32_t)(d1 > t3);
  }
  const uint32_t nib = q0 | (q1 << 2);   // channels 2 lane, 2 lane + 1

  // ---- pack and store into the page-head block (layout in oscar_kv.h)
  uint8_t* base = c.pages + ((size_t)phys * c.hkv + h) * c.page_bytes;
  if (w == 0) {
    // word (8t + l / 8): channels 16 (l / 8) .. + 15 = the nibbles of lanes 8 (l / 8) .. + 7
    uint32_t word = nib << (4 * (lane & 7));
#pragma unroll
    for (int d = 1; d < 8; d <<= 1) word |= (uint32_t)__shfl_xor((int)word, d);
    if ((lane & 7) == 0) ((uint32_t*)base)[8 * t + lane / 8] = word;
  } else {
    // half-word of channels 8L .. 8L + 7 of slot t = the nibbles of lanes 4L .. 4L + 3
    uint32_t hw = nib << (4 * (lane & 3));
#pragma unroll
    for (int d = 1; d < 4; d <<= 1) hw |= (uint32_t)__shfl_xor((int)hw, d);
    if ((lane & 3) == 0) {
      const int L = lane / 4;
      const int u = 2 * (16 * (t >> 2) + L) + ((t & 3) >> 1);
      ((uint16_t*)(base + 512))[2 * u + (t & 1)] = (uint16_t)hw;
    }
  }
  if ((2 * lane) % G == 0) {
    uint32_t* prm = (uint32_t*)(base + (w == 0 ? 1024 : v_param_offset(c)));
    prm[16 * gi + t] = s16 | (z16 << 16);
  }
}

__global__ __launch_bounds__(128) void quantize_kernel(CacheArgs c, QuantArgs clip, SeqArgs s,
                                                       const uint16_t* __restrict__ stage_k,
                                                       const uint16_t* __restrict__ stage_v) {
  quantize_item(c, clip, s, stage_k, stage_v, blockIdx.x, blockIdx.y);
}

hipError_t launch_quantize(const CacheArgs& c, const QuantArgs& clip, const SeqArgs& s,
                           const uint16_t* stage_k, const uint16_t* stage_v, int total_q,
                           hipStream_t stream) {
  if (total_q <= 0 || s.n_seqs <= 0) return hipSuccess;
  dim3 grid(total_q, c.hkv);
  hipLaunchKernelGGL(quantize_kernel, grid, dim3(128), 0, stream, c, clip, s, stage_k, stage_v);
  return hipGetLastError();
}

// OScaR key block `blk` of KV head h: the append's quantized positions
// 32 blk .. 32 blk + 31 (one sequence: its count is a multiple of 32), i.e.
// INT2 tokens that fill logical pages m0 and m0 + 1 (OScaR notes, step two
// "Omni-Token Scaling" and "KIVI and the per-channel paradigm").  256
// threads; thread (t = tid / 8, part = tid % 8) first holds channels
// 16 part .. 16 part + 15 of the block's token t:
//  1. s = bf16(sqrt(sum of squares)) of the rotated bf16 row (fp64; the
//     squares are exact and the sum is exact whenever their bits span at
//     most 53 positions, so the fixed summation order does not matter then),
//     u = bf16(k / s) (fp64 quotient, 0 when s = 0) to LDS;
//  2. thread (hh = tid / 128, j = tid % 128): min / max of channel j over
//     tokens 16 hh .. 16 hh + 15, combined through LDS; Delta = bf16((max -
//     min) / 3), z = bf16(-min / Delta) (bf16(min) when Delta = 0), and the
//     codes of its 16 tokens against the exact fp64 thresholds;
//  3. thread (t, part) packs the 16 codes of its word.
__device__ __forceinline__ void ots_key_block(const CacheArgs& c, const QuantArgs& clip,
                                              const SeqArgs& s,
                                              const uint16_t* __restrict__ stage_k, int blk,
                                              int h) {
#pragma clang fp contract(off)
  __shared__ __align__(16) uint16_t s_u[kOtsBlock][kD];   // normalized rows (bf16 bits)
  __shared__ float s_mm[2][2][kD];                         // [token half][min, max][channel]
  __shared__ __align__(16) uint8_t s_code[kOtsBlock][kD];
  __shared__ uint16_t s_scale[kOtsBlock];
  const int tid = threadIdx.x, lane = tid & 63;
  const int item0 = kOtsBlock * blk;
  int i, before, slot, lb, cu0;
  // (every wave finds the same sequence: the result is uniform over the work-group)
  if (!locate_quant_position(c, clip, s, item0, lane, i, before, slot, lb, cu0)) return;
  const int sqb = s_quant_of(lb, c.s_sink, c.s_keep, c.s_flush);
  const int p0 = sqb + (item0 - before);
  const int m0 = (p0 - c.s_sink) / kPage;   // even: p0 - S_sink is a multiple of 32
  auto phys_of = [&](int m) {
    const int ph = m < c.max_pages ? c.block_table[(size_t)slot * c.max_pages + m] : -1;
    return (ph >= 0 && ph < c.num_pages) ? ph : -1;
  };
  const int page_a = phys_of(m0), page_b = phys_of(m0 + 1);
  auto block_of = [&](int t) -> uint8_t* {   // page-head block holding token t, or null
    const int ph = t < kPage ? page_a : page_b;
    return ph < 0 ? nullptr : c.pages + ((size_t)ph * c.hkv + h) * c.page_bytes;
  };

  // ---- 1. token scale and normalized row
  {
    const int t = tid >> 3, part = tid & 7;
    const int p = p0 + t;
    const uint16_t* src;
    if (p < lb) {   // an old row, still in the recent ring
      const int r = (p - c.s_sink) % c.ring_cap;
      src = c.win + (((size_t)slot * c.hkv + h) * c.win_blocks + c.sink_blocks + r / kPage) *
                        (2 * kPage * kD) + (r % kPage) * kD;
    } else {        // a new row of this append
      src = stage_k + ((size_t)cu0 + (p - lb)) * c.hkv * kD + (size_t)h * kD;
    }
    const u32x4_r w0 = *(const u32x4_r*)(src + 16 * part);
    const u32x4_r w1 = *(const u32x4_r*)(src + 16 * part + 8);
    double x[16];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = (double)bf16_bits_to_f32(w0[e] & 0xFFFFu);
      x[2 * e + 1] = (double)bf16_bits_to_f32(w0[e] >> 16);
      x[8 + 2 * e] = (double)bf16_bits_to_f32(w1[e] & 0xFFFFu);
      x[9 + 2 * e] = (double)bf16_bits_to_f32(w1[e] >> 16);
    }
    double ss = 0.0;
#pragma unroll
    for (int e = 0; e < 16; ++e) ss += x[e] * x[e];
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
    ss += __shfl_xor(ss, 4);
    const uint32_t s16 = f64_to_bf16_rne(__builtin_sqrt(ss));
    const double sv = (double)bf16_bits_to_f32(s16);
    uint32_t packed[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t a = sv > 0.0 ? f64_to_bf16_rne(x[2 * e] / sv) : 0u;
      const uint32_t b = sv > 0.0 ? f64_to_bf16_rne(x[2 * e + 1] / sv) : 0u;
      packed[e] = a | (b << 16);
    }
    *(u32x4_r*)&s_u[t][16 * part] = u32x4_r{packed[0], packed[1], packed[2], packed[3]};
    *(u32x4_r*)&s_u[t][16 * part + 8] = u32x4_r{packed[4], packed[5], packed[6], packed[7]};
    if (part == 0) s_scale[t] = (uint16_t)s16;
  }
  __syncthreads();

  // ---- 2. per-channel parameters and codes
  {
    const int j = tid & (kD - 1), hh = tid >> 7;
    float mn = __builtin_inff(), mx = -__builtin_inff();
    float u[kPage];
#pragma unroll
    for (int r = 0; r < kPage; ++r) {
      u[r] = bf16_bits_to_f32(s_u[kPage * hh + r][j]);
      mn = fminf(mn, u[r]);
      mx = fmaxf(mx, u[r]);
    }
    s_mm[hh][0][j] = mn;
    s_mm[hh][1][j] = mx;
    __syncthreads();
    // a zero extreme is taken as +0
    mn = fminf(s_mm[0][0][j], s_mm[1][0][j]) + 0.0f;
    mx = fmaxf(s_mm[0][1][j], s_mm[1][1][j]) + 0.0f;
    const double dmn = (double)mn, dmx = (double)mx;
    const uint32_t d16 = f64_to_bf16_rne((dmx - dmn) / 3.0);
    const double dl = (double)bf16_bits_to_f32(d16);
    const uint32_t z16 = dl == 0.0 ? f64_to_bf16_rne(dmn) : f64_to_bf16_rne(-dmn / dl);
    const double z = (double)bf16_bits_to_f32(z16);
    const double t1 = dl * (0.5 - z), t2 = dl * (1.5 - z), t3 = dl * (2.5 - z);
#pragma unroll
    for (int r = 0; r < kPage; ++r) {
      const double v = (double)u[r];
      const uint32_t q = dl == 0.0 ? 0u : (uint32_t)(v > t1) + (uint32_t)(v >= t2) + (uint32_t)(v > t3);
      s_code[kPage * hh + r][j] = (uint8_t)q;
    }
    if (hh == 0) {   // channel j's (Delta, z) in the page of its half
      uint8_t* base = block_of(j < 64 ? 0 : kPage);
      if (base) ((uint32_t*)(base + kOtsChanOffset))[j & 63] = d16 | (z16 << 16);
    }
  }
  __syncthreads();

  // ---- 3. pack codes (word 8 t + part: channels 16 part + e at bits 2e) and scales
  {
    const int t = tid >> 3, part = tid & 7;
    const u32x4_r cw = *(const u32x4_r*)&s_code[t][16 * part];   // 16 codes, one per byte
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t b = cw[e];
#pragma unroll
      for (int k = 0; k < 4; ++k) word |= ((b >> (8 * k)) & 3u) << (2 * (4 * e + k));
    }
    uint8_t* base = block_of(t);
    if (base) {
      ((uint32_t*)base)[8 * (t % kPage) + part] = word;
      if (part == 0) ((uint16_t*)(base + kOtsScaleOffset))[t % kPage] = s_scale[t];
    }
  }
}

__global__ __launch_bounds__(256) void ots_key_kernel(CacheArgs c, QuantArgs clip, SeqArgs s,
                                                      const uint16_t* __restrict__ stage_k) {
  ots_key_block(c, clip, s, stage_k, blockIdx.x, blockIdx.y);
}

hipError_t launch_ots_keys(const CacheArgs& c, const QuantArgs& clip, const SeqArgs& s,
                           const uint16_t* stage_k, int total_q, hipStream_t stream) {
  if (total_q <= 0 || s.n_seqs <= 0) return hipSuccess;
  dim3 grid(total_q / kOtsBlock, c.hkv);
  hipLaunchKernelGGL(ots_key_kernel, grid, dim3(256), 0, stream, c, clip, s, stage_k);
  return hipGetLastError();
}

// New rows that stay in BF16: sink positions and positions at or beyond S_quant
// (work-group x = ti enumerates them; the host sizes the grid by the largest
// such count of the call).
__device__ __forceinline__ void place_item(const CacheArgs& c, const SeqArgs& s,
                                           const uint16_t* __restrict__ stage_k,
                                           const uint16_t* __restrict__ stage_v, int ti, int h,
                                           int i) {
  const int ch = threadIdx.x;
  const int slot = s.slots[i];
  const int lb = s.lens[i];
  const int n_new = s.cu_new[i + 1] - s.cu_new[i];
  if (slot < 0 || slot >= c.max_seqs || lb < 0 || n_new <= 0) return;
  const int sqa = s_quant_of(lb + n_new, c.s_sink, c.s_keep, c.s_flush);
  // ti enumerates the new rows that stay in BF16: the sink part first, then
  // the rows from S_quant on
  const int in_sink = max(0, min(lb + n_new, c.s_sink) - lb);
  const int p = ti < in_sink ? lb + ti : max(lb, sqa) + (ti - in_sink);
  if (p >= lb + n_new) return;
  int blk, tt;
  if (p < c.s_sink) {
    blk = p / kPage;
    tt = p % kPage;
  } else if (p >= sqa) {
    const int r = (p - c.s_sink) % c.ring_cap;
    blk = c.sink_blocks + r / kPage;
    tt = r % kPage;
  } else {
    return;  // quantized straight into the pages
  }
  uint16_t* wb = c.win + (((size_t)slot * c.hkv + h) * c.win_blocks + blk) * (2 * kPage * kD);
  const size_t tok = (size_t)s.cu_new[i] + (p - lb);
  const size_t src = (tok * c.hkv + h) * kD + ch;
  wb[tt * kD + ch] = stage_k[src];
  wb[kPage * kD + v_window_index(tt, ch)] = stage_v[src];
}

constexpr int kPlaceRows = 4;   // rows per work-group of place_kernel

__global__ __launch_bounds__(128) void place_kernel(CacheArgs c, SeqArgs s,
                                                    const uint16_t* __restrict__ stage_k,
                                                    const uint16_t* __restrict__ stage_v) {
#pragma unroll
  for (int r = 0; r < kPlaceRows; ++r)
    place_item(c, s, stage_k, stage_v, blockIdx.x * kPlaceRows + r, blockIdx.y, blockIdx.z);
}

// Quantize and place in one launch, for appends where no new row lands on a
// ring slot that the flush reads (the two sets of work-groups then touch
// disjoint memory).  Work-groups [0, total_q Hkv) quantize, the rest place.
__global__ __launch_bounds__(128) void flush_place_kernel(CacheArgs c, QuantArgs clip, SeqArgs s,
                                                          const uint16_t* __restrict__ stage_k,
                                                          const uint16_t* __restrict__ stage_v,
                                                          int total_q, int max_new) {
  const int nq = total_q * c.hkv;
  const int b = blockIdx.x;
  if (b < nq) {
    quantize_item(c, clip, s, stage_k, stage_v, b / c.hkv, b % c.hkv);
  } else {
    const int pb = b - nq;
    place_item(c, s, stage_k, stage_v, pb % max_new, (pb / max_new) % c.hkv, pb / (max_new * c.hkv));
  }
}

hipError_t launch_flush_place(const CacheArgs& c, const QuantArgs& clip, const SeqArgs& s,
                              const uint16_t* stage_k, const uint16_t* stage_v, int total_q,
                              int max_new, hipStream_t stream) {
  if (s.n_seqs <= 0 || (total_q <= 0 && max_new <= 0)) return hipSuccess;
  const long long grid = (long long)total_q * c.hkv + (long long)max_new * c.hkv * s.n_seqs;
  hipLaunchKernelGGL(flush_place_kernel, dim3((unsigned)grid), dim3(128), 0, stream, c, clip, s,
                     stage_k, stage_v, total_q, max_new > 0 ? max_new : 1);
  return hipGetLastError();
}

hipError_t launch_place(const CacheArgs& c, const SeqArgs& s, const uint16_t* stage_k,
                        const uint16_t* stage_v, int max_new, hipStream_t stream) {
  if (max_new <= 0 || s.n_seqs <= 0) return hipSuccess;
  dim3 grid((max_new + kPlaceRows - 1) / kPlaceRows, c.hkv, s.n_seqs);
  hipLaunchKernelGGL(place_kernel, grid, dim3(128), 0, stream, c, s, stage_k, stage_v);
  return hipGetLastError();
}

// Appends of exactly one token per sequence in which no new row is flushed
// and the new rows' ring slots are not among the flushed ones (every decode
// step with S_keep >= 1): rotation, flush and placement in one launch.
// Work-groups [0, total_q Hkv) quantize flushed ring rows; the others rotate
// the new rows, 32 output columns each (whole rows for the structured
// rotation), writing keys and values straight
// into their window slot and queries to q_rot.  jobs: 0 = keys, 1 = values,
// 2 = queries (optional); dst_b of keys / values receives the rotated rows
// if not null.
__global__ __launch_bounds__(128) void append_one_kernel(CacheArgs c, QuantArgs clip, SeqArgs s,
                                                         RotateJobs jobs, int total_q,
                                                         const uint16_t* __restrict__ stage_k,
                                                         const uint16_t* __restrict__ stage_v) {
  __shared__ uint16_t xs[16][kD + 8];
  const int nq = total_q * c.hkv;
  int b = blockIdx.x;
  if (b < nq) {   // uniform
    quantize_item(c, clip, s, stage_k, stage_v, b / c.hkv, b % c.hkv);
    return;
  }
  b -= nq;
  const int n_tok = s.n_seqs;   // token t is sequence t's new token
  const int blocks = (n_tok + 15) / 16;
  const int zc = jobs.kind ? 1 : 4;   // dense: four 32-column quarters
  const int z = b % zc;
  b /= zc;
  const int tb = b % blocks;
  int y = b / blocks;
  int job = 0;
  RotateJob jd = jobs.job[0];
  if (y >= jobs.job[0].heads) {
    y -= jobs.job[0].heads;
    job = 1;
    jd = jobs.job[1];
    if (jobs.n > 2 && y >= jobs.job[1].heads) {
      y -= jobs.job[1].heads;
      job = 2;
      jd = jobs.job[2];
    }
  }
  const int h = y;
  if (jobs.kind) {   // structured rotation: whole rows, thread rows tid / 16 and tid / 16 + 8
    int tslot[2], tpos[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {   // (loads from a clamped index, all issued together)
      const int tok = 16 * tb + (threadIdx.x >> 4) + 8 * k;
      const int tc = min(tok, n_tok - 1);
      const int none = job != 2 && tok < n_tok ? 0 : -1;   // (or-ed in: the loads stay unconditional)
      tslot[k] = s.slots[tc] | none;
      tpos[k] = s.lens[tc] | none;
    }
    auto out8 = [&](int tok, int c0, const uint16_t (&bits)[8]) {
      u32x4_r w;
#pragma unroll
      for (int q = 0; q < 4; ++q) w[q] = (uint32_t)bits[2 * q] | ((uint32_t)bits[2 * q + 1] << 16);
      const size_t o = ((size_t)tok * jd.heads + h) * kD + c0;
      if (job == 2) {
        *(u32x4_r*)(jd.dst_a + o) = w;
        return;
      }
      if (jd.dst_b) *(u32x4_r*)(jd.dst_b + o) = w;
      const int k = (tok - 16 * tb) >> 3;
      const int slot = tslot[k], p = tpos[k];
      if (slot < 0 || slot >= c.max_seqs || p < 0) return;
      int blk, tt;
      if (p < c.s_sink) {
        blk = p / kPage;
        tt = p % kPage;
      } else if (p >= s_quant_of(p + 1, c.s_sink, c.s_keep, c.s_flush)) {
        const int r = (p - c.s_sink) % c.ring_cap;
        blk = c.sink_blocks + r / kPage;
        tt = r % kPage;
      } else {
        return;   // excluded by the host: flushed in the same call
      }
      uint16_t* wb = c.win + (((size_t)slot * c.hkv + h) * c.win_blocks + blk) * (2 * kPage * kD);
      if (job == 0) {
        *(u32x4_r*)(wb + tt * kD + c0) = w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) wb[kPage * kD + v_window_index(tt, c0 + e)] = bits[e];
      }
    };
    fwht_block<128>(jd.src, jd.heads, h, 16 * tb, n_tok, jobs.kind, xs, out8);
    return;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = 32 * z + 16 * wave + (lane & 15);
  // the cache rows and positions of this lane's four output tokens, loaded
  // ahead of the rotation (they only decide where the results go)
  // (loads from a clamped index, unconditional: a load under a branch makes
  // the compiler wait for it at the branch's end, one round trip per token)
  int tslot[4], tpos[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int tok = 16 * tb + (lane >> 4) + 4 * v;
    const int tc = min(tok, n_tok - 1);
    const int none = job != 2 && tok < n_tok ? 0 : -1;   // (or-ed in: the loads stay unconditional)
    tslot[v] = s.slots[tc] | none;
    tpos[v] = s.lens[tc] | none;
  }
  float rb[kD / 4];
  load_r_slice(jd.r + (size_t)(h / jd.g) * kD * kD, j, rb);
  auto out = [&](int tok, int col, uint16_t bits) {
    const size_t o = ((size_t)tok * jd.heads + h) * kD + col;
    if (job == 2) {
      jd.dst_a[o] = bits;
      return;
    }
    if (jd.dst_b) jd.dst_b[o] = bits;
    const int v = (tok - 16 * tb) >> 2;   // tok = 16 tb + lane / 16 + 4 v
    const int slot = tslot[v];
    const int p = tpos[v];   // the new token's position
    if (slot < 0 || slot >= c.max_seqs || p < 0) return;
    int blk, tt;
    if (p < c.s_sink) {
      blk = p / kPage;
      tt = p % kPage;
    } else if (p >= s_quant_of(p + 1, c.s_sink, c.s_keep, c.s_flush)) {
      const int r = (p - c.s_sink) % c.ring_cap;
      blk = c.sink_blocks + r / kPage;
      tt = r % kPage;
    } else {
      return;   // excluded by the host: flushed in the same call
    }
    uint16_t* wb = c.win + (((size_t)slot * c.hkv + h) * c.win_blocks + blk) * (2 * kPage * kD);
    if (job == 0) wb[tt * kD + col] = bits;
    else wb[kPage * kD + v_window_index(tt, col)] = bits;
  };
  rotate_block<128>(jd.src, jd.heads, h, 16 * tb, n_tok, j, rb, xs, out);
}

hipError_t launch_append_one(const CacheArgs& c, const QuantArgs& clip, const SeqArgs& s,
                             const RotateJobs& jobs, int total_q, const uint16_t* stage_k,
                             const uint16_t* stage_v, hipStream_t stream) {
  if (s.n_seqs <= 0) return hipSuccess;
  int rows = 0;
  for (int k = 0; k < jobs.n; ++k) rows += jobs.job[k].heads;
  const long long zc = jobs.kind ? 1 : 4;
  const long long grid = (long long)total_q * c.hkv + zc * ((s.n_seqs + 15) / 16) * rows;
  hipLaunchKernelGGL(append_one_kernel, dim3((unsigned)grid), dim3(128), 0, stream, c, clip, s,
                     jobs, total_q, stage_k, stage_v);
  return hipGetLastError();
}

}  // namespace oscar
