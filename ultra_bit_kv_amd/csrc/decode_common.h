// Pieces shared by the split-K decode kernels (INT2 mixed cache and plain
// BF16 pages): wave-level reductions, the online softmax, the compact-grid
// item lookup and the log-sum-exp merge of split partial records.
#pragma once
#include "device_common.h"

namespace oscar {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

template <int SH>
__device__ __forceinline__ float row_ror(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x120 + SH, 0xF, 0xF, false));
}

// all-reduce over the four 16-lane rows (lanes n, n+16, n+32, n+48)
__device__ __forceinline__ float rows_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                            false, false);
  x = fmaxf(__builtin_bit_cast(float, (int)a[0]), __builtin_bit_cast(float, (int)a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                            false, false);
  return fmaxf(__builtin_bit_cast(float, (int)b[0]), __builtin_bit_cast(float, (int)b[1]));
}

__device__ __forceinline__ float rows_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                            false, false);
  x = __builtin_bit_cast(float, (int)a[0]) + __builtin_bit_cast(float, (int)a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                            false, false);
  return __builtin_bit_cast(float, (int)b[0]) + __builtin_bit_cast(float, (int)b[1]);
}

__device__ __forceinline__ half8 codes_as_half8(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3,
                                                uint32_t mask) {
  u32x4 v = {w0 & mask, w1 & mask, w2 & mask, w3 & mask};
  return __builtin_bit_cast(half8, v);
}

__device__ __forceinline__ float f16lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// hi16(w) (an fp16 value) times b in fp32 with one rounding, as one
// mixed-precision multiply-add (a zero product gives +0).  w must not come
// straight from the exp unit or a matrix instruction (no wait states).
__device__ __forceinline__ float f16hi_mul(uint32_t w, float b) {
  float r;
  asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(w), "v"(b));
  return r;
}
typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));

// Bit pattern of the largest fp16 scale (low halves) of eight scale | zero
// words.  Scales are (hi - lo) / 3 >= 0, and the bit patterns of
// non-negative fp16 values are ordered like the values.
__device__ __forceinline__ uint32_t max_scale_bits(const u32x4& a, const u32x4& b) {
  auto m = [](uint32_t x, uint32_t y) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(ushort2_t, x),
                                                                  __builtin_bit_cast(ushort2_t, y)));
  };
  return m(m(m(a[0], a[1]), m(a[2], a[3])), m(m(b[0], b[1]), m(b[2], b[3]))) & 0xFFFFu;
}

// The products a * lo16(wa) and b * lo16(wb) (fp16 scales) as fp16 pairs
// split in two: hi = the products rounded to fp16, lo = the remainders
// a * s - hi (one fused multiply-add each) rounded to fp16, so hi + lo
// carries about 22 significant bits.  Mixed-precision fused multiply-adds
// that write one fp16 half each.  The leading s_nop gives a and b, which
// come from the exp unit, the wait state such a result needs before a VALU
// reads it; the trailing one the two wait states a matrix instruction needs
// before it reads a VGPR a VALU wrote (the compiler does not see into the
// asm, and hi / lo feed MFMAs).
__device__ __forceinline__ void mul_by_f16lo_split(float a, uint32_t wa, float b, uint32_t wb,
                                                   uint32_t& hi, uint32_t& lo) {
  uint32_t h, l;
  asm("s_nop 0\n\t"
      "v_fma_mixlo_f16 %0, %2, %3, 0 op_sel:[0,0,0] op_sel_hi:[0,1,0]\n\t"
      "v_fma_mixhi_f16 %0, %4, %5, 0 op_sel:[0,0,0] op_sel_hi:[0,1,0]\n\t"
      "v_fma_mixlo_f16 %1, %2, %3, -%0 op_sel:[0,0,0] op_sel_hi:[0,1,1]\n\t"
      "v_fma_mixhi_f16 %1, %4, %5, -%0 op_sel:[0,0,1] op_sel_hi:[0,1,1]\n\t"
      "s_nop 1"
      : "=&v"(h), "=&v"(l)
      : "v"(a), "v"(wa), "v"(b), "v"(wb));
  hi = h;
  lo = l;
}

// q (two fp16 values) times (d0, d1) (fp32) as fp16 pairs split in two:
// hi = the products rounded to fp16, lo = the remainders q d - hi (one fused
// multiply-add each) rounded to fp16.  For an 11-bit q and an 8-bit d the
// product has at most 19 bits, so hi + lo holds it exactly (22 bits) while
// both stay in the fp16 normal range.  The trailing s_nop gives the matrix
// instructions that read hi / lo the two wait states after a VALU write.
__device__ __forceinline__ void mul_f16pair_split(uint32_t q, float d0, float d1, uint32_t& hi,
                                                  uint32_t& lo) {
  uint32_t h, l;
  asm("v_fma_mixlo_f16 %0, %2, %3, 0 op_sel:[0,0,0] op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixhi_f16 %0, %2, %4, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixlo_f16 %1, %2, %3, -%0 op_sel:[0,0,0] op_sel_hi:[1,0,1]\n\t"
      "v_fma_mixhi_f16 %1, %2, %4, -%0 op_sel:[1,0,1] op_sel_hi:[1,0,1]\n\t"
      "s_nop 1"
      : "=&v"(h), "=&v"(l)
      : "v"(q), "v"(d0), "v"(d1));
  hi = h;
  lo = l;
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

struct SoftmaxState {
  float m;    // running max (log2 domain), same in every lane of a column
  float l;    // this lane's share of the running sum
  float z;    // this lane's share of sum_t p_t * zero_v[t][group]
  float mr;   // the max subtracted before exp2: m, or 0 while m = -inf
};

// Online-softmax update with a lazy max.  x holds logits in raw units; the
// log2-domain logit is scale * x (scale > 0).  The reference max only moves
// when a logit exceeds it by more than `slack` (so p <= 2^slack), which keeps
// most tiles free of the accumulator rescale; slack = 0 keeps every p <= 1.
template <int N>
__device__ __forceinline__ void softmax_step(const float (&x)[N], float scale, float (&p)[N],
                                             SoftmaxState& st, float4_t (&acc)[8],
                                             float slack = 8.0f) {
  float lmax = x[0];
#pragma unroll
  for (int k = 1; k < N; ++k) lmax = fmaxf(lmax, x[k]);
  // a column's maximum passes the bound exactly when one of its lanes'
  // maxima does (scale > 0), so the cross-lane reduction only runs then
  if (__any(lmax * scale > st.m + slack)) {
    const float tmax = rows_max(lmax) * scale;
    const float m_new = fmaxf(st.m, tmax);
    const float alpha = m_new > st.m ? __builtin_amdgcn_exp2f(st.m - m_new) : 1.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= alpha;
    st.l *= alpha;
    st.z *= alpha;
    st.m = m_new;
    st.mr = m_new == kNegInf ? 0.0f : m_new;
  }
#pragma unroll
  for (int k = 0; k < N; ++k) {
    p[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[k], scale, -st.mr));
    st.l += p[k];
  }
}

constexpr int kMaxWgPages = 2 * kMaxPairsPerSplit;   // page ids staged per work-group


// Issue priority of the calling wave from its remaining share of the work
// and its dispatch round (work-group b of a launch that fills the device
// runs as the (b / cus)-th one on its compute unit).  Waves of one SIMD
// otherwise issue oldest-first, so the work-groups placed first on a compute
// unit run ahead and the last ones finish alone: a wave with more work
// left, or placed later, gets a higher priority (4 levels; a round is worth
// a third of a level).
__device__ __forceinline__ void set_priority(int remaining, int total, int round) {
  const int p = ((12 * remaining - 1) / total + (round < 3 ? round : 3)) / 3;
  if (p >= 3) __builtin_amdgcn_s_setprio(3);
  else if (p == 2) __builtin_amdgcn_s_setprio(2);
  else if (p == 1) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// The same priorities for a fixed total and round, as thresholds on the
// remaining work: the level is the number of thresholds reached.
struct PrioSteps {
  int r1, r2, r3;
};
__device__ __forceinline__ PrioSteps prio_steps(int total, int round) {
  const int rr = round < 3 ? round : 3;
  auto at = [&](int level) {   // least remaining work whose level is >= `level`
    const int x = 3 * level - rr;
    return x > 0 ? (total * x + 12) / 12 : 0;
  };
  return PrioSteps{at(1), at(2), at(3)};
}
__device__ __forceinline__ void set_priority(const PrioSteps& t, int remaining) {
  if (remaining >= t.r3) __builtin_amdgcn_s_setprio(3);
  else if (remaining >= t.r2) __builtin_amdgcn_s_setprio(2);
  else if (remaining >= t.r1) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// Where work item `item` of a compact grid lies: items are numbered
// sequence-major and sequence k has items_of(slot, len) of them, so a
// block-wide prefix sum over the sequences' counts finds the sequence.
// s_item receives {sequence, item within it, its slot, its length}, or
// s_item[0] = -1 when the device lengths give fewer items than the grid.
// Ends with a barrier.
template <int NT, class F>
__device__ __forceinline__ void locate_item(const SeqArgs& s, F items_of, int item, int* s_wsum,
                                            int* s_item) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = s.n_seqs, per = (n + NT - 1) / NT;
  const int k0 = min(tid * per, n), k1 = min(k0 + per, n);
  int run = 0;
  for (int k = k0; k < k1; ++k) run += items_of(s.slots[k], s.lens[k]);
  int incl = run;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  if (lane == 63) s_wsum[wave] = incl;
  if (tid == 0) s_item[0] = -1;
  __syncthreads();
  int off = incl - run;
  for (int w2 = 0; w2 < wave; ++w2) off += s_wsum[w2];
  for (int k = k0; k < k1; ++k) {
    const int sl = s.slots[k], ln = s.lens[k];
    const int q = items_of(sl, ln);
    if (item >= off && item < off + q) {   // exactly one (k, thread) matches
      s_item[0] = k;
      s_item[1] = item - off;
      s_item[2] = sl;
      s_item[3] = ln;
    }
    off += q;
  }
  __syncthreads();
}

// The work item of this work-group: from the host's table when the launch
// has one, otherwise located on the device (locate_item).  Returns false
// when the device lengths give fewer items than the grid (uniform).
struct WgItem {
  int seq, local, slot, len;
};
template <int NT, class F>
__device__ __forceinline__ bool work_item(const SeqArgs& s, const ItemOrder& order, F items_of,
                                          int* s_wsum, int* s_item, WgItem& it) {
  if (order.n > 0) {
    const uint32_t w = order.item_of[blockIdx.x];
    it.seq = (int)(w >> 16);
    it.local = (int)(w & 0xFFFFu);
    it.slot = order.slot[blockIdx.x];
    it.len = order.len[blockIdx.x];
    return true;
  }
  locate_item<NT>(s, items_of, (int)blockIdx.x, s_wsum, s_item);
  if (s_item[0] < 0) return false;
  it.seq = __builtin_amdgcn_readfirstlane(s_item[0]);
  it.local = __builtin_amdgcn_readfirstlane(s_item[1]);
  it.slot = __builtin_amdgcn_readfirstlane(s_item[2]);
  it.len = __builtin_amdgcn_readfirstlane(s_item[3]);
  return true;
}

// Log-sum-exp merge of partial records (OSCAR summary page, section 4
// "Decoding Attention Kernel": segments of the sequence are processed by
// separate launches and their partial results merged afterwards).  A record
// holds, per head, m (log2 domain), l = sum 2^(x - m) and the unnormalized
// o' = sum 2^(x - m) v'; two records combine exactly as
//   M = max(m1, m2), l = l1 2^(m1 - M) + l2 2^(m2 - M), o' likewise.

// Split records of sequence i: the host's count when the launch carries the
// table, else from the device length.
__device__ __forceinline__ int split_records(const CacheArgs& c, const SeqArgs& s,
                                             const SplitCounts& sc, int i, int quota, int smax) {
  if (sc.n > 0) return sc.ns[i];
  const int slot = s.slots[i], len = s.lens[i];
  const bool ok = slot >= 0 && slot < c.max_seqs && len >= 1;
  return decode_splits(decode_work(ok ? len : 0, c.s_sink, c.s_keep, c.s_flush, c.ring_cap), quota,
                       smax);
}

// Lane slice of R_V for the un-rotation o = o' . R_V^T on the fp32 matrix
// cores: rb[u][e] = R_V[j][32 kq + 4u + e] of output channel j.  The
// structured rotations generate their entries (R = H / sqrt(128) or
// H P_br / sqrt(128), the same for every head) instead of reading a matrix.
__device__ __forceinline__ void load_unrotation(const CacheArgs& c, int h, int j, int kq,
                                                float4_t (&rb)[8]) {
  if (c.rot) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) rb[u][e] = hadamard_entry(c.rot, j, 32 * kq + 4 * u + e);
    return;
  }
  const float4_t* rg = (const float4_t*)(c.r_v + ((size_t)h * kD + j) * kD + 32 * kq);
#pragma unroll
  for (int u = 0; u < 8; ++u) rb[u] = rg[u];
}

// Final merge, then (UNROT) o = o' . R_V^T.
//
// Work-group = (KV head, pass, block of SB sequences): its 16 rows are the
// (sequence, query head) pairs of the block, one MFMA tile of rows, and all
// 128 output columns.  Thread = (row, 4 channels): it folds the row's
// records in rounds of 8 with a running maximum, loading the maxima and
// sums itself.  Without UNROT the thread stores its 4 channels.  With it,
// the merged o' rows go to LDS and wave w computes output columns
// 16w .. 16w+15 on the fp32 matrix cores, with lane (i, q) holding
// R_V[16w + i][32q .. 32q+31] in registers (loaded at entry, before any
// wait), so the contraction index of step (u, e) is k = 32q + 4u + e.
template <int HP, bool UNROT>
__global__ __launch_bounds__(512) void lse_merge_kernel(CacheArgs c, SeqArgs s, SplitCounts sc,
                                                        int quota, int passes, int smax, int chunk,
                                                        int stride, int sb,
                                                        const float* __restrict__ recs,
                                                        float* __restrict__ out) {
  constexpr int W = rec_words(HP), OO = rec_o_offset(HP);
  constexpr int kRound = 8;
  __shared__ float fin[16][kD + 4];
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int li = lane & 15, kq = lane >> 4;
  const int h = blockIdx.x / passes, pass = blockIdx.x % passes;
  const int nh = min(HP, c.g - pass * HP);
  const int s0 = blockIdx.y * sb;

  float4_t rb[8];
  if constexpr (UNROT) load_unrotation(c, h, 16 * wave + li, kq, rb);

  const int r = t >> 5, c4 = t & 31;
  const int i = s0 + r / nh;
  const bool valid = r < sb * nh && i < s.n_seqs;
  int nrec = 0;
  bool ok = false;
  const float* rec = recs;
  if (valid) {
    if (sc.n > 0) {
      ok = true;   // the host checked every slot and length of the call
    } else {
      const int slot = s.slots[i], len = s.lens[i];
      ok = slot >= 0 && slot < c.max_seqs && len >= 1;
    }
    const int ns = split_records(c, s, sc, i, quota, smax);
    nrec = (ns + chunk - 1) / chunk;
    rec = recs + (((size_t)i * c.hkv + h) * passes + pass) * stride * W;
  }
  const int hr = r % nh;
  float M = kNegInf, L = 0.0f;
  float4_t O = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < nrec; j0 += kRound) {
    float m[kRound], l[kRound];
    float4_t o[kRound];
#pragma unroll
    for (int j = 0; j < kRound; ++j) {
      const float* rj = rec + (size_t)(j0 + j < nrec ? j0 + j : j0) * W;
      m[j] = rj[hr];
      l[j] = rj[HP + hr];
      o[j] = *(const float4_t*)(rj + OO + hr * kD + 4 * c4);
    }
    float Mn = M;
#pragma unroll
    for (int j = 0; j < kRound; ++j)
      if (j0 + j < nrec) Mn = fmaxf(Mn, m[j]);
    const float sc = M == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(M - Mn);
    L *= sc;
    O[0] *= sc;
    O[1] *= sc;
    O[2] *= sc;
    O[3] *= sc;
#pragma unroll
    for (int j = 0; j < kRound; ++j) {
      const float w = (j0 + j < nrec && m[j] != kNegInf) ? __builtin_amdgcn_exp2f(m[j] - Mn) : 0.0f;
      L = __builtin_fmaf(w, l[j], L);
      O[0] = __builtin_fmaf(w, o[j][0], O[0]);
      O[1] = __builtin_fmaf(w, o[j][1], O[1]);
      O[2] = __builtin_fmaf(w, o[j][2], O[2]);
      O[3] = __builtin_fmaf(w, o[j][3], O[3]);
    }
    M = Mn;
  }
  float4_t f = {0.f, 0.f, 0.f, 0.f};
  if (nrec > 0) {
    f[0] = O[0] / L;
    f[1] = O[1] / L;
    f[2] = O[2] / L;
    f[3] = O[3] / L;
  }
  if constexpr (!UNROT) {
    if (valid && ok)
      *(float4_t*)(out + ((size_t)i * c.hq + (size_t)h * c.g + pass * HP + hr) * kD + 4 * c4) = f;
    return;
  }
  *(float4_t*)(&fin[r][4 * c4]) = f;
  __syncthreads();

  float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < 8; ++u) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fin[li][32 * kq + 4 * u + e], rb[u][e], acc, 0, 0,
                                                 0);
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int rr = 4 * kq + v;   // output row of this lane's v-th value
    const int ii = s0 + rr / nh;
    if (rr >= sb * nh || ii >= s.n_seqs) continue;
    if (sc.n == 0) {
      const int slot = s.slots[ii];
      if (slot < 0 || slot >= c.max_seqs || s.lens[ii] < 1) continue;
    }
    float* o = out + ((size_t)ii * c.hq + (size_t)h * c.g + pass * HP + rr % nh) * kD;
    o[16 * wave + li] = acc[v];
  }
}


// One launch for rows with many splits: work-group = (sequence, KV head,
// pass, query head of the pass), 1024 threads = 32 split groups x 32
// channel quads.  Thread (g, c4) folds splits g, g + 32, ... (8 per load
// round, all 8 loads issued together) with a running maximum, the 32 group
// states are folded through LDS, and (UNROT) output channel n = t / 8 of
// o = o' . R_V^T is the sum of 8 partial products of 16 channels each (its
// R_V row slice is loaded at entry, before any record).
template <int HP, bool UNROT>
__global__ __launch_bounds__(1024) void lse_wide_kernel(CacheArgs c, SeqArgs s, SplitCounts sc,
                                                        int quota, int passes, int smax,
                                                        const float* __restrict__ partials,
                                                        float* __restrict__ out) {
  constexpr int W = rec_words(HP), OO = rec_o_offset(HP);
  constexpr int kG = 32, kRound = 8;
  __shared__ float s_o[kG][kD];
  __shared__ float s_ml[kG][2];
  __shared__ float s_fin[kD];
  const int t = threadIdx.x, g = t >> 5, c4 = t & 31;
  const int x = blockIdx.x, hr = blockIdx.y;
  const int pass = x % passes, h = (x / passes) % c.hkv, i = x / (passes * c.hkv);
  const int nh = min(HP, c.g - pass * HP);
  if (hr >= nh) return;   // (uniform)

  const int n_out = t >> 3, part = t & 7;   // output channel, its 16-channel share of the sum
  float rv[16];
  if constexpr (UNROT) {
    if (c.rot) {
#pragma unroll
      for (int e = 0; e < 16; ++e) rv[e] = hadamard_entry(c.rot, n_out, 16 * part + e);
    } else {
      const float4_t* rg = (const float4_t*)(c.r_v + ((size_t)h * kD + n_out) * kD + 16 * part);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float4_t q = rg[u];
#pragma unroll
        for (int e = 0; e < 4; ++e) rv[4 * u + e] = q[e];
      }
    }
  }
  bool ok;
  if (sc.n > 0) {
    ok = true;   // the host checked every slot and length of the call
  } else {
    const int slot = s.slots[i], len = s.lens[i];
    ok = slot >= 0 && slot < c.max_seqs && len >= 1;
  }
  const int ns = split_records(c, s, sc, i, quota, smax);
  const float* rec = partials + (((size_t)i * c.hkv + h) * passes + pass) * smax * W;
  float M = kNegInf, L = 0.0f;
  float4_t O = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = g; j0 < ns; j0 += kG * kRound) {
    float m[kRound], l[kRound];
    float4_t o[kRound];
#pragma unroll
    for (int r = 0; r < kRound; ++r) {
      const int j = j0 + kG * r;
      const float* rj = rec + (size_t)(j < ns ? j : j0) * W;
      m[r] = rj[hr];
      l[r] = rj[HP + hr];
      o[r] = *(const float4_t*)(rj + OO + hr * kD + 4 * c4);
    }
    float Mn = M;
#pragma unroll
    for (int r = 0; r < kRound; ++r)
      if (j0 + kG * r < ns) Mn = fmaxf(Mn, m[r]);
    const float sc0 = M == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(M - Mn);
    L *= sc0;
    O[0] *= sc0;
    O[1] *= sc0;
    O[2] *= sc0;
    O[3] *= sc0;
#pragma unroll
    for (int r = 0; r < kRound; ++r) {
      const float w =
          (j0 + kG * r < ns && m[r] != kNegInf) ? __builtin_amdgcn_exp2f(m[r] - Mn) : 0.0f;
      L = __builtin_fmaf(w, l[r], L);
      O[0] = __builtin_fmaf(w, o[r][0], O[0]);
      O[1] = __builtin_fmaf(w, o[r][1], O[1]);
      O[2] = __builtin_fmaf(w, o[r][2], O[2]);
      O[3] = __builtin_fmaf(w, o[r][3], O[3]);
    }
    M = Mn;
  }
  *(float4_t*)&s_o[g][4 * c4] = O;
  if (c4 == 0) {
    s_ml[g][0] = M;
    s_ml[g][1] = L;
  }
  __syncthreads();
  if (t < kD) {
    float Mf = kNegInf;
#pragma unroll 8
    for (int gg = 0; gg < kG; ++gg) Mf = fmaxf(Mf, s_ml[gg][0]);
    float Lf = 0.0f, of = 0.0f;
#pragma unroll 8
    for (int gg = 0; gg < kG; ++gg) {
      const float mg = s_ml[gg][0];
      const float w = mg == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(mg - Mf);
      Lf = __builtin_fmaf(w, s_ml[gg][1], Lf);
      of = __builtin_fmaf(w, s_o[gg][t], of);
    }
    s_fin[t] = ns > 0 ? of / Lf : 0.0f;
  }
  __syncthreads();
  if (!ok) return;   // (uniform)
  float* orow = out + ((size_t)i * c.hq + (size_t)h * c.g + pass * HP + hr) * kD;
  if constexpr (!UNROT) {
    if (t < kD) orow[t] = s_fin[t];
    return;
  }
  float acc = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc = __builtin_fmaf(s_fin[16 * part + e], rv[e], acc);
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  if (part == 0) orow[n_out] = acc;
}

// The merge launch of a split-K decode step: the wide merge when a row may
// have more than kMergeDirect splits, else the 16-row final merge.
template <int HP, bool UNROT>
hipError_t launch_merge(const CacheArgs& c, const SeqArgs& s, const DecodePlan& plan,
                        float* partials, float* out, hipStream_t stream) {
  if (plan.smax > kMergeDirect) {
    const dim3 g1(s.n_seqs * c.hkv * plan.passes, HP);
    hipLaunchKernelGGL((lse_wide_kernel<HP, UNROT>), g1, dim3(1024), 0, stream, c, s, *plan.counts,
                       plan.quota, plan.passes, plan.smax, partials, out);
    return hipGetLastError();
  }
  const int nh_full = c.g < HP ? c.g : HP;
  const int sb = 16 / nh_full;   // sequences per final-merge work-group (16 rows)
  const dim3 mgrid(c.hkv * plan.passes, (s.n_seqs + sb - 1) / sb);
  hipLaunchKernelGGL((lse_merge_kernel<HP, UNROT>), mgrid, dim3(512), 0, stream, c, s,
                     *plan.counts, plan.quota,
                     plan.passes, plan.smax, 1, plan.smax, sb, partials, out);
  return hipGetLastError();
}

}  // namespace oscar
