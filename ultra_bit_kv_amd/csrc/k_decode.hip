// Split-K decode attention over the mixed INT2 / BF16 paged cache (gfx950).
//
// What is computed (OSCAR summary page, section 2 "Attention and KV cache" and
// section 4 "Decoding Attention Kernel"; OScaR notes, "KV cache"):
//   o = softmax(q' K^T / sqrt(128)) V . R_V^T
// over the BF16 sink rows, the INT2 middle (dequantized as scale * code +
// zero) and the BF16 recent rows of one cache row, for the g query heads of
// each KV head.  As in the pages' decoder, segments of the context are
// processed by separate work-groups of one launch, each writing a partial
// (max, sum, unnormalized output), and a second launch merges them by
// log-sum-exp and applies R_V^T.
//
// Work-group = (sequence, context split, group of adjacent KV heads), one
// wave per KV head.  Column n (0..15) of every MFMA tile is (group gi = n / HP,
// head hl = n % HP).
//
// INT2 page pair (32 tokens), per wave:
//   QK^T: A = K codes [16 tokens x 32 channels] per instruction, taken as fp16
//         subnormals straight from the code bits (code * 4^v * 2^-24, one AND
//         per two codes), B = the rotated query scaled by 4^-v and masked to
//         the column's group.  Scale and zero-point enter after the MFMA:
//         q.k_hat = sum_g s_g (q_g . c_g) + z_g sum_{j in g} q_j.
//   P.V:  A = V codes [16 channels x 32 tokens] (the page layout stores each
//         lane's 32 codes contiguously), B = p * scale_v as fp16; the zero
//         point term sum_t p_t z_t is accumulated on the VALU.
// BF16 window block (16 tokens): bf16 MFMA for q.k, P split into bf16 hi + lo
// for P.V.
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

// fp16 pair (a * lo16(wa), b * lo16(wb)), rounded to fp16.
__device__ __forceinline__ uint32_t mul_f32_by_f16lo_pack(float a, uint32_t wa, float b,
                                                          uint32_t wb) {
  const half2_t ha = __builtin_bit_cast(half2_t, wa);
  const half2_t hb = __builtin_bit_cast(half2_t, wb);
  half2_t r;
  r.x = (_Float16)(a * (float)ha.x);
  r.y = (_Float16)(b * (float)hb.x);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

struct SoftmaxState {
  float m;   // running max (log2 domain), same in every lane of a column
  float l;   // this lane's share of the running sum
  float z;   // this lane's share of sum_t p_t * zero_v[t][group]
};

// Online-softmax update with a lazy max.  x holds logits in raw units; the
// log2-domain logit is scale * x (scale > 0).  The reference max only moves
// when a logit exceeds it by more than 8 (so p <= 2^8), which keeps most
// tiles free of the accumulator rescale.
template <int N>
__device__ __forceinline__ void softmax_step(const float (&x)[N], float scale, float (&p)[N],
                                             SoftmaxState& st, float4_t (&acc)[8]) {
  float tmax = x[0];
#pragma unroll
  for (int k = 1; k < N; ++k) tmax = fmaxf(tmax, x[k]);
  tmax = rows_max(tmax) * scale;
  if (__any(tmax > st.m + 8.0f)) {
    const float m_new = fmaxf(st.m, tmax);
    const float alpha = m_new > st.m ? __builtin_amdgcn_exp2f(st.m - m_new) : 1.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= alpha;
    st.l *= alpha;
    st.z *= alpha;
    st.m = m_new;
  }
  const float mref = st.m == kNegInf ? 0.0f : st.m;
#pragma unroll
  for (int k = 0; k < N; ++k) {
    p[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[k], scale, -mref));
    st.l += p[k];
  }
}

constexpr int kMaxWgPages = 2 * kMaxPairsPerSplit;   // page ids staged per work-group
constexpr int kPrefetch = 2;       // page pairs in flight per wave ahead of the one processed


// Issue priority of the calling wave from its remaining share of the work:
// waves of one SIMD otherwise issue oldest-first, so the first work-groups
// on a compute unit run ahead and the last ones finish alone.
__device__ __forceinline__ void set_priority(int remaining, int total) {
  const int p = (4 * remaining - 1) / total;   // 0..3
  if (p >= 3) __builtin_amdgcn_s_setprio(3);
  else if (p == 2) __builtin_amdgcn_s_setprio(2);
  else if (p == 1) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// Work-group = one work item (sequence, context split, group of WH adjacent
// KV heads, query-head pass); items are numbered sequence-major, then split,
// then head group, and the launch has exactly one work-group per item.  A
// work-group finds its item from a prefix sum over the sequences' item
// counts.  Wave w owns KV head WH * group + w; all waves walk the same pages,
// so each page is fetched as one contiguous run of WH page-head blocks.
template <int NG, int HP, int PF, int WH>
__global__ __launch_bounds__(64 * WH) void int2_decode_kernel(CacheArgs c, SeqArgs s, int quota,
                                                              int passes, int smax,
                                                              const uint16_t* __restrict__ q_rot,
                                                              float* __restrict__ partials) {
  constexpr int PW = HP * kD + 2 * HP;   // floats per partial record
  constexpr int NT = 64 * WH;
  __shared__ int s_pages[kMaxWgPages];
  __shared__ int s_wsum[WH];
  __shared__ int s_item[4];   // sequence, item within it, its slot and length

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, qd = lane >> 4;
  const int rows = (c.hkv / WH) * passes;

  // ---- the item of this work-group: sequence i with prefix(i) <= item < prefix(i + 1)
  {
    auto seq_items = [&](int sl, int ln) {
      const bool ok = sl >= 0 && sl < c.max_seqs && ln >= 1;
      const DecodeWork wk = decode_work(ok ? ln : 0, c.s_sink, c.s_keep, c.s_flush, c.ring_cap);
      return decode_splits(wk, quota, smax) * rows;
    };
    const int n = s.n_seqs, per = (n + NT - 1) / NT;
    const int k0 = min(tid * per, n), k1 = min(k0 + per, n);
    int run = 0;
    for (int k = k0; k < k1; ++k) run += seq_items(s.slots[k], s.lens[k]);
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
    const int item = blockIdx.x;
    for (int k = k0; k < k1; ++k) {
      const int sl = s.slots[k], ln = s.lens[k];
      const int q = seq_items(sl, ln);
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
  if (s_item[0] < 0) return;   // uniform: the device lengths give fewer items than the grid
  const int i = __builtin_amdgcn_readfirstlane(s_item[0]);
  const int local = __builtin_amdgcn_readfirstlane(s_item[1]);
  const int split = local / rows, row = local % rows;
  const int hgrp = row / passes, pass = row % passes;
  const int h = hgrp * WH + wave;

  const int slot = __builtin_amdgcn_readfirstlane(s_item[2]);
  int len = __builtin_amdgcn_readfirstlane(s_item[3]);
  const bool row_ok = slot >= 0 && slot < c.max_seqs && len >= 1;
  if (!row_ok) len = 0;
  const int nh = min(HP, c.g - pass * HP);   // valid heads in this pass

  // ---- this split's share of the context: INT2 page pairs and BF16 window blocks
  const int sq = s_quant_of(len, c.s_sink, c.s_keep, c.s_flush);
  const int nq = sq > c.s_sink ? sq - c.s_sink : 0;               // INT2 tokens
  const int n_pages = (nq + kPage - 1) / kPage;
  const int n_pairs = (n_pages + 1) / 2;
  const int32_t* bt = c.block_table + (size_t)(row_ok ? slot : 0) * c.max_pages;

  const int nsink = min(len, c.s_sink);
  const int sb_n = (nsink + kPage - 1) / kPage;
  const int ring_lo = max(sq, c.s_sink);
  const int cnt = len > ring_lo ? len - ring_lo : 0;
  const int b0 = (ring_lo - c.s_sink) % c.ring_cap;
  const int rb_n = cnt > 0 ? c.ring_cap / kPage : 0;
  const int n_wu = sb_n + rb_n;
  const int n_split = decode_splits(DecodeWork{n_pairs, n_wu}, quota, smax);
  // (products stay below 2^31 within the config limits)
  const int pb = (int)((unsigned)(split * n_pairs) / (unsigned)n_split);
  const int pe = (int)((unsigned)((split + 1) * n_pairs) / (unsigned)n_split);
  const int wb = (int)((unsigned)(split * n_wu) / (unsigned)n_split);
  const int we = (int)((unsigned)((split + 1) * n_wu) / (unsigned)n_split);
  const int total_units = max(1, (pe - pb) + kWinCost * (we - wb));
  set_priority(total_units, total_units);
  const uint16_t* wbase = c.win + ((size_t)(row_ok ? slot : 0) * c.hkv + h) * c.win_blocks *
                                      (2 * kPage * kD);
  struct Win {
    u32x4 kl[4], vl[4];
    int u;
  };
  auto win_block = [&](int u) { return u < sb_n ? u : c.sink_blocks + (u - sb_n); };
  auto win_slot_ok = [&](int u, int t) {
    if (u < sb_n) return kPage * u + t < nsink;
    const int off = (kPage * (u - sb_n) + t - b0 + c.ring_cap) % c.ring_cap;
    return off < cnt;
  };
  auto load_win = [&](int u, Win& W) {
    W.u = u;
    const uint16_t* bp = wbase + (size_t)win_block(u) * (2 * kPage * kD);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      W.kl[k] = *(const u32x4*)(bp + r16 * kD + 32 * qd + 8 * k);
      W.vl[k] = *(const u32x4*)(bp + kPage * kD + 32 * (16 * qd + r16) + 8 * k);
    }
  };
  // ---- per-lane MFMA column n = (group gi, head hl)
  const int n = r16, gi = n / HP, hl = n % HP;
  const bool colv = (gi < NG) && (hl < nh);
  const int grp_q = (NG == 1) ? 0 : (NG == 2 ? (qd >> 1) : qd);   // group of channels 32qd..32qd+31
  const bool bval = colv && (gi == grp_q);
  const float C2 = kLog2e * 0.08838834764831845f;                // log2(e) / sqrt(128)
  const float K1 = C2 * 16777216.0f;                              // undo the 2^-24 code scaling

  // ---- the lane's 32 query channels straight into registers; the split's page ids to LDS
  u32x4 wq[4];
  {
    const u32x4 z = {0u, 0u, 0u, 0u};
    const uint16_t* qp = q_rot + ((size_t)i * c.hq + (size_t)h * c.g + (size_t)pass * HP +
                                  (colv ? hl : 0)) * kD + 32 * qd;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) wq[cc] = colv ? *(const u32x4*)(qp + 8 * cc) : z;
  }
  const int n_wg_pages = min(2 * (pe - pb), kMaxWgPages);
  for (int t = tid; t < n_wg_pages; t += 64 * WH) {
    const int pg = 2 * pb + t;
    int ph = -1;
    if (pg < n_pages && pg < c.max_pages) ph = bt[pg];
    s_pages[t] = (ph >= 0 && ph < c.num_pages) ? ph : -1;
  }
  // group sums of q' for the zero-point term: each lane adds its 32 channels
  // if they lie in its column's group, then the four lanes of the column add up
  float qsum = 0.0f;
  if (bval) {
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        qsum += bf16_bits_to_f32(wq[cc][e] & 0xFFFFu) + bf16_bits_to_f32(wq[cc][e] >> 16);
  }
  qsum = rows_sum(qsum);
  // INT2 logits in raw units x = s * D + z * qsum * 2^-24, log2 logit = K1 * x
  const float qz = colv ? qsum * (1.0f / 16777216.0f) : 0.0f;
  __syncthreads();   // page ids visible

  bf16x8 bw[4];
  half8 bq[4];
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) {
    bw[cc] = __builtin_bit_cast(bf16x8, wq[cc]);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        // K index 8 qd + 2v + e of chunk cc <-> channel 32 qd + cl
        const int cl = 16 * (cc >> 1) + 4 * (cc & 1) + v + 8 * e;
        const uint32_t word = wq[cl >> 3][(cl & 7) >> 1];
        const uint32_t bits = (cl & 1) ? (word >> 16) : (word & 0xFFFFu);
        const float qv = bval ? bf16_bits_to_f32(bits) : 0.0f;
        bq[cc][2 * v + e] = (_Float16)(qv * (1.0f / (float)(1 << (2 * v))));
      }
    }
  }

  const size_t head_off = (size_t)h * c.page_bytes;
  const size_t page_stride = (size_t)c.hkv * c.page_bytes;
  const int gsel = gi < NG ? gi : 0;                              // in-bounds group for params

  float4_t acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = float4_t{0.f, 0.f, 0.f, 0.f};
  SoftmaxState st{kNegInf, 0.0f, 0.0f};

  struct Pair {
    u32x2 ka, kb, va, vb;
    u32x4 kpa, kpb, vpa, vpb;
    int tok;      // INT2 token index of slot 0 of page A
    bool oka, okb;
  };
  const int np = min(pe - pb, kMaxPairsPerSplit);                 // pairs of this split
  const int koff = (r16 * 8 + 2 * qd) * 4;
  const int poff = 1024 + 4 * (16 * gsel + 4 * qd);
  const int vpoff = poff + 64 * NG;
  auto load_pair = [&](int k, Pair& d) {
    const int local = min(k, np - 1);                             // tail loads re-read the last pair
    int pa = s_pages[2 * local], pbq = s_pages[2 * local + 1];
    d.oka = pa >= 0;
    d.okb = pbq >= 0;
    if (!d.oka) pa = 0;
    if (!d.okb) pbq = pa;
    d.tok = 32 * (pb + local);
    const uint8_t* A = c.pages + (size_t)pa * page_stride + head_off;
    const uint8_t* B = c.pages + (size_t)pbq * page_stride + head_off;
    d.ka = *(const u32x2*)(A + koff);
    d.kb = *(const u32x2*)(B + koff);
    d.va = *(const u32x2*)(A + 512 + 8 * lane);
    d.vb = *(const u32x2*)(B + 512 + 8 * lane);
    d.kpa = *(const u32x4*)(A + poff);
    d.kpb = *(const u32x4*)(B + poff);
    d.vpa = *(const u32x4*)(A + vpoff);
    d.vpb = *(const u32x4*)(B + vpoff);
  };

  auto qk_tile = [&](u32x2 kw) {
    float4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      uint32_t w = (cc < 2) ? kw[0] : kw[1];
      if (cc & 1) w >>= 8;
      const u32x4 v = {w & 0x00030003u, w & 0x000C000Cu, w & 0x00300030u, w & 0x00C000C0u};
      d = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, v), bq[cc], d, 0, 0, 0);
    }
    return d;
  };

  auto process_pair = [&](const Pair& d) {
    const float4_t da = qk_tile(d.ka);
    const float4_t db = qk_tile(d.kb);
    float x[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = __builtin_fmaf(f16lo(d.kpa[r]), da[r], f16hi(d.kpa[r]) * qz);
      x[4 + r] = __builtin_fmaf(f16lo(d.kpb[r]), db[r], f16hi(d.kpb[r]) * qz);
    }
    if constexpr (NG > 1) {   // sum the group partials: lanes n, n +- HP, ... of a 16-lane row
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if constexpr (HP <= 8) x[k] += row_ror<8>(x[k]);
        if constexpr (HP <= 4) x[k] += row_ror<4>(x[k]);
        if constexpr (HP <= 2) x[k] += row_ror<2>(x[k]);
        if constexpr (HP <= 1) x[k] += row_ror<1>(x[k]);
      }
    }
    if (!(d.oka && d.okb && d.tok + 32 <= nq)) {   // the pair holds slots past S_quant
      const int ta = d.tok + 4 * qd;   // INT2 token index of row 0 of tile A in this lane
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (!(d.oka && ta + r < nq)) x[r] = kNegInf;
        if (!(d.okb && ta + 16 + r < nq)) x[4 + r] = kNegInf;
      }
    }
    float p[8];
    softmax_step<8>(x, K1, p, st, acc);
    u32x4 pw;   // P' = p * scale_v as fp16, k index 8 qd + e <-> (e < 4 ? A : B) row e % 4
    pw[0] = mul_f32_by_f16lo_pack(p[0], d.vpa[0], p[1], d.vpa[1]);
    pw[1] = mul_f32_by_f16lo_pack(p[2], d.vpa[2], p[3], d.vpa[3]);
    pw[2] = mul_f32_by_f16lo_pack(p[4], d.vpb[0], p[5], d.vpb[1]);
    pw[3] = mul_f32_by_f16lo_pack(p[6], d.vpb[2], p[7], d.vpb[3]);
    const half8 pv = __builtin_bit_cast(half8, pw);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      st.z = __builtin_fmaf(p[r], f16hi(d.vpa[r]), st.z);
      st.z = __builtin_fmaf(p[4 + r], f16hi(d.vpb[r]), st.z);
    }
    const uint32_t w0 = d.va[0], w1 = d.va[1], w2 = d.vb[0], w3 = d.vb[1];
    const uint32_t s0 = w0 >> 8, s1 = w1 >> 8, s2 = w2 >> 8, s3 = w3 >> 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t mask = 0x00030003u << (2 * (j & 3));
      const half8 a = (j < 4) ? codes_as_half8(w0, w1, w2, w3, mask)
                              : codes_as_half8(s0, s1, s2, s3, mask);
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pv, acc[j], 0, 0, 0);
    }
  };

  auto process_win = [&](const Win& W) {
    float4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, W.kl[cc]), bw[cc], d,
                                                  0, 0, 0);
    float x[4], p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = win_slot_ok(W.u, 4 * qd + r) ? d[r] : kNegInf;
    softmax_step<4>(x, C2, p, st, acc);
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      hi[r] = f32_to_bf16_rne(p[r]);
      lo[r] = f32_to_bf16_rne(p[r] - __uint_as_float(hi[r] << 16));
    }
    const short4_t phi = {(short)hi[0], (short)hi[1], (short)hi[2], (short)hi[3]};
    const short4_t plo = {(short)lo[0], (short)lo[1], (short)lo[2], (short)lo[3]};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const u32x4 src = W.vl[j >> 1];
      const u32x2 pr = (j & 1) ? u32x2{src[2], src[3]} : u32x2{src[0], src[1]};
      const short4_t a = __builtin_bit_cast(short4_t, pr);
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, phi, acc[j], 0, 0, 0);
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, plo, acc[j], 0, 0, 0);
    }
  };

  // ---- INT2 ring: PF page pairs in flight ahead of the one being processed
  Pair ring[PF];
  if (np > 0) {
#pragma unroll
    for (int j = 0; j < PF; ++j) load_pair(j, ring[j]);
  }

  // ---- INT2 page pairs: accumulate in code units (code * 4^(j%4) * 2^-24)
  if (np > 0) {
    for (int k = 0; k < np; k += PF) {
      set_priority(total_units - k, total_units);
#pragma unroll
      for (int j = 0; j < PF; ++j) {
        if (k + j < np) process_pair(ring[j]);
        load_pair(k + j + PF, ring[j]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] *= 16777216.0f / (float)(1 << (2 * (j & 3)));

  // ---- BF16 window blocks (true scale), one block in flight ahead
  if (wb < we) {
    Win wa, wn;
    load_win(wb, wa);
    for (int u = wb; u < we; ++u) {
      set_priority(kWinCost * (we - u), total_units);
      if (u + 1 < we) load_win(u + 1, wn);
      if (__any(win_slot_ok(u, r16))) process_win(wa);
      wa = wn;
    }
  }

  // ---- this wave's partial record: (max, sum, unnormalized o') per head of the pass
  st.l = rows_sum(st.l);
  st.z = rows_sum(st.z);
  float* rec = partials + ((((size_t)i * c.hkv + h) * passes + pass) * smax + split) * PW;
  if (qd == 0 && gi == 0 && hl < nh) {
    rec[hl] = st.m;
    rec[HP + hl] = st.l;
  }
  if (bval) {   // lane holds channels 32qd .. 32qd+31 of its head, in its own group
    float* o = rec + 2 * HP + hl * kD + 32 * qd;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float4_t lo = {acc[0][r] + st.z, acc[1][r] + st.z, acc[2][r] + st.z, acc[3][r] + st.z};
      const float4_t hi = {acc[4][r] + st.z, acc[5][r] + st.z, acc[6][r] + st.z, acc[7][r] + st.z};
      *(float4_t*)(o + 8 * r) = lo;
      *(float4_t*)(o + 8 * r + 4) = hi;
    }
  }
}

// Log-sum-exp merge of the split partials, then o = o' . R_V^T.
//
// Work-group = (KV head, pass, block of SB sequences, half of the output
// columns); its 16 rows are the (sequence, query head) pairs of the block,
// which is exactly one MFMA tile of rows.  All global loads (the half of R_V,
// every split's max and sum, the first kChunk split outputs of each row
// channel) are issued before the first wait; both column halves merge the
// same rows.  The un-rotation runs on the fp32 matrix cores: o'[16 x 128]
// times the R_V^T columns of the half, with those R_V rows staged in LDS
// (padded to 132 floats so the operand reads of a wave fall in distinct
// banks).
template <int HP>
__global__ __launch_bounds__(256) void merge_unrotate_kernel(CacheArgs c, SeqArgs s, int quota,
                                                             int passes, int smax, int sb,
                                                             const float* __restrict__ partials,
                                                             float* __restrict__ out) {
  constexpr int PW = HP * kD + 2 * HP;
  constexpr int kChunk = 8;                      // split outputs per channel per load round
  constexpr int kRows = 16;
  constexpr int kLd = kD + 4;
  __shared__ float rv[kD / 2][kLd];   // the half of R_V's rows (output columns) of this work-group
  __shared__ float fin[kRows][kLd];
  __shared__ float s_M[kRows], s_L[kRows];
  __shared__ int s_ns[kRows];
  // per-split maxima and sums, [kRows][smax] each, in dynamic LDS
  extern __shared__ float s_dyn[];
  float* s_m = s_dyn;
  float* s_l = s_dyn + (size_t)kRows * smax;
  const int tid = threadIdx.x;
  const int h = blockIdx.x / passes, pass = blockIdx.x % passes;
  const int nh = min(HP, c.g - pass * HP);
  const int s0 = blockIdx.y * sb;
  const int jh = 64 * blockIdx.z;   // output columns jh .. jh + 63

  // row r <-> (sequence s0 + r / nh, head hh = r % nh)
  auto row_seq = [&](int r) { return s0 + r / nh; };
  auto row_valid = [&](int r) { return r < sb * nh && row_seq(r) < s.n_seqs; };
  auto rec_of = [&](int r) {
    return partials + (((size_t)row_seq(r) * c.hkv + h) * passes + pass) * smax * PW;
  };
  // ---- issue every load first: R_V, the split maxima / sums and the first
  // kChunk split outputs of each (row, channel).  Records exist for all smax
  // splits of every row, so the loads need not wait for the split counts.
  const float4* rg = (const float4*)(c.r_v + ((size_t)h * kD + jh) * kD);
  float4 rvv[kD * kD / 8 / 256];
#pragma unroll
  for (int t = 0; t < kD * kD / 8 / 256; ++t) rvv[t] = rg[tid + 256 * t];
  const int nml = kRows * smax;
  const int t_ml = tid < nml ? tid : 0;
  float ml_m = 0.0f, ml_l = 0.0f;
  if (tid < nml && row_valid(t_ml / smax)) {
    const float* rec = rec_of(t_ml / smax) + (size_t)(t_ml % smax) * PW;
    ml_m = rec[(t_ml / smax) % nh];
    ml_l = rec[HP + (t_ml / smax) % nh];
  }
  constexpr int kPer = kRows * kD / 256;   // (row, channel) pairs per thread
  const int ch = tid % kD;
  const int jmax = smax < kChunk ? smax : kChunk;
  float ov[kPer][kChunk];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int r = tid / kD + 2 * k;
    const bool rv_ok = row_valid(r);
    const float* o = rec_of(rv_ok ? r : 0) + 2 * HP + (r % nh) * kD + ch;
#pragma unroll
    for (int j = 0; j < kChunk; ++j) ov[k][j] = (rv_ok && j < jmax) ? o[(size_t)j * PW] : 0.0f;
  }
  int my_ns = 0;
  if (tid < kRows && row_valid(tid)) {
    const int i = row_seq(tid);
    const int slot = s.slots[i];
    const int len = s.lens[i];
    const bool ok = slot >= 0 && slot < c.max_seqs && len >= 1;
    my_ns = decode_splits(decode_work(ok ? len : 0, c.s_sink, c.s_keep, c.s_flush, c.ring_cap),
                          quota, smax);
  }
#pragma unroll
  for (int t = 0; t < kD * kD / 8 / 256; ++t) {
    const int e = 4 * (tid + 256 * t);
    *(float4*)(&rv[e / kD][e % kD]) = rvv[t];
  }
  if (tid < nml) {
    s_m[tid] = ml_m;
    s_l[tid] = ml_l;
  }
  for (int t = tid + 256; t < nml; t += 256) {   // more than 16 splits: remaining maxima / sums
    const int r = t / smax, sp = t % smax;
    float m = 0.0f, l = 0.0f;
    if (row_valid(r)) {
      const float* rec = rec_of(r) + (size_t)sp * PW;
      m = rec[r % nh];
      l = rec[HP + r % nh];
    }
    s_m[t] = m;
    s_l[t] = l;
  }
  if (tid < kRows) s_ns[tid] = my_ns;
  __syncthreads();
  if (tid < kRows) {   // log-sum-exp of row tid over its splits
    const int ns = s_ns[tid];
    float M = kNegInf;
    for (int sp = 0; sp < ns; ++sp) M = fmaxf(M, s_m[tid * smax + sp]);
    float L = 0.0f;
    for (int sp = 0; sp < ns; ++sp) {   // the split's weight replaces its maximum
      const float wt = M == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(s_m[tid * smax + sp] - M);
      L += wt * s_l[tid * smax + sp];
      s_m[tid * smax + sp] = wt;
    }
    s_M[tid] = M;
    s_L[tid] = L;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int r = tid / kD + 2 * k;
    const int ns = s_ns[r];
    auto weight = [&](int sp) { return s_m[r * smax + sp]; };
    float O = 0.0f;
#pragma unroll
    for (int j = 0; j < kChunk; ++j)
      if (j < ns) O = __builtin_fmaf(weight(j), ov[k][j], O);
    if (ns > kChunk) {   // long contexts: more load rounds
      const float* o = rec_of(r) + 2 * HP + (r % nh) * kD + ch;
      for (int sp0 = kChunk; sp0 < ns; sp0 += kChunk) {
        float v[kChunk];
#pragma unroll
        for (int j = 0; j < kChunk; ++j) v[j] = sp0 + j < ns ? o[(size_t)(sp0 + j) * PW] : 0.0f;
#pragma unroll
        for (int j = 0; j < kChunk; ++j)
          if (sp0 + j < ns) O = __builtin_fmaf(weight(sp0 + j), v[j], O);
      }
    }
    fin[r][ch] = ns > 0 ? O / s_L[r] : 0.0f;
  }
  __syncthreads();

  // ---- o = o' . R_V^T on the fp32 matrix cores: wave w computes columns jh + 16w .. +15
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, kq = lane >> 4;
  float4_t acc0 = {0.f, 0.f, 0.f, 0.f};
  const int j0 = 16 * wave;
#pragma unroll
  for (int kb = 0; kb < kD / 4; ++kb)
    acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(fin[li][4 * kb + kq], rv[j0 + li][4 * kb + kq], acc0,
                                                0, 0, 0);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int r = 4 * kq + v;   // output row of this lane's v-th value
    if (!row_valid(r)) continue;
    const int i = row_seq(r);
    const int slot = s.slots[i];
    if (slot < 0 || slot >= c.max_seqs || s.lens[i] < 1) continue;
    float* o = out + ((size_t)i * c.hq + (size_t)h * c.g + pass * HP + r % nh) * kD;
    o[jh + j0 + li] = acc0[v];
  }
}

template <int NG, int HP>
static hipError_t launch_decode_t(const CacheArgs& c, const SeqArgs& s, const DecodePlan& plan,
                                  const uint16_t* q_rot, float* out, float* partials,
                                  int phases, hipStream_t stream) {
  const int wh = plan.wh;
  if (phases & kDecodeSplit) {
    const dim3 grid(plan.grid);
    switch (wh) {
      case 4:
        hipLaunchKernelGGL((int2_decode_kernel<NG, HP, kPrefetch, 4>), grid, dim3(256), 0, stream,
                           c, s, plan.quota, plan.passes, plan.smax, q_rot, partials);
        break;
      case 2:
        hipLaunchKernelGGL((int2_decode_kernel<NG, HP, kPrefetch, 2>), grid, dim3(128), 0, stream,
                           c, s, plan.quota, plan.passes, plan.smax, q_rot, partials);
        break;
      default:
        hipLaunchKernelGGL((int2_decode_kernel<NG, HP, kPrefetch, 1>), grid, dim3(64), 0, stream,
                           c, s, plan.quota, plan.passes, plan.smax, q_rot, partials);
        break;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (phases & kDecodeMerge) {
    const int nh_full = c.g < HP ? c.g : HP;
    const int sb = 16 / nh_full;   // sequences per merge work-group (16 rows)
    dim3 mgrid(c.hkv * plan.passes, (s.n_seqs + sb - 1) / sb, 2);
    const size_t dyn = 2 * sizeof(float) * 16 * (size_t)plan.smax;
    hipLaunchKernelGGL((merge_unrotate_kernel<HP>), mgrid, dim3(256), dyn, stream, c, s,
                       plan.quota, plan.passes, plan.smax, sb, partials, out);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <int NG, int HP>
static int wgs_per_cu_t(int wh) {
  int nb = 0;
  hipError_t e = hipErrorInvalidValue;
  switch (wh) {
    case 4:
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, int2_decode_kernel<NG, HP, kPrefetch, 4>, 256, 0);
      break;
    case 2:
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, int2_decode_kernel<NG, HP, kPrefetch, 2>, 128, 0);
      break;
    default:
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, int2_decode_kernel<NG, HP, kPrefetch, 1>, 64, 0);
      break;
  }
  return e == hipSuccess && nb > 0 ? nb : 1;
}

template <int NG>
static int wgs_per_cu_ng(const DecodePlan& plan) {
  switch (plan.hp) {
    case 1: return wgs_per_cu_t<NG, 1>(plan.wh);
    case 2: return wgs_per_cu_t<NG, 2>(plan.wh);
    case 4: return wgs_per_cu_t<NG, 4>(plan.wh);
    case 8:
      if constexpr (NG <= 2) return wgs_per_cu_t<NG, 8>(plan.wh);
      break;
    case 16:
      if constexpr (NG == 1) return wgs_per_cu_t<NG, 16>(plan.wh);
      break;
  }
  return 1;
}

int decode_wgs_per_cu(const CacheArgs& c, const DecodePlan& plan) {
  switch (c.ng) {
    case 1: return wgs_per_cu_ng<1>(plan);
    case 2: return wgs_per_cu_ng<2>(plan);
    case 4: return wgs_per_cu_ng<4>(plan);
  }
  return 1;
}

template <int NG>
static hipError_t dispatch_hp(const CacheArgs& c, const SeqArgs& s, const DecodePlan& plan,
                              const uint16_t* q_rot, float* out, float* partials,
                              int phases, hipStream_t stream) {
  switch (plan.hp) {
    case 1: return launch_decode_t<NG, 1>(c, s, plan, q_rot, out, partials, phases, stream);
    case 2: return launch_decode_t<NG, 2>(c, s, plan, q_rot, out, partials, phases, stream);
    case 4: return launch_decode_t<NG, 4>(c, s, plan, q_rot, out, partials, phases, stream);
    case 8:
      if constexpr (NG <= 2) return launch_decode_t<NG, 8>(c, s, plan, q_rot, out, partials, phases, stream);
      break;
    case 16:
      if constexpr (NG == 1) return launch_decode_t<NG, 16>(c, s, plan, q_rot, out, partials, phases, stream);
      break;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const CacheArgs& c, const SeqArgs& s, const DecodePlan& plan,
                         const uint16_t* q_rot, float* out, float* partials, int phases,
                         hipStream_t stream) {
  if (s.n_seqs <= 0 || plan.grid <= 0) return hipSuccess;
  switch (c.ng) {
    case 1: return dispatch_hp<1>(c, s, plan, q_rot, out, partials, phases, stream);
    case 2: return dispatch_hp<2>(c, s, plan, q_rot, out, partials, phases, stream);
    case 4: return dispatch_hp<4>(c, s, plan, q_rot, out, partials, phases, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace oscar
