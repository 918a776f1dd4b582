// Split-K decode attention over the mixed INT2 / BF16 paged cache (gfx950).
//
// What is computed (OSCAR summary page, section 2 "Attention and KV cache" and
// section 4 "Decoding Attention Kernel"; OScaR notes, "KV cache"):
//   o = softmax(q' K^T / sqrt(128)) V . R_V^T
// over the BF16 sink rows, the INT2 middle (dequantized as scale * code +
// zero) and the BF16 recent rows of one cache row, for the g query heads of
// each KV head.  The pages' decoder processes sequence segments in two
// launches and merges them; here the context of each (sequence, KV head) is
// split over work-groups, each writes a partial (max, sum, unnormalized
// output), and the last work-group to finish merges them by log-sum-exp and
// applies R_V^T, all in one launch.
//
// Work-group = 4 waves; one (sequence, KV head, query-head pass, split).
// Column n (0..15) of every MFMA tile is (group gi = n / HP, head hl = n % HP).
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

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

struct SoftmaxState {
  float m;   // running max (log2 domain), same in every lane of a column
  float l;   // this lane's share of the running sum
  float z;   // this lane's share of sum_t p_t * zero_v[t][group]
};

// Online-softmax update with a lazy max: the reference max only moves when a
// logit exceeds it by more than 8 (so p <= 2^8), which keeps most tiles free
// of the accumulator rescale.
template <int N>
__device__ __forceinline__ void softmax_step(float (&x)[N], float (&p)[N], SoftmaxState& st,
                                             float4_t (&acc)[8]) {
  float tmax = x[0];
#pragma unroll
  for (int k = 1; k < N; ++k) tmax = fmaxf(tmax, x[k]);
  tmax = rows_max(tmax);
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
    p[k] = __builtin_amdgcn_exp2f(x[k] - mref);
    st.l += p[k];
  }
}

template <int NG, int HP>
__global__ __launch_bounds__(256) void int2_decode_kernel(CacheArgs c, SeqArgs s, int splits,
                                                          int passes,
                                                          const uint16_t* __restrict__ q_rot,
                                                          float* __restrict__ out,
                                                          float* __restrict__ partials,
                                                          uint32_t* __restrict__ counters) {
  constexpr int G = kD / NG;
  constexpr int PW = HP * kD + 2 * HP;   // floats per partial record
  __shared__ float red_m[4][HP];
  __shared__ float red_l[4][HP];
  __shared__ float red_o[4][HP][kD];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int split = blockIdx.x;
  const int h = blockIdx.y / passes, pass = blockIdx.y % passes;
  const int i = blockIdx.z;
  const int r16 = lane & 15, qd = lane >> 4;

  const int slot = s.slots[i];
  int len = s.lens[i];
  const bool row_ok = slot >= 0 && slot < c.max_seqs && len >= 1;
  if (!row_ok) len = 0;
  const int nh = min(HP, c.g - pass * HP);   // valid heads in this pass

  // ---- columns and query operands
  const int n = r16, gi = n / HP, hl = n % HP;
  const int hqi = pass * HP + hl;
  const bool colv = (gi < NG) && (hl < nh);
  const uint16_t* qrow =
      q_rot + ((size_t)(row_ok ? i : 0) * c.hq + (size_t)h * c.g + (colv ? hqi : pass * HP)) * kD;
  const int grp_q = (NG == 1) ? 0 : (NG == 2 ? (qd >> 1) : qd);   // group of channels 32qd..32qd+31
  const bool bval = colv && (gi == grp_q);
  const float C2 = kLog2e * 0.08838834764831845f;                // log2(e) / sqrt(128)
  const float K1 = C2 * 16777216.0f;                              // undo the 2^-24 code scaling

  half8 bq[4];
  bf16x8 bw[4];
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int ch = 32 * qd + 16 * (cc >> 1) + 4 * (cc & 1) + v + 8 * e;
        const float qv = bval ? bf16_bits_to_f32(qrow[ch]) : 0.0f;
        bq[cc][2 * v + e] = (_Float16)(qv * (1.0f / (float)(1 << (2 * v))));
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint16_t bits = colv ? qrow[32 * qd + 8 * cc + e] : (uint16_t)0;
      bw[cc][e] = __builtin_bit_cast(__bf16, bits);
    }
  }
  float qsum = 0.0f;
  if (colv) {
    for (int ch = gi * G; ch < (gi + 1) * G; ++ch) qsum += bf16_bits_to_f32(qrow[ch]);
  }
  const float qsC = qsum * C2;

  // ---- this split's share of the context
  const int sq = s_quant_of(len, c.s_sink, c.s_keep, c.s_flush);
  const int nq = sq > c.s_sink ? sq - c.s_sink : 0;               // INT2 tokens
  const int n_pages = (nq + kPage - 1) / kPage;
  const int n_pairs = (n_pages + 1) / 2;
  const int pb = (int)((long long)split * n_pairs / splits);
  const int pe = (int)((long long)(split + 1) * n_pairs / splits);
  const int32_t* bt = c.block_table + (size_t)(row_ok ? slot : 0) * c.max_pages;
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
    int pa;
    bool oka, okb;
  };
  auto load_pair = [&](int pp, Pair& d) {
    const int pa = 2 * pp, pbq = 2 * pp + 1;
    int phys_a = pa < c.max_pages ? bt[pa] : -1;
    int phys_b = (pbq < n_pages && pbq < c.max_pages) ? bt[pbq] : -1;
    d.oka = phys_a >= 0 && phys_a < c.num_pages;
    d.okb = phys_b >= 0 && phys_b < c.num_pages;
    if (!d.oka) phys_a = 0;
    if (!d.okb) phys_b = phys_a;
    d.pa = pa;
    const uint8_t* A = c.pages + (size_t)phys_a * page_stride + head_off;
    const uint8_t* B = c.pages + (size_t)phys_b * page_stride + head_off;
    const int koff = (r16 * 8 + 2 * qd) * 4;
    const int poff = 1024 + 4 * (16 * gsel + 4 * qd);
    const int vpoff = poff + 64 * NG;
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
      x[r] = f16lo(d.kpa[r]) * (da[r] * K1) + f16hi(d.kpa[r]) * qsC;
      x[4 + r] = f16lo(d.kpb[r]) * (db[r] * K1) + f16hi(d.kpb[r]) * qsC;
    }
    if constexpr (NG > 1) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if constexpr (HP <= 8) x[k] += row_ror<8>(x[k]);
        if constexpr (HP <= 4) x[k] += row_ror<4>(x[k]);
        if constexpr (HP <= 2) x[k] += row_ror<2>(x[k]);
        if constexpr (HP <= 1) x[k] += row_ror<1>(x[k]);
      }
    }
    const int ta = 16 * d.pa + 4 * qd;   // INT2 token index of row 0 of tile A in this lane
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (!(d.oka && ta + r < nq)) x[r] = kNegInf;
      if (!(d.okb && ta + 16 + r < nq)) x[4 + r] = kNegInf;
    }
    float p[8];
    softmax_step<8>(x, p, st, acc);
    half8 pv;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pv[r] = (_Float16)(p[r] * f16lo(d.vpa[r]));
      pv[4 + r] = (_Float16)(p[4 + r] * f16lo(d.vpb[r]));
      st.z += p[r] * f16hi(d.vpa[r]) + p[4 + r] * f16hi(d.vpb[r]);
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

  {
    int pp = pb + wave;
    Pair cur, nxt;
    if (pp < pe) load_pair(pp, cur);
    for (; pp < pe; pp += 4) {
      if (pp + 4 < pe) load_pair(pp + 4, nxt);
      process_pair(cur);
      cur = nxt;
    }
  }
  // INT2 accumulators carry code * 4^(j%4) * 2^-24: bring them to true scale
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] *= 16777216.0f / (float)(1 << (2 * (j & 3)));

  // ---- BF16 window blocks (sink, then ring)
  const int nsink = min(len, c.s_sink);
  const int sb_n = (nsink + kPage - 1) / kPage;
  const int ring_lo = max(sq, c.s_sink);
  const int cnt = len > ring_lo ? len - ring_lo : 0;
  const int b0 = (ring_lo - c.s_sink) % c.ring_cap;
  const int rb_n = cnt > 0 ? c.ring_cap / kPage : 0;
  const int n_wu = sb_n + rb_n;
  const int wb = (int)((long long)split * n_wu / splits);
  const int we = (int)((long long)(split + 1) * n_wu / splits);
  const uint16_t* wbase = c.win + ((size_t)(row_ok ? slot : 0) * c.hkv + h) * c.win_blocks *
                                      (2 * kPage * kD);
  for (int u = wb + wave; u < we; u += 4) {
    int blk, first;   // window block and the slot index of its slot 0 in its segment
    const bool is_sink = u < sb_n;
    if (is_sink) {
      blk = u;
      first = kPage * u;
    } else {
      blk = c.sink_blocks + (u - sb_n);
      first = kPage * (u - sb_n);
    }
    auto slot_ok = [&](int t) {
      if (is_sink) return first + t < nsink;
      const int off = (first + t - b0 + c.ring_cap) % c.ring_cap;
      return off < cnt;
    };
    if (!__any(slot_ok(r16))) continue;
    const uint16_t* bp = wbase + (size_t)blk * (2 * kPage * kD);
    u32x4 kl[4], vl[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      kl[k] = *(const u32x4*)(bp + r16 * kD + 32 * qd + 8 * k);
      vl[k] = *(const u32x4*)(bp + kPage * kD + 32 * (16 * qd + r16) + 8 * k);
    }
    float4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kl[cc]), bw[cc], d, 0,
                                                  0, 0);
    float x[4], p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = slot_ok(4 * qd + r) ? d[r] * C2 : kNegInf;
    softmax_step<4>(x, p, st, acc);
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
      const u32x4 src = vl[j >> 1];
      const u32x2 pr = (j & 1) ? u32x2{src[2], src[3]} : u32x2{src[0], src[1]};
      const short4_t a = __builtin_bit_cast(short4_t, pr);
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, phi, acc[j], 0, 0, 0);
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, plo, acc[j], 0, 0, 0);
    }
  }

  // ---- wave totals -> LDS
  st.l = rows_sum(st.l);
  st.z = rows_sum(st.z);
  if (qd == 0 && gi == 0) {
    red_m[wave][hl] = st.m;
    red_l[wave][hl] = st.l;
  }
  if (bval) {   // lane holds channels 32qd .. 32qd+31 of its head, in its own group
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int j = 0; j < 8; ++j) red_o[wave][hl][32 * qd + 8 * r + j] = acc[j][r] + st.z;
  }
  __syncthreads();

  // ---- merge the 4 waves -> this work-group's partial record
  const size_t rec_base = (((size_t)i * c.hkv + h) * passes + pass) * splits;
  float* rec = partials + (rec_base + split) * PW;
  for (int idx = tid; idx < nh * kD; idx += 256) {
    const int hh = idx / kD, ch = idx % kD;
    float M = red_m[0][hh];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, red_m[w][hh]);
    float L = 0.0f, O = 0.0f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float wt = __builtin_amdgcn_exp2f(red_m[w][hh] - M);
        L += wt * red_l[w][hh];
        O += wt * red_o[w][hh][ch];
      }
    }
    if (ch == 0) {
      rec[hh] = M;
      rec[HP + hh] = L;
    }
    rec[2 * HP + hh * kD + ch] = O;
  }

  // ---- the last work-group of this (sequence, KV head, pass) merges all splits
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = atomicAdd(&counters[((size_t)i * c.hkv + h) * passes + pass], 1u);
    s_last = (prev == (uint32_t)(splits - 1));
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  float(*fin)[kD] = red_o[0];
  const float* recs = partials + rec_base * PW;
  for (int idx = tid; idx < nh * kD; idx += 256) {
    const int hh = idx / kD, ch = idx % kD;
    float M = kNegInf;
    for (int sp = 0; sp < splits; ++sp) M = fmaxf(M, recs[(size_t)sp * PW + hh]);
    float L = 0.0f, O = 0.0f;
    for (int sp = 0; sp < splits; ++sp) {
      const float* r = recs + (size_t)sp * PW;
      const float wt = M == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(r[hh] - M);
      L += wt * r[HP + hh];
      O += wt * r[2 * HP + hh * kD + ch];
    }
    fin[hh][ch] = O / L;
  }
  __syncthreads();
  const float* rv = c.r_v + (size_t)h * kD * kD;
  for (int idx = tid; idx < nh * kD; idx += 256) {
    const int hh = idx / kD, jo = idx % kD;
    const float* row = rv + (size_t)jo * kD;   // o_j = sum_c o'_c R_V[j][c]
    float sum = 0.0f;
#pragma unroll 8
    for (int cc = 0; cc < kD; ++cc) sum = __builtin_fmaf(fin[hh][cc], row[cc], sum);
    if (row_ok)
      out[((size_t)i * c.hq + (size_t)h * c.g + pass * HP + hh) * kD + jo] = sum;
  }
  if (tid == 0) counters[((size_t)i * c.hkv + h) * passes + pass] = 0u;
}

template <int NG, int HP>
static hipError_t launch_decode_t(const CacheArgs& c, const SeqArgs& s, const DecodePlan& plan,
                                  const uint16_t* q_rot, float* out, float* partials,
                                  uint32_t* counters, hipStream_t stream) {
  dim3 grid(plan.splits, c.hkv * plan.passes, s.n_seqs);
  hipLaunchKernelGGL((int2_decode_kernel<NG, HP>), grid, dim3(256), 0, stream, c, s, plan.splits,
                     plan.passes, q_rot, out, partials, counters);
  return hipGetLastError();
}

template <int NG>
static hipError_t dispatch_hp(const CacheArgs& c, const SeqArgs& s, const DecodePlan& plan,
                              const uint16_t* q_rot, float* out, float* partials,
                              uint32_t* counters, hipStream_t stream) {
  switch (plan.hp) {
    case 1: return launch_decode_t<NG, 1>(c, s, plan, q_rot, out, partials, counters, stream);
    case 2: return launch_decode_t<NG, 2>(c, s, plan, q_rot, out, partials, counters, stream);
    case 4: return launch_decode_t<NG, 4>(c, s, plan, q_rot, out, partials, counters, stream);
    case 8:
      if constexpr (NG <= 2)
        return launch_decode_t<NG, 8>(c, s, plan, q_rot, out, partials, counters, stream);
      break;
    case 16:
      if constexpr (NG == 1)
        return launch_decode_t<NG, 16>(c, s, plan, q_rot, out, partials, counters, stream);
      break;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const CacheArgs& c, const SeqArgs& s, const DecodePlan& plan,
                         const uint16_t* q_rot, float* out, float* partials, uint32_t* counters,
                         hipStream_t stream) {
  if (s.n_seqs <= 0) return hipSuccess;
  switch (c.ng) {
    case 1: return dispatch_hp<1>(c, s, plan, q_rot, out, partials, counters, stream);
    case 2: return dispatch_hp<2>(c, s, plan, q_rot, out, partials, counters, stream);
    case 4: return dispatch_hp<4>(c, s, plan, q_rot, out, partials, counters, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace oscar
