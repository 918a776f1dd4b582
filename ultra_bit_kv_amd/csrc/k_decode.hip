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

constexpr int kMaxWgPages = 512;   // page ids staged per work-group (<= 256 pairs per split)

template <int NG, int HP>
__global__ __launch_bounds__(256) void int2_decode_kernel(CacheArgs c, SeqArgs s, int splits,
                                                          int passes,
                                                          const uint16_t* __restrict__ q_rot,
                                                          float* __restrict__ partials) {
  constexpr int G = kD / NG;
  constexpr int PW = HP * kD + 2 * HP;   // floats per partial record
  __shared__ float red_m[4][HP];
  __shared__ float red_l[4][HP];
  __shared__ float red_o[4][HP][kD];
  __shared__ __attribute__((aligned(16))) uint16_t s_q[HP][kD];
  __shared__ float s_qsum[HP * NG];
  __shared__ int s_pages[kMaxWgPages];

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

  // ---- this split's share of the INT2 pages
  const int sq = s_quant_of(len, c.s_sink, c.s_keep, c.s_flush);
  const int nq = sq > c.s_sink ? sq - c.s_sink : 0;               // INT2 tokens
  const int n_pages = (nq + kPage - 1) / kPage;
  const int n_pairs = (n_pages + 1) / 2;
  const int pb = (int)((long long)split * n_pairs / splits);
  const int pe = (int)((long long)(split + 1) * n_pairs / splits);
  const int32_t* bt = c.block_table + (size_t)(row_ok ? slot : 0) * c.max_pages;

  // ---- stage the query rows of this pass and the split's page ids in LDS
  const uint16_t* qbase =
      q_rot + ((size_t)(row_ok ? i : 0) * c.hq + (size_t)h * c.g + (size_t)pass * HP) * kD;
  for (int t = tid; t < HP * 16; t += 256) {
    const int hh = t >> 4, part = t & 15;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (hh < nh) v = *(const u32x4*)(qbase + (size_t)hh * kD + 8 * part);
    *(u32x4*)(&s_q[hh][8 * part]) = v;
  }
  const int n_wg_pages = min(2 * (pe - pb), kMaxWgPages);
  for (int t = tid; t < n_wg_pages; t += 256) {
    const int pg = 2 * pb + t;
    int ph = -1;
    if (pg < n_pages && pg < c.max_pages) ph = bt[pg];
    s_pages[t] = (ph >= 0 && ph < c.num_pages) ? ph : -1;
  }
  __syncthreads();
  if (tid < HP * NG) {   // sum of each (group, head) slice of q', column n = group * HP + head
    const int hh = tid % HP, gg = tid / HP;
    float sum = 0.0f;
    for (int ch = gg * G; ch < (gg + 1) * G; ++ch) sum += bf16_bits_to_f32(s_q[hh][ch]);
    s_qsum[tid] = sum;
  }
  __syncthreads();

  // ---- per-lane MFMA operands for column n = (group gi, head hl)
  const int n = r16, gi = n / HP, hl = n % HP;
  const bool colv = (gi < NG) && (hl < nh);
  const int grp_q = (NG == 1) ? 0 : (NG == 2 ? (qd >> 1) : qd);   // group of channels 32qd..32qd+31
  const bool bval = colv && (gi == grp_q);
  const float C2 = kLog2e * 0.08838834764831845f;                // log2(e) / sqrt(128)
  const float K1 = C2 * 16777216.0f;                              // undo the 2^-24 code scaling
  const float qsC = colv ? s_qsum[n] * C2 : 0.0f;

  u32x4 wq[4];
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    wq[cc] = colv ? *(const u32x4*)(&s_q[hl][32 * qd + 8 * cc]) : z;
  }
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
  // pairs of this wave: local index wave + 4k, k < npw (interleaved over the 4 waves)
  const int nw = pe - pb;
  const int npw = nw > wave ? (nw - wave + 3) / 4 : 0;
  const int koff = (r16 * 8 + 2 * qd) * 4;
  const int poff = 1024 + 4 * (16 * gsel + 4 * qd);
  const int vpoff = poff + 64 * NG;
  auto load_pair = [&](int k, Pair& d) {
    const int local = wave + 4 * min(k, npw - 1);     // tail loads re-read the last pair
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
    const int ta = d.tok + 4 * qd;   // INT2 token index of row 0 of tile A in this lane
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

  if (npw > 0) {   // ping-pong: the loads of the next pair are in flight while one is processed
    Pair pa_, pb_;
    load_pair(0, pa_);
    for (int k = 0; k < npw; k += 2) {
      load_pair(k + 1, pb_);
      process_pair(pa_);
      load_pair(k + 2, pa_);
      if (k + 1 < npw) process_pair(pb_);
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
  float* rec = partials + ((((size_t)i * c.hkv + h) * passes + pass) * splits + split) * PW;
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
}

// Log-sum-exp merge of the split partials of one (sequence, KV head, pass),
// then o = o' . R_V^T with R_V staged in LDS (rows padded to 129 floats so the
// row-per-thread reads of a wave fall in distinct banks).
template <int HP>
__global__ __launch_bounds__(256) void merge_unrotate_kernel(CacheArgs c, SeqArgs s, int splits,
                                                             int passes,
                                                             const float* __restrict__ partials,
                                                             float* __restrict__ out) {
  constexpr int PW = HP * kD + 2 * HP;
  __shared__ float rv[kD][kD + 1];
  __shared__ float fin[HP][kD];
  const int tid = threadIdx.x;
  const int h = blockIdx.x / passes, pass = blockIdx.x % passes;
  const int i = blockIdx.y;
  const int slot = s.slots[i];
  const bool row_ok = slot >= 0 && slot < c.max_seqs && s.lens[i] >= 1;
  const int nh = min(HP, c.g - pass * HP);

  const float4* rg = (const float4*)(c.r_v + (size_t)h * kD * kD);
  for (int t = tid; t < kD * kD / 4; t += 256) {
    const float4 v = rg[t];
    const int row = (4 * t) / kD, col = (4 * t) % kD;
    rv[row][col] = v.x;
    rv[row][col + 1] = v.y;
    rv[row][col + 2] = v.z;
    rv[row][col + 3] = v.w;
  }
  const float* recs = partials + (((size_t)i * c.hkv + h) * passes + pass) * splits * PW;
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
  if (!row_ok) return;
  for (int idx = tid; idx < nh * kD; idx += 256) {
    const int hh = idx / kD, jo = idx % kD;
    float sum = 0.0f;
#pragma unroll 8
    for (int cc = 0; cc < kD; ++cc) sum = __builtin_fmaf(fin[hh][cc], rv[jo][cc], sum);
    out[((size_t)i * c.hq + (size_t)h * c.g + pass * HP + hh) * kD + jo] = sum;
  }
}

template <int NG, int HP>
static hipError_t launch_decode_t(const CacheArgs& c, const SeqArgs& s, const DecodePlan& plan,
                                  const uint16_t* q_rot, float* out, float* partials,
                                  hipStream_t stream) {
  dim3 grid(plan.splits, c.hkv * plan.passes, s.n_seqs);
  hipLaunchKernelGGL((int2_decode_kernel<NG, HP>), grid, dim3(256), 0, stream, c, s, plan.splits,
                     plan.passes, q_rot, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 mgrid(c.hkv * plan.passes, s.n_seqs);
  hipLaunchKernelGGL((merge_unrotate_kernel<HP>), mgrid, dim3(256), 0, stream, c, s, plan.splits,
                     plan.passes, partials, out);
  return hipGetLastError();
}

template <int NG>
static hipError_t dispatch_hp(const CacheArgs& c, const SeqArgs& s, const DecodePlan& plan,
                              const uint16_t* q_rot, float* out, float* partials,
                              hipStream_t stream) {
  switch (plan.hp) {
    case 1: return launch_decode_t<NG, 1>(c, s, plan, q_rot, out, partials, stream);
    case 2: return launch_decode_t<NG, 2>(c, s, plan, q_rot, out, partials, stream);
    case 4: return launch_decode_t<NG, 4>(c, s, plan, q_rot, out, partials, stream);
    case 8:
      if constexpr (NG <= 2) return launch_decode_t<NG, 8>(c, s, plan, q_rot, out, partials, stream);
      break;
    case 16:
      if constexpr (NG == 1) return launch_decode_t<NG, 16>(c, s, plan, q_rot, out, partials, stream);
      break;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const CacheArgs& c, const SeqArgs& s, const DecodePlan& plan,
                         const uint16_t* q_rot, float* out, float* partials, hipStream_t stream) {
  if (s.n_seqs <= 0) return hipSuccess;
  switch (c.ng) {
    case 1: return dispatch_hp<1>(c, s, plan, q_rot, out, partials, stream);
    case 2: return dispatch_hp<2>(c, s, plan, q_rot, out, partials, stream);
    case 4: return dispatch_hp<4>(c, s, plan, q_rot, out, partials, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace oscar
