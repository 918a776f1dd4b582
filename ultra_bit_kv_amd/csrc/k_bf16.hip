// Split-K decode attention over a plain BF16 paged cache (gfx950): the
// uncompressed baseline the INT2 cache is measured against (OSCAR summary
// page, abstract and section 5: memory and throughput against BF16; OScaR
// notes, efficiency: latency against BF16 FlashDecoding).
//
//   o = softmax(q K^T / sqrt(128)) V        (no rotation, no windows)
//
// Page-head block (8 KB): K rows [16 tokens][128], then V rows [16][128],
// bf16, row-major.  Work-group = (sequence, context split, group of WH
// adjacent KV heads, query-head pass), one wave per KV head; items come from
// the same compact grid and split rule as the INT2 kernel, a unit of work
// being a pair of pages.  Column n (0..15) of every MFMA tile is query head
// n of the pass.
//
// Per page, per wave:
//   q.K^T: bf16 MFMA 16x16x32, A = K rows (lane: token, 32 channels), B = q.
//   P.V:   bf16 MFMA 16x16x16 with P split into bf16 hi + lo; A row i of
//          output tile j is channel 8i + j, so lane (i, quad) loads
//          channels 8i .. 8i+7 of tokens 4 quad .. 4 quad + 3 (four 16-byte
//          loads, each token row read whole by 16 lanes) and regroups them
//          per channel with byte permutes.  Accumulators match the INT2
//          kernel's (lane (i, quad), tile j, value v <-> channel
//          32 quad + 8 v + j), and so do the partial records.
#include "decode_common.h"

namespace oscar {

constexpr int kBfPrefetch = 2;   // pages in flight per wave ahead of the one processed

template <int HP, int PF, int WH>
__global__ __launch_bounds__(64 * WH) void bf16_decode_kernel(CacheArgs c, SeqArgs s, int quota,
                                                              int passes, int smax, int cus, ItemOrder order,
                                                              const uint16_t* __restrict__ q,
                                                              float* __restrict__ partials) {
  constexpr int PW = rec_words(HP);
  constexpr int NT = 64 * WH;
  constexpr int kBlk = 2 * kPage * kD;   // bf16 elements of one page-head block
  __shared__ int s_pages[kMaxWgPages];
  __shared__ int s_wsum[WH];
  __shared__ int s_item[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, qd = lane >> 4;
  const int rows = (c.hkv / WH) * passes;

  WgItem it;
  if (!work_item<NT>(
          s, order,
          [&](int sl, int ln) {
            const bool ok = sl >= 0 && sl < c.max_seqs && ln >= 1;
            const DecodeWork wk = decode_work(ok ? ln : 0, c.s_sink, c.s_keep, c.s_flush, c.ring_cap);
            return decode_splits(wk, quota, smax) * rows;
          },
          s_wsum, s_item, it))
    return;   // uniform
  const int i = it.seq;
  const int local = it.local;
  const int split = local / rows, row = local % rows;
  const int hgrp = row / passes, pass = row % passes;
  const int h = hgrp * WH + wave;
  const int slot = it.slot;
  int len = it.len;
  const bool row_ok = slot >= 0 && slot < c.max_seqs && len >= 1;
  if (!row_ok) len = 0;
  const int nh = min(HP, c.g - pass * HP);

  // ---- this split's pages: pairs [pb, pe) of the row's ceil(len / 16) pages
  const int n_pages = (len + kPage - 1) / kPage;
  const int n_pairs = (n_pages + 1) / 2;
  const int n_split = decode_splits(DecodeWork{n_pairs, 0}, quota, smax);
  const int pb = (int)((unsigned)(split * n_pairs) / (unsigned)n_split);
  const int pe = (int)((unsigned)((split + 1) * n_pairs) / (unsigned)n_split);
  const int pg0 = 2 * pb;
  const int npg = max(0, min(min(2 * pe, n_pages) - pg0, kMaxWgPages));
  const int rnd = blockIdx.x / cus;
  set_priority(max(1, pe - pb), max(1, pe - pb), rnd);
  const int32_t* bt = c.block_table + (size_t)(row_ok ? slot : 0) * c.max_pages;

  const int hl = r16;              // this lane's MFMA column: query head hl of the pass
  const bool colv = hl < nh;
  const float C2 = kLog2e * 0.08838834764831845f;   // log2(e) / sqrt(128)

  u32x4 wq[4];
  {
    const u32x4 z = {0u, 0u, 0u, 0u};
    const uint16_t* qp =
        q + ((size_t)i * c.hq + (size_t)h * c.g + (size_t)pass * HP + (colv ? hl : 0)) * kD + 32 * qd;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) wq[cc] = colv ? *(const u32x4*)(qp + 8 * cc) : z;
  }
  for (int t = tid; t < npg; t += NT) {
    const int pg = pg0 + t;
    int ph = -1;
    if (pg < c.max_pages) ph = bt[pg];
    s_pages[t] = (ph >= 0 && ph < c.num_pages) ? ph : -1;
  }
  __syncthreads();   // page ids visible
  bf16x8 bw[4];
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) bw[cc] = __builtin_bit_cast(bf16x8, wq[cc]);

  const uint16_t* pages = (const uint16_t*)c.pages;
  const size_t page_stride = (size_t)c.hkv * kBlk;
  const size_t head_off = (size_t)h * kBlk;

  float4_t acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = float4_t{0.f, 0.f, 0.f, 0.f};
  SoftmaxState st{kNegInf, 0.0f, 0.0f, 0.0f};

  struct Page {
    u32x4 k[4], v[4];
    int tok;   // token index of slot 0
    bool ok;
  };
  auto load_page = [&](int k, Page& d) {
    const int t = min(k, npg - 1);   // tail loads re-read the last page
    int ph = s_pages[t];
    d.ok = ph >= 0;
    if (!d.ok) ph = 0;
    d.tok = kPage * (pg0 + t);
    const uint16_t* P = pages + (size_t)ph * page_stride + head_off;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) d.k[cc] = *(const u32x4*)(P + r16 * kD + 32 * qd + 8 * cc);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      d.v[u] = *(const u32x4*)(P + kPage * kD + (4 * qd + u) * kD + 8 * r16);
  };
  auto process_page = [&](const Page& d) {
    float4_t dd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
      dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, d.k[cc]), bw[cc], dd,
                                                   0, 0, 0);
    float x[4], p[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) x[v] = (d.ok && d.tok + 4 * qd + v < len) ? dd[v] : kNegInf;
    softmax_step<4>(x, C2, p, st, acc);
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      hi[v] = f32_to_bf16_rne(p[v]);
      lo[v] = f32_to_bf16_rne(p[v] - __uint_as_float(hi[v] << 16));
    }
    const short4_t phi = {(short)hi[0], (short)hi[1], (short)hi[2], (short)hi[3]};
    const short4_t plo = {(short)lo[0], (short)lo[1], (short)lo[2], (short)lo[3]};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // tokens 4 qd + 0..3 of channel 8 r16 + j: half (j & 1) of word j / 2 of each row
      const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
      const uint32_t w01 = __builtin_amdgcn_perm(d.v[1][j >> 1], d.v[0][j >> 1], sel);
      const uint32_t w23 = __builtin_amdgcn_perm(d.v[3][j >> 1], d.v[2][j >> 1], sel);
      const short4_t a = __builtin_bit_cast(short4_t, u32x2{w01, w23});
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, phi, acc[j], 0, 0, 0);
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, plo, acc[j], 0, 0, 0);
    }
  };

  if (npg > 0) {
    Page ring[PF];
#pragma unroll
    for (int j = 0; j < PF; ++j) load_page(j, ring[j]);
    for (int k = 0; k < npg; k += PF) {
      set_priority(max(1, (npg - k + 1) / 2), max(1, pe - pb), rnd);
#pragma unroll
      for (int j = 0; j < PF; ++j) {
        if (k + j < npg) process_page(ring[j]);
        load_page(k + j + PF, ring[j]);
      }
    }
  }

  // ---- this wave's partial record: (max, sum, unnormalized o) per head of the pass
  st.l = rows_sum(st.l);
  float* rec = partials + ((((size_t)i * c.hkv + h) * passes + pass) * smax + split) * PW;
  if (qd == 0 && colv) {
    rec[hl] = st.m;
    rec[HP + hl] = st.l;
  }
  if (colv) {   // lane holds channels 32qd .. 32qd+31 of its head
    float* o = rec + rec_o_offset(HP) + hl * kD + 32 * qd;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float4_t lo4 = {acc[0][r], acc[1][r], acc[2][r], acc[3][r]};
      const float4_t hi4 = {acc[4][r], acc[5][r], acc[6][r], acc[7][r]};
      *(float4_t*)(o + 8 * r) = lo4;
      *(float4_t*)(o + 8 * r + 4) = hi4;
    }
  }
}

template <int HP, int WH>
static void launch_split_t(const CacheArgs& c, const SeqArgs& s, const DecodePlan& plan,
                           const uint16_t* q, float* partials, hipStream_t stream) {
  hipLaunchKernelGGL((bf16_decode_kernel<HP, kBfPrefetch, WH>), dim3(plan.grid), dim3(64 * WH), 0,
                     stream, c, s, plan.quota, plan.passes, plan.smax, plan.cus, *plan.order, q, partials);
}

template <int HP>
static hipError_t launch_bf16_t(const CacheArgs& c, const SeqArgs& s, const DecodePlan& plan,
                                const uint16_t* q, float* out, float* partials, int phases,
                                hipStream_t stream) {
  if (phases & kDecodeSplit) {
    switch (plan.wh) {
      case 4: launch_split_t<HP, 4>(c, s, plan, q, partials, stream); break;
      case 2: launch_split_t<HP, 2>(c, s, plan, q, partials, stream); break;
      default: launch_split_t<HP, 1>(c, s, plan, q, partials, stream); break;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (phases & kDecodeMerge) return launch_merge<HP, false>(c, s, plan, partials, out, stream);
  return hipSuccess;
}

hipError_t launch_bf16_decode(const CacheArgs& c, const SeqArgs& s, const DecodePlan& plan,
                              const uint16_t* q, float* out, float* partials, int phases,
                              hipStream_t stream) {
  if (s.n_seqs <= 0 || plan.grid <= 0) return hipSuccess;
  switch (plan.hp) {
    case 1: return launch_bf16_t<1>(c, s, plan, q, out, partials, phases, stream);
    case 2: return launch_bf16_t<2>(c, s, plan, q, out, partials, phases, stream);
    case 4: return launch_bf16_t<4>(c, s, plan, q, out, partials, phases, stream);
    case 8: return launch_bf16_t<8>(c, s, plan, q, out, partials, phases, stream);
    case 16: return launch_bf16_t<16>(c, s, plan, q, out, partials, phases, stream);
  }
  return hipErrorInvalidValue;
}

template <int HP>
static int bf16_wgs_t(int wh) {
  int nb = 0;
  hipError_t e = hipErrorInvalidValue;
  switch (wh) {
    case 4:
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, bf16_decode_kernel<HP, kBfPrefetch, 4>, 256, 0);
      break;
    case 2:
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, bf16_decode_kernel<HP, kBfPrefetch, 2>, 128, 0);
      break;
    default:
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, bf16_decode_kernel<HP, kBfPrefetch, 1>, 64, 0);
      break;
  }
  return e == hipSuccess && nb > 0 ? nb : 1;
}

int bf16_decode_wgs_per_cu(const DecodePlan& plan) {
  switch (plan.hp) {
    case 1: return bf16_wgs_t<1>(plan.wh);
    case 2: return bf16_wgs_t<2>(plan.wh);
    case 4: return bf16_wgs_t<4>(plan.wh);
    case 8: return bf16_wgs_t<8>(plan.wh);
    case 16: return bf16_wgs_t<16>(plan.wh);
  }
  return 1;
}

}  // namespace oscar
