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
//         lane's 32 codes contiguously), B = p * scale_v as fp16 hi + lo (two
//         MFMAs, about 22 significant bits); the zero point term
//         sum_t p_t z_t is accumulated on the VALU.
// BF16 window block (16 tokens): bf16 MFMA for q.k, P split into bf16 hi + lo
// for P.V.
#include "decode_common.h"

namespace oscar {

constexpr int kPrefetch = 2;   // page pairs in flight per wave ahead of the one processed

// Work-group = one work item (sequence, context split, group of WH adjacent
// KV heads, query-head pass); items are numbered sequence-major, then split,
// then head group, and the launch has exactly one work-group per item.  A
// work-group finds its item from a prefix sum over the sequences' item
// counts.  Wave w owns KV head WH * group + w; all waves walk the same pages,
// so each page is fetched as one contiguous run of WH page-head blocks.
template <int NG, int HP, int KH, int PF, int WH>
__global__ __launch_bounds__(64 * WH) void int2_decode_kernel(CacheArgs c, SeqArgs s, int quota,
                                                              int passes, int smax, int cus, ItemOrder order,
                                                              const uint16_t* __restrict__ q_rot,
                                                              float* __restrict__ partials) {
  constexpr int PW = rec_words(HP);   // floats per partial record
  constexpr int NT = 64 * WH;
  __shared__ __align__(8) int s_pages[kMaxWgPages];
  __shared__ int s_wsum[WH];
  __shared__ int s_item[4];   // sequence, item within it, its slot and length

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, qd = lane >> 4;
  const int rows = (c.hkv / (WH * KH)) * passes;

  // ---- the item of this work-group
  WgItem it;
  if (!work_item<NT>(
          s, order,
          [&](int sl, int ln) {
            const bool ok = sl >= 0 && sl < c.max_seqs && ln >= 1;
            const DecodeWork wk = decode_work(ok ? ln : 0, c.s_sink, c.s_keep, c.s_flush, c.ring_cap);
            return decode_splits(wk, quota, smax) * rows;
          },
          s_wsum, s_item, it))
    return;   // uniform: the device lengths give fewer items than the grid
  const int i = it.seq;
  const int local = it.local;
  const int split = local / rows, row = local % rows;
  const int hgrp = row / passes, pass = row % passes;
  const int hw = (hgrp * WH + wave) * KH;   // first KV head of this wave

  const int slot = it.slot;
  int len = it.len;
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
  const int rnd = blockIdx.x / cus;   // dispatch round on its compute unit
  set_priority(total_units, total_units, rnd);
  const uint16_t* wbase = c.win + ((size_t)(row_ok ? slot : 0) * c.hkv + hw) * c.win_blocks *
                                      (2 * kPage * kD);
  struct Win {
    u32x4 kl[4], vl[4];
    int u, k;   // block, KV head of the wave
  };
  auto win_block = [&](int u) { return u < sb_n ? u : c.sink_blocks + (u - sb_n); };
  auto win_slot_ok = [&](int u, int t) {
    if (u < sb_n) return kPage * u + t < nsink;
    const int off = (kPage * (u - sb_n) + t - b0 + c.ring_cap) % c.ring_cap;
    return off < cnt;
  };
  auto load_win = [&](int u, int k, Win& W) {
    W.u = u;
    W.k = k;
    const uint16_t* bp = wbase + ((size_t)k * c.win_blocks + win_block(u)) * (2 * kPage * kD);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      W.kl[k] = *(const u32x4*)(bp + r16 * kD + 32 * qd + 8 * k);
      W.vl[k] = *(const u32x4*)(bp + kPage * kD + 32 * (16 * qd + r16) + 8 * k);
    }
  };
  // ---- per-lane MFMA column n = (group gi, KV head kh of the wave, head hl of the pass)
  const int n = r16, gi = n / (KH * HP), kh = (n / HP) % KH, hl = n % HP;
  const int h = hw + kh;                                          // this column's KV head
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
  // The split's first BF16 window block is loaded before anything that waits
  // on the block table: the window blocks are processed first, while the
  // page ids and the first INT2 page pairs are on their way.
  const int nw = (we - wb) * KH;   // window blocks of this wave (each KV head in turn)
  Win wa, wn;
  if (nw > 0) load_win(wb, 0, wa);
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

  // B operands of the q.k MFMAs on KV head k: this column's q' if it belongs to head k
  half8 bqk[KH][4];
#pragma unroll
  for (int k = 0; k < KH; ++k)
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) bqk[k][cc] = (KH == 1 || kh == k) ? bq[cc] : half8{};

  const size_t head_off = (size_t)hw * c.page_bytes;              // the wave's first head
  const size_t col_off = (size_t)kh * c.page_bytes;               // this column's head, relative
  const size_t page_stride = (size_t)c.hkv * c.page_bytes;
  const int gsel = gi < NG ? gi : 0;                              // in-bounds group for params

  float4_t acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = float4_t{0.f, 0.f, 0.f, 0.f};
  SoftmaxState st{kNegInf, 0.0f, 0.0f};

  struct Pair {
    u32x2 ka[KH], kb[KH], va[KH], vb[KH];   // codes of each KV head of the wave
    u32x4 kpa, kpb, vpa, vpb;                // scale / zero of this column's head and group
    int tok;      // INT2 token index of slot 0 of page A
    bool oka, okb;
  };
  const int np = min(pe - pb, kMaxPairsPerSplit);                 // pairs of this split
  const int koff = (r16 * 8 + 2 * qd) * 4;
  const int poff = 1024 + 4 * (16 * gsel + 4 * qd);
  const int vpoff = poff + 64 * NG;
  // Page ids of the next pair to load, read from LDS one load ahead so the
  // LDS latency stays off the path that issues the page loads (loads are
  // issued in order k = 0, 1, 2, ...; the tail re-reads the last pair).
  int nx_a = 0, nx_b = 0;
  auto fetch_ids = [&](int k) {
    const int local = min(k, np - 1);
    nx_a = s_pages[2 * local];
    nx_b = s_pages[2 * local + 1];
  };
  auto load_pair = [&](int k, Pair& d) {
    const int local = min(k, np - 1);
    int pa = nx_a, pbq = nx_b;
    fetch_ids(k + 1);
    d.oka = pa >= 0;
    d.okb = pbq >= 0;
    if (!d.oka) pa = 0;
    if (!d.okb) pbq = pa;
    d.tok = 32 * (pb + local);
    const uint8_t* A = c.pages + (size_t)pa * page_stride + head_off;
    const uint8_t* B = c.pages + (size_t)pbq * page_stride + head_off;
#pragma unroll
    for (int k = 0; k < KH; ++k) {
      d.ka[k] = *(const u32x2*)(A + k * c.page_bytes + koff);
      d.kb[k] = *(const u32x2*)(B + k * c.page_bytes + koff);
      d.va[k] = *(const u32x2*)(A + k * c.page_bytes + 512 + 8 * lane);
      d.vb[k] = *(const u32x2*)(B + k * c.page_bytes + 512 + 8 * lane);
    }
    d.kpa = *(const u32x4*)(A + col_off + poff);
    d.kpb = *(const u32x4*)(B + col_off + poff);
    d.vpa = *(const u32x4*)(A + col_off + vpoff);
    d.vpb = *(const u32x4*)(B + col_off + vpoff);
  };

  auto qk_tile = [&](const u32x2 (&kw)[KH]) {
    float4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KH; ++k)
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        uint32_t w = (cc < 2) ? kw[k][0] : kw[k][1];
        if (cc & 1) w >>= 8;
        const u32x4 v = {w & 0x00030003u, w & 0x000C000Cu, w & 0x00300030u, w & 0x00C000C0u};
        d = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, v), bqk[k][cc], d, 0,
                                                   0, 0);
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
    if constexpr (NG > 1) {   // sum the group partials: lanes n, n +- KH HP, ... of a 16-lane row
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if constexpr (KH * HP <= 8) x[k] += row_ror<8>(x[k]);
        if constexpr (KH * HP <= 4) x[k] += row_ror<4>(x[k]);
        if constexpr (KH * HP <= 2) x[k] += row_ror<2>(x[k]);
        if constexpr (KH * HP <= 1) x[k] += row_ror<1>(x[k]);
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
    // P' = p * scale_v enters the MFMA as fp16: with p <= 2^8 (the lazy
    // max) a value scale of 128 or more could overflow it, so such a pair
    // takes the exact max (p <= 1, P' <= scale <= 65504)
    const bool big_scale = max_scale_bits(d.vpa, d.vpb) >= 0x5800u;   // fp16 128.0
    float p[8];
    softmax_step<8>(x, K1, p, st, acc, __any(big_scale) ? 0.0f : 8.0f);
    uint32_t ph[4], pl[4];
    mul_by_f16lo_split(p[0], d.vpa[0], p[1], d.vpa[1], ph[0], pl[0]);
    mul_by_f16lo_split(p[2], d.vpa[2], p[3], d.vpa[3], ph[1], pl[1]);
    mul_by_f16lo_split(p[4], d.vpb[0], p[5], d.vpb[1], ph[2], pl[2]);
    mul_by_f16lo_split(p[6], d.vpb[2], p[7], d.vpb[3], ph[3], pl[3]);
    // B operands of the P.V MFMAs on KV head k: this column's P' if it belongs to head k
    half8 pv[KH], pvl[KH];
#pragma unroll
    for (int k = 0; k < KH; ++k) {
      const bool mine = KH == 1 || kh == k;
      pv[k] = __builtin_bit_cast(half8, mine ? u32x4{ph[0], ph[1], ph[2], ph[3]} : u32x4{});
      pvl[k] = __builtin_bit_cast(half8, mine ? u32x4{pl[0], pl[1], pl[2], pl[3]} : u32x4{});
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      st.z = __builtin_fmaf(p[r], f16hi(d.vpa[r]), st.z);
      st.z = __builtin_fmaf(p[4 + r], f16hi(d.vpb[r]), st.z);
    }
#pragma unroll
    for (int k = 0; k < KH; ++k) {
      const uint32_t w0 = d.va[k][0], w1 = d.va[k][1], w2 = d.vb[k][0], w3 = d.vb[k][1];
      const uint32_t s0 = w0 >> 8, s1 = w1 >> 8, s2 = w2 >> 8, s3 = w3 >> 8;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t mask = 0x00030003u << (2 * (j & 3));
        const half8 a = (j < 4) ? codes_as_half8(w0, w1, w2, w3, mask)
                                : codes_as_half8(s0, s1, s2, s3, mask);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pv[k], acc[j], 0, 0, 0);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pvl[k], acc[j], 0, 0, 0);
      }
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
    for (int r = 0; r < 4; ++r)   // only the columns of the block's KV head
      x[r] = ((KH == 1 || kh == W.k) && win_slot_ok(W.u, 4 * qd + r)) ? d[r] : kNegInf;
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
  // (issued now, so they arrive while the window blocks are processed)
  Pair ring[PF];
  if (np > 0) {
    fetch_ids(0);
#pragma unroll
    for (int j = 0; j < PF; ++j) load_pair(j, ring[j]);
  }

  // ---- BF16 window blocks (true scale), each KV head of the wave in turn,
  // one block in flight ahead
  for (int t = 0; t < nw; ++t) {
    const int u = wb + t / KH;
    set_priority(kWinCost * (we - u) + np, total_units, rnd);
    if (t + 1 < nw) load_win(wb + (t + 1) / KH, (t + 1) % KH, wn);
    if (__any(win_slot_ok(u, r16))) process_win(wa);
    wa = wn;
  }

  // ---- INT2 page pairs: accumulate in code units (code * 4^(j%4) * 2^-24);
  // the window sums are moved to those units and back (powers of two, exact)
  if (np > 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= (float)(1 << (2 * (j & 3))) * (1.0f / 16777216.0f);
    for (int k = 0; k < np; k += PF) {
      set_priority(np - k, total_units, rnd);
#pragma unroll
      for (int j = 0; j < PF; ++j) {
        if (k + j < np) process_pair(ring[j]);
        load_pair(k + j + PF, ring[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= 16777216.0f / (float)(1 << (2 * (j & 3)));
  }

  // ---- this wave's partial record: (max, sum, unnormalized o') per head of the pass
  st.l = rows_sum(st.l);
  st.z = rows_sum(st.z);
  float* rec = partials + ((((size_t)i * c.hkv + h) * passes + pass) * smax + split) * PW;
  if (qd == 0 && gi == 0 && hl < nh) {   // one lane per (KV head, query head) column
    rec[hl] = st.m;
    rec[HP + hl] = st.l;
  }
  if (bval) {   // lane holds channels 32qd .. 32qd+31 of its head, in its own group
    float* o = rec + rec_o_offset(HP) + hl * kD + 32 * qd;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float4_t lo = {acc[0][r] + st.z, acc[1][r] + st.z, acc[2][r] + st.z, acc[3][r] + st.z};
      const float4_t hi = {acc[4][r] + st.z, acc[5][r] + st.z, acc[6][r] + st.z, acc[7][r] + st.z};
      *(float4_t*)(o + 8 * r) = lo;
      *(float4_t*)(o + 8 * r + 4) = hi;
    }
  }
}

template <int NG, int HP, int KH>
static hipError_t launch_decode_t(const CacheArgs& c, const SeqArgs& s, const DecodePlan& plan,
                                  const uint16_t* q_rot, float* out, float* partials,
                                  int phases, hipStream_t stream) {
  const int wh = plan.wh;
  if (phases & kDecodeSplit) {
    const dim3 grid(plan.grid);
    switch (wh) {
      case 4:
        hipLaunchKernelGGL((int2_decode_kernel<NG, HP, KH, kPrefetch, 4>), grid, dim3(256), 0, stream,
                           c, s, plan.quota, plan.passes, plan.smax, plan.cus, *plan.order, q_rot,
                           partials);
        break;
      case 2:
        hipLaunchKernelGGL((int2_decode_kernel<NG, HP, KH, kPrefetch, 2>), grid, dim3(128), 0, stream,
                           c, s, plan.quota, plan.passes, plan.smax, plan.cus, *plan.order, q_rot,
                           partials);
        break;
      default:
        hipLaunchKernelGGL((int2_decode_kernel<NG, HP, KH, kPrefetch, 1>), grid, dim3(64), 0, stream,
                           c, s, plan.quota, plan.passes, plan.smax, plan.cus, *plan.order, q_rot,
                           partials);
        break;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (phases & kDecodeMerge)
    return c.unrot ? launch_merge<HP, true>(c, s, plan, partials, out, stream)
                   : launch_merge<HP, false>(c, s, plan, partials, out, stream);
  return hipSuccess;
}

template <int NG, int HP, int KH>
static int wgs_per_cu_t(int wh) {
  int nb = 0;
  hipError_t e = hipErrorInvalidValue;
  switch (wh) {
    case 4:
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, int2_decode_kernel<NG, HP, KH, kPrefetch, 4>, 256, 0);
      break;
    case 2:
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, int2_decode_kernel<NG, HP, KH, kPrefetch, 2>, 128, 0);
      break;
    default:
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, int2_decode_kernel<NG, HP, KH, kPrefetch, 1>, 64, 0);
      break;
  }
  return e == hipSuccess && nb > 0 ? nb : 1;
}

// The (groups, heads per pass, KV heads per wave) shapes the planner uses:
// one group: any power-of-two pass, two KV heads per wave up to 8 heads;
// with ng groups the columns (group, KV head, head) fill the tile exactly.
template <class F>
static auto with_shape(int ng, int hp, int kh, F&& f) {
  if (ng == 1) {
    if (kh == 2) {
      switch (hp) {
        case 1: return f.template operator()<1, 1, 2>();
        case 2: return f.template operator()<1, 2, 2>();
        case 4: return f.template operator()<1, 4, 2>();
        case 8: return f.template operator()<1, 8, 2>();
      }
    } else {
      switch (hp) {
        case 1: return f.template operator()<1, 1, 1>();
        case 2: return f.template operator()<1, 2, 1>();
        case 4: return f.template operator()<1, 4, 1>();
        case 8: return f.template operator()<1, 8, 1>();
        case 16: return f.template operator()<1, 16, 1>();
      }
    }
  } else if (ng == 2) {
    if (kh == 2 && hp == 4) return f.template operator()<2, 4, 2>();
    if (kh == 1 && hp == 8) return f.template operator()<2, 8, 1>();
  } else if (ng == 4) {
    if (kh == 2 && hp == 2) return f.template operator()<4, 2, 2>();
    if (kh == 1 && hp == 4) return f.template operator()<4, 4, 1>();
  }
  return f.fail();
}

struct OccupancyQuery {
  const DecodePlan& plan;
  template <int NG, int HP, int KH>
  int operator()() const { return wgs_per_cu_t<NG, HP, KH>(plan.wh); }
  int fail() const { return 1; }
};

int decode_wgs_per_cu(const CacheArgs& c, const DecodePlan& plan) {
  return with_shape(c.ng, plan.hp, plan.kh, OccupancyQuery{plan});
}

struct DecodeLaunch {
  const CacheArgs& c;
  const SeqArgs& s;
  const DecodePlan& plan;
  const uint16_t* q_rot;
  float* out;
  float* partials;
  int phases;
  hipStream_t stream;
  template <int NG, int HP, int KH>
  hipError_t operator()() const {
    return launch_decode_t<NG, HP, KH>(c, s, plan, q_rot, out, partials, phases, stream);
  }
  hipError_t fail() const { return hipErrorInvalidValue; }
};

hipError_t launch_decode(const CacheArgs& c, const SeqArgs& s, const DecodePlan& plan,
                         const uint16_t* q_rot, float* out, float* partials, int phases,
                         hipStream_t stream) {
  if (s.n_seqs <= 0 || plan.grid <= 0) return hipSuccess;
  return with_shape(c.ng, plan.hp, plan.kh,
                    DecodeLaunch{c, s, plan, q_rot, out, partials, phases, stream});
}

}  // namespace oscar
