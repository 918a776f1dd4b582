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

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) const u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;

// One direct-to-LDS load: each lane's 16 bytes at src + OFF go to
// dst + OFF + 16 * lane (dst is the same for the whole wave; the immediate
// offset applies to both addresses).
template <int OFF = 0>
__device__ __forceinline__ void load_lds16(const uint8_t* src, lds_u8* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, OFF, 0);
}

// A wave-uniform address kept in scalar registers, so that a per-lane 32-bit
// offset added to it gives a scalar-base + vector-offset load address.
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  const uint64_t a = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return (const uint8_t*)(((uint64_t)hi << 32) | lo);
}

// Bytes of one page for the KH consecutive KV heads of a wave (their
// page-head blocks are contiguous in a page), and the direct-to-LDS loads
// (1 KB per wave instruction, 16 bytes per lane) that bring it in.
template <int NG, int KH, int KM>
struct PairGeom {
  static constexpr int PB = KM ? kOtsPageBytes : 1024 + 128 * NG;   // page-head block
  static constexpr int RB = KH * PB;                  // one page of the wave's heads
  static constexpr int NI = (RB + 1023) / 1024;       // loads per page
  static constexpr int LAST_LANES = (RB - 1024 * (NI - 1)) / 16;   // lanes of the last load
  static constexpr int PAIR_LOADS = 2 * NI;
  static constexpr int WIN_LOADS = 4;                 // one window half: 16 rows x 256 B
  static constexpr int SLOT = 2 * RB > 4096 ? 2 * RB : 4096;
};

// LDS of the split kernel: the ring, the split's page ids, the item lookup
// and (QS) a query block of 256 * KH * HP bytes per wave.  The query gets
// its own block when three work-groups per compute unit still fit (1 KB per
// work-group kept for allocation granularity); otherwise it passes through
// the ring's last slot before that slot's first item is requested.
template <int NG, int HP, int KH, int WH, int D, int KM>
struct DecodeLds {
  using G = PairGeom<NG, KH, KM>;
  static constexpr int BASE = WH * D * G::SLOT + 4 * kMaxWgPages + 64;
  static constexpr int QB = 256 * KH * HP;
  static constexpr bool QS = 3 * (BASE + WH * QB + 1024) <= 160 * 1024;
};

// s_waitcnt vmcnt for na loads groups in flight of which w are window halves
// (WL loads each) and na - w page pairs (PL loads each), 0 <= w <= na < D.
template <int WL, int PL, int NA, int W>
__device__ __forceinline__ void vm_wait_n() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(W * WL + (NA - W) * PL) : "memory");
}
template <int D, int WL, int PL>
__device__ __forceinline__ void wait_loads(int na, int w) {
  static_assert(D >= 2 && D <= 4, "ring depth");
  if (na == 0) return vm_wait_n<WL, PL, 0, 0>();
  if (na == 1) return w ? vm_wait_n<WL, PL, 1, 1>() : vm_wait_n<WL, PL, 1, 0>();
  if constexpr (D >= 3) {
    if (na == 2) {
      if (w == 2) return vm_wait_n<WL, PL, 2, 2>();
      return w ? vm_wait_n<WL, PL, 2, 1>() : vm_wait_n<WL, PL, 2, 0>();
    }
  }
  if constexpr (D >= 4) {
    if (w == 3) return vm_wait_n<WL, PL, 3, 3>();
    if (w == 2) return vm_wait_n<WL, PL, 3, 2>();
    return w ? vm_wait_n<WL, PL, 3, 1>() : vm_wait_n<WL, PL, 3, 0>();
  }
  vm_wait_n<WL, PL, 0, 0>();   // (not reached)
}

// Work-group = one work item (sequence, context split, group of WH adjacent
// KV head groups, query-head pass); items are numbered sequence-major, then
// split, then head group, and the launch has exactly one work-group per
// item.  Wave w owns KV heads KH (WH group + w) ...; all waves walk the same
// blocks and pages.
//
// Everything a wave reads from the cache streams through a ring of D slots
// in LDS, one ring per wave, filled by direct-to-LDS loads (data in flight
// costs no registers): first the split's BF16 window blocks, each as two
// ring items per KV head of the wave (its 16 K rows, then its 16 V rows),
// then its INT2 page pairs (one item: the wave's KV heads' bytes of both
// pages).  Item j + D is requested as soon as item j has been read out of its
// slot into registers, so D items are in flight while one is processed.
// Each item is waited for with an exact vmcnt: the loads of the items after
// it (up to j + D - 1 and the last item) are counted from their types (a
// window half is 4 loads, a pair 2 NI), and no other vector memory access of
// the wave is outstanding meanwhile.
template <int NG, int HP, int KH, int WH, int D, int KM, int PS>
__global__ __launch_bounds__(64 * WH) void int2_decode_kernel(CacheArgs c, SeqArgs s, int quota,
                                                              int passes, int smax, int cus, ItemOrder order,
                                                              const uint16_t* __restrict__ q_rot,
                                                              float* __restrict__ partials) {
  using G = PairGeom<NG, KH, KM>;
  static_assert(KM == 0 || (NG == 4 && KH == 1), "OScaR keys: G = 32 values, one KV head per wave");
  constexpr int PW = rec_words(HP);   // floats per partial record
  constexpr int NT = 64 * WH;
  static_assert(D >= 2 && D <= 4, "ring depth");
  static_assert((D - 1) * G::PAIR_LOADS <= 63, "vmcnt limit");
  __shared__ __align__(16) uint8_t s_ring[WH * D * G::SLOT];
  __shared__ __align__(8) int s_pages[kMaxWgPages];
  using L = DecodeLds<NG, HP, KH, WH, D, KM>;
  __shared__ __align__(16) uint8_t s_qblk[L::QS ? WH * L::QB : 16];
  __shared__ int s_wsum[WH];
  __shared__ int s_item[4];   // sequence, item within it, its slot and length

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, qd = lane >> 4;
  // PS = 0: the WH waves take WH groups of KH adjacent KV heads, all walking
  // the split's blocks and pages; PS = 1 (small batches): the waves share one
  // group of KH heads and divide the split's pairs and window blocks, then
  // combine their softmax states (fewer, larger work-groups' worth of
  // records; three work-groups per compute unit even for one sequence)
  const int rows = (PS ? c.hkv / KH : c.hkv / (WH * KH)) * passes;

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
  const int hw = (PS ? hgrp : hgrp * WH + wave) * KH;   // first KV head of this wave

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
  const int b0 = cnt > 0 ? (ring_lo - c.s_sink) % c.ring_cap : 0;
  const int rb_n = ring_blocks_live(len, ring_lo, c.s_sink, c.ring_cap);
  const int n_wu = sb_n + rb_n;
  const int n_split = decode_splits(DecodeWork{n_pairs, n_wu}, quota, smax);
  // (products stay below 2^31 within the config limits)
  const int pb = (int)((unsigned)(split * n_pairs) / (unsigned)n_split);
  const int pe = (int)((unsigned)((split + 1) * n_pairs) / (unsigned)n_split);
  const int wb = (int)((unsigned)(split * n_wu) / (unsigned)n_split);
  const int we = (int)((unsigned)((split + 1) * n_wu) / (unsigned)n_split);
  const int total_units = max(1, (pe - pb) + kWinCost * (we - wb));
  const PrioSteps prio = prio_steps(total_units, blockIdx.x / cus);   // (dispatch round on its CU)
  set_priority(prio, total_units);
  // window block u: sink block u, then the live ring blocks from the one
  // holding the oldest live row (b0), in ring order
  auto ring_blk = [&](int u) { return (b0 / kPage + (u - sb_n)) % (c.ring_cap / kPage); };
  auto win_block = [&](int u) { return u < sb_n ? u : c.sink_blocks + ring_blk(u); };
  auto win_slot_ok = [&](int u, int t) {
    if (u < sb_n) return kPage * u + t < nsink;
    const int off = (kPage * ring_blk(u) + t - b0 + c.ring_cap) % c.ring_cap;
    return off < cnt;
  };
  // ---- per-lane MFMA column n = (group gi, KV head kh of the wave, head hl of the pass)
  const int n = r16, gi = n / (KH * HP), kh = (n / HP) % KH, hl = n % HP;
  const int h = hw + kh;                                          // this column's KV head
  const bool colv = (gi < NG) && (hl < nh);
  const int grp_q = (NG == 1) ? 0 : (NG == 2 ? (qd >> 1) : qd);   // group of channels 32qd..32qd+31
  const bool bval = colv && (gi == grp_q);
  const float C2 = kLog2e * 0.08838834764831845f;                // log2(e) / sqrt(128)
  const float K1 = C2 * 16777216.0f;                              // undo the 2^-24 code scaling

  // ---- the ring of this wave.  Its address is passed through an empty asm
  // statement: the compiler then cannot assume anything about the ring's
  // contents, which only the direct-to-LDS loads write.
  lds_u8* ring = (lds_u8*)(s_ring + wave * (D * G::SLOT));
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+s"(ring)::"memory");   // (an SGPR operand: device code only)
#endif
  // this wave's pairs k (split pair pair_of(k)) and window blocks (win_u)
  const int sp_pairs = min(pe - pb, kMaxPairsPerSplit);           // pairs of this split
  const int np = PS ? (sp_pairs > wave ? (sp_pairs - wave + WH - 1) / WH : 0) : sp_pairs;
  const int nwb = PS ? (we - wb > wave ? (we - wb - wave + WH - 1) / WH : 0) : we - wb;
  const int nwin = 2 * nwb * KH;                                  // window items (K, V halves)
  auto pair_of = [&](int k) { return PS ? wave + WH * k : k; };
  auto win_u = [&](int tt) { return PS ? wb + wave + WH * (tt / KH) : wb + tt / KH; };
  const int n_items = nwin + np;
  const size_t page_stride = (size_t)c.hkv * G::PB;
  const uint8_t* wave_base = c.pages + (size_t)hw * G::PB;        // the wave's first head of page 0
  const uint8_t* win_base = (const uint8_t*)(c.win + ((size_t)(row_ok ? slot : 0) * c.hkv + hw) *
                                                         c.win_blocks * (2 * kPage * kD));
  // page ids of pair k (the split's last pair for k >= np); -1: unmapped
  auto pair_ids = [&](int k) {
    return *(const u32x2*)&s_pages[2 * pair_of(max(0, min(k, np - 1)))];
  };
  // Window half placement in LDS: 16-byte chunk (t, j) of a half (row t, bytes
  // 16 j .. 16 j + 15 of its 256) sits at chunk 16 t + (j ^ t), so the 16
  // lanes that read one column of chunks hit 16 different bank groups.  Load
  // m of a half writes LDS chunks 64 m + lane, i.e. row t = 4 m + lane / 16;
  // woff[m] is where that lane's (swizzled) chunk of row t lies in the half.
  uint32_t woff[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint32_t jj = lane & 15, t0 = lane >> 4;
    woff[m] = 256 * t0 + 16 * (jj ^ (t0 + 4 * m));
  }
  auto request_win = [&](int item, lds_u8* dst) {
    const int tt = item >> 1, half = item & 1;
    const int u = win_u(tt), k = tt % KH;
    const uint8_t* src = uniform_ptr(win_base + ((size_t)k * c.win_blocks + win_block(u)) *
                                                    (4 * kPage * kD) + half * (2 * kPage * kD));
    load_lds16<0>(src + woff[0], dst);
    load_lds16<1024>(src + woff[1], dst);
    load_lds16<2048>(src + woff[2], dst);
    load_lds16<3072>(src + woff[3], dst);
  };
  auto request_pair = [&](u32x2 ids, lds_u8* dst) {
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
      int ph = __builtin_amdgcn_readfirstlane((int)ids[pg]);
      if (ph < 0) ph = 0;   // unmapped: any valid page, its logits are masked
      const uint8_t* src = uniform_ptr(wave_base + (size_t)ph * page_stride) + (uint32_t)(16 * lane);
      lds_u8* d = dst + pg * G::RB;
      load_lds16<0>(src, d);
      if (G::NI > 2 || lane < G::LAST_LANES) load_lds16<1024>(src, d);
      if constexpr (G::NI > 2) {
        if (G::NI > 3 || lane < G::LAST_LANES) load_lds16<2048>(src, d);
      }
      if constexpr (G::NI > 3) {
        static_assert(G::NI == 4, "at most four loads per page");
        if (lane < G::LAST_LANES) load_lds16<3072>(src, d);
      }
    }
  };
  // request item j into slot j % D (nothing past the last item)
  auto request = [&](int j, u32x2 ids) {
    if (j >= n_items) return;
    lds_u8* dst = ring + (j % D) * G::SLOT;
    if (j < nwin) request_win(j, dst);
    else request_pair(ids, dst);
  };
  // wait until item j is in its slot: the items after it up to j + D - 1
  // that exist may still be loading (windows first, then pairs)
  auto wait_item = [&](int j) {
    const int last = min(j + D - 1, n_items - 1);
    const int na = max(0, last - j);                      // items in flight after j
    const int wins = max(0, min(last, nwin - 1) - j);     // window halves among them
    wait_loads<D, G::WIN_LOADS, G::PAIR_LOADS>(na, wins);
  };

  // ---- start-up, in this order (all direct-to-LDS): the split's page ids
  // (wave w: ids 64 w .. 64 w + 63), the query rows of the wave's columns
  // (into the wave's query block, or ring slot D - 1), the first window
  // items (into slots 0 .. D - 2 when the query uses slot D - 1); then, once
  // the ids and the query are in, the window item of slot D - 1 if it was
  // held back, the check of the ids, one barrier and the first pairs.
  // Nothing waits for window data before the barrier, and the ring requests
  // stay in item order.
  const int n_wg_pages = min(2 * (pe - pb), kMaxWgPages);
  const int id_lim = min(n_pages, c.max_pages) - 2 * pb;   // ids t < id_lim lie in the row, with INT2 tokens
  if (64 * wave < n_wg_pages) {
    const int t = 64 * wave + lane;
    if (t < id_lim && t < n_wg_pages)
      __builtin_amdgcn_global_load_lds(bt + 2 * pb + t, (lds_u8*)(s_pages + 64 * wave), 4, 0, 0);
    else if (t < n_wg_pages)
      s_pages[t] = -1;
  }
  // Query block: row kk * HP + hl = query head (hw + kk) g + pass HP + hl,
  // 256 bytes each; load m brings 16-byte chunks 64 m + lane.
  lds_u8* const qblk = L::QS ? (lds_u8*)(s_qblk + wave * L::QB) : ring + (D - 1) * G::SLOT;
  {
    lds_u8* qdst = qblk;
    constexpr int QR = KH * HP;
    static_assert(256 * QR <= G::SLOT, "the query block fits a ring slot");
#pragma unroll
    for (int m = 0; m < (QR + 3) / 4; ++m) {
      const int x = 64 * m + lane, r = x >> 4;
      const int kk = r / HP, hq_l = r % HP;
      if (r < QR && hq_l < nh) {
        const uint8_t* src = (const uint8_t*)(q_rot + ((size_t)i * c.hq + (size_t)(hw + kk) * c.g +
                                                        (size_t)pass * HP + hq_l) * kD) + 16 * (x & 15);
        load_lds16<0>(src, qdst + 1024 * m);
      }
    }
  }
  // items that need no page id: the windows
  const int d_win = np == 0 ? D : min(D, nwin);
  const int d_a = L::QS ? d_win : min(d_win, D - 1);   // requested before the query is read
  if (n_items > 0) {
#pragma unroll
    for (int d = 0; d < D; ++d)
      if (d < d_a) request(d, u32x2{0u, 0u});
  }
  // wait for the ids and the query: only the d_a window items (4 loads each) are younger
  {
    const int after = min(d_a, n_items);
    if (after == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if (after == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(G::WIN_LOADS) : "memory");
    else if (after == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * G::WIN_LOADS) : "memory");
    else if (after == 3) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * G::WIN_LOADS) : "memory");
    else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * G::WIN_LOADS) : "memory");
  }
  u32x4 wq[4];
  {
    const lds_u8* qrow = qblk + 256 * (kh * HP + hl) + 64 * qd;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const u32x4 v = *(lds_u32x4*)(qrow + 16 * cc);
      wq[cc] = colv ? v : z;
    }
  }
  u32x4 wqo = {0u, 0u, 0u, 0u};   // OScaR keys: channels 32 gi + 8 qd .. + 7 of the column's head
  if constexpr (KM) {
    const u32x4 v = *(lds_u32x4*)(qblk + 256 * (kh * HP + hl) + 2 * (32 * (gi < NG ? gi : 0) + 8 * qd));
    if (colv) wqo = v;
  }
  // slot D - 1 is free once the query is in registers
  if constexpr (!L::QS) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (n_items > 0 && d_win == D) request(D - 1, u32x2{0u, 0u});
  }

  // check the wave's ids in place (-1: unmapped); longer splits load the
  // rest here
  int bad_ids = 0;   // a page holding INT2 tokens without a valid page id
  auto check_ids = [&](int t) {
    if (t < n_wg_pages) {
      int ph = s_pages[t];
      const bool ok = t < id_lim && ph >= 0 && ph < c.num_pages;
      if (!ok) s_pages[t] = -1;
      bad_ids |= (!ok && t < n_pages - 2 * pb);
    }
  };
  check_ids(64 * wave + lane);
  for (int t = 64 * (wave + WH) + lane; t - lane < n_wg_pages; t += 64 * WH) {   // long splits
    if (t < n_wg_pages) s_pages[t] = t < id_lim ? bt[2 * pb + t] : -1;
    check_ids(t);
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
  // OScaR keys: q . k_hat = s_t (sum_j q_j Delta_j c_tj - C), C = sum_j q_j o_j
  // with o_j = Delta_j z_j (-z_j for a constant channel), per key block.  The
  // query enters the MFMA scaled by 2^sh (wave-uniform), chosen so that
  // |q| 2^sh < 2^14: q 2^sh 4^-v Delta stays in the fp16 normal range.  qo:
  // this lane's column's query at channels 32 gi + 8 qd .. + 7, times
  // 2^(sh - 24), for its share of C.
  int sh = 0;
  float qo[KM ? 8 : 1];
  if constexpr (KM) {
    uint32_t m = 0;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
#pragma unroll
      for (int e = 0; e < 4; ++e) m = max(m, max(wq[cc][e] & 0x7FFFu, (wq[cc][e] >> 16) & 0x7FFFu));
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, d));
    sh = min(100, max(-100, 13 - ((int)(m >> 7) - 127)));
    sh = __builtin_amdgcn_readfirstlane(sh);
    const float f = __builtin_ldexpf(1.0f, sh - 24);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qo[2 * e] = bf16_bits_to_f32(wqo[e] & 0xFFFFu) * f;
      qo[2 * e + 1] = bf16_bits_to_f32(wqo[e] >> 16) * f;
    }
  }

  // page ids visible; ids_ok: every page of the split's pairs with INT2
  // tokens is mapped, so only the last pairs (past S_quant) need masks.  The
  // barrier carries no memory fence (a fence would wait for the window loads
  // in flight): the ids' loads were waited for with the query, and the LDS
  // writes of this wave complete with lgkmcnt(0).
  const bool wbad = __any(bad_ids);
  if (lane == 0) s_wsum[wave] = wbad ? 1 : 0;   // (free: the item lookup is done)
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  int any_bad = 0;
#pragma unroll
  for (int w = 0; w < WH; ++w) any_bad |= s_wsum[w];
  const bool ids_ok = !any_bad;

  if (n_items > 0) {
#pragma unroll
    for (int d = 0; d < D; ++d)
      if (d >= d_win) request(d, pair_ids(d - nwin));
  }

  // ---- B operands: the bf16 query for the window blocks, and for the INT2
  // codes q' scaled by 4^-v (chunk cc, K index 8 qd + 2v + e <-> channel
  // 32 qd + 16 (cc/2) + 4 (cc%2) + v + 8 e), zero outside the column's group
  bf16x8 bw[4];
  half8 bq[4];
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) {
    bw[cc] = __builtin_bit_cast(bf16x8, wq[cc]);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int cl = 16 * (cc >> 1) + 4 * (cc & 1) + v + 8 * e;
        const uint32_t word = wq[cl >> 3][(cl & 7) >> 1];
        const uint32_t bits = (cl & 1) ? (word >> 16) : (word & 0xFFFFu);
        // (OScaR keys have no channel groups: every column takes all 128
        // channels of its head, so no group partials need adding up)
        const float qv = (KM ? colv : bval) ? bf16_bits_to_f32(bits) : 0.0f;
        bq[cc][2 * v + e] = (_Float16)(KM ? qv * __builtin_ldexpf(1.0f, sh - 2 * v)
                                          : qv * (1.0f / (float)(1 << (2 * v))));
      }
    }
  }
  const int gsel = gi < NG ? gi : 0;                              // in-bounds group for params

  float4_t acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = float4_t{0.f, 0.f, 0.f, 0.f};
  SoftmaxState st{kNegInf, 0.0f, 0.0f, 0.0f};

  const int koff = (r16 * 8 + 2 * qd) * 4;                        // K codes of this lane
  const int poff = 1024 + 4 * (16 * gsel + 4 * qd);               // K params of this lane's column
  const int vpoff = (KM ? 1024 : 1024 + 64 * NG) + 4 * (16 * gsel + 4 * qd);   // V params
  const float K1o = KM ? C2 * __builtin_ldexpf(1.0f, 24 - sh) : K1;   // log2 logit per raw unit

  // ---- BF16 window blocks (true scale), each KV head of the wave in turn
  // K half: lane (r16, qd) reads row r16, channels 32 qd + 8 cc .. + 7, i.e.
  // chunk (r16, 4 qd + cc); V half: the bf16 P.V operand order of the window
  // layout, chunk (lane / 4 .. , ...): lane (r16, qd) reads chunks
  // 4 (16 qd + r16) + cc, i.e. row t = (16 qd + r16) / 4, j = 4 ((16 qd + r16) % 4) + cc.
  short4_t win_phi = {0, 0, 0, 0}, win_plo = {0, 0, 0, 0};
  for (int it_w = 0; it_w < nwin; ++it_w) {
    const int tt = it_w >> 1, half = it_w & 1;
    const int u = win_u(tt), k = tt % KH;
    set_priority(prio, kWinCost * (we - u) + np);
    wait_item(it_w);
    const lds_u8* P = ring + (it_w % D) * G::SLOT;
    u32x4 rv[4];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      int t, j;
      if (half == 0) {
        t = r16;
        j = 4 * qd + cc;
      } else {
        const int a = 16 * qd + r16;
        t = a >> 2;
        j = 4 * (a & 3) + cc;
      }
      rv[cc] = *(lds_u32x4*)(P + 16 * (16 * t + (j ^ t)));
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    request(it_w + D, pair_ids(it_w + D - nwin));
    const bool live = __any(win_slot_ok(u, r16));   // uniform
    if (!live) continue;
    if (half == 0) {
      float4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cc = 0; cc < 4; ++cc)
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, rv[cc]), bw[cc], d,
                                                    0, 0, 0);
      float x[4], p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)   // only the columns of the block's KV head
        x[r] = ((KH == 1 || kh == k) && win_slot_ok(u, 4 * qd + r)) ? d[r] : kNegInf;
      softmax_step<4>(x, C2, p, st, acc);
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        hi[r] = f32_to_bf16_rne(p[r]);
        lo[r] = f32_to_bf16_rne(p[r] - __uint_as_float(hi[r] << 16));
      }
      win_phi = short4_t{(short)hi[0], (short)hi[1], (short)hi[2], (short)hi[3]};
      win_plo = short4_t{(short)lo[0], (short)lo[1], (short)lo[2], (short)lo[3]};
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const u32x4 src = rv[j >> 1];
        const u32x2 pr = (j & 1) ? u32x2{src[2], src[3]} : u32x2{src[0], src[1]};
        const short4_t a = __builtin_bit_cast(short4_t, pr);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, win_phi, acc[j], 0, 0, 0);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, win_plo, acc[j], 0, 0, 0);
      }
    }
  }

  // q.k of one page (16 tokens) for the wave's KV heads: each head's codes
  // against the same query operand; each column keeps the sum of its head
  auto qk_page = [&](const u32x2 (&kw)[KH]) {
    float4_t sel = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KH; ++k) {
      float4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        uint32_t w = (cc < 2) ? kw[k][0] : kw[k][1];
        if (cc & 1) w >>= 8;
        const u32x4 v = {w & 0x00030003u, w & 0x000C000Cu, w & 0x00300030u, w & 0x00C000C0u};
        d = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, v), bq[cc], d, 0, 0, 0);
      }
      if (KH == 1 || kh == k) sel = d;
    }
    return sel;
  };

  // ---- INT2 page pairs: accumulate in code units (code * 4^(j%4) * 2^-24);
  // the window sums are moved to those units and back (powers of two, exact)
  if (np > 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= (float)(1 << (2 * (j & 3))) * (1.0f / 16777216.0f);
  }
  // page ids of the pair requested next, read from LDS one iteration ahead
  // so that no LDS round trip lies between the wait for a slot and the
  // request that refills it
  u32x2 nxt = pair_ids(D);
  for (int k = 0; k < np; ++k) {
    const int item = nwin + k;
    const u32x2 req = nxt;
    nxt = pair_ids(k + D + 1);
    set_priority(prio, np - k);
    wait_item(item);
    const lds_u8* P = ring + (item % D) * G::SLOT;
    u32x2 ka[KH], kb[KH], va[KH], vb[KH];
#pragma unroll
    for (int kk = 0; kk < KH; ++kk) {
      ka[kk] = *(lds_u32x2*)(P + kk * G::PB + koff);
      kb[kk] = *(lds_u32x2*)(P + G::RB + kk * G::PB + koff);
      va[kk] = *(lds_u32x2*)(P + kk * G::PB + 512 + 8 * lane);
      vb[kk] = *(lds_u32x2*)(P + G::RB + kk * G::PB + 512 + 8 * lane);
    }
    const u32x4 vpa = *(lds_u32x4*)(P + kh * G::PB + vpoff);
    const u32x4 vpb = *(lds_u32x4*)(P + G::RB + kh * G::PB + vpoff);
    // sum the group partials: lanes n, n +- KH HP, ... of a 16-lane row
    auto group_sum = [&](float (&y)[8]) {
      if constexpr (NG > 1) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          if constexpr (KH * HP <= 8) y[t] += row_ror<8>(y[t]);
          if constexpr (KH * HP <= 4) y[t] += row_ror<4>(y[t]);
          if constexpr (KH * HP <= 2) y[t] += row_ror<2>(y[t]);
          if constexpr (KH * HP <= 1) y[t] += row_ror<1>(y[t]);
        }
      }
    };
    float x[8];
    if constexpr (!KM) {
      const u32x4 kpa = *(lds_u32x4*)(P + kh * G::PB + poff);
      const u32x4 kpb = *(lds_u32x4*)(P + G::RB + kh * G::PB + poff);
      // the slot is free again once its contents are in registers
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      request(item + D, req);
      const float4_t da = qk_page(ka);
      const float4_t db = qk_page(kb);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x[r] = __builtin_fmaf(f16lo(kpa[r]), da[r], f16hi_mul(kpa[r], qz));
        x[4 + r] = __builtin_fmaf(f16lo(kpb[r]), db[r], f16hi_mul(kpb[r], qz));
      }
      group_sum(x);
    } else {
      // OScaR key block = this pair.  B operand per chunk: q 2^sh 4^-v times
      // the channel's Delta, as fp16 hi + lo (the 16-bit product, exactly
      // up to fp16 range); the channels of the lane's group (32 qd ..) have
      // their (Delta, z) words in page qd / 2.
      const lds_u8* pbw = P + (qd >> 1) * G::RB + kOtsChanOffset + 4 * 32 * (qd & 1);
      float4_t da = {0.f, 0.f, 0.f, 0.f}, db = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const int base = 16 * (cc >> 1) + 4 * (cc & 1);   // channel 32 qd + base + v + 8 e
        const u32x4 w0 = *(lds_u32x4*)(pbw + 4 * base);
        const u32x4 w1 = *(lds_u32x4*)(pbw + 4 * (base + 8));
        const u32x4 qb = __builtin_bit_cast(u32x4, bq[cc]);
        uint32_t hv[4], lv[4];
#pragma unroll
        for (int v = 0; v < 4; ++v)
          mul_f16pair_split(qb[v], __uint_as_float(w0[v] << 16), __uint_as_float(w1[v] << 16), hv[v],
                            lv[v]);
        const u32x4 hi = {hv[0], hv[1], hv[2], hv[3]}, lo = {lv[0], lv[1], lv[2], lv[3]};
        uint32_t wa = (cc < 2) ? ka[0][0] : ka[0][1];
        uint32_t wb2 = (cc < 2) ? kb[0][0] : kb[0][1];
        if (cc & 1) {
          wa >>= 8;
          wb2 >>= 8;
        }
        const u32x4 ca = {wa & 0x00030003u, wa & 0x000C000Cu, wa & 0x00300030u, wa & 0x00C000C0u};
        const u32x4 cb = {wb2 & 0x00030003u, wb2 & 0x000C000Cu, wb2 & 0x00300030u, wb2 & 0x00C000C0u};
        const half8 h8 = __builtin_bit_cast(half8, hi), l8 = __builtin_bit_cast(half8, lo);
        da = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, ca), h8, da, 0, 0, 0);
        da = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, ca), l8, da, 0, 0, 0);
        db = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, cb), h8, db, 0, 0, 0);
        db = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, cb), l8, db, 0, 0, 0);
      }
      // this column group's share of C: channels 32 gi + 8 qd .. + 7, then
      // the four lanes of the column
      const lds_u8* pcw = P + (gsel >> 1) * G::RB + kOtsChanOffset + 4 * (32 * (gsel & 1) + 8 * qd);
      const u32x4 c0 = *(lds_u32x4*)pcw, c1 = *(lds_u32x4*)(pcw + 16);
      const u32x2 tsa = *(lds_u32x2*)(P + kOtsScaleOffset + 8 * qd);
      const u32x2 tsb = *(lds_u32x2*)(P + G::RB + kOtsScaleOffset + 8 * qd);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      request(item + D, req);
      float cp = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w = e < 4 ? c0[e] : c1[e - 4];
        const float dl = __uint_as_float(w << 16), z = __uint_as_float(w & 0xFFFF0000u);
        cp = __builtin_fmaf(qo[e], dl != 0.0f ? dl * z : -z, cp);
      }
      cp = rows_sum(cp);
      // C over all channels: the four group columns of the head add up
      if constexpr (KH * HP <= 8) cp += row_ror<8>(cp);
      if constexpr (KH * HP <= 4) cp += row_ror<4>(cp);
      if constexpr (KH * HP <= 2) cp += row_ror<2>(cp);
      if constexpr (KH * HP <= 1) cp += row_ror<1>(cp);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x[r] = da[r] - cp;
        x[4 + r] = db[r] - cp;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {   // token scales of rows 4 qd + r
        const uint32_t wa = tsa[r >> 1], wb3 = tsb[r >> 1];
        x[r] *= bf16_bits_to_f32((r & 1) ? wa >> 16 : wa & 0xFFFFu);
        x[4 + r] *= bf16_bits_to_f32((r & 1) ? wb3 >> 16 : wb3 & 0xFFFFu);
      }
    }
    const int tok = 32 * (pb + pair_of(k));   // INT2 token index of slot 0 of page A
    if (!(ids_ok && tok + 32 <= nq)) {   // slots past S_quant, or unmapped pages
      const u32x2 own = pair_ids(k);
      const bool oka = (int)own[0] >= 0, okb = (int)own[1] >= 0;
      const int ta = tok + 4 * qd;   // INT2 token index of row 0 of tile A in this lane
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (!(oka && ta + r < nq)) x[r] = kNegInf;
        if (!(okb && ta + 16 + r < nq)) x[4 + r] = kNegInf;
      }
    }
    // P' = p * scale_v enters the MFMA as fp16: with p <= 2^8 (the lazy
    // max) a value scale of 128 or more could overflow it, so such a pair
    // takes the exact max (p <= 1, P' <= scale <= 65504)
    const bool big_scale = max_scale_bits(vpa, vpb) >= 0x5800u;   // fp16 128.0
    float p[8];
    softmax_step<8>(x, K1o, p, st, acc, __any(big_scale) ? 0.0f : 8.0f);
    uint32_t ph[4], pl[4];
    mul_by_f16lo_split(p[0], vpa[0], p[1], vpa[1], ph[0], pl[0]);
    mul_by_f16lo_split(p[2], vpa[2], p[3], vpa[3], ph[1], pl[1]);
    mul_by_f16lo_split(p[4], vpb[0], p[5], vpb[1], ph[2], pl[2]);
    mul_by_f16lo_split(p[6], vpb[2], p[7], vpb[3], ph[3], pl[3]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      st.z = __builtin_fmaf(p[r], f16hi(vpa[r]), st.z);
      st.z = __builtin_fmaf(p[4 + r], f16hi(vpb[r]), st.z);
    }
#pragma unroll
    for (int kk = 0; kk < KH; ++kk) {
      // B operands of the P.V MFMAs on KV head kk: this column's P' if it belongs to head kk
      const bool mine = KH == 1 || kh == kk;
      const half8 pv = __builtin_bit_cast(half8, mine ? u32x4{ph[0], ph[1], ph[2], ph[3]} : u32x4{});
      const half8 pvl = __builtin_bit_cast(half8, mine ? u32x4{pl[0], pl[1], pl[2], pl[3]} : u32x4{});
      const uint32_t w0 = va[kk][0], w1 = va[kk][1], w2 = vb[kk][0], w3 = vb[kk][1];
      const uint32_t s0 = w0 >> 8, s1 = w1 >> 8, s2 = w2 >> 8, s3 = w3 >> 8;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t mask = 0x00030003u << (2 * (j & 3));
        const half8 a = (j < 4) ? codes_as_half8(w0, w1, w2, w3, mask)
                                : codes_as_half8(s0, s1, s2, s3, mask);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pv, acc[j], 0, 0, 0);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pvl, acc[j], 0, 0, 0);
      }
    }
  }
  if (np > 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= 16777216.0f / (float)(1 << (2 * (j & 3)));
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- this wave's partial record: (max, sum, unnormalized o') per head of the pass
  st.l = rows_sum(st.l);
  st.z = rows_sum(st.z);
  if constexpr (PS && WH > 1) {
    // the waves hold partial states of the same columns: rescale each to the
    // common maximum and add them up in wave 0, through the idle ring's LDS
    // ([WH][16] maxima, then waves 1.. : 32 accumulator values, l and z per lane)
    float* sm = (float*)s_ring;
    float* sb = sm + WH * 16;
    static_assert((WH * 16 + (WH - 1) * 64 * 34) * 4 <= WH * D * G::SLOT, "combine space");
    __syncthreads();   // every wave's ring is idle (each has waited for all its loads)
    if (qd == 0) sm[wave * 16 + r16] = st.m;
    __syncthreads();
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < WH; ++w) M = fmaxf(M, sm[w * 16 + r16]);
    const float sc = st.m == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(st.m - M);
    if (wave > 0) {
      float* dst = sb + ((wave - 1) * 64 + lane) * 34;
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[4 * j + r] = acc[j][r] * sc;
      dst[32] = st.l * sc;
      dst[33] = st.z * sc;
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= sc;
    st.l *= sc;
    st.z *= sc;
#pragma unroll
    for (int w = 1; w < WH; ++w) {
      const float* src = sb + ((w - 1) * 64 + lane) * 34;
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[j][r] += src[4 * j + r];
      st.l += src[32];
      st.z += src[33];
    }
    st.m = M;
  }
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

// Calls f.template run<WH, D>() for the plan's waves per work-group; the
// ring has two slots, three in OScaR key mode (its pair loop frees a slot
// only after the key dot products, which read the block's channel
// parameters from the slot).
template <int KM, class F>
static auto with_waves_ring(int wh, F&& f) {
  constexpr int D = KM ? 3 : 2;
  if (wh == 4) return f.template run<4, D>();
  if (wh == 2) return f.template run<2, D>();
  return f.template run<1, D>();
}

template <int NG, int HP, int KH, int KM, int PS>
struct SplitLaunch {
  const CacheArgs& c;
  const SeqArgs& s;
  const DecodePlan& plan;
  const uint16_t* q_rot;
  float* partials;
  hipStream_t stream;
  template <int WH, int D>
  hipError_t run() const {
    hipLaunchKernelGGL((int2_decode_kernel<NG, HP, KH, WH, D, KM, PS>), dim3(plan.grid), dim3(64 * WH), 0,
                       stream, c, s, plan.quota, plan.passes, plan.smax, plan.cus, *plan.order, q_rot,
                       partials);
    return hipGetLastError();
  }
};

template <int NG, int HP, int KH, int KM, int PS>
struct SplitOccupancy {
  template <int WH, int D>
  int run() const {
    int nb = 0;
    auto* kernel = &int2_decode_kernel<NG, HP, KH, WH, D, KM, PS>;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, 64 * WH, 0);
    return e == hipSuccess && nb > 0 ? nb : 1;
  }
};

template <int NG, int HP, int KH, int KM>
static hipError_t launch_decode_t(const CacheArgs& c, const SeqArgs& s, const DecodePlan& plan,
                                  const uint16_t* q_rot, float* out, float* partials,
                                  int phases, hipStream_t stream) {
  if (phases & kDecodeSplit) {
    const hipError_t e =
        plan.ps ? with_waves_ring<KM>(plan.wh, SplitLaunch<NG, HP, KH, KM, 1>{c, s, plan, q_rot, partials, stream})
                : with_waves_ring<KM>(plan.wh, SplitLaunch<NG, HP, KH, KM, 0>{c, s, plan, q_rot, partials, stream});
    if (e != hipSuccess) return e;
  }
  if (phases & kDecodeMerge)
    return c.unrot ? launch_merge<HP, true>(c, s, plan, partials, out, stream)
                   : launch_merge<HP, false>(c, s, plan, partials, out, stream);
  return hipSuccess;
}

template <int NG, int HP, int KH, int KM>
static int wgs_per_cu_t(int wh, int ps) {
  return ps ? with_waves_ring<KM>(wh, SplitOccupancy<NG, HP, KH, KM, 1>{})
            : with_waves_ring<KM>(wh, SplitOccupancy<NG, HP, KH, KM, 0>{});
}

// The (groups, heads per pass, KV heads per wave, key mode) shapes the
// planner uses: one group: any power-of-two pass, two KV heads per wave up
// to 8 heads; with ng groups the columns (group, KV head, head) fill the
// tile exactly; OScaR keys: G = 32, one KV head per wave, 4 heads per pass.
template <class F>
static auto with_shape(int ng, int hp, int kh, int km, F&& f) {
  if (km) {
    if (ng == 4 && kh == 1 && hp == 4) return f.template operator()<4, 4, 1, 1>();
    return f.fail();
  }
  if (ng == 1) {
    if (kh == 2) {
      switch (hp) {
        case 1: return f.template operator()<1, 1, 2, 0>();
        case 2: return f.template operator()<1, 2, 2, 0>();
        case 4: return f.template operator()<1, 4, 2, 0>();
        case 8: return f.template operator()<1, 8, 2, 0>();
      }
    } else {
      switch (hp) {
        case 1: return f.template operator()<1, 1, 1, 0>();
        case 2: return f.template operator()<1, 2, 1, 0>();
        case 4: return f.template operator()<1, 4, 1, 0>();
        case 8: return f.template operator()<1, 8, 1, 0>();
        case 16: return f.template operator()<1, 16, 1, 0>();
      }
    }
  } else if (ng == 2) {
    if (kh == 2 && hp == 4) return f.template operator()<2, 4, 2, 0>();
    if (kh == 1 && hp == 8) return f.template operator()<2, 8, 1, 0>();
  } else if (ng == 4) {
    if (kh == 2 && hp == 2) return f.template operator()<4, 2, 2, 0>();
    if (kh == 1 && hp == 4) return f.template operator()<4, 4, 1, 0>();
  }
  return f.fail();
}

struct OccupancyQuery {
  const DecodePlan& plan;
  template <int NG, int HP, int KH, int KM>
  int operator()() const { return wgs_per_cu_t<NG, HP, KH, KM>(plan.wh, plan.ps); }
  int fail() const { return 1; }
};

int decode_wgs_per_cu(const CacheArgs& c, const DecodePlan& plan) {
  return with_shape(c.ng, plan.hp, plan.kh, c.key_mode, OccupancyQuery{plan});
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
  template <int NG, int HP, int KH, int KM>
  hipError_t operator()() const {
    return launch_decode_t<NG, HP, KH, KM>(c, s, plan, q_rot, out, partials, phases, stream);
  }
  hipError_t fail() const { return hipErrorInvalidValue; }
};

hipError_t launch_decode(const CacheArgs& c, const SeqArgs& s, const DecodePlan& plan,
                         const uint16_t* q_rot, float* out, float* partials, int phases,
                         hipStream_t stream) {
  if (s.n_seqs <= 0 || plan.grid <= 0) return hipSuccess;
  return with_shape(c.ng, plan.hp, plan.kh, c.key_mode,
                    DecodeLaunch{c, s, plan, q_rot, out, partials, phases, stream});
}

}  // namespace oscar
