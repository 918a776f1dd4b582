// Chunked-prefill attention over the mixed INT2 / BF16 paged cache (gfx950).
//
// What is computed (WUSH-KV notes, "method step details", inference
// (Algorithm 2): new keys and queries of a chunk are transformed, the chunk
// joins the cache at full precision and grouped-query attention runs over the
// mixed-precision cache; OSCAR summary page, section 2 "Attention and KV
// cache": row-wise softmax(Q K^T / sqrt(d)) V):
//   the query at chunk row j of a sequence (position P = len_before + j)
//   attends to positions 0 .. P: positions below len_before as the cache holds
//   them after the chunk's append (bf16 sink / recent rows, INT2 rows as
//   scale * code + zero), the chunk's own rows at their bf16 rotated values
//   (the append's k_rot / v_rot outputs), then o = o' . R_V^T.
//
// Work-group = (sequence, tile of 16 W query rows, KV head), W = 8 waves, or
// 16 when the chunks attend mostly to a cached prefix (each staged key block
// then serves more rows); query row r of a (sequence, KV head) is (chunk
// row r / g, head r % g), and wave w owns rows 16w .. 16w+15 as the 16
// columns of its MFMA tiles.  The key stream is
// staged 64 positions per barrier, processed in 32-position steps; the
// work-group stages the keys in LDS as fp16
// (K rows [token][channel] as fp16 hi + lo, V transposed [row][token] with
// row 16 j + u holding channel 8 u + j),
// decoding every
// position from wherever it lives (sink, INT2 page, ring, chunk rows), one
// block ahead in registers.  Per block and wave:
//   S^T = K . Q^T   v_mfma_f32_16x16x32_f16, A = keys (hi, then lo), B = the
//                   wave's query rows (fp16 from bf16, exact in the normal range)
//   online softmax per column (query row) over 32 keys, causal mask p <= P
//   O^T += V^T . P^T  v_mfma_f32_16x16x32_f16 with P split into fp16 hi + lo
// then the normalized o' rows go through LDS (reusing the staging space) and
// the bf16 matrix cores apply R_V^T as hi + lo products (wave w computes output channels
// 16 (w % 8) .. 16 (w % 8) + 15 of its share of the rows).
#include "decode_common.h"

namespace oscar {

namespace {

// Work-group shape: W waves of 16 RB query rows each (RB blocks of 16, the
// columns of RB MFMA tiles that share every key and value operand read from
// LDS).  Staging: 512 threads, thread (token pair tp, channel octet u) takes
// positions 2 tp, 2 tp + 1 of a 64-position stage, channels 8 u .. 8 u + 7.
template <int W, int RB = 1>
struct PfShape {
  static constexpr int kWaves = W;
  static constexpr int kThreads = 64 * W;
  static constexpr int kRows = 16 * W * RB;        // query rows per work-group
  static constexpr int kStage = 64;                // key positions staged per barrier
  static constexpr int kStageThreads = 512;        // (kStage / 2) pairs x 16 octets
  static constexpr int kKRow = kD + 8;   // staged key row in fp16 (padded: rows start 4 banks apart)
  static constexpr int kVRow = kStage + 4;   // staged value row (one channel), 34 dwords: the
                                             // 16 rows one instruction writes start on distinct banks
  // bf16 mode: value rows of 72 (16-byte aligned, 16 rows on distinct bank
  // quads), each 32-key group ordered so that a lane's 8 keys of a P.V
  // step (4 qd .. 4 qd + 3, 16 + 4 qd .. 16 + 4 qd + 3) are adjacent
  static constexpr int kVRowBF = kStage + 8;
  static_assert(kThreads >= kStageThreads, "a stage is 64 positions");
};

// LDS: the staging buffers during the key loop, the normalized o' rows after it.
template <int W>
struct PfStage {
  using S = PfShape<W>;
  _Float16 k[S::kStage][S::kKRow];    // keys [token][channel], fp16 part
  _Float16 kl[S::kStage][S::kKRow];   // remainders k - fp16(k)
  _Float16 vt[kD][S::kVRow];          // values [row][token], row 16 j + u = channel 8 u + j
  int skip[S::kStage];                // position unreadable (unmapped page or past the row)
};
// bf16 mode: two stage buffers (keys as bf16 bits, values transposed), so a
// stage is deposited while the previous one is read, one barrier per stage
template <int W>
struct PfStageBF {
  using S = PfShape<W>;
  _Float16 k[2][S::kStage][S::kKRow];
  _Float16 vt[2][kD][S::kVRowBF];
};
template <int W, int RB>
struct PfFinal {
  float o[PfShape<W, RB>::kRows][kD + 4];
};
template <int W, bool BF, int RB>
constexpr int pf_lds() {
  constexpr int st = BF ? (int)sizeof(PfStageBF<W>) : (int)sizeof(PfStage<W>);
  return st > (int)sizeof(PfFinal<W, RB>) ? st : (int)sizeof(PfFinal<W, RB>);
}

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_v __attribute__((ext_vector_type(2)));

// One position's K and V row slice (8 channels) as fetched from HBM, before
// decoding: kind 0 = zero row (past the end or an unmapped page), 1 = bf16
// words, 2 = INT2 code words with their scale / zero words.
struct RawSlice {
  u32x4 k, v;
  int kind;
};

__device__ __forceinline__ void bf16x2_to_f32(uint32_t w, float& lo, float& hi) {
  lo = __uint_as_float(w << 16);
  hi = __uint_as_float(w & 0xFFFF0000u);
}

// x as bf16 hi + lo: hi = RNE(x), lo = RNE(x - hi) (x - hi is exact in fp32)
__device__ __forceinline__ void split_bf16(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 b = (__bf16)x[e];
    hi[e] = b;
    lo[e] = (__bf16)(x[e] - (float)b);
  }
}

}  // namespace

// BF: no sequence of the launch has INT2 rows below its chunk, so every key
// and value is a bf16 row (sink, ring, the chunk itself): they are staged as
// their own bits and run on the bf16 matrix cores (exact keys and values,
// P as bf16 hi + lo).  Otherwise keys are staged as fp16 (hi + lo for the
// steps that hold INT2 rows) and values as fp16, on the fp16 matrix cores.
template <int W, bool BF, int RB>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(RB == 1 ? 4 : 2))) void prefill_attn_kernel(CacheArgs c, PrefillArgs a) {
  static_assert(RB == 1 || BF, "two row blocks per wave: bf16 mode");
  using S = PfShape<W, RB>;
  constexpr int kPfWaves = S::kWaves, kPfThreads = S::kThreads, kPfRows = S::kRows;
  constexpr int kStage = S::kStage;
  __shared__ __align__(16) char smem[pf_lds<W, BF, RB>()];
  PfStage<W>& sg = *reinterpret_cast<PfStage<W>*>(smem);
  PfStageBF<W>& sbf = *reinterpret_cast<PfStageBF<W>*>(smem);
  float(&fin)[kPfRows][kD + 4] = reinterpret_cast<PfFinal<W, RB>*>(smem)->o;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, qd = lane >> 4;
  // work-group b takes tile rank b / (sequences x KV heads): the tiles with
  // the longest causal ranges of every (sequence, KV head) first, the
  // shortest last, so the launch does not end on a long tile
  const int groups = a.n_seqs * c.hkv;
  const int b = (int)blockIdx.x, grp = b % groups;
  const int i = grp / c.hkv, h = grp % c.hkv;
  const int tile = a.tiles - 1 - b / groups;
  const int slot = a.slots[i], lb = a.len_before[i];
  const int t0 = a.cu_new[i], n_new = a.cu_new[i + 1] - t0;
  const int rows = n_new * c.g;
  if (slot < 0 || slot >= c.max_seqs || lb < 0 || n_new <= 0 || tile * kPfRows >= rows) return;
  const int len = lb + n_new;                                     // cache length after the append
  const int sq = s_quant_of(len, c.s_sink, c.s_keep, c.s_flush);  // INT2 below this position
  const int32_t* bt = c.block_table + (size_t)slot * c.max_pages;
  const uint16_t* wrow = c.win + ((size_t)slot * c.hkv + h) * c.win_blocks * (2 * kPage * kD);

  // ---- this lane's query rows (MFMA column r16 of each of the wave's RB
  // row blocks) and the keys the work-group reads
  const int wrow0 = tile * kPfRows + 16 * RB * wave;              // the wave's first row
  bool colv[RB];
  int qpos[RB];
  // (row / g and row % g by a magic multiplier: a plain division would keep
  // a reciprocal in a vector register through the key loop)
  auto div_g = [&](int x, uint32_t& rem) {
    return (int)div_by_magic((uint32_t)x, (uint32_t)c.g, a.g_magic, rem);
  };
  uint32_t rem_;
  const int wg_last = min(rows, (tile + 1) * kPfRows) - 1;
  const int kend = lb + div_g(wg_last, rem_) + 1;                 // keys [0, kend)
  const int w_last = min(rows, wrow0 + 16 * RB) - 1;
  const int wave_kend = w_last >= wrow0 ? lb + div_g(w_last, rem_) + 1 : 0;
  const int wave_qmin = lb + div_g(wrow0, rem_);                  // position of the wave's first row

  half8 bq[RB][4];     // the query in fp16 (exact in the normal range), for the INT2 steps
  bf16x8 bqb[RB][4];   // and its bf16 bits, for the steps over bf16 rows
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = wrow0 + 16 * rb + r16;
    colv[rb] = row < rows;
    uint32_t hl_u;
    const int pj_u = div_g(row, hl_u);
    const int pj = colv[rb] ? pj_u : 0, hl = colv[rb] ? (int)hl_u : 0;
    qpos[rb] = lb + pj;
    const uint16_t* qp = a.q_rot + ((size_t)(t0 + pj) * c.hq + (size_t)h * c.g + hl) * kD + 8 * qd;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const u32x4 w = colv[rb] ? *(const u32x4*)(qp + 32 * cc) : u32x4{0u, 0u, 0u, 0u};
      bqb[rb][cc] = __builtin_bit_cast(bf16x8, w);
      if constexpr (BF) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float lo, hi;
        bf16x2_to_f32(w[e], lo, hi);
        bq[rb][cc][2 * e] = (_Float16)lo;
        bq[rb][cc][2 * e + 1] = (_Float16)hi;
      }
    }
  }

  // fp16 staging: a 32-position step holding INT2 rows of the prefix
  // ([S_sink, int2_end)) also gets the keys' fp16 remainders (bf16 rows are
  // exact in fp16 alone)
  const int int2_end = min(sq, lb);
  auto step_int2 = [&](int p0) { return p0 + 2 * kPage > c.s_sink && p0 < int2_end; };

  // ---- staging: thread (token pair tp, channels 8u .. 8u+7) takes staged
  // rows 2 tp + m (m < 2) of a stage; threads from 512 on do not stage
  const bool stager = tid < S::kStageThreads;
  const int st_tp = tid >> 4, st_u = tid & 15;
  auto fetch = [&](int p0, int m, RawSlice& r) {
    const int p = p0 + 2 * st_tp + m;
    r.kind = 0;
    r.k = r.v = u32x4{0u, 0u, 0u, 0u};
    if (p >= len) return;
    if (p >= lb) {   // a row of this chunk: the append's bf16 rotated row
      const size_t o = ((size_t)(t0 + p - lb) * c.hkv + h) * kD + 8 * st_u;
      r.k = *(const u32x4*)(a.k_rot + o);
      r.v = *(const u32x4*)(a.v_rot + o);
      r.kind = 1;
    } else if (p < c.s_sink || p >= sq) {   // sink slot p, or ring slot (p - S_sink) mod R
      uint32_t rs;   // ring slot (p - S_sink) mod R
      div_by_magic((uint32_t)max(p - c.s_sink, 0), (uint32_t)c.ring_cap, a.ring_magic, rs);
      const int bs = p < c.s_sink ? p : c.sink_blocks * kPage + (int)rs;
      const uint16_t* blk = wrow + (size_t)(bs / kPage) * (2 * kPage * kD);
      const int tt = bs % kPage;
      r.k = *(const u32x4*)(blk + tt * kD + 8 * st_u);
      // V part: (token tt, channel 8u + j) at 32 (16 (tt / 4) + u) + 4 j + tt % 4
      const uint16_t* vb = blk + kPage * kD + 32 * (16 * (tt >> 2) + st_u) + (tt & 3);
      r.v = u32x4{(uint32_t)vb[0] | ((uint32_t)vb[4] << 16), (uint32_t)vb[8] | ((uint32_t)vb[12] << 16),
                  (uint32_t)vb[16] | ((uint32_t)vb[20] << 16), (uint32_t)vb[24] | ((uint32_t)vb[28] << 16)};
      r.kind = 1;
    } else {   // INT2: logical page (p - S_sink) / 16, slot (p - S_sink) % 16
      if constexpr (BF) return;   // (none below a bf16-mode chunk)
      const int m = (p - c.s_sink) / kPage, sl = (p - c.s_sink) % kPage;
      const int ph = m < c.max_pages ? bt[m] : -1;
      if (ph < 0 || ph >= c.num_pages) return;
      const uint32_t* pg = (const uint32_t*)(c.pages + ((size_t)ph * c.hkv + h) * c.page_bytes);
      const int gr = (st_u * c.ng) >> 4;   // group of channels 8u .. 8u + 7: 8u / G with G = 128 / ng
      r.k = u32x4{pg[8 * sl + (st_u >> 1)] >> (16 * (st_u & 1)), pg[256 + 16 * gr + sl], 0u, 0u};
      r.v = u32x4{pg[128 + 2 * (16 * (sl >> 2) + st_u) + ((sl & 3) >> 1)] >> (16 * (sl & 1)),
                  pg[256 + 16 * c.ng + 16 * gr + sl], 0u, 0u};
      r.kind = 2;
    }
  };
  // K rows as fp16 hi / lo of one position; returns its values as fp16
  auto deposit = [&](const RawSlice& r, int m, half8& vh) {
    const int row = 2 * st_tp + m;
    float kv[8], vv[8];
    if (st_u == 0) sg.skip[row] = r.kind == 0 ? 1 : 0;
    if (r.kind == 1) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bf16x2_to_f32(r.k[e], kv[2 * e], kv[2 * e + 1]);
        bf16x2_to_f32(r.v[e], vv[2 * e], vv[2 * e + 1]);
      }
    } else if (r.kind == 2) {
      // scale * code + zero: the product is exact, so fmaf rounds once
      const float ks = f16lo(r.k[1]), kz = f16hi(r.k[1]);
      const float vs = f16lo(r.v[1]), vz = f16hi(r.v[1]);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        kv[j] = __builtin_fmaf(ks, (float)((r.k[0] >> (2 * j)) & 3u), kz);
        vv[j] = __builtin_fmaf(vs, (float)((r.v[0] >> (2 * j)) & 3u), vz);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) kv[j] = vv[j] = 0.0f;
    }
    // keys as fp16 hi + lo (about 22 significant bits): a logit is sensitive
    // to the key's rounding; bf16 rows are exact in hi alone
    half8 kh, kl = {};
#pragma unroll
    for (int j = 0; j < 8; ++j) kh[j] = (_Float16)kv[j];
    if (r.kind == 2) {   // bf16 rows are exact in hi (up to fp16 subnormals)
#pragma unroll
      for (int j = 0; j < 8; ++j) kl[j] = (_Float16)(kv[j] - (float)kh[j]);
    }
    *(half8*)&sg.k[row][8 * st_u] = kh;
    *(half8*)&sg.kl[row][8 * st_u] = kl;
#pragma unroll
    for (int j = 0; j < 8; ++j) vh[j] = (_Float16)vv[j];
  };
  // both positions: the values go out as one 32-bit word (two tokens) per
  // channel, channel 8u + j to row 16 j + u
  auto deposit2 = [&](const RawSlice (&r)[2], int buf) {
    if constexpr (BF) {
      // the rows' own bits (kind 1) or zeros (kind 0: fetch leaves the
      // words zero; no kind 2 below a bf16-mode chunk)
      const u32x4 k0 = r[0].k, k1 = r[1].k, a0 = r[0].v, a1 = r[1].v;
      __builtin_memcpy(&sbf.k[buf][2 * st_tp][8 * st_u], &k0, 16);
      __builtin_memcpy(&sbf.k[buf][2 * st_tp + 1][8 * st_u], &k1, 16);
      // staged column of stage positions 2 tp, 2 tp + 1 (key kk of its
      // 32-key group goes to 8 ((kk % 16) / 4) + 4 (kk / 16) + kk % 4)
      const int kk = (2 * st_tp) & 31;
      const int vc = (2 * st_tp - kk) + 8 * ((kk & 15) >> 2) + 4 * (kk >> 4) + (kk & 3);
#pragma unroll
      for (int e = 0; e < 4; ++e) {   // channels 8u + 2e (low halves), 8u + 2e + 1 (high halves)
        const uint32_t wl = __builtin_amdgcn_perm(a1[e], a0[e], 0x05040100u);
        const uint32_t wh = __builtin_amdgcn_perm(a1[e], a0[e], 0x07060302u);
        __builtin_memcpy(&sbf.vt[buf][16 * (2 * e) + st_u][vc], &wl, 4);
        __builtin_memcpy(&sbf.vt[buf][16 * (2 * e + 1) + st_u][vc], &wh, 4);
      }
      return;
    }
    half8 v0, v1;
    deposit(r[0], 0, v0);
    deposit(r[1], 1, v1);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // (the vector elements go through locals: a bit cast of an element
      // of an ext_vector value compiles to element 0 for every j here)
      const _Float16 e0 = v0[j], e1 = v1[j];
      const uint32_t w = (uint32_t)__builtin_bit_cast(uint16_t, e0) |
                         ((uint32_t)__builtin_bit_cast(uint16_t, e1) << 16);
      __builtin_memcpy(&sg.vt[16 * j + st_u][2 * st_tp], &w, 4);   // (a byte copy: no type punning)
    }
  };

  float4_t acc[RB][8];
  SoftmaxState st[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[rb][j] = float4_t{0.f, 0.f, 0.f, 0.f};
    st[rb] = SoftmaxState{kNegInf, 0.0f, 0.0f, 0.0f};
  }
  const float C2 = kLog2e * 0.08838834764831845f;   // log2(e) / sqrt(128)

  // Unmapped INT2 pages are read as zero rows with zero weight (as in decode):
  // a per-stage mask of such positions, built by the staging threads.
  const int nstage = (kend + kStage - 1) / kStage;
  // the 64 positions of stage ks, from buffer buf (bf16 mode; else the one buffer)
  // mid() runs before the first step in every wave (bf16 mode: the staging
  // of later stages), whatever the wave's key range
  auto run_stage = [&](int ks, int buf, auto&& mid) {
    const int s0 = ks * kStage;
#pragma unroll
    for (int sb = 0; sb < kStage / (2 * kPage); ++sb) {
      // two 16-position blocks per softmax step: block b of the pair is
      // staged rows tb + 16 b; K slot 8 qd + 4 b + r of the 32-key P.V MFMA
      // is key 16 b + 4 qd + r, the lane's own softmax values
      const int p0 = s0 + 2 * kPage * sb, tb = 2 * kPage * sb;
      if (sb == 0) mid();
      if (p0 >= wave_kend) continue;
      float x[RB][8], p[RB][8];
      // fp16 mode: no unreadable row (unmapped page) among the step's 32
      bool clean = true;
      if constexpr (!BF) clean = !__any(sg.skip[tb + (lane & 31)]);
      // the whole step lies below every row of the wave: no causal mask
      const bool below = p0 + 2 * kPage - 1 <= wave_qmin;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        float4_t d[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) d[rb] = float4_t{0.f, 0.f, 0.f, 0.f};
        if constexpr (BF) {
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) {
            bf16x8 kb;
            __builtin_memcpy(&kb, &sbf.k[buf][tb + kPage * b + r16][32 * cc + 8 * qd], 16);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
              d[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, bqb[rb][cc], d[rb], 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int cc = 0; cc < 4; ++cc)
            d[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                *(const half8*)&sg.k[tb + kPage * b + r16][32 * cc + 8 * qd], bq[0][cc], d[0], 0, 0, 0);
          if (step_int2(p0)) {
#pragma unroll
            for (int cc = 0; cc < 4; ++cc)
              d[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                  *(const half8*)&sg.kl[tb + kPage * b + r16][32 * cc + 8 * qd], bq[0][cc], d[0], 0, 0, 0);
          }
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          if constexpr (BF) {
            // (rows past the end, the only zero rows here, lie past every
            // query position; a column past the last query row has a zero
            // query, finite logits and an output that is never stored)
            if (below) {
#pragma unroll
              for (int r = 0; r < 4; ++r) x[rb][4 * b + r] = d[rb][r];
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                x[rb][4 * b + r] = s0 + tb + kPage * b + 4 * qd + r <= qpos[rb] ? d[rb][r] : kNegInf;
            }
          } else if (clean && below) {
#pragma unroll
            for (int r = 0; r < 4; ++r) x[rb][4 * b + r] = colv[rb] ? d[rb][r] : kNegInf;
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int row = tb + kPage * b + 4 * qd + r;
              x[rb][4 * b + r] =
                  (colv[rb] && s0 + row <= qpos[rb] && !sg.skip[row]) ? d[rb][r] : kNegInf;
            }
          }
        }
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) softmax_step<8>(x[rb], C2, p[rb], st[rb], acc[rb]);
      if constexpr (!BF) {
        half8 ph, pl;
#pragma unroll
        for (int r = 0; r < 8; r += 2) {   // fp16 hi / lo, one packed conversion per pair
          const half2_t h2 = __builtin_convertvector(float2_v{p[0][r], p[0][r + 1]}, half2_t);
          const float2_v hf = __builtin_convertvector(h2, float2_v);
          const half2_t l2 = __builtin_convertvector(float2_v{p[0][r] - hf[0], p[0][r + 1] - hf[1]}, half2_t);
          ph[r] = h2[0];
          ph[r + 1] = h2[1];
          pl[r] = l2[0];
          pl[r + 1] = l2[1];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const half4_t a0 = *(const half4_t*)&sg.vt[16 * j + r16][tb + 4 * qd];
          const half4_t a1 = *(const half4_t*)&sg.vt[16 * j + r16][tb + kPage + 4 * qd];
          const half8 av = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
          acc[0][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, ph, acc[0][j], 0, 0, 0);
          acc[0][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pl, acc[0][j], 0, 0, 0);
        }
      } else {
        // P as bf16 hi + lo (about 16 significant bits): one packed
        // conversion per pair, the hi halves back to fp32 by shift and mask
        bf16x8 ph[RB], pl[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int r = 0; r < 8; r += 2) {
            const bf16x2_t h2 = __builtin_convertvector(float2_v{p[rb][r], p[rb][r + 1]}, bf16x2_t);
            const uint32_t hb = __builtin_bit_cast(uint32_t, h2);
            const float h0 = __builtin_bit_cast(float, hb << 16);
            const float h1 = __builtin_bit_cast(float, hb & 0xFFFF0000u);
            const bf16x2_t l2 = __builtin_convertvector(float2_v{p[rb][r] - h0, p[rb][r + 1] - h1}, bf16x2_t);
            ph[rb][r] = h2[0];
            ph[rb][r + 1] = h2[1];
            pl[rb][r] = l2[0];
            pl[rb][r + 1] = l2[1];
          }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          bf16x8 av;   // keys tb + 4 qd .. + 3, then tb + 16 + 4 qd .. + 3
          __builtin_memcpy(&av, &sbf.vt[buf][16 * j + r16][tb + 8 * qd], 16);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            acc[rb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, ph[rb], acc[rb][j], 0, 0, 0);
            acc[rb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pl[rb], acc[rb][j], 0, 0, 0);
          }
        }
      }
    }
  };
  RawSlice cur[2], nxt[2];
  // Every thread waits here for its query loads (and a stager for its first
  // stage).  The query feeds the first MFMA of the key loop; left to the
  // compiler, the wait for it lands inside the loop, where it becomes a wait
  // for every load in flight (the next stages' rows) once per stage.
  constexpr int kWaitVm0 = 0x0F70;   // s_waitcnt vmcnt(0) expcnt(7) lgkmcnt(15)
  if constexpr (BF) {
    if (stager) {
#pragma unroll
      for (int m = 0; m < 2; ++m) fetch(0, m, cur[m]);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    if (stager) {
      deposit2(cur, 0);
      if (1 < nstage) {
#pragma unroll
        for (int m = 0; m < 2; ++m) fetch(kStage, m, nxt[m]);
      }
    }
    __syncthreads();
    // Stage ks + 1 goes into the other buffer (free: every wave has passed
    // the barrier after reading it as stage ks - 1) and stage ks + 2 is
    // fetched between the two steps of stage ks: the loads then have a whole
    // stage of work to arrive before the next wait for them
    // (unconditional: every thread stages, a fetch past the row gives zero
    // rows, and the last deposits land in a buffer no step reads; a branch
    // here makes the compiler wait for these loads at the next MFMA)
    static_assert(!BF || S::kThreads == S::kStageThreads, "bf16 mode: every thread stages");
    for (int ks = 0; ks < nstage; ++ks) {
      run_stage(ks, ks & 1, [&] {
        deposit2(nxt, (ks + 1) & 1);
#pragma unroll
        for (int m = 0; m < 2; ++m) fetch((ks + 2) * kStage, m, nxt[m]);
      });
      __syncthreads();   // stage ks + 1 in, stage ks read by every wave
    }
  } else {
    if (stager) {
#pragma unroll
      for (int m = 0; m < 2; ++m) fetch(0, m, cur[m]);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    for (int ks = 0; ks < nstage; ++ks) {
      if (stager) {
        deposit2(cur, 0);
        if (ks + 1 < nstage) {   // next stage in flight during this one
#pragma unroll
          for (int m = 0; m < 2; ++m) fetch((ks + 1) * kStage, m, nxt[m]);
        }
      }
      __syncthreads();
      run_stage(ks, 0, [] {});
      __syncthreads();   // the stage is consumed before the next one is deposited
#pragma unroll
      for (int m = 0; m < 2; ++m) cur[m] = nxt[m];
    }
  }

  // ---- normalize, then o = o' . R_V^T (or o' when the value transform is absorbed)
  // acc[rb][j][r] is staged value row 16 j + 4 qd + r, i.e. channel 32 qd + 8 r + j
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float l = rows_sum(st[rb].l);
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        fin[16 * (RB * wave + rb) + r16][32 * qd + 8 * r + j] = acc[rb][j][r] * inv;
  }
  __syncthreads();
  auto out_row = [&](int rr) {   // output row of work-group row rr, or nullptr
    const int R = tile * kPfRows + rr;
    if (R >= rows) return (float*)nullptr;
    uint32_t hr_;
    const int pr = div_g(R, hr_);
    return a.out + ((size_t)(t0 + pr) * c.hq + (size_t)h * c.g + hr_) * kD;
  };
  if (!c.unrot) {
    for (int k = tid; k < kPfRows * (kD / 4); k += kPfThreads) {
      const int rr = k / (kD / 4), c4 = k % (kD / 4);
      float* o = out_row(rr);
      if (o) *(float4_t*)(o + 4 * c4) = *(const float4_t*)&fin[rr][4 * c4];
    }
    return;
  }
  // Wave w computes output channels 16 (w % 8) .. 16 (w % 8) + 15 of the row
  // tiles rt = w / 8, w / 8 + kPfWaves / 8, ... on the bf16 matrix cores:
  // both operands as bf16 hi + lo (o' . R = o'_hi R_hi + o'_hi R_lo + o'_lo
  // R_hi, each factor held to about 16 bits; a sixteenth of the fp32
  // matrix cores' time for the same product).  For the 32-channel chunk kc,
  // lane (li, kq) holds o' row 16 rt + li and R_V row 16 (w % 8) + li at
  // channels 32 kc + 8 kq .. + 7.
  constexpr int kColBlocks = kD / 16;
  static_assert(kPfWaves % kColBlocks == 0, "the epilogue splits the 128 output channels over the waves");
  const int cb = wave % kColBlocks;
  const int li = r16, kq = qd;
  bf16x8 rh[4], rl[4];
  {
    const int j = 16 * cb + li;
    const float* rg = c.r_v + ((size_t)h * kD + j) * kD;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      float f[8];
      if (c.rot) {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = hadamard_entry(c.rot, j, 32 * kc + 8 * kq + e);
      } else {
        __builtin_memcpy(f, rg + 32 * kc + 8 * kq, 32);
      }
      split_bf16(f, rh[kc], rl[kc]);
    }
  }
  for (int rt = wave / kColBlocks; rt < kPfRows / 16; rt += kPfWaves / kColBlocks) {
    if (tile * kPfRows + 16 * rt >= rows) break;
    float4_t o4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      float f[8];
      __builtin_memcpy(f, &fin[16 * rt + li][32 * kc + 8 * kq], 32);
      bf16x8 ah, al;
      split_bf16(f, ah, al);
      o4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, rh[kc], o4, 0, 0, 0);
      o4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, rl[kc], o4, 0, 0, 0);
      o4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, rh[kc], o4, 0, 0, 0);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float* o = out_row(16 * rt + 4 * kq + v);
      if (o) o[16 * cb + li] = o4[v];
    }
  }
}

hipError_t launch_prefill(const CacheArgs& c, const PrefillArgs& a, hipStream_t stream) {
  if (a.n_seqs <= 0 || a.tiles <= 0) return hipSuccess;
  const dim3 grid((unsigned)a.tiles * (unsigned)a.n_seqs * (unsigned)c.hkv);
  // (the host sizes the tiles for these shapes: 8 row blocks in bf16 mode)
  if (a.bf16_only) {
    if (a.blocks != 8) return hipErrorInvalidValue;
    hipLaunchKernelGGL((prefill_attn_kernel<8, true, 1>), grid, dim3(64 * 8), 0, stream, c, a);
  } else if (a.blocks == 16) {
    hipLaunchKernelGGL((prefill_attn_kernel<16, false, 1>), grid, dim3(64 * 16), 0, stream, c, a);
  } else if (a.blocks == 8) {
    hipLaunchKernelGGL((prefill_attn_kernel<8, false, 1>), grid, dim3(64 * 8), 0, stream, c, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int prefill_tiles(int n_new, int g, int blocks) {
  const int rows = 16 * blocks;
  return (n_new * g + rows - 1) / rows;
}

}  // namespace oscar
