// Internal declarations shared by the host library and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace oscar {

constexpr int kD = 128;          // head dim
constexpr int kPage = 16;        // tokens per page / window block
constexpr int kMaxKvHeads = 64;

// Everything a kernel needs to address one cache, passed by value.
struct CacheArgs {
  uint8_t* pages;
  const int32_t* block_table;
  uint16_t* win;
  const float* r_k;
  const float* r_v;
  int hq, hkv, g;                // query heads, KV heads, hq / hkv
  int group, ng;                 // quantization group size and groups per row
  int s_sink, s_keep, s_flush;
  int ring_cap;                  // roundup16(s_keep + s_flush)
  int sink_blocks, win_blocks;   // ceil(s_sink / 16), sink_blocks + ring_cap / 16
  int max_seqs, max_pages, num_pages;
  int page_bytes;                // bytes of one page-head block
  int key_mode;                  // 0: per-token clipped key groups; 1: OScaR token scale + channel blocks
  int unrot;                     // apply R_V^T after the merge (0: output in the rotated basis)
  int rot;                       // 0: dense r_k / r_v; 1: H / sqrt(128); 2: H P_br / sqrt(128)
};

// Clip ratios, and the host's per-sequence table: where each sequence's
// quantized positions start among the call's, its cache row, length before
// the call and first new token (qn = 0: the kernels read the device arrays).
constexpr int kMaxQuantSeqs = 512;
struct QuantSeq {
  int32_t before, slot, len_before, cu_new;
};
struct QuantArgs {
  float k[kMaxKvHeads];
  float v[kMaxKvHeads];
  int qn;
  QuantSeq q[kMaxQuantSeqs + 1];   // q[qn].before = the call's quantized positions
};

// Per-call sequence metadata (device arrays provided by the caller).
struct SeqArgs {
  const int32_t* slots;
  const int32_t* lens;           // len_before (append) or seq_len (decode)
  const int32_t* cu_new;         // append only
  int n_seqs;
};

// ---- launchers (each returns hipGetLastError() of its launch) -------------

// One rotation job: dst[t][h][:] = bf16_rne(src[t][h][:] . r[h / g]) for
// t < n_tok, h < heads; dst_b (optional) receives a copy.
struct RotateJob {
  const uint16_t* src;
  const float* r;
  uint16_t* dst_a;
  uint16_t* dst_b;
  int heads, g;
};
struct RotateJobs {
  RotateJob job[3];
  int n;
  int kind;                      // 0: dense (the jobs' r); 1, 2: structured (r unused)
};
hipError_t launch_rotate(const RotateJobs& jobs, int n_tok, hipStream_t stream);

// Quantize every position that moves to INT2 in this append, from the ring
// (old rows) or the staging rows (new tokens), into the pages.  total_q =
// sum over sequences of S_quant(after) - S_quant(before) (< 2^31).
hipError_t launch_quantize(const CacheArgs& c, const QuantArgs& clip, const SeqArgs& s,
                           const uint16_t* stage_k, const uint16_t* stage_v, int total_q,
                           hipStream_t stream);

// Both of the above in one launch; only valid when no new row lands on a ring
// slot that the flush still reads.
hipError_t launch_flush_place(const CacheArgs& c, const QuantArgs& clip, const SeqArgs& s,
                              const uint16_t* stage_k, const uint16_t* stage_v, int total_q,
                              int max_new, hipStream_t stream);

// OScaR key mode: the key blocks (32 INT2 positions, one KV head) that move
// to INT2 in this append, from the ring (old rows) or the staging rows (new
// tokens), into the pages; total_q as for launch_quantize (a multiple of 32
// per sequence).
hipError_t launch_ots_keys(const CacheArgs& c, const QuantArgs& clip, const SeqArgs& s,
                           const uint16_t* stage_k, int total_q, hipStream_t stream);

// Byte offset of the value parameters in a page-head block.
__host__ __device__ inline int v_param_offset(const CacheArgs& c) {
  return c.key_mode ? 1024 : 1024 + 64 * c.ng;
}
constexpr int kOtsBlock = 32;         // OScaR key block: INT2 tokens per channel (Delta, z)
constexpr int kOtsPageBytes = 1568;   // OScaR page-head block
constexpr int kOtsScaleOffset = 1280; // token scales (bf16) in the block
constexpr int kOtsChanOffset = 1312;  // channel (Delta, z) words in the block

// Copy staging rows of new tokens that land in the sink or the ring.
hipError_t launch_place(const CacheArgs& c, const SeqArgs& s, const uint16_t* stage_k,
                        const uint16_t* stage_v, int max_new, hipStream_t stream);

// One-token append in one launch (rotate, flush, place): every sequence
// appends exactly one token, none is flushed in the same call and no new row
// lands on a ring slot the flush reads.  jobs: keys, values, queries (opt.).
hipError_t launch_append_one(const CacheArgs& c, const QuantArgs& clip, const SeqArgs& s,
                             const RotateJobs& jobs, int total_q, const uint16_t* stage_k,
                             const uint16_t* stage_v, hipStream_t stream);

// Chunked-prefill attention: the new rows of each sequence (just appended)
// attend causally to the cache before them and to each other.
struct PrefillArgs {
  const int32_t* slots;          // [n_seqs] cache rows
  const int32_t* len_before;     // [n_seqs] tokens before the chunk
  const int32_t* cu_new;         // [n_seqs + 1] chunk rows of sequence i: cu_new[i] .. cu_new[i+1]-1
  const uint16_t* q_rot;         // bf16 [cu_new[n]][hq][128]
  const uint16_t* k_rot;         // bf16 [cu_new[n]][hkv][128]
  const uint16_t* v_rot;         // bf16 [cu_new[n]][hkv][128]
  float* out;                    // fp32 [cu_new[n]][hq][128]
  int n_seqs;
  int tiles;                     // most query tiles of any sequence (grid x)
  int blocks;                    // query rows per work-group / 16: 8 or 16 (bf16 mode: 8)
  int bf16_only;                 // no sequence has INT2 rows below its chunk
  uint32_t g_magic;              // floor(2^32 / g), 0 for g = 1 (see div_magic)
  uint32_t ring_magic;           // floor(2^32 / ring_cap), 0 for ring_cap = 1
};
// floor(2^32 / d) for d >= 2, 0 for d = 1: with it a kernel divides without
// a reciprocal held in vector registers (div_by_magic).
inline uint32_t div_magic(uint32_t d) { return d > 1 ? (uint32_t)((1ull << 32) / d) : 0u; }
int prefill_tiles(int n_new, int g, int blocks);
hipError_t launch_prefill(const CacheArgs& c, const PrefillArgs& a, hipStream_t stream);

// Decoded rows of one cache row.
hipError_t launch_dequant(const CacheArgs& c, int slot, int len, int t0, int t1, float* k_out,
                          float* v_out, hipStream_t stream);

// ---- decode work split (shared by the host planner and the kernels) ------
//
// The decode work of one (sequence, group of KV heads, query-head pass) is
// its INT2 page pairs plus its BF16 window blocks; a window block (8 KB per
// head) counts as kWinCost page pairs (2.5 KB per head at G = 64): measured
// per work-group, a window block takes about twice a pair's time.  The work is cut into splits of at most
// quota16 / 16 units (the quota is fixed point with 4 fraction bits, so the
// planner can fill the device closely); every split is one work-group of the
// split launch.
constexpr int kWinCost = 2;
constexpr int kMaxSplits = 256;            // splits per (sequence, row), merge LDS bound
constexpr int kMaxPairsPerSplit = 256;     // page ids staged per work-group
constexpr int kMaxScanSeqs = 2048;         // sequences per decode launch
constexpr int kMergeDirect = 32;           // most splits per row merged by one launch

// Partial record of a (sequence, KV head, pass, split): the log2-domain
// maxima and the sums of the pass's HP query heads, then their
// unnormalized o' rows, which start 16 bytes into the record and stay
// 16-byte aligned (the record length is a multiple of 4 floats).
__host__ __device__ constexpr int rec_o_offset(int hp) { return 2 * hp < 4 ? 4 : 2 * hp; }
__host__ __device__ constexpr int rec_words(int hp) { return rec_o_offset(hp) + hp * kD; }

struct DecodeWork {
  int n_pairs;                   // INT2 page pairs
  int n_wu;                      // BF16 window blocks visited (sink blocks, then live ring blocks)
};

// Ring blocks that hold live rows: the live slots are the cnt = len -
// ring_lo offsets b0, b0 + 1, ... (mod R) from b0 = (ring_lo - S_sink) mod R;
// the blocks visited are b0 / 16, b0 / 16 + 1, ... (mod R / 16).
__host__ __device__ inline int ring_blocks_live(int len, int ring_lo, int s_sink, int ring_cap) {
  if (ring_cap <= 0 || len <= ring_lo) return 0;
  const int cnt = len - ring_lo, b0 = (ring_lo - s_sink) % ring_cap;
  const int nb = (b0 % kPage + cnt + kPage - 1) / kPage;
  return nb < ring_cap / kPage ? nb : ring_cap / kPage;
}

__host__ __device__ inline DecodeWork decode_work(int len, int s_sink, int s_keep, int s_flush,
                                                  int ring_cap) {
  DecodeWork w{0, 0};
  if (len < 1) return w;
  const int num = len - s_sink - s_keep;
  const int sq = s_sink + s_flush * (num >= 0 ? num / s_flush : 0);
  const int nq = sq > s_sink ? sq - s_sink : 0;
  w.n_pairs = ((nq + kPage - 1) / kPage + 1) / 2;
  const int nsink = len < s_sink ? len : s_sink;
  const int ring_lo = sq > s_sink ? sq : s_sink;
  w.n_wu = (nsink + kPage - 1) / kPage + ring_blocks_live(len, ring_lo, s_sink, ring_cap);
  return w;
}

__host__ __device__ inline int decode_splits(DecodeWork w, int quota16, int smax) {
  const int cost = w.n_pairs + kWinCost * w.n_wu;
  const int n = cost > 0 ? (16 * cost + quota16 - 1) / quota16 : 1;
  return n < smax ? n : smax;
}

// Work item of each work-group of a split launch, chosen on the host (n > 0):
// work-group b takes item `local` of sequence `seq` (item_of[b] = seq << 16 |
// local), whose cache row and length are slot[b] and len[b] (the host copies
// of the call's arrays, which the device copies must equal), so a
// work-group starts its loads without reading the sequence arrays first.
// With n = 0 work-group b takes item b and finds its sequence on the device.
// Work-group b of a launch that fills the device runs on compute unit
// b % cus, so the planner deals the items out largest first, in alternating
// directions, to even out the work of each compute unit.
constexpr int kMaxOrder = 1024;
struct ItemOrder {
  int n;
  uint32_t item_of[kMaxOrder];
  int32_t slot[kMaxOrder];
  int32_t len[kMaxOrder];
};

// Split records of each sequence of a decode launch, as planned on the host,
// for the merge launch: it then starts loading records without reading the
// sequence arrays first.  n = 0: the merge kernels derive the counts from
// the device lengths.
struct SplitCounts {
  int n;
  uint16_t ns[kMaxScanSeqs];
};

// INT2 split-K decode (partials to the workspace) and the merge / un-rotation launch.
struct DecodePlan {
  int quota;                     // work per context split in 1/16 page pairs (a window block = kWinCost pairs)
  int smax;                      // most splits of any sequence
  int hp;                        // query heads handled per pass (ng * kh * hp <= 16)
  int passes;                    // ceil(g / hp)
  int kh;                        // KV heads per wave (1, or 2 when a head's columns fill half a tile)
  int wh;                        // waves per work-group
  int ring;                      // INT2 split kernel: page pairs per wave in its LDS ring (2 or 4)
  int ps;                        // INT2 split kernel: 1 = the waves of a work-group share one KV-head group
  int grid;                      // work-groups of the split launch (= its work items)
  int cus;                       // compute units: work-group b runs in dispatch round b / cus
  const ItemOrder* order;        // work item of each work-group (host memory, passed by value)
  const SplitCounts* counts;     // split records per sequence (host memory, passed by value)
};
// Work-groups of the split kernel that fit on one compute unit.
int decode_wgs_per_cu(const CacheArgs& c, const DecodePlan& plan);
constexpr int kDecodeSplit = 1;   // the split kernel: partial records to the workspace
constexpr int kDecodeMerge = 2;   // the merge / un-rotation kernel: partials to out
hipError_t launch_decode(const CacheArgs& c, const SeqArgs& s, const DecodePlan& plan,
                         const uint16_t* q_rot, float* out, float* partials, int phases,
                         hipStream_t stream);

// Split-K decode over a plain BF16 paged cache (c.pages = bf16
// [num_pages][hkv][2][16][128], c.s_sink = c.s_keep = c.ring_cap = 0,
// c.s_flush = 1, so decode_work counts its page pairs): split kernel and the
// same merge, without un-rotation.
hipError_t launch_bf16_decode(const CacheArgs& c, const SeqArgs& s, const DecodePlan& plan,
                              const uint16_t* q, float* out, float* partials, int phases,
                              hipStream_t stream);
int bf16_decode_wgs_per_cu(const DecodePlan& plan);

}  // namespace oscar
