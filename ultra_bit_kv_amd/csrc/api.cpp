// liboscar_kv host side: argument checks, the closed-form flush planner, the
// split-K planner, workspace layout and kernel launches.  See oscar_kv.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <mutex>
#include <vector>

#include "device_common.h"
#include "oscar_check.h"
#include "oscar_internal.h"
#include "oscar_kv.h"

namespace {

using namespace oscar;

constexpr size_t kAlign = 256;
// Config limits: with them every row's decode work fits kMaxSplits splits of
// kMaxPairsPerSplit units (32768 pairs + 3 * 1281 window blocks < 65536).
constexpr int kMaxSink = 4096, kMaxKeep = 8192, kMaxFlush = 8192;
constexpr int kMaxPagesPerSeq = 65536;
static_assert((kMaxPagesPerSeq / 2) +
                      kWinCost * (kMaxSink / kPage + (kMaxKeep + kMaxFlush) / kPage + 1) <=
                  (int64_t)kMaxSplits * (kMaxPairsPerSplit - 1),
              "decode work of the largest row must fit the split limits");
// Split launch sizing: the work-groups of a launch fill this share of the
// resident slots, so none waits for a second round.
constexpr int kFillPercent = 100;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// S_quant of the flush rule (WUSH-KV notes, "method step details").
int64_t s_quant(int64_t len, const oscar_kv_config& c) {
  const int64_t num = len - c.s_sink - c.s_keep;
  const int64_t k = num >= 0 ? num / c.s_flush : 0;
  return c.s_sink + (int64_t)c.s_flush * k;
}

int64_t int2_pages(int64_t len, const oscar_kv_config& c) {
  const int64_t nq = s_quant(len, c) - c.s_sink;
  return nq > 0 ? (nq + kPage - 1) / kPage : 0;
}

int ring_cap(const oscar_kv_config& c) {
  return (c.s_keep + c.s_flush + kPage - 1) / kPage * kPage;
}

int ng_of(const oscar_kv_config& c) { return kD / c.group_size; }

size_t page_bytes_of(const oscar_kv_config& c) {
  return c.key_mode == OSCAR_KEYS_OTS ? (size_t)kOtsPageBytes
                                      : 1024 + 128 * (size_t)(kD / c.group_size);
}

// Query heads per decode pass and KV heads per wave: columns of a 16-wide
// MFMA tile are (group, KV head of the wave, query head) triples, so
// ng * kh * hp <= 16.  With more than one group the columns of one head are
// kh * hp apart and the group sum is a cycle of DPP rotations, so
// ng * kh * hp = 16.  A wave takes two KV heads when one head's columns
// fill at most half a tile without a second pass (each pass re-reads the
// codes), which halves the per-column work per byte.
DecodePlan head_passes(const oscar_kv_config& c) {
  const int g = c.num_q_heads / c.num_kv_heads;
  const int ng = ng_of(c);
  int pow2 = 1;
  while (pow2 < g && pow2 < 16) pow2 *= 2;
  const bool even = c.num_kv_heads % 2 == 0;
  int hp, kh;
  if (c.key_mode == OSCAR_KEYS_OTS) {   // (G = 32) one KV head per wave, 4 heads per pass
    kh = 1;
    hp = 4;
  } else if (ng == 1) {
    hp = pow2;
    kh = (even && hp <= 8) ? 2 : 1;
  } else if (even && pow2 <= 8 / ng) {
    kh = 2;
    hp = 8 / ng;
  } else {
    kh = 1;
    hp = 16 / ng;
  }
  DecodePlan p{};
  p.hp = hp;
  p.kh = kh;
  p.passes = (g + hp - 1) / hp;
  const int waves = c.num_kv_heads / kh;   // KV head groups, one wave each
  p.wh = waves % 4 == 0 ? 4 : (waves % 2 == 0 ? 2 : 1);
  p.ring = 2;
  p.quota = 1;
  p.smax = 1;
  return p;
}

// What the split limits of a decode call depend on: KV heads, query-head
// passes and heads per pass, and the largest decode work of any row.
struct DecodeShape {
  int hkv, passes, hp;
  int64_t max_cost;   // page pairs, a window block = kWinCost
};

DecodeShape int2_shape(const oscar_kv_config& c) {
  const DecodePlan p = head_passes(c);
  const int64_t pairs = ((int64_t)c.max_pages_per_seq + 1) / 2;
  const int64_t wu = (c.s_sink + kPage - 1) / kPage + ring_cap(c) / kPage;
  return DecodeShape{c.num_kv_heads, p.passes, p.hp, pairs + kWinCost * wu};
}

// Fewest splits that keep every split within kMaxPairsPerSplit - 1 units
// (the page-id list a work-group stages in LDS; the planner's largest quota).
int min_splits(const DecodeShape& sh) {
  return (int)std::max<int64_t>(1, (sh.max_cost + kMaxPairsPerSplit - 2) / (kMaxPairsPerSplit - 1));
}

// Most splits per (sequence, KV head, pass) the workspace is sized for:
// about 16K partial records per launch, at most kMaxSplits, and never fewer
// than min_splits (the config limits keep min_splits <= kMaxSplits).
int max_splits(const DecodeShape& sh, int n_seqs) {
  const int ns = std::min(std::max(1, n_seqs), kMaxScanSeqs);
  const long long rows = (long long)ns * sh.hkv * sh.passes;
  long long s = (16384 + rows - 1) / rows;
  s = std::max(1LL, std::min((long long)kMaxSplits, s));
  return (int)std::max<long long>(s, min_splits(sh));
}

// Split partial records of one decode launch (at most kMaxScanSeqs sequences).
size_t partials_bytes(const DecodeShape& sh, int n_seqs) {
  const size_t rec = (size_t)rec_words(sh.hp);
  const int ns = std::min(std::max(1, n_seqs), kMaxScanSeqs);
  const int cap = max_splits(sh, ns);
  return align_up((size_t)ns * sh.hkv * sh.passes * (size_t)cap * rec * sizeof(float));
}

size_t staging_bytes(const oscar_kv_config& c, int64_t n_tok) {
  return 2 * align_up((size_t)n_tok * c.num_kv_heads * kD * sizeof(uint16_t));
}

CacheArgs make_args(const oscar_kv_cache& k) {
  const oscar_kv_config& c = k.cfg;
  CacheArgs a{};
  a.pages = k.pages;
  a.block_table = k.block_table;
  a.win = k.win;
  a.r_k = k.r_k;
  a.r_v = k.r_v;
  a.unrot = k.out_rotated ? 0 : 1;
  a.rot = k.rotation;
  a.hq = c.num_q_heads;
  a.hkv = c.num_kv_heads;
  a.g = c.num_q_heads / c.num_kv_heads;
  a.group = c.group_size;
  a.ng = ng_of(c);
  a.s_sink = c.s_sink;
  a.s_keep = c.s_keep;
  a.s_flush = c.s_flush;
  a.ring_cap = ring_cap(c);
  a.sink_blocks = (c.s_sink + kPage - 1) / kPage;
  a.win_blocks = a.sink_blocks + a.ring_cap / kPage;
  a.max_seqs = c.max_seqs;
  a.max_pages = c.max_pages_per_seq;
  a.num_pages = c.num_pages;
  a.page_bytes = (int)page_bytes_of(c);
  a.key_mode = c.key_mode;
  return a;
}

// gfx950 check and compute-unit count, once per device.
int check_device(int* cus = nullptr) {
  static std::mutex mu;
  static int known[64] = {0};   // 0 unknown, 1 ok, -1 not gfx950
  static int n_cu[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return OSCAR_ERR_HIP;
  if (dev < 0 || dev >= 64) return OSCAR_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(mu);
  if (known[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return OSCAR_ERR_HIP;
    known[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    n_cu[dev] = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
  }
  if (cus) *cus = n_cu[dev];
  return known[dev] == 1 ? OSCAR_OK : OSCAR_ERR_DEVICE;
}

// Decode work of a row of len tokens (page pairs, a window block = kWinCost);
// the kernels compute the same numbers from the device lengths with the same
// function.
int64_t decode_cost(int64_t len, const CacheArgs& a) {
  const DecodeWork w = decode_work((int)len, a.s_sink, a.s_keep, a.s_flush, a.ring_cap);
  return w.n_pairs + (int64_t)kWinCost * w.n_wu;
}

// Resident split work-groups per compute unit, once per (device, kernel shape).
int decode_slots_per_cu(const CacheArgs& a, const DecodePlan& plan, bool bf16) {
  static std::mutex mu;
  static std::vector<std::pair<long long, int>> memo;
  int dev = 0;
  (void)hipGetDevice(&dev);
  const long long key =
      ((((((((long long)dev * 2 + (bf16 ? 1 : 0)) * 8 + a.ng) * 32 + plan.hp) * 8 + plan.wh) * 4 +
         plan.kh) * 8 + plan.ring) * 2 + (bf16 ? 0 : a.key_mode)) * 2 + (bf16 ? 0 : plan.ps);
  std::lock_guard<std::mutex> lock(mu);
  for (const auto& m : memo)
    if (m.first == key) return m.second;
  const int n = bf16 ? bf16_decode_wgs_per_cu(plan) : decode_wgs_per_cu(a, plan);
  memo.emplace_back(key, n);
  return n;
}

// Kernels read rows and page blocks with 16-byte vector loads.
bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }
bool cache_aligned(const oscar_kv_cache& k) {
  return aligned16(k.pages) && aligned16(k.win) && aligned16(k.r_k) && aligned16(k.r_v) &&
         aligned16(k.r_q) &&
         aligned16(k.block_table);
}

// The rotation kind is one of the three, and the structured kinds take no
// matrices.
bool rotation_ok(const oscar_kv_cache& k) {
  if (k.rotation == OSCAR_ROT_DENSE) return true;
  return (k.rotation == OSCAR_ROT_HADAMARD || k.rotation == OSCAR_ROT_HADAMARD_BITREV) && !k.r_k &&
         !k.r_v && !k.r_q;
}
bool dense(const oscar_kv_cache& k) { return k.rotation == OSCAR_ROT_DENSE; }

thread_local char g_last_hip[160] = "";

int hip_status(hipError_t e) {
  if (e == hipSuccess) return OSCAR_OK;
  std::snprintf(g_last_hip, sizeof g_last_hip, "HIP runtime error: %s", hipGetErrorString(e));
  return OSCAR_ERR_HIP;
}

}  // namespace

extern "C" {

int oscar_check_config(const oscar_kv_config* c) {
  if (!c) return OSCAR_ERR_NULL;
  if (c->head_dim != kD || c->page_size != kPage) return OSCAR_ERR_SHAPE;
  if (c->num_kv_heads < 1 || c->num_kv_heads > OSCAR_MAX_KV_HEADS) return OSCAR_ERR_SHAPE;
  if (c->num_q_heads < c->num_kv_heads || c->num_q_heads % c->num_kv_heads != 0)
    return OSCAR_ERR_SHAPE;
  if (c->num_q_heads / c->num_kv_heads > 256) return OSCAR_ERR_SHAPE;
  if (c->group_size != 32 && c->group_size != 64 && c->group_size != 128) return OSCAR_ERR_GROUP;
  for (int h = 0; h < c->num_kv_heads; ++h) {
    const float a = c->clip_k[h], b = c->clip_v[h];
    if (!(a >= 0.5f && a <= 1.0f) || !(b >= 0.5f && b <= 1.0f)) return OSCAR_ERR_CLIP;
  }
  if (c->s_sink < 0 || c->s_keep < 0 || c->s_flush < 1) return OSCAR_ERR_WINDOW;
  if (c->s_sink > kMaxSink || c->s_keep > kMaxKeep || c->s_flush > kMaxFlush) return OSCAR_ERR_WINDOW;
  if (c->max_seqs < 1 || c->max_pages_per_seq < 0 || c->num_pages < 0) return OSCAR_ERR_CAPACITY;
  if (c->max_pages_per_seq > kMaxPagesPerSeq) return OSCAR_ERR_CAPACITY;
  if (c->key_mode != OSCAR_KEYS_CLIP && c->key_mode != OSCAR_KEYS_OTS) return OSCAR_ERR_ARG;
  if (c->key_mode == OSCAR_KEYS_OTS) {
    // one (Delta, z) per channel per block of 32 INT2 tokens; flushes move whole blocks
    if (c->group_size != kOtsBlock) return OSCAR_ERR_GROUP;
    if (c->s_flush % kOtsBlock != 0) return OSCAR_ERR_WINDOW;
  }
  return OSCAR_OK;
}

size_t oscar_page_head_bytes(int32_t group_size) {
  if (group_size != 32 && group_size != 64 && group_size != 128) return 0;
  return 1024 + 128 * (size_t)(kD / group_size);
}

size_t oscar_config_page_head_bytes(const oscar_kv_config* c) {
  if (oscar_check_config(c) != OSCAR_OK) return 0;
  return page_bytes_of(*c);
}

size_t oscar_pages_bytes(const oscar_kv_config* c) {
  if (oscar_check_config(c) != OSCAR_OK) return 0;
  return (size_t)c->num_pages * c->num_kv_heads * page_bytes_of(*c);
}

int32_t oscar_ring_capacity(const oscar_kv_config* c) {
  if (oscar_check_config(c) != OSCAR_OK) return 0;
  return ring_cap(*c);
}

size_t oscar_win_bytes(const oscar_kv_config* c) {
  if (oscar_check_config(c) != OSCAR_OK) return 0;
  const size_t blocks = (c->s_sink + kPage - 1) / kPage + ring_cap(*c) / kPage;
  return (size_t)c->max_seqs * c->num_kv_heads * blocks * 2 * kPage * kD * sizeof(uint16_t);
}

int64_t oscar_max_seq_len(const oscar_kv_config* c) {
  if (oscar_check_config(c) != OSCAR_OK) return 0;
  // largest len with S_quant(len) - S_sink <= 16 * max_pages_per_seq
  const int64_t kmax = (int64_t)kPage * c->max_pages_per_seq / c->s_flush;
  return (int64_t)c->s_sink + c->s_keep + (kmax + 1) * c->s_flush - 1;
}

size_t oscar_workspace_size(const oscar_kv_config* c, int32_t n_seqs, int64_t max_new_tokens) {
  if (oscar_check_config(c) != OSCAR_OK || n_seqs < 0 || max_new_tokens < 0) return 0;
  return std::max(partials_bytes(int2_shape(*c), std::max(1, (int)n_seqs)),
                  staging_bytes(*c, max_new_tokens));
}

const char* oscar_status_string(int status) {
  switch (status) {
    case OSCAR_OK: return "ok";
    case OSCAR_ERR_NULL: return "a required pointer is NULL";
    case OSCAR_ERR_SHAPE: return "unsupported shape (head_dim, page_size or head counts)";
    case OSCAR_ERR_GROUP: return "group_size must be 32, 64 or 128";
    case OSCAR_ERR_CLIP: return "clip ratios must lie in [0.5, 1]";
    case OSCAR_ERR_WINDOW: return "invalid window sizes (s_sink, s_keep >= 0, s_flush >= 1)";
    case OSCAR_ERR_CAPACITY: return "slot, length or page count exceeds the cache";
    case OSCAR_ERR_WORKSPACE: return "workspace too small";
    case OSCAR_ERR_DEVICE: return "current device is not gfx950";
    case OSCAR_ERR_HIP: return g_last_hip[0] ? g_last_hip : "HIP runtime error";
    case OSCAR_ERR_ARG: return "invalid argument";
  }
  return "unknown status";
}

int oscar_rotate_quant_append(const oscar_kv_cache* cache, int32_t n_seqs,
                              const int32_t* seq_slots_host, const int32_t* len_before_host,
                              const int32_t* cu_new_host, const int32_t* seq_slots,
                              const int32_t* len_before, const int32_t* cu_new, const uint16_t* k,
                              const uint16_t* v, const uint16_t* q, uint16_t* q_rot,
                              uint16_t* k_rot, uint16_t* v_rot, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (!cache) return OSCAR_ERR_NULL;
  const oscar_kv_config& c = cache->cfg;
  int st = oscar_check_config(&c);
  if (st != OSCAR_OK) return st;
  if (!seq_slots_host || !len_before_host || !cu_new_host || !seq_slots || !len_before ||
      !cu_new || !k || !v || !workspace || !cache->pages || !cache->block_table || !cache->win ||
      (dense(*cache) && (!cache->r_k || !cache->r_v)))
    return OSCAR_ERR_NULL;
  if (!rotation_ok(*cache)) return OSCAR_ERR_ARG;
  if (q_rot && !q) return OSCAR_ERR_NULL;
  if (!aligned16(k) || !aligned16(v) || !aligned16(q) || !aligned16(q_rot) || !aligned16(k_rot) ||
      !aligned16(v_rot) || !cache_aligned(*cache) || !aligned16(workspace))
    return OSCAR_ERR_ARG;
  if (n_seqs < 1 || n_seqs > c.max_seqs) return OSCAR_ERR_ARG;
  if (cu_new_host[0] != 0) return OSCAR_ERR_ARG;
  const int64_t max_len = oscar_max_seq_len(&c);
  std::vector<char> seen(c.max_seqs, 0);
  int64_t total_q = 0;
  int max_keep = 0;   // most new rows of one sequence that stay in BF16
  for (int i = 0; i < n_seqs; ++i) {
    const int slot = seq_slots_host[i];
    if (slot < 0 || slot >= c.max_seqs) return OSCAR_ERR_CAPACITY;
    if (seen[slot]) return OSCAR_ERR_ARG;
    seen[slot] = 1;
    const int64_t n_new = (int64_t)cu_new_host[i + 1] - cu_new_host[i];
    const int64_t lb = len_before_host[i];
    if (n_new < 0 || lb < 0) return OSCAR_ERR_ARG;
    if (lb + n_new > max_len) return OSCAR_ERR_CAPACITY;
    if (int2_pages(lb + n_new, c) > c.max_pages_per_seq) return OSCAR_ERR_CAPACITY;
    if (int2_pages(lb + n_new, c) > 0 && c.num_pages < 1) return OSCAR_ERR_CAPACITY;
    total_q += s_quant(lb + n_new, c) - s_quant(lb, c);
    // new rows that stay in BF16: the sink part and the part from S_quant on
    const int64_t in_sink = std::max<int64_t>(0, std::min<int64_t>(lb + n_new, c.s_sink) - lb);
    const int64_t in_ring = std::max<int64_t>(0, lb + n_new - std::max(lb, s_quant(lb + n_new, c)));
    max_keep = std::max<int>(max_keep, (int)(in_sink + in_ring));
  }
  const int64_t n_tok = cu_new_host[n_seqs];
  if (n_tok > (int64_t)1 << 30 || total_q > (int64_t)1 << 30) return OSCAR_ERR_ARG;
  const size_t need = staging_bytes(c, n_tok);
  if (workspace_bytes < need) return OSCAR_ERR_WORKSPACE;
  if ((st = check_device()) != OSCAR_OK) return st;
  if (n_tok == 0) return OSCAR_OK;

  hipStream_t sm = (hipStream_t)stream;
  const CacheArgs a = make_args(*cache);
  QuantArgs clip{};
  for (int h = 0; h < c.num_kv_heads; ++h) {
    clip.k[h] = c.clip_k[h];
    clip.v[h] = c.clip_v[h];
  }
  if (n_seqs <= kMaxQuantSeqs) {
    clip.qn = n_seqs;
    int64_t run = 0;
    for (int i = 0; i < n_seqs; ++i) {
      const int64_t lb = len_before_host[i];
      clip.q[i] = QuantSeq{(int32_t)run, seq_slots_host[i], (int32_t)lb, cu_new_host[i]};
      run += s_quant(lb + (int64_t)cu_new_host[i + 1] - cu_new_host[i], c) - s_quant(lb, c);
    }
    clip.q[n_seqs] = QuantSeq{(int32_t)run, -1, 0, cu_new_host[n_seqs]};
  }
  SeqArgs sa{seq_slots, len_before, cu_new, n_seqs};
  uint8_t* ws = (uint8_t*)workspace;
  uint16_t* stage_k = (uint16_t*)ws;
  uint16_t* stage_v = (uint16_t*)(ws + staging_bytes(c, n_tok) / 2);

  // One launch for one-token appends (decode steps): no new row is flushed
  // in the same call and no new row lands on a ring slot the flush reads.
  // (in OScaR key mode only when nothing is quantized: keys move to INT2 in
  // whole blocks through the key-block kernel)
  bool one = c.key_mode == OSCAR_KEYS_CLIP || total_q == 0;
  for (int i = 0; one && i < n_seqs; ++i) {
    const int64_t n_new = (int64_t)cu_new_host[i + 1] - cu_new_host[i];
    const int64_t lb = len_before_host[i];
    one = n_new == 1 && (lb < s_quant(lb, c) || s_quant(lb + 1, c) <= lb) &&
          lb - s_quant(lb, c) < a.ring_cap;
  }
  if (one) {
    RotateJobs jobs{};
    jobs.job[0] = RotateJob{k, cache->r_k, nullptr, k_rot, c.num_kv_heads, 1};
    jobs.job[1] = RotateJob{v, cache->r_v, nullptr, v_rot, c.num_kv_heads, 1};
    jobs.n = 2;
    jobs.kind = cache->rotation;
    if (q_rot)
      jobs.job[jobs.n++] = RotateJob{q, cache->r_q ? cache->r_q : cache->r_k, q_rot, nullptr,
                                     c.num_q_heads, c.num_q_heads / c.num_kv_heads};
    return hip_status(
        launch_append_one(a, clip, sa, jobs, (int)total_q, stage_k, stage_v, sm));
  }
  // 1. rotate new rows: keys and values to staging, queries straight to q_rot
  RotateJobs jobs{};
  jobs.job[0] = RotateJob{k, cache->r_k, stage_k, k_rot, c.num_kv_heads, 1};
  jobs.job[1] = RotateJob{v, cache->r_v, stage_v, v_rot, c.num_kv_heads, 1};
  jobs.n = 2;
  jobs.kind = cache->rotation;
  if (q_rot)
    jobs.job[jobs.n++] = RotateJob{q, cache->r_q ? cache->r_q : cache->r_k, q_rot, nullptr,
                                   c.num_q_heads, c.num_q_heads / c.num_kv_heads};
  if ((st = hip_status(launch_rotate(jobs, (int)n_tok, sm))) != OSCAR_OK) return st;
  // OScaR keys: whole blocks, before any new row can overwrite a ring slot
  // they read (the value rows follow in the quantize launch)
  if (c.key_mode == OSCAR_KEYS_OTS &&
      (st = hip_status(launch_ots_keys(a, clip, sa, stage_k, (int)total_q, sm))) != OSCAR_OK)
    return st;
  // 2+3 in one launch when no new row lands on a ring slot the flush reads
  bool disjoint = true;
  for (int i = 0; disjoint && i < n_seqs; ++i) {
    const int64_t n_new = (int64_t)cu_new_host[i + 1] - cu_new_host[i];
    const int64_t lb = len_before_host[i];
    if (n_new > 0 && (lb + n_new - 1) - s_quant(lb, c) >= a.ring_cap) disjoint = false;
  }
  if (disjoint)
    return hip_status(launch_flush_place(a, clip, sa, stage_k, stage_v, (int)total_q, max_keep, sm));
  // 2. quantize every position that crosses S_quant (reads the ring first)
  if ((st = hip_status(launch_quantize(a, clip, sa, stage_k, stage_v, (int)total_q, sm))) != OSCAR_OK)
    return st;
  // 3. new rows that stay BF16 go to the sink / ring
  return hip_status(launch_place(a, sa, stage_k, stage_v, max_keep, sm));
}

}  // extern "C"

namespace {

// Checks and the split plan shared by the decode entry points.  The plan
// depends only on the configuration, the host lengths and the device, so the
// split and merge calls of one decode step compute the same plan.
// Plans and enqueues one split-K decode call (INT2 or BF16 pages) of
// n_seqs checked sequences.
// cap_override > 0: the most splits per row the workspace holds (a fixed
// scratch buffer), instead of the limit oscar_workspace_size sizes for.
int plan_and_launch(const CacheArgs& a, DecodePlan plan, const DecodeShape& sh, bool bf16,
                    int n_seqs, const int32_t* seq_slots_host, const int32_t* seq_lens_host,
                    const int32_t* seq_slots, const int32_t* seq_lens, const uint16_t* q,
                    float* out, void* workspace, void* stream, int phases, int cap_override = 0) {
  int cus = 256;
  int st = check_device(&cus);
  if (st != OSCAR_OK) return st;
  // Every launch keeps to the split limit the workspace is sized for (that
  // of a full launch), so a short last launch fits in it too.
  const int cap = cap_override > 0 ? cap_override : max_splits(sh, std::min(n_seqs, kMaxScanSeqs));
  // Work-group rows: WH groups of KH KV heads per work-group, or (when such
  // items cannot fill the device within the split limit: small batches) one
  // group of KH heads whose pairs the WH waves divide.
  const int64_t rows_heads = (int64_t)(a.hkv / (plan.wh * plan.kh)) * plan.passes;
  plan.ps = 0;
  if (!bf16 && plan.wh > 1) {
    plan.ps = 1;
    const int64_t slots_ps =
        std::max<int64_t>(1, (int64_t)cus * decode_slots_per_cu(a, plan, bf16) * kFillPercent / 100);
    plan.ps = (int64_t)std::min(n_seqs, kMaxScanSeqs) * rows_heads * cap < slots_ps ? 1 : 0;
  }
  const int64_t rows = plan.ps ? (int64_t)(a.hkv / plan.kh) * plan.passes : rows_heads;
  const int64_t slots =
      std::max<int64_t>(1, (int64_t)cus * decode_slots_per_cu(a, plan, bf16) * kFillPercent / 100);
  static thread_local ItemOrder order;
  static thread_local SplitCounts counts;
  // Launches of at most kMaxScanSeqs sequences, in stream order.
  for (int s0 = 0; s0 < n_seqs; s0 += kMaxScanSeqs) {
    const int ns = std::min(kMaxScanSeqs, n_seqs - s0);
    // Context splits: a work quota per split.  The smallest quota whose work
    // items (one work-group each) all fit in one round of resident
    // work-groups, so none waits for a second round; long sequences get
    // more splits.  The quota never leaves the split limits.
    static thread_local std::vector<int64_t> cost;
    cost.resize(ns);
    int64_t total = 0, max_cost = 0;
    for (int i = 0; i < ns; ++i) {
      cost[i] = decode_cost(seq_lens_host[s0 + i], a);
      total += cost[i];
      max_cost = std::max(max_cost, cost[i]);
    }
    // Small batches whose work gives a full round of work-groups fewer than
    // two units per wave: two thirds of the round (fewer records to merge,
    // the split no slower; measured on a 32K bs1 row: split -0.6 us, merge
    // -0.7 us; a 128K bs1 row keeps the full round)
    int64_t slots_l = slots;
    if (plan.ps && total * rows < 2 * slots * plan.wh) slots_l = std::max<int64_t>(1, slots * 2 / 3);
    // quota in 1/16 units; at most 255 pairs per split (the LDS page list)
    auto splits_of = [&](int64_t c16, int64_t q16) {
      return std::max<int64_t>(1, (16 * c16 + q16 - 1) / q16);
    };
    auto items_of = [&](int64_t q16) {
      int64_t n = 0;
      for (int i = 0; i < ns; ++i) n += splits_of(cost[i], q16);
      return n * rows;
    };
    const int64_t q_max = 16 * (kMaxPairsPerSplit - 1);
    int64_t quota = std::max<int64_t>(32, (16 * total * rows + slots_l - 1) / slots_l);
    quota = std::max<int64_t>(quota, (16 * max_cost + cap - 1) / cap);
    quota = std::min<int64_t>(quota, q_max);
    if (items_of(quota) > slots_l) {   // smallest quota in (quota, limit] that fits (items fall as quota grows)
      int64_t lo = quota, hi = q_max;
      while (hi - lo > 1) {
        const int64_t mid = (lo + hi) / 2;
        (items_of(mid) > slots_l ? lo : hi) = mid;
      }
      quota = hi;
    }
    int64_t smax = 1;
    for (int i = 0; i < ns; ++i) smax = std::max<int64_t>(smax, splits_of(cost[i], quota));
    // unreachable: cap >= min_splits, or (fixed scratch) checked by the caller
    if (smax > cap) return cap_override > 0 ? OSCAR_ERR_WORKSPACE : OSCAR_ERR_CAPACITY;
    plan.quota = (int)quota;
    plan.smax = (int)smax;
    plan.grid = (int)items_of(quota);
    plan.cus = cus;
    // Deal the items out largest first: work-group b takes the b-th largest
    // in its dispatch round, rounds alternating in direction, so the items
    // sharing a compute unit (b, b + cus, ...) add up to about equal work.
    order.n = 0;
    if (plan.grid <= kMaxOrder) {
      static thread_local std::vector<std::pair<int, uint32_t>> items;   // (work units, sequence << 16 | item in it)
      items.clear();
      items.reserve(plan.grid);
      for (int i = 0; i < ns; ++i) {
        const DecodeWork w =
            decode_work(seq_lens_host[s0 + i], a.s_sink, a.s_keep, a.s_flush, a.ring_cap);
        const int nsp = (int)splits_of(cost[i], quota);
        for (int sp = 0; sp < nsp; ++sp) {
          const int pb = (int)((int64_t)sp * w.n_pairs / nsp), pe = (int)((int64_t)(sp + 1) * w.n_pairs / nsp);
          const int wb = (int)((int64_t)sp * w.n_wu / nsp), we = (int)((int64_t)(sp + 1) * w.n_wu / nsp);
          const int units = (pe - pb) + kWinCost * (we - wb);
          for (int r = 0; r < rows; ++r)
            items.emplace_back(units, ((uint32_t)i << 16) | (uint32_t)(sp * rows + r));
        }
      }
      std::stable_sort(items.begin(), items.end(),
                       [](const std::pair<int, uint32_t>& x, const std::pair<int, uint32_t>& y) {
                         return x.first > y.first;
                       });
      for (int b = 0; b < plan.grid; ++b) {
        const int r = b / cus, col = b % cus;
        const int in_round = std::min(cus, plan.grid - r * cus);   // items of this round
        const int k = r * cus + ((r & 1) ? in_round - 1 - col : col);
        const uint32_t it = items[k].second;
        order.item_of[b] = it;
        order.slot[b] = seq_slots_host[s0 + (it >> 16)];
        order.len[b] = seq_lens_host[s0 + (it >> 16)];
      }
      order.n = plan.grid;
    }
    plan.order = &order;
    counts.n = ns;
    for (int i = 0; i < ns; ++i) counts.ns[i] = (uint16_t)splits_of(cost[i], quota);
    plan.counts = &counts;
    const SeqArgs sa{seq_slots + s0, seq_lens + s0, nullptr, ns};
    const size_t qo = (size_t)s0 * a.hq * kD;
    const uint16_t* qs = q ? q + qo : nullptr;
    float* os = out ? out + qo : nullptr;
    const hipError_t e =
        bf16 ? launch_bf16_decode(a, sa, plan, qs, os, (float*)workspace, phases, (hipStream_t)stream)
             : launch_decode(a, sa, plan, qs, os, (float*)workspace, phases, (hipStream_t)stream);
    st = hip_status(e);
    if (st != OSCAR_OK) return st;
  }
  return OSCAR_OK;
}

// ---- plain BF16 paged cache (the uncompressed comparison point) ----------

int check_bf16(const oscar_bf16_cache* b) {
  if (!b) return OSCAR_ERR_NULL;
  if (b->head_dim != kD || b->page_size != kPage) return OSCAR_ERR_SHAPE;
  if (b->num_kv_heads < 1 || b->num_kv_heads > OSCAR_MAX_KV_HEADS) return OSCAR_ERR_SHAPE;
  if (b->num_q_heads < b->num_kv_heads || b->num_q_heads % b->num_kv_heads != 0)
    return OSCAR_ERR_SHAPE;
  if (b->num_q_heads / b->num_kv_heads > 256) return OSCAR_ERR_SHAPE;
  if (b->max_seqs < 1 || b->max_pages_per_seq < 0 || b->num_pages < 0) return OSCAR_ERR_CAPACITY;
  if (b->max_pages_per_seq > kMaxPagesPerSeq) return OSCAR_ERR_CAPACITY;
  return OSCAR_OK;
}

// Query heads per pass: a power of two covering g, at most the 16 columns of
// an MFMA tile.
DecodePlan bf16_plan(const oscar_bf16_cache& b) {
  const int g = b.num_q_heads / b.num_kv_heads;
  int hp = 1;
  while (hp < g && hp < 16) hp *= 2;
  DecodePlan p{};
  p.hp = hp;
  p.passes = (g + hp - 1) / hp;
  p.kh = 1;
  p.wh = b.num_kv_heads % 4 == 0 ? 4 : (b.num_kv_heads % 2 == 0 ? 2 : 1);
  p.quota = 1;
  p.smax = 1;
  return p;
}

DecodeShape bf16_shape(const oscar_bf16_cache& b) {
  const DecodePlan p = bf16_plan(b);
  return DecodeShape{b.num_kv_heads, p.passes, p.hp, ((int64_t)b.max_pages_per_seq + 1) / 2};
}

// The BF16 cache as kernel arguments: no windows (s_sink = s_keep = 0,
// s_flush = 1, so every token is a "page" token and decode_work counts the
// row's page pairs); one page-head block = 16 K rows + 16 V rows of bf16.
CacheArgs make_bf16_args(const oscar_bf16_cache& b) {
  CacheArgs a{};
  a.pages = (uint8_t*)b.pages;
  a.block_table = b.block_table;
  a.hq = b.num_q_heads;
  a.hkv = b.num_kv_heads;
  a.g = b.num_q_heads / b.num_kv_heads;
  a.group = kD;
  a.ng = 1;
  a.s_sink = 0;
  a.s_keep = 0;
  a.s_flush = 1;
  a.ring_cap = 0;
  a.max_seqs = b.max_seqs;
  a.max_pages = b.max_pages_per_seq;
  a.num_pages = b.num_pages;
  a.page_bytes = 2 * kPage * kD * (int)sizeof(uint16_t);
  return a;
}

// ---- fixed device scratch of oscar_int2_decode_attn_noalloc ---------------
// A file-scope device array: each GPU the library runs on holds its own copy
// until the process ends.  Host code never uses the array's name as an
// address: the per-device address comes from hipGetSymbolAddress, taken once
// per device with that device current.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

hipError_t device_scratch(void** out) {
  static std::mutex mu;
  static void* addr[64] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

// Most splits per row whose partial records fit in the scratch for a launch
// of n_seqs sequences.
int scratch_splits(const DecodeShape& sh, int n_seqs) {
  const int ns = std::min(std::max(1, n_seqs), kMaxScanSeqs);
  const size_t per_split = (size_t)ns * sh.hkv * sh.passes * rec_words(sh.hp) * sizeof(float);
  return (int)std::min<size_t>(kMaxSplits, kScratchBytes / per_split);
}

// noalloc: the split records go to the fixed scratch instead of `workspace`.
int decode_step(const oscar_kv_cache* cache, int32_t n_seqs, const int32_t* seq_slots_host,
                const int32_t* seq_lens_host, const int32_t* seq_slots, const int32_t* seq_lens,
                const uint16_t* q_rot, float* out, void* workspace, size_t workspace_bytes,
                void* stream, int phases, bool noalloc = false) {
  if (!cache) return OSCAR_ERR_NULL;
  const oscar_kv_config& c = cache->cfg;
  int st = oscar_check_config(&c);
  if (st != OSCAR_OK) return st;
  if (!seq_slots_host || !seq_lens_host || !seq_slots || !seq_lens || (!noalloc && !workspace) ||
      !cache->pages || !cache->block_table || !cache->win ||
      (dense(*cache) && !cache->r_v && !cache->out_rotated))
    return OSCAR_ERR_NULL;
  if (!rotation_ok(*cache)) return OSCAR_ERR_ARG;
  if (((phases & kDecodeSplit) && !q_rot) || ((phases & kDecodeMerge) && !out)) return OSCAR_ERR_NULL;
  if (!aligned16(q_rot) || !aligned16(out) || !cache_aligned(*cache) ||
      (!noalloc && !aligned16(workspace)))
    return OSCAR_ERR_ARG;
  if (n_seqs < 1 || n_seqs > c.max_seqs) return OSCAR_ERR_ARG;
  // separate split and merge calls share one launch's workspace
  if (phases != (kDecodeSplit | kDecodeMerge) && n_seqs > kMaxScanSeqs) return OSCAR_ERR_ARG;
  const int64_t max_len = oscar_max_seq_len(&c);
  for (int i = 0; i < n_seqs; ++i) {
    const int slot = seq_slots_host[i];
    const int64_t len = seq_lens_host[i];
    if (slot < 0 || slot >= c.max_seqs) return OSCAR_ERR_CAPACITY;
    if (len < 1) return OSCAR_ERR_ARG;
    if (len > max_len || int2_pages(len, c) > c.max_pages_per_seq) return OSCAR_ERR_CAPACITY;
    if (int2_pages(len, c) > 0 && c.num_pages < 1) return OSCAR_ERR_CAPACITY;
  }
  const CacheArgs args = make_args(*cache);
  int cap = 0;
  if (noalloc) {
    // the longest row must fit its splits in the scratch at the largest
    // split quota (kMaxPairsPerSplit - 1 work units per split)
    cap = scratch_splits(int2_shape(c), n_seqs);
    int64_t max_cost = 0;
    for (int i = 0; i < n_seqs; ++i) max_cost = std::max(max_cost, decode_cost(seq_lens_host[i], args));
    if (cap < 1 || (max_cost + kMaxPairsPerSplit - 2) / (kMaxPairsPerSplit - 1) > cap)
      return OSCAR_ERR_WORKSPACE;
    if ((st = check_device()) != OSCAR_OK) return st;
    if ((st = hip_status(device_scratch(&workspace))) != OSCAR_OK) return st;
  } else if (workspace_bytes < partials_bytes(int2_shape(c), n_seqs)) {
    return OSCAR_ERR_WORKSPACE;
  }
  return plan_and_launch(args, head_passes(c), int2_shape(c), false, n_seqs, seq_slots_host,
                         seq_lens_host, seq_slots, seq_lens, q_rot, out, workspace, stream, phases,
                         cap);
}


}  // namespace

extern "C" {

int oscar_int2_decode_attn(const oscar_kv_cache* cache, int32_t n_seqs,
                           const int32_t* seq_slots_host, const int32_t* seq_lens_host,
                           const int32_t* seq_slots, const int32_t* seq_lens,
                           const uint16_t* q_rot, float* out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return decode_step(cache, n_seqs, seq_slots_host, seq_lens_host, seq_slots, seq_lens, q_rot, out,
                     workspace, workspace_bytes, stream, kDecodeSplit | kDecodeMerge);
}

int oscar_int2_decode_partials(const oscar_kv_cache* cache, int32_t n_seqs,
                               const int32_t* seq_slots_host, const int32_t* seq_lens_host,
                               const int32_t* seq_slots, const int32_t* seq_lens,
                               const uint16_t* q_rot, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return decode_step(cache, n_seqs, seq_slots_host, seq_lens_host, seq_slots, seq_lens, q_rot,
                     nullptr, workspace, workspace_bytes, stream, kDecodeSplit);
}

int oscar_int2_decode_merge(const oscar_kv_cache* cache, int32_t n_seqs,
                            const int32_t* seq_slots_host, const int32_t* seq_lens_host,
                            const int32_t* seq_slots, const int32_t* seq_lens, float* out,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return decode_step(cache, n_seqs, seq_slots_host, seq_lens_host, seq_slots, seq_lens, nullptr,
                     out, workspace, workspace_bytes, stream, kDecodeMerge);
}


int oscar_int2_decode_attn_noalloc(const oscar_kv_cache* cache, int32_t n_seqs,
                                   const int32_t* seq_slots_host, const int32_t* seq_lens_host,
                                   const int32_t* seq_slots, const int32_t* seq_lens,
                                   const uint16_t* q_rot, float* out, void* stream) {
  return decode_step(cache, n_seqs, seq_slots_host, seq_lens_host, seq_slots, seq_lens, q_rot, out,
                     nullptr, 0, stream, kDecodeSplit | kDecodeMerge, true);
}

size_t oscar_bf16_workspace_size(const oscar_bf16_cache* cache, int32_t n_seqs) {
  if (check_bf16(cache) != OSCAR_OK) return 0;
  return partials_bytes(bf16_shape(*cache), std::max(1, (int)n_seqs));
}

int oscar_bf16_paged_decode_attn(const oscar_bf16_cache* cache, int32_t n_seqs,
                                 const int32_t* seq_slots_host, const int32_t* seq_lens_host,
                                 const int32_t* seq_slots, const int32_t* seq_lens,
                                 const uint16_t* q, float* out, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  int st = check_bf16(cache);
  if (st != OSCAR_OK) return st;
  const oscar_bf16_cache& b = *cache;
  if (!seq_slots_host || !seq_lens_host || !seq_slots || !seq_lens || !q || !out || !workspace ||
      !b.pages || !b.block_table)
    return OSCAR_ERR_NULL;
  if (!aligned16(q) || !aligned16(out) || !aligned16(workspace) || !aligned16(b.pages) ||
      !aligned16(b.block_table))
    return OSCAR_ERR_ARG;
  if (n_seqs < 1 || n_seqs > b.max_seqs) return OSCAR_ERR_ARG;
  for (int i = 0; i < n_seqs; ++i) {
    const int slot = seq_slots_host[i];
    const int64_t len = seq_lens_host[i];
    if (slot < 0 || slot >= b.max_seqs) return OSCAR_ERR_CAPACITY;
    if (len < 1) return OSCAR_ERR_ARG;
    if ((len + kPage - 1) / kPage > b.max_pages_per_seq || b.num_pages < 1) return OSCAR_ERR_CAPACITY;
  }
  if (workspace_bytes < partials_bytes(bf16_shape(b), n_seqs)) return OSCAR_ERR_WORKSPACE;
  return plan_and_launch(make_bf16_args(b), bf16_plan(b), bf16_shape(b), true, n_seqs,
                         seq_slots_host, seq_lens_host, seq_slots, seq_lens, q, out, workspace,
                         stream, kDecodeSplit | kDecodeMerge);
}

int oscar_int2_prefill_attn(const oscar_kv_cache* cache, int32_t n_seqs,
                            const int32_t* seq_slots_host, const int32_t* len_before_host,
                            const int32_t* cu_new_host, const int32_t* seq_slots,
                            const int32_t* len_before, const int32_t* cu_new,
                            const uint16_t* q_rot, const uint16_t* k_rot, const uint16_t* v_rot,
                            float* out, void* stream) {
  if (!cache) return OSCAR_ERR_NULL;
  const oscar_kv_config& c = cache->cfg;
  int st = oscar_check_config(&c);
  if (st != OSCAR_OK) return st;
  if (!seq_slots_host || !len_before_host || !cu_new_host || !seq_slots || !len_before ||
      !cu_new || !q_rot || !k_rot || !v_rot || !out || !cache->pages || !cache->block_table ||
      !cache->win || (dense(*cache) && !cache->out_rotated && !cache->r_v))
    return OSCAR_ERR_NULL;
  if (!rotation_ok(*cache) || c.key_mode != OSCAR_KEYS_CLIP) return OSCAR_ERR_ARG;
  if (!aligned16(q_rot) || !aligned16(k_rot) || !aligned16(v_rot) || !aligned16(out) ||
      !cache_aligned(*cache))
    return OSCAR_ERR_ARG;
  if (n_seqs < 1 || n_seqs > c.max_seqs || n_seqs > 65535) return OSCAR_ERR_ARG;
  if (cu_new_host[0] != 0) return OSCAR_ERR_ARG;
  const int64_t max_len = oscar_max_seq_len(&c);
  const int g = c.num_q_heads / c.num_kv_heads;
  std::vector<char> seen(c.max_seqs, 0);
  int64_t prefix = 0, chunk = 0;
  int bf16_only = 1;   // every key below the chunks is a bf16 row
  for (int i = 0; i < n_seqs; ++i) {
    const int slot = seq_slots_host[i];
    if (slot < 0 || slot >= c.max_seqs) return OSCAR_ERR_CAPACITY;
    if (seen[slot]) return OSCAR_ERR_ARG;
    seen[slot] = 1;
    const int64_t n_new = (int64_t)cu_new_host[i + 1] - cu_new_host[i];
    const int64_t lb = len_before_host[i];
    if (n_new < 0 || lb < 0) return OSCAR_ERR_ARG;
    if (lb + n_new > max_len || int2_pages(lb + n_new, c) > c.max_pages_per_seq)
      return OSCAR_ERR_CAPACITY;
    if (n_new * g > ((int64_t)1 << 30)) return OSCAR_ERR_ARG;
    prefix += lb * n_new;
    chunk += n_new * n_new / 2;
    if (std::min(s_quant(lb + n_new, c), lb) > c.s_sink) bf16_only = 0;
  }
  // Query rows per work-group: 256 when the chunks attend mostly to a cached
  // INT2 prefix (a staged key block then serves twice the rows), else 128
  // (smaller tiles waste less of the causal triangle; bf16 mode always)
  const int blocks = (!bf16_only && prefix > chunk) ? 16 : 8;
  int tiles = 0;
  for (int i = 0; i < n_seqs; ++i)
    tiles = std::max(tiles, prefill_tiles(cu_new_host[i + 1] - cu_new_host[i], g, blocks));
  const int64_t n_tok = cu_new_host[n_seqs];
  if (n_tok > (int64_t)1 << 30) return OSCAR_ERR_ARG;
  if ((st = check_device()) != OSCAR_OK) return st;
  if (n_tok == 0) return OSCAR_OK;
  const PrefillArgs pa{seq_slots, len_before, cu_new, q_rot, k_rot, v_rot, out, n_seqs, tiles,
                       blocks, bf16_only, div_magic((uint32_t)g),
                       div_magic((uint32_t)std::max(1, ring_cap(c)))};
  return hip_status(launch_prefill(make_args(*cache), pa, (hipStream_t)stream));
}

int oscar_dequant(const oscar_kv_cache* cache, int32_t seq_slot, int32_t seq_len,
                  int32_t tok_begin, int32_t tok_end, float* k_out, float* v_out, void* stream) {
  if (!cache) return OSCAR_ERR_NULL;
  const oscar_kv_config& c = cache->cfg;
  int st = oscar_check_config(&c);
  if (st != OSCAR_OK) return st;
  if (!k_out || !v_out || !cache->pages || !cache->block_table || !cache->win)
    return OSCAR_ERR_NULL;
  if (seq_slot < 0 || seq_slot >= c.max_seqs) return OSCAR_ERR_CAPACITY;
  if (seq_len < 0 || seq_len > oscar_max_seq_len(&c) ||
      int2_pages(seq_len, c) > c.max_pages_per_seq)
    return OSCAR_ERR_CAPACITY;
  if (tok_begin < 0 || tok_end < tok_begin || tok_end > seq_len) return OSCAR_ERR_ARG;
  if ((st = check_device()) != OSCAR_OK) return st;
  return hip_status(launch_dequant(make_args(*cache), seq_slot, seq_len, tok_begin, tok_end, k_out,
                                   v_out, (hipStream_t)stream));
}

}  // extern "C"

extern "C" int oscar_round_f64_host(int32_t target, const double* x, uint16_t* out, int64_t n) {
  if (!x || !out) return OSCAR_ERR_NULL;
  if (n < 0 || target < 0 || target > 2) return OSCAR_ERR_ARG;
  for (int64_t i = 0; i < n; ++i)
    out[i] = target == 0 ? oscar::f64_to_bf16_rne(x[i])
                         : (target == 1 ? oscar::f64_to_f16_rne(x[i]) : oscar::f64_to_bf16_rne_normal(x[i]));
  return OSCAR_OK;
}
