/*
 * liboscar_kv -- INT2 KV cache with a fixed per-head rotation and clipped
 * asymmetric 2-bit quantization, BF16 sink / recent windows, and paged GQA
 * decode attention over the mixed cache.  MI355X (gfx950) only.
 *
 * Sources (the pages this library implements):
 *  [OSCAR]  "OSCAR: Offline Spectral Covariance-Aware Rotation for 2-bit KV
 *           Cache Quantization", paperlayer.ai summary: section 3 (fixed
 *           rotations and clipping thresholds, affine asymmetric INT2 with
 *           scale and zero point, per-token groups), section 4 (mixed
 *           precision paged cache with BF16 sink and recent windows, fused
 *           clip-quantize-pack writing four 2-bit codes per byte, demotion
 *           of the oldest recent tokens, decode attention that unpacks INT2
 *           and accumulates in floating point, segments merged after two
 *           launches), section 5 (R = U . H_Had . P_br), appendix B
 *           (Algorithm 1: rotate before the cache write).
 *  [OScaR]  OScaR reading notes (zhongzhuzhou.org): uniform quantizer and
 *           dequantizer formulas, orthogonal transforms preserve q.k.
 *  [WUSH]   WUSH-KV notes (paper.rainbus.top), "method step details": the
 *           key transform is applied after RoPE to new keys and queries;
 *           S_quant advances over S_flush-aligned segments beyond the
 *           S_sink / S_keep windows; kappa-quantile clipped affine quantizer.
 *
 * Conventions
 *  - head_dim D = 128, page size P = 16, G in {32, 64, 128}, ng = 128 / G.
 *  - Rows are row vectors: x' = x . R with R row-major [128][128] fp32.
 *    Keys and queries use R_K of their KV head (query head hq belongs to KV
 *    head hq / g, g = Hq / Hkv); values use R_V.  The decode output is
 *    returned in the original basis: o = o' . R_V^T.
 *  - bf16 and fp16 values travel as uint16_t bit patterns.
 *  - Every pointer argument is a DEVICE pointer unless its name ends in
 *    _host.  Device buffers (cache arrays, rows, workspace, output) must be
 *    16-byte aligned (OSCAR_ERR_ARG otherwise).  The caller owns all memory;
 *    the library allocates nothing and keeps no state between calls (the one
 *    exception is the fixed device scratch of
 *    oscar_int2_decode_attn_noalloc, declared below).
 *  - Calls enqueue work on `stream` (a hipStream_t; NULL = default stream)
 *    and return without waiting.  Calls that touch the same cache or the
 *    same workspace must be ordered on one stream by the caller.
 *  - All argument checks run on the host before anything is enqueued; on a
 *    non-zero status nothing was enqueued (except OSCAR_ERR_HIP, which
 *    reports a failed launch).  Non-finite inputs, and rotated values whose
 *    magnitude exceeds the fp16 range, are outside the contract.
 *
 * Cache placement (per cache row, after `len` tokens)            [OSCAR s4, WUSH]
 *  S_quant(len) = S_sink + S_flush * max(0, floor((len - S_sink - S_keep) / S_flush))
 *  position p < min(len, S_sink)          -> sink window, bf16, slot p
 *  S_sink <= p < S_quant                   -> INT2, logical page (p - S_sink) / 16,
 *                                            slot (p - S_sink) % 16
 *  max(S_quant, S_sink) <= p < len         -> recent ring, bf16,
 *                                            slot (p - S_sink) mod R,
 *                                            R = roundup16(S_keep + S_flush)
 *  Rows are always the bf16 rounding of the exact x . R; INT2 rows are the
 *  quantization of that bf16 row, so the cache does not depend on how the
 *  tokens were grouped into append calls.
 *
 * Quantizer (one token, one KV head, one group of G channels)    [OSCAR s3, OScaR, WUSH]
 *  s = the group's values sorted; for q in {kappa, 1 - kappa}:
 *  h = (G - 1) q, i = floor(h), v(q) = s[i] + (h - i) (s[min(i+1, G-1)] - s[i])
 *  (fp64, in this order); hi = v(kappa), lo = v(1 - kappa);
 *  scale = fp16_rne((hi - lo) / 3), zero = fp16_rne(lo) (one rounding from fp64);
 *  code = [x > zero + scale/2] + [x >= zero + 3 scale/2] + [x > zero + 5 scale/2],
 *  or 0 when scale == 0; dequantized value = scale * code + zero.
 *
 * On-HBM layout
 *  pages: uint8 [num_pages][Hkv][PB], PB = 1024 + 128 * ng bytes per page-head:
 *   [0, 512)           K codes, uint32 word (8 t + w) holds channels 16 w + i
 *                      (i = 0..15) of slot t at bits 2i .. 2i+1.
 *   [512, 1024)        V codes, uint32 word u = 2 (16 a + m) + e holds
 *                      code(slot 4a + 2e,     channel 8m + j) at bits 2j .. 2j+1,
 *                      code(slot 4a + 2e + 1, channel 8m + j) at bits 16+2j .. 17+2j
 *                      (a = 0..3, m = 0..15, e = 0..1, j = 0..7).
 *   [1024, 1024+64ng)  K params, uint32 word (16 gr + t): fp16 scale (bits 0..15),
 *                      fp16 zero (bits 16..31) of group gr, slot t.
 *   [1024+64ng, PB)    V params, same order.
 *  block_table: int32 [max_seqs][max_pages_per_seq]: physical page of logical
 *   INT2 page m of a cache row.  Entries outside [0, num_pages) are skipped.
 *  win: bf16 [max_seqs][Hkv][NB][2][16][128], NB = ceil(S_sink/16) + R/16;
 *   block b < ceil(S_sink/16) holds sink slots 16b + t, the rest hold ring
 *   slots 16 (b - ceil(S_sink/16)) + t.  Part 0 (K) is row-major (element
 *   128 t + c); part 1 (V) holds (t, c) at element
 *   32 (16 (t/4) + c/8) + 4 (c%8) + t%4.
 *  pages and win must be zero-filled once when allocated (slots that were
 *  never written are read with zero weight, so they must hold finite data).
 *
 * OScaR key mode (cfg.key_mode = OSCAR_KEYS_OTS)                 [OScaR]
 *  Keys of the INT2 segment are quantized as in the OScaR notes (step two
 *  "Omni-Token Scaling" and the background "KIVI and the per-channel
 *  paradigm"): for each rotated bf16 key row k~ (one token, one KV head),
 *  s = bf16_rne(sqrt(sum_j k~_j^2)) (squares summed in fp64, correctly
 *  rounded square root) and u_j = bf16_rne(k~_j / s) (u = 0 when s = 0);
 *  then over each block of 32 consecutive INT2 positions (INT2 tokens
 *  32b .. 32b + 31, i.e. logical pages 2b and 2b + 1) and each channel j:
 *  Delta_j = bf16_rne((max_t u - min_t u) / 3), z_j = bf16_rne(-min_t u /
 *  Delta_j) and code = [u > Delta (1/2 - z)] + [u >= Delta (3/2 - z)] +
 *  [u > Delta (5/2 - z)] (fp64, exact); a constant channel (Delta_j = 0)
 *  keeps z_j = bf16_rne(min_t u) and codes 0.  Dequantized key:
 *  s * Delta_j * (code - z_j), or s * z_j when Delta_j = 0.  Values are
 *  quantized per token exactly as in the default mode (clip_v, G = 32);
 *  clip_k is not used.  Requires group_size = 32 and s_flush a multiple of
 *  32 (a flush then moves whole key blocks).  Page-head block of 1568 bytes:
 *   [0, 512)      K codes, the layout above
 *   [512, 1024)   V codes, the layout above
 *   [1024, 1280)  V params, the layout above (ng = 4)
 *   [1280, 1312)  the 16 token scales s (bf16; slot t at bytes 1280 + 2t)
 *   [1312, 1568)  uint32 word i: bf16 Delta (bits 0..15) | bf16 z (bits 16..31)
 *                 of channel 64 (m % 2) + i of the key block of logical page m
 *  98 bytes per INT2 token and KV head (5.2x fewer than bf16).
 *
 * Status codes: 0 on success, a negative OSCAR_ERR_* otherwise.
 */
#ifndef OSCAR_KV_H
#define OSCAR_KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define OSCAR_HEAD_DIM 128
#define OSCAR_PAGE_SIZE 16
#define OSCAR_MAX_KV_HEADS 64

enum oscar_status {
  OSCAR_OK = 0,
  OSCAR_ERR_NULL = -1,       /* a required pointer is NULL */
  OSCAR_ERR_SHAPE = -2,      /* head_dim != 128, page_size != 16, Hq % Hkv, Hkv out of range */
  OSCAR_ERR_GROUP = -3,      /* group_size not in {32, 64, 128} */
  OSCAR_ERR_CLIP = -4,       /* a clip ratio is not in [0.5, 1] */
  OSCAR_ERR_WINDOW = -5,     /* s_sink < 0, s_keep < 0 or s_flush < 1 */
  OSCAR_ERR_CAPACITY = -6,   /* slot, length or page count beyond the cache */
  OSCAR_ERR_WORKSPACE = -7,  /* workspace smaller than oscar_workspace_size() */
  OSCAR_ERR_DEVICE = -8,     /* current device is not gfx950 */
  OSCAR_ERR_HIP = -9,        /* a HIP runtime call or launch failed */
  OSCAR_ERR_ARG = -10        /* other invalid argument (counts, ranges, duplicates) */
};

typedef struct {
  int32_t head_dim;           /* must be 128 */
  int32_t num_q_heads;        /* Hq, a multiple of num_kv_heads */
  int32_t num_kv_heads;       /* Hkv, 1 .. 64 */
  int32_t group_size;         /* G: 32, 64 or 128 channels per quantization group */
  int32_t page_size;          /* must be 16 */
  int32_t s_sink;             /* BF16 sink window (first tokens), >= 0 */
  int32_t s_keep;             /* BF16 recent window kept after a flush, >= 0 */
  int32_t s_flush;            /* flush granularity, >= 1 */
  int32_t max_seqs;           /* cache rows */
  int32_t max_pages_per_seq;  /* block table width */
  int32_t num_pages;          /* physical pages in the pool */
  float clip_k[OSCAR_MAX_KV_HEADS]; /* kappa for keys, per KV head, in [0.5, 1] */
  float clip_v[OSCAR_MAX_KV_HEADS]; /* kappa for values, per KV head, in [0.5, 1] */
  int32_t key_mode;           /* OSCAR_KEYS_CLIP (0) or OSCAR_KEYS_OTS (1), see above */
} oscar_kv_config;

enum oscar_key_mode {
  OSCAR_KEYS_CLIP = 0,        /* per-token clipped groups of G channels (OSCAR) */
  OSCAR_KEYS_OTS = 1          /* per-token scale, per-channel blocks of 32 tokens (OScaR) */
};

typedef struct {
  oscar_kv_config cfg;
  uint8_t* pages;             /* [num_pages][Hkv][PB] INT2 pages (layout above) */
  const int32_t* block_table; /* [max_seqs][max_pages_per_seq] */
  uint16_t* win;              /* [max_seqs][Hkv][NB][2][16][128] bf16 windows */
  const float* r_k;           /* [Hkv][128][128] fp32 key/query rotation */
  const float* r_v;           /* [Hkv][128][128] fp32 value rotation */
  /* Query transform [Hkv][128][128] fp32, or NULL: queries then use r_k.  A
   * general invertible key transform T (WUSH-KV notes, "core method": any
   * mutually inverse pair between the two factors of K^T Q leaves the scores
   * unchanged) takes r_k = T and r_q = T^-T, so q' . k' = q . k. */
  const float* r_q;
  /* Non-zero: the value transform is absorbed into the output projection
   * (OSCAR summary s4 "KV Cache Layout", WUSH-KV notes: W_O absorbs the
   * inverse value transform), so decode returns o' in the rotated basis and
   * does not read r_v. */
  int32_t out_rotated;
  /* Rotation kind.  OSCAR_ROT_DENSE: the matrices above.  The structured
   * kinds rotate keys, values and queries of every head by one fixed
   * orthogonal matrix built from Sylvester's Hadamard matrix H (entries
   * H[i][k] = (-1)^popcount(i & k)), with no matrix in memory (r_k, r_v and
   * r_q must be NULL, OSCAR_ERR_ARG otherwise):
   *   OSCAR_ROT_HADAMARD         R = H / sqrt(128)  (OScaR notes, step one
   *                              "Canalized Rotation"; the QuaRot-style baseline)
   *   OSCAR_ROT_HADAMARD_BITREV  R = H P_br / sqrt(128), P_br the 7-bit
   *                              bit-reversal permutation of the channels
   *                              (OSCAR summary page, section 5 "Rotation
   *                              Analysis": the Hadamard and bit-reversal
   *                              factors of R = U H P_br)
   * The rotated row is the bf16 rounding of x . R: the transform runs as a
   * fast Walsh-Hadamard transform (7 butterfly stages, exact fp64 sums for
   * rows whose magnitudes span less than 2^38) scaled once by fp64
   * 1/sqrt(128).  The decode merge and the prefill epilogue un-rotate with
   * R^T = R^-1 generated in registers. */
  int32_t rotation;
} oscar_kv_cache;

enum oscar_rotation {
  OSCAR_ROT_DENSE = 0,
  OSCAR_ROT_HADAMARD = 1,
  OSCAR_ROT_HADAMARD_BITREV = 2
};

/* Checks a configuration; returns OSCAR_OK or the first failing OSCAR_ERR_*
 * (an unknown key_mode is OSCAR_ERR_ARG; OScaR key mode with group_size != 32
 * is OSCAR_ERR_GROUP and with s_flush % 32 != 0 OSCAR_ERR_WINDOW). */
int oscar_check_config(const oscar_kv_config* cfg);

/* Byte sizes of the caller-allocated cache buffers (0 for an invalid cfg).
 * oscar_page_head_bytes: PB of the default key mode for a group size;
 * oscar_config_page_head_bytes: PB of a configuration (1568 in OScaR key mode). */
size_t oscar_page_head_bytes(int32_t group_size);
size_t oscar_config_page_head_bytes(const oscar_kv_config* cfg);
size_t oscar_pages_bytes(const oscar_kv_config* cfg);
size_t oscar_win_bytes(const oscar_kv_config* cfg);
int32_t oscar_ring_capacity(const oscar_kv_config* cfg);
/* Longest sequence a cache row can hold (INT2 pages + ring + sink). */
int64_t oscar_max_seq_len(const oscar_kv_config* cfg);

/* Workspace bytes needed by oscar_rotate_quant_append with at most
 * `max_new_tokens` new tokens per call and by oscar_int2_decode_attn with at
 * most `n_seqs` sequences per call.  The workspace holds scratch data of one
 * call only (staged rotated rows, split partials); its content need not be
 * initialized and is not used across calls. */
size_t oscar_workspace_size(const oscar_kv_config* cfg, int32_t n_seqs, int64_t max_new_tokens);

/* Append new tokens of n_seqs sequences: rotate, place, flush, quantize.
 * [OSCAR s4 "KV Cache Update", appendix B; WUSH "method step details"]
 *  seq_slots[i]   cache row of sequence i (distinct, < max_seqs)
 *  len_before[i]  tokens already in that row
 *  cu_new[i]      prefix sums of new-token counts, cu_new[0] = 0,
 *                 new tokens of sequence i are rows cu_new[i] .. cu_new[i+1]-1
 *  (_host arrays are read on the host for checks, launch sizes and the
 *  per-sequence table passed in the kernel arguments of calls with at most
 *  512 sequences; the device arrays must hold the same values)
 *  k, v           bf16 [cu_new[n]][Hkv][128] post-RoPE keys / values
 *  q              bf16 [cu_new[n]][Hq][128] post-RoPE queries, or NULL
 *  q_rot          bf16 [cu_new[n]][Hq][128] out: q . R_K (q . r_q when the cache
 *                 has a query transform), or NULL (needs q)
 *  k_rot, v_rot   bf16 [cu_new[n]][Hkv][128] out: the rotated rows, or NULL
 * Positions that the flush rule moves to INT2 are quantized into the pages
 * (previously recent rows are read from the ring before it is overwritten),
 * the rest go to the sink or the ring.  The block table must already map
 * every logical page below ceil((S_quant(len_after) - S_sink) / 16). */
int oscar_rotate_quant_append(const oscar_kv_cache* cache, int32_t n_seqs,
                              const int32_t* seq_slots_host, const int32_t* len_before_host,
                              const int32_t* cu_new_host,
                              const int32_t* seq_slots, const int32_t* len_before,
                              const int32_t* cu_new,
                              const uint16_t* k, const uint16_t* v, const uint16_t* q,
                              uint16_t* q_rot, uint16_t* k_rot, uint16_t* v_rot,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Decode attention of one query token per sequence over its whole cache row.
 * [OSCAR s2, s4 "Decoding Attention Kernel"; OScaR "KV cache"]
 *  seq_lens[i]    tokens in the row, including the token just appended (>= 1)
 *  q_rot          bf16 [n_seqs][Hq][128] rotated queries (from the append call)
 *  out            fp32 [n_seqs][Hq][128]: softmax(q' K^T / sqrt(128)) V . R_V^T, or
 *                 without the final R_V^T when cache->out_rotated is set
 * Split-K over the context: one launch writes partial results (max, sum,
 * unnormalized output) of each context split to the workspace, a second
 * launch merges them (log-sum-exp) and applies R_V^T.  In OScaR key mode
 * the INT2 keys enter as s * Delta_j * (code - z_j) [OScaR, "Omni-Token
 * Scaling": the token scale multiplies the per-channel dequantized row]. */
int oscar_int2_decode_attn(const oscar_kv_cache* cache, int32_t n_seqs,
                           const int32_t* seq_slots_host, const int32_t* seq_lens_host,
                           const int32_t* seq_slots, const int32_t* seq_lens,
                           const uint16_t* q_rot, float* out,
                           void* workspace, size_t workspace_bytes, void* stream);

/* The two launches of oscar_int2_decode_attn as separate calls, for callers
 * that schedule or time them apart [OSCAR s4 "Decoding Attention Kernel":
 * the split-K partials and their log-sum-exp merge].  A merge call must
 * follow the partials call of the same step on the same stream, with the
 * same cache, sequence arguments and workspace; together they compute
 * exactly what oscar_int2_decode_attn computes.
 *  oscar_int2_decode_partials: q_rot as above; writes the partial records
 *                              (max, sum, unnormalized o' per context split)
 *                              to the workspace.
 *  oscar_int2_decode_merge:    out as above; reads those records.
 * These two calls take at most 2048 sequences (OSCAR_ERR_ARG otherwise). */
int oscar_int2_decode_partials(const oscar_kv_cache* cache, int32_t n_seqs,
                               const int32_t* seq_slots_host, const int32_t* seq_lens_host,
                               const int32_t* seq_slots, const int32_t* seq_lens,
                               const uint16_t* q_rot,
                               void* workspace, size_t workspace_bytes, void* stream);
int oscar_int2_decode_merge(const oscar_kv_cache* cache, int32_t n_seqs,
                            const int32_t* seq_slots_host, const int32_t* seq_lens_host,
                            const int32_t* seq_slots, const int32_t* seq_lens, float* out,
                            void* workspace, size_t workspace_bytes, void* stream);

/* oscar_int2_decode_attn without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, serving loops
 * and harnesses that forbid hipMalloc).  It computes what
 * oscar_int2_decode_attn computes with the same kernels; the split records
 * go to a fixed 64 MiB scratch array that the library holds on each GPU it
 * runs on until the process ends.  The call allocates nothing.
 * Limit: the records of a launch (at most 2048 sequences) must fit in the
 * scratch: a launch of n sequences keeps at most S splits per (sequence, KV
 * head, query-head pass) with n * Hkv * passes * S * record bytes <= 64 MiB,
 * and a call whose longest row needs more splits
 * returns OSCAR_ERR_WORKSPACE with nothing enqueued.  Every call on a GPU
 * shares that GPU's scratch: calls that overlap on one GPU (different
 * streams, or different host threads without ordering) race and must not be
 * made.  The scratch needs no clearing: every record the merge reads is
 * written by the split launch of the same call.  Other errors as for
 * oscar_int2_decode_attn. */
int oscar_int2_decode_attn_noalloc(const oscar_kv_cache* cache, int32_t n_seqs,
                                   const int32_t* seq_slots_host, const int32_t* seq_lens_host,
                                   const int32_t* seq_slots, const int32_t* seq_lens,
                                   const uint16_t* q_rot, float* out, void* stream);

/* Chunked-prefill attention: the new tokens of each sequence, just added by
 * oscar_rotate_quant_append, attend causally over the mixed cache.
 * [WUSH "method step details" (inference, Algorithm 2): the chunk's rows join
 * the cache at full precision and grouped-query attention runs over the
 * mixed-precision cache; OSCAR s2: softmax(Q K^T / sqrt(d)) V row by row]
 *  seq_slots, len_before, cu_new  the arguments of that append call (host and
 *                 device copies holding the same values)
 *  q_rot          bf16 [cu_new[n]][Hq][128] rotated queries (the append's q_rot)
 *  k_rot, v_rot   bf16 [cu_new[n]][Hkv][128] the chunk's rotated rows (the
 *                 append's k_rot / v_rot outputs)
 *  out            fp32 [cu_new[n]][Hq][128]: the query at chunk row j of sequence
 *                 i (position P = len_before[i] + j) attends to positions 0 .. P:
 *                 positions below len_before[i] as the cache holds them after the
 *                 append (bf16 sink / recent rows, INT2 rows as scale * code +
 *                 zero), the chunk's rows at their bf16 values whether or not the
 *                 append moved them to INT2; softmax(q' K^T / sqrt(128)) V . R_V^T,
 *                 without the R_V^T when cache->out_rotated is set.
 * Unmapped INT2 pages (block-table entries outside [0, num_pages)) are skipped
 * as in decode.  Keys and values are staged in fp16 (INT2 rows rounded once
 * from the fp32 dequantized value) and accumulated in fp32.  Errors:
 * OSCAR_ERR_NULL, OSCAR_ERR_ARG (misaligned pointers, cu_new[0] != 0, negative
 * counts, repeated slots, n_seqs outside [1, min(max_seqs, 65535)]),
 * OSCAR_ERR_CAPACITY (slot or length beyond the cache), OSCAR_ERR_DEVICE,
 * OSCAR_ERR_HIP; a cache in OScaR key mode is OSCAR_ERR_ARG (prefill over
 * such a cache is not provided).  Needs no workspace. */
int oscar_int2_prefill_attn(const oscar_kv_cache* cache, int32_t n_seqs,
                            const int32_t* seq_slots_host, const int32_t* len_before_host,
                            const int32_t* cu_new_host,
                            const int32_t* seq_slots, const int32_t* len_before,
                            const int32_t* cu_new,
                            const uint16_t* q_rot, const uint16_t* k_rot, const uint16_t* v_rot,
                            float* out, void* stream);

/* For checking: the decoded rows of positions [tok_begin, tok_end) of one
 * cache row holding seq_len tokens, in the rotated basis: bf16 window rows
 * widened to fp32, INT2 rows as scale * code + zero rounded once to fp32 (in
 * OScaR key mode INT2 keys as s * (Delta_j * (code - z_j)) in fp64, rounded
 * once to fp32) -- the values the decode kernel reads.
 * [OSCAR s4 "Decoding Attention Kernel": INT2 segments are unpacked to
 * floating point (scale times code plus zero point) and BF16 segments read
 * as they are; OScaR "integer quantization basics": the dequantizer]
 *  k_out, v_out   fp32 [tok_end - tok_begin][Hkv][128] */
int oscar_dequant(const oscar_kv_cache* cache, int32_t seq_slot, int32_t seq_len,
                  int32_t tok_begin, int32_t tok_end, float* k_out, float* v_out, void* stream);

/* ---- Plain BF16 paged cache: the uncompressed comparison point ----------
 * [OSCAR abstract and s5: KV memory and throughput against BF16; OScaR
 * "efficiency": decode latency against BF16 FlashDecoding]
 * No rotation, no windows: every token of a row sits in its logical page
 * m = p / 16, slot p % 16, and the kernel computes
 *   out = softmax(q K^T / sqrt(128)) V
 * with the same split-K / log-sum-exp scheme as oscar_int2_decode_attn.
 *  pages: bf16 [num_pages][Hkv][2][16][128]; part 0 holds the K rows of the
 *         page's 16 slots (row-major, element 128 t + c), part 1 the V rows
 *         in the same order.  Slots at or beyond a row's length are ignored.
 *  block_table: int32 [max_seqs][max_pages_per_seq]: physical page of logical
 *         page m; entries outside [0, num_pages) are skipped (their tokens
 *         get zero weight). */
typedef struct {
  int32_t head_dim;           /* must be 128 */
  int32_t num_q_heads;        /* Hq, a multiple of num_kv_heads, Hq / Hkv <= 256 */
  int32_t num_kv_heads;       /* Hkv, 1 .. 64 */
  int32_t page_size;          /* must be 16 */
  int32_t max_seqs;           /* cache rows */
  int32_t max_pages_per_seq;  /* block table width, <= 65536 */
  int32_t num_pages;          /* physical pages in the pool */
  const uint16_t* pages;      /* bf16 [num_pages][Hkv][2][16][128] */
  const int32_t* block_table; /* [max_seqs][max_pages_per_seq] */
} oscar_bf16_cache;

/* Workspace bytes for oscar_bf16_paged_decode_attn with at most n_seqs
 * sequences per call (0 for an invalid cache description). */
size_t oscar_bf16_workspace_size(const oscar_bf16_cache* cache, int32_t n_seqs);

/* Decode attention of one query per sequence over a BF16 paged cache row.
 *  seq_slots[i], seq_lens[i]  cache row and its token count (>= 1); host and
 *                             device copies as for oscar_int2_decode_attn
 *  q      bf16 [n_seqs][Hq][128] queries (query head hq reads KV head hq / g)
 *  out    fp32 [n_seqs][Hq][128]
 * Errors: OSCAR_ERR_SHAPE / CAPACITY for an invalid description, slot or
 * length, OSCAR_ERR_ARG for misaligned pointers or n_seqs outside
 * [1, max_seqs], OSCAR_ERR_WORKSPACE, OSCAR_ERR_DEVICE, OSCAR_ERR_HIP. */
int oscar_bf16_paged_decode_attn(const oscar_bf16_cache* cache, int32_t n_seqs,
                                 const int32_t* seq_slots_host, const int32_t* seq_lens_host,
                                 const int32_t* seq_slots, const int32_t* seq_lens,
                                 const uint16_t* q, float* out,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Text for a status code (static storage). */
const char* oscar_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* OSCAR_KV_H */
