/*
 * eta.h - C ABI of the ETA (Elastic Threshold Attention) decode library for
 * AMD Instinct MI355X (gfx950).
 *
 * Method: "Elastic Threshold Attention: Learned Contextual Sparsity for
 * Long-Context Decoding" (paperpeel.com/paper/2609.20888). One decode step,
 * for every sequence n and query head h (KV head g = h / G, G = H_Q / H_KV):
 *   threshold  tau~ = w_h . q + b_h - a   (learned, Sections 1 and D.1)
 *              tau~ = c_h - a             (calibrated, Section 4.7)
 *   screen     every complete 64-token block whose bound
 *              s (q . mu^ + ||q|| R^) is not below tau~ is admitted
 *              (Sections 3, 3.1, F.1); the partial last block and the `lwb`
 *              most recent complete blocks always are (Section 4.8, F.4); if
 *              nothing is admitted, the block with the largest bound is
 *              (top-1 rescue, Section 3.2 and F.4);
 *   attention  over the tokens t < T of admitted blocks:
 *              S = s q.k,  S~ = S * sigmoid(beta (S - tau~)),
 *              o = sum exp(S~) v / sum exp(S~)   (Sections 2.2, E.3, G.1),
 *   with s = 1/sqrt(d). A KV block is read once for all G heads that admit
 *   it; each head accumulates only the blocks it admitted (Section 4.3, F.1).
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless the comment says "host".
 *   - The caller owns all memory. The library allocates nothing and keeps no
 *     state between calls apart from a per-device launch-geometry cache and
 *     the per-device array that serves eta_decode_noalloc as its workspace.
 *     A decode workspace carries the previous call's per-die work weights
 *     and range timings to the next call on it; they steer only how the work
 *     is split, never what is computed.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = default
 *     stream) except eta_stats, which synchronises the stream.
 *   - Host-checkable arguments are validated before any device work; a
 *     failing call returns a negative eta_status and launches nothing.
 *     Device-resident values (sequence lengths, block-table entries) are
 *     checked by the kernels: offending blocks are skipped, and eta_stats
 *     reports ETA_ERR_DEVICE_DATA for the decode step that met them.
 *   - Nothing aborts and no C++ exception crosses this interface.
 *   - Calls that share a workspace or a cache region must be ordered on one
 *     stream (or by the caller's events); the library is re-entrant otherwise.
 */
#ifndef ETA_H_
#define ETA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* eta_stream_t; /* same type as hipStream_t */

typedef enum {
  ETA_OK = 0,
  ETA_ERR_INVALID_ARGUMENT = -1,   /* bad pointer, size, alignment or value */
  ETA_ERR_UNSUPPORTED = -2,        /* valid but not implemented (block size, head dim, group size) */
  ETA_ERR_WORKSPACE_TOO_SMALL = -3,
  ETA_ERR_HIP = -4,                /* a HIP runtime call failed */
  ETA_ERR_DEVICE_DATA = -5         /* a kernel met an out-of-range length or page id */
} eta_status;

enum { ETA_F32 = 0, ETA_BF16 = 1 };                 /* K/V/q element type */
enum { ETA_TAU_LEARNED = 0, ETA_TAU_CALIBRATED = 1 }; /* threshold mode */
enum { ETA_PHASE_ALL = -1, ETA_PHASE_SCREEN = 0, ETA_PHASE_ATTEND = 1, ETA_PHASE_MERGE = 2 };
enum { ETA_BOUND_GEOMETRIC = 0, ETA_BOUND_DUAL = 1, ETA_BOUND_QUEST = 2, ETA_BOUND_GEOMETRIC_FP8 = 3,
       ETA_BOUND_GEOMETRIC_SUB = 4 };
                                                      /* block screen, see eta_screen_opts */
enum { ETA_FP8_E4M3 = 0, ETA_FP8_E5M2 = 1 };          /* FP8 record formats (OCP 8-bit floats) */

/* Paged KV cache plus its per-block records (caller-owned device buffers).
 *   k_pages, v_pages : [num_pages][num_kv_heads][block_size][head_dim] of
 *                      kv_dtype (bf16 as raw 16-bit patterns), 16-byte aligned.
 *   mu               : [num_pages][num_kv_heads][head_dim] float16 bit patterns,
 *                      the block centroid rounded to nearest even (Section 3.2,
 *                      F.1), 16-byte aligned.
 *   radius           : [num_pages][num_kv_heads] float32, an upper bound on the
 *                      distance of every key of the block to mu (rounded up;
 *                      +inf for blocks holding non-finite keys), 4-byte aligned.
 *   sigma            : NULL, or [num_pages][num_kv_heads][head_dim] float16 bit
 *                      patterns, 16-byte aligned: the coordinate standard
 *                      deviation of the block's keys (population, about their
 *                      mean), rounded to nearest even; +inf where not finite
 *                      (Section F.1; only the dual screen reads it). When not
 *                      NULL, the record builders fill it too.
 *   kmin, kmax       : NULL (both), or [num_pages][num_kv_heads][head_dim]
 *                      float16 bit patterns each, 16-byte aligned: per key
 *                      coordinate the least value of the block rounded down
 *                      and the greatest rounded up to float16, NaN in both for
 *                      a block holding a non-finite key (the per-block extrema
 *                      of the comparator of Section 4.3; only ETA_BOUND_QUEST
 *                      reads them). When not NULL, the record builders fill them.
 *   mu8, radius8     : NULL (both), or an FP8 copy of the geometric record
 *                      (Section 5 names FP8 metadata as future work; the reading
 *                      taken): mu8 [num_pages][num_kv_heads][head_dim] bytes,
 *                      16-byte aligned, the block mean rounded to nearest even
 *                      in format mu8_format and saturated at its largest finite
 *                      value; radius8 [num_pages][num_kv_heads] float32, the
 *                      farthest key's distance to that stored centroid, rounded
 *                      up (zero centroid, +inf radius for a block holding a
 *                      non-finite key). Only ETA_BOUND_GEOMETRIC_FP8 reads them;
 *                      when not NULL, the record builders fill them.
 *   mu8_format       : ETA_FP8_E4M3 (3 mantissa bits, largest 448) or
 *                      ETA_FP8_E5M2 (2 mantissa bits, largest 57344); read only
 *                      when mu8 is not NULL.
 *   sub_block, mu_sub, radius_sub : screen blocks of another size than the
 *                      page (Appendix F.3 ablates the block size; the reading
 *                      taken): sub_block 16 or 32 tokens, so a page holds
 *                      64/sub_block consecutive blocks, or 128 tokens, so a
 *                      block spans the entries 2j and 2j + 1 of a sequence's
 *                      block table. mu_sub [num_pages][num_kv_heads][slots]
 *                      [head_dim] float16 bits (16-byte aligned) and radius_sub
 *                      [num_pages][num_kv_heads][slots] float32, slots =
 *                      64/sub_block (16, 32) or 1 (128): the record of each such
 *                      block, by the same rule as mu/radius over its keys. A
 *                      128-token block's record lives with its first page
 *                      (entry 2j); every table that holds that page at an even
 *                      entry must hold the same second page after it. Both
 *                      NULL, or both set; only ETA_BOUND_GEOMETRIC_SUB reads
 *                      them; when set, the record builders fill them (the
 *                      append path builds a 128-token block's record when the
 *                      token completing its second page arrives).
 * Supported: head_dim 64 or 128, block_size 64 (Section 4.8 and F.3 use 64). */
typedef struct {
  int kv_dtype;
  int head_dim;
  int num_kv_heads;
  int block_size;
  int num_pages;
  void* k_pages;
  void* v_pages;
  uint16_t* mu;
  float* radius;
  uint16_t* sigma;
  uint16_t* kmin;
  uint16_t* kmax;
  uint8_t* mu8;
  float* radius8;
  int mu8_format;
  int sub_block;
  uint16_t* mu_sub;
  float* radius_sub;
} eta_cache;

/* Sequences of a batch.
 *   seq_lens    : [num_seqs] int32 token counts, 1 <= T <= block_size*max_blocks_per_seq.
 *   block_table : [num_seqs][max_blocks_per_seq] int32; entry j of row n is the
 *                 page holding tokens [64j, 64j+64) of sequence n. Entries past
 *                 the last block may hold anything: they are read but never
 *                 used, so the whole row must be addressable.               */
typedef struct {
  int num_seqs;
  int max_blocks_per_seq;
  const int32_t* seq_lens;
  const int32_t* block_table;
} eta_seqs;

/* Build the record (mu, radius) of every complete block of every sequence and
 * KV head, reading the keys in k_pages. Idempotent; records of partial blocks
 * are left untouched. (Section 3.2 and F.1: metadata per KV head, built from the
 * cache; Section 4.8: built during prefill.) Rows of blocks with an
 * out-of-range page id are skipped. */
eta_status eta_build_block_summaries(const eta_cache* cache, const eta_seqs* seqs,
                                     eta_stream_t stream);

/* Append one token per sequence (Section 3.2: the block records sit in a
 * table beside the paged cache; Section 4.8: they are built as the cache
 * grows, so a decode step reads the records of every block completed so far).
 * k_new, v_new are [num_seqs][num_kv_heads][head_dim]
 * of kv_dtype (16-byte aligned). seqs->seq_lens holds the lengths BEFORE the
 * append; the token goes to row T%64 of page block_table[n][T/64], which the
 * caller has assigned. When that fills the block (T%64 == 63) its record is
 * built in the same launch, bit-identical to eta_build_block_summaries. The
 * caller increments seq_lens afterwards. Sequences with T >= 64*max_blocks or
 * an out-of-range page id are skipped. */
eta_status eta_append_kv(const eta_cache* cache, const eta_seqs* seqs, const void* k_new,
                         const void* v_new, eta_stream_t stream);

/* Bytes of device workspace eta_decode needs for these sizes (0 if they are
 * invalid or unsupported). The workspace carries the screen's compacted block
 * lists and counts, the split partial results and the statistics; it must be
 * 256-byte aligned and may be reused by later calls of the same or smaller
 * size. */
size_t eta_decode_workspace_size(const eta_cache* cache, int num_seqs, int max_blocks_per_seq,
                                 int num_q_heads);

/* One decode step: out[n][h][:] (float32, [num_seqs][num_q_heads][head_dim])
 * for every sequence and query head.
 *   q          [num_seqs][num_q_heads][head_dim] of kv_dtype, 16-byte aligned.
 *   tau_mode   ETA_TAU_LEARNED: w [num_q_heads][head_dim] float32 and
 *              b_or_c [num_q_heads] float32 (bias b_h) are required;
 *              ETA_TAU_CALIBRATED: w is ignored, b_or_c holds c_h. c_h = -inf
 *              admits every block and leaves logits unfiltered (plain softmax
 *              attention: the dense comparator).
 *   a          threshold adjustment (tau~ = tau - a), finite.
 *   beta       gate sharpness, finite and > 0 (5 at inference, B.1).
 *   lwb        number of most recent complete blocks always admitted, >= 0.
 *   block_size must equal cache->block_size (64).
 * num_q_heads must be a multiple of num_kv_heads with G = num_q_heads /
 * num_kv_heads in {1, 2, 4, 8}. Equivalent to the three phases below in order
 * (short segments run them as one launch: see eta_decode_launches).
 * Values of V: those of a block a head did not admit never reach that head's
 * output (with ETA_BOUND_GEOMETRIC_SUB, per screen block, also between the
 * blocks of one page); a non-finite element i of V at a token a head attends
 * to makes element i of that head's output non-finite (inf or NaN, as the
 * exact weighted sum is), and the other elements are unaffected. */
eta_status eta_decode(const eta_cache* cache, const eta_seqs* seqs, const void* q,
                      int num_q_heads, int tau_mode, const float* w, const float* b_or_c,
                      float a, float beta, int lwb, int block_size, float* out,
                      void* workspace, size_t ws_bytes, eta_stream_t stream);

/* Bytes of the device array that eta_decode_noalloc uses as its workspace. */
#define ETA_NOALLOC_WORKSPACE_BYTES ((size_t)32 << 20)

/* eta_decode for callers that cannot allocate device memory (code under stream
 * capture, tight serving loops, hosts that forbid allocation): the same
 * arguments without the workspace, which is instead a fixed array of
 * ETA_NOALLOC_WORKSPACE_BYTES in the library's device memory. Each GPU holds its
 * own copy from its first call until the process ends. The call allocates
 * nothing. Sizes whose workspace (eta_decode_workspace_size) exceeds the array
 * return ETA_ERR_WORKSPACE_TOO_SMALL before any launch; every other argument is
 * checked as by eta_decode. All calls on one GPU share its array: calls that
 * overlap in time on one GPU (on different streams, or from several threads
 * without ordering) race and give wrong results. Counts of these calls are not
 * available through eta_stats. */
eta_status eta_decode_noalloc(const eta_cache* cache, const eta_seqs* seqs, const void* q,
                              int num_q_heads, int tau_mode, const float* w, const float* b_or_c,
                              float a, float beta, int lwb, int block_size, float* out,
                              eta_stream_t stream);

/* Block screen of a decode step (Sections 3.1 and F.1).
 *   ETA_BOUND_GEOMETRIC : score s (q . mu + ||q|| R), an upper bound on the
 *                         scaled logit of every key of the block (the default).
 *   ETA_BOUND_DUAL      : score min(geometric, s (q . mu + z ||q * sigma||)), the
 *                         geometric bound tightened by a z-deviation estimate
 *                         (the reading of the paper's dual bound, Eq. 7, whose
 *                         display did not survive). Not a bound: a block whose
 *                         best key lies more than z deviations out can be
 *                         missed. Needs cache->sigma; z finite and >= 0
 *                         (2.0 in the paper's B.1 tables).
 *   ETA_BOUND_QUEST     : score s sum_i max(q_i kmax_i, q_i kmin_i), the best
 *                         corner of the block's stored key box: the comparator
 *                         bound of Section 4.3 (sound, like the geometric one;
 *                         each term takes the IEEE maximum, in which a NaN
 *                         product yields to the other). Needs cache->kmin and
 *                         cache->kmax.
 *   ETA_BOUND_GEOMETRIC_FP8 : the geometric bound over the FP8 records,
 *                         s (q . mu8 + ||q|| radius8): half the record bytes of
 *                         the float16 centroid, a coarser centroid and so a
 *                         larger radius. Needs cache->mu8 and cache->radius8.
 *   ETA_BOUND_GEOMETRIC_SUB : the geometric bound on blocks of cache->sub_block
 *                         tokens (records mu_sub/radius_sub). Screen, forced
 *                         blocks (the partial last block, the lwb most recent
 *                         complete ones), rescue and counts work on those
 *                         blocks; with 16 or 32 tokens the attention loads a
 *                         page's rows only for the blocks some head of the group
 *                         admitted and each head attends only to the tokens of
 *                         its own blocks; with 128 it loads both pages of every
 *                         block some head admitted. eta_stats then reports
 *                         per-head counts, union counts and the bitmap in these
 *                         blocks (ceil(max_blocks_per_seq * 64 / sub_block) bits
 *                         per head).
 * The score also ranks blocks for the top-1 rescue. */
typedef struct {
  int bound;
  float z;
} eta_screen_opts;

/* eta_decode / eta_decode_phase with a screen choice: phase is ETA_PHASE_ALL
 * for the whole step or one ETA_PHASE_*; screen NULL means the geometric bound.
 * Returns ETA_ERR_INVALID_ARGUMENT for an unknown bound, a negative or
 * non-finite z, the dual bound without cache->sigma, the comparator bound
 * without cache->kmin and cache->kmax, the FP8 bound without cache->mu8
 * and cache->radius8, or the sub_block bound without cache->mu_sub. */
eta_status eta_decode_ex(int phase, const eta_screen_opts* screen, const eta_cache* cache,
                         const eta_seqs* seqs, const void* q, int num_q_heads, int tau_mode,
                         const float* w, const float* b_or_c, float a, float beta, int lwb,
                         int block_size, float* out, void* workspace, size_t ws_bytes,
                         eta_stream_t stream);

/* How eta_decode (eta_decode_ex with ETA_PHASE_ALL) runs a step of these
 * sizes on the current device: 1 = as one launch, 2 = as the screen phase
 * followed by the attend phase. Short segments (at most 512 screen blocks,
 * i.e. 32,768 tokens, per sequence) with the geometric bound on page blocks
 * run in one launch: each (sequence, KV head) gets several workgroups, each
 * of which screens and finalizes the whole segment on its own (the records of
 * such a segment are a few hundred KB) and attends to its share of the
 * admitted blocks; the last of them merges. Results and statistics are those
 * of the two phases up to float32 rounding. ETA_FUSED=0 in the environment
 * keeps the two phases. A negative value is the eta_status of invalid sizes
 * (checked as by eta_decode_ex). */
int eta_decode_launches(const eta_screen_opts* screen, const eta_cache* cache, const eta_seqs* seqs,
                        int num_q_heads);

/* One phase of eta_decode with the same arguments, for callers that overlap or
 * time the phases: ETA_PHASE_SCREEN (thresholds, bound screen, compaction of
 * admitted block ids, rescue, counts), ETA_PHASE_ATTEND (split flash-decode over
 * the compacted lists, Section 3.2 and F.3 chunked decoding, followed by the
 * associative merge of the splits into out, done by the workgroup that
 * completes each (sequence, KV head)), ETA_PHASE_MERGE (accepted for
 * compatibility; no work, the merge is part of ETA_PHASE_ATTEND). Phases must
 * run in this order on one workspace; ATTEND reads what SCREEN wrote. */
eta_status eta_decode_phase(int phase, const eta_cache* cache, const eta_seqs* seqs,
                            const void* q, int num_q_heads, int tau_mode, const float* w,
                            const float* b_or_c, float a, float beta, int lwb, int block_size,
                            float* out, void* workspace, size_t ws_bytes, eta_stream_t stream);

/* Synchronise `stream`, then copy the counts of the last eta_decode on this
 * workspace to host memory (Section F.4 validates exactly these integers):
 *   admitted_per_head [num_seqs][num_q_heads] int32  blocks admitted per head
 *   union_per_kv      [num_seqs][num_kv_heads] int32 blocks loaded per KV head
 *   tokens_per_head   [num_seqs][num_q_heads] int64  attended tokens (nullable)
 *   rescued           [num_seqs][num_q_heads] uint8  1 if top-1 rescue fired (nullable)
 *   admitted_bitmap   [num_seqs][num_q_heads][ceil(max_blocks_per_seq/32)]
 *                     uint32, bit j%32 of word j/32 = block j admitted (nullable)
 * Blocks are the screen's blocks: after a decode with ETA_BOUND_GEOMETRIC_SUB
 * they are the cache's sub_block-token blocks, and the bitmap has
 * ceil(ceil(max_blocks_per_seq * 64 / sub_block) / 32) words per head (the
 * sizes passed stay those of the decode call). All output pointers are host pointers. Returns ETA_ERR_DEVICE_DATA (after
 * filling the outputs) if that decode met invalid lengths or page ids, and
 * ETA_ERR_INVALID_ARGUMENT if the sizes do not match that decode. */
eta_status eta_stats(const void* workspace, int num_seqs, int max_blocks_per_seq, int num_q_heads,
                     int num_kv_heads, int32_t* admitted_per_head, int32_t* union_per_kv,
                     int64_t* tokens_per_head, uint8_t* rescued, uint32_t* admitted_bitmap,
                     eta_stream_t stream);

/* Offline calibration of per-head constants c_h for the calibrated mode
 * (Section 4.7 and Appendix D.2, Algorithm 1, whose body did not survive; the
 * reading taken): over the sequences of `seqs` (keys from `cache`), every
 * position t (0-based) is a query row over the keys s <= t with scaled scores
 * S = q_t . k_s / sqrt(d); each key of row t weighs floor(2^31 / (t + 1)) (the
 * 1/t row weighting, in integers). Scores fall in opts->num_bins equal bins
 * over [opts->lo, opts->hi) (outside: the end bins; NaN: bin 0). The target is
 * the weighted count of scores at or above the learned threshold
 * w_h . q_t + b_h (the head's training density; w, b given, rho NULL) or
 * floor(rho_h * total) (rho given, w and b NULL). c_h is the lowest bin edge
 * whose weighted tail (the weight of the bins at or above it) does not exceed
 * the target.
 *   q        [num_seqs][64*max_blocks_per_seq][num_q_heads][head_dim] kv_dtype,
 *            a query for every position (positions >= seq_len unused), 16-byte aligned.
 *   w, b     [num_q_heads][head_dim], [num_q_heads] float32 (device), or NULL.
 *   rho      [num_q_heads] float32 (device) densities in [0, 1], or NULL.
 *   hist     [num_q_heads][num_bins] uint64 out: weighted bin counts.
 *   above    [num_q_heads] uint64 out: weighted count at or above the learned
 *            threshold (zero without a predictor).
 *   total    [num_q_heads] uint64 out: weight of all scores.
 *   c_out    [num_q_heads] float32 out: the constants.
 *   err_flag [1] int32 device out: 1 if an out-of-range page id was met.
 * All outputs are device buffers the library overwrites (8-byte aligned for the
 * uint64 ones). Requires 2 <= num_bins and G * num_bins <= 8192 (the
 * per-workgroup histogram lives in 64 KB of LDS), lo < hi, both finite.
 * Asynchronous on `stream`. */
typedef struct {
  int num_bins;
  float lo;
  float hi;
} eta_calib_opts;

eta_status eta_calibrate(const eta_cache* cache, const eta_seqs* seqs, const void* q, int num_q_heads,
                         const float* w, const float* b, const float* rho, const eta_calib_opts* opts,
                         uint64_t* hist, uint64_t* above, uint64_t* total, float* c_out, int32_t* err_flag,
                         eta_stream_t stream);

/* Causal prompt pass (Sections 2.2 and 2.3, the fused causal forward; E.1,
 * E.3 and G.1, the gate inside the softmax; 4.8, records built while the
 * prompt is processed). For every position t < seq_len of every sequence and
 * every query head h, over the keys s <= t of the sequence's pages:
 *   S = q_t . k_s / sqrt(d),  S~ = S sigmoid(beta (S - tau~_t)),
 *   out_t = sum_s exp(S~) v_s / sum_s exp(S~),
 * with tau~_t = w_h . q_t + b_h - a (ETA_TAU_LEARNED) or c_h - a
 * (ETA_TAU_CALIBRATED; c_h = -inf gives plain causal attention). Dense: no
 * block is skipped, the gate alone filters. In the same launch the records
 * (centroid, radius, and the deviation if cache->sigma is set) of every
 * complete block (64 j + 64 <= seq_len) are written, bit-identical to
 * eta_build_block_summaries'; the cache must hold the prompt's keys and values.
 *   q        [num_seqs][64*max_blocks_per_seq][num_q_heads][head_dim] of
 *            kv_dtype (device, 16-byte aligned); positions >= seq_len are not
 *            read.
 *   w, b_or_c  as for eta_decode (device float32; w ignored when calibrated).
 *   out      [num_seqs][64*max_blocks_per_seq][num_q_heads][head_dim] float32
 *            (device, 16-byte aligned); rows at positions >= seq_len are NaN.
 *   err_flag [1] int32 device out: 1 if a length outside [0, 64*max_blocks]
 *            (that sequence's rows are then NaN) or an out-of-range page id
 *            (the block reads as zeros and its record is left alone) was met.
 * bfloat16 caches: products on the matrix cores, S with bfloat16 operands;
 * the weights times V in float16 (one term, V converted exactly) when every
 * value of V in the prompts lies within +-65280, else in two bfloat16 terms of
 * each weight (a range check over V picks the path for the whole call). A
 * non-finite element i of V at key s makes element i of the outputs of s's
 * (sequence, KV head) non-finite at every position of s's 64-token key block
 * and later: from s on as the exact rule gives, and at the block's positions
 * before s as well, where the exact rule does not use key s (the block's
 * masked keys enter the products with weight 0, and 0 times a non-finite
 * value is NaN). Earlier positions and the other elements are unaffected.
 * float32 caches: float32 arithmetic on the vector units; keys after a
 * position are skipped, so a non-finite element i of V at key s reaches
 * element i of the outputs at positions s and later only, as the exact rule
 * gives.
 * Requires beta > 0 finite, a finite, and num_seqs * num_q_heads <= 65535
 * (ETA_ERR_UNSUPPORTED otherwise). Asynchronous on `stream`. */
eta_status eta_prefill(const eta_cache* cache, const eta_seqs* seqs, const void* q, int num_q_heads,
                       int tau_mode, const float* w, const float* b_or_c, float a, float beta, float* out,
                       int32_t* err_flag, eta_stream_t stream);

/* Static text for a status code. */
const char* eta_status_string(eta_status status);

#ifdef __cplusplus
}
#endif

#endif /* ETA_H_ */
