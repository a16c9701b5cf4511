// Internal declarations shared by the host library and the kernel files:
// workspace layout and kernel launchers. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace eta {

constexpr int kBlock = 64;          // tokens per KV block (one page)
constexpr int kTile = 64;           // blocks screened per wavefront
constexpr int kClaim = 2;           // entries per wavefront claim inside a workgroup
constexpr int kMaxAttendWgs = 4096; // upper bound of the attend grid (workspace sizing)
constexpr int kMaxBlocksPerSeq = 1 << 16;
constexpr int kMaxGroup = 8;
constexpr int kXcdClasses = 8;       // attend workgroup k runs on accelerator complex die k % 8
constexpr int kWeightOne = 1024;     // fixed-point unit of the per-die work weights
constexpr int kStatMagic = 0x45544131;
constexpr int kFusedTiles = 8;       // segments of at most this many tiles are screened in one workgroup
constexpr int kFusedMaxWgs = 512;    // largest grid of the one-launch decode of short segments
constexpr int kArrivalStride = 32;   // 64-bit words between two segments' arrival words (own 256-byte line)

// header of the workspace: the sizes the last decode laid it out for, and
// whether the attend timings of the last decode are present
enum Glob : int {
  kGlobN = 0,
  kGlobMB = 1,
  kGlobHQ = 2,
  kGlobHKV = 3,
  kGlobD = 4,
  kGlobStatMagic = 5,  // kStatMagic once an attend kernel has written rng_stat
  kGlobStatW = 6,      // ranges that attend kernel had
  kGlobSB = 7,         // screen blocks per page of the last decode (1, 2 or 4)
  kGlobPB = 8,         // pages per screen block of the last decode (1 or 2)
  kGlobCount = 16
};

struct Dims {
  int N, MB, HQ, HKV, D, G, S, NT;  // S = N*HKV segments, NT = tiles of 64 screen blocks per segment
  int SB;                           // screen blocks per 64-token page: 1 (b = 64, 128), 2 (b = 32) or 4 (b = 16)
  int PB;                           // pages per screen block: 1, or 2 (b = 128; the screen's lanes stay pages)
};

// Device pointers into one caller-provided workspace.
struct Ws {
  int32_t* glob;        // [kGlobCount]
  float* tau;           // [N*HQ]       effective thresholds
  int32_t* tile_cnt;    // [S][NT+1]    admitted union blocks per tile (tile NT: rescue entries)
  int2* tile_ent;       // [S][NT+1][64] (page, (j << 8) | head mask), ascending page index j within a tile
  uint32_t* tile_sub;   // [S][NT+1][64] with screen blocks smaller than a page: bit q G + h = head h
                        //              admitted block q of the entry's page
  int32_t* tile_off;    // [S][NT+2]    exclusive prefix of tile_cnt over the segment's used tiles,
                        //              the rescue tile last (index ntn), total at ntn+1
  int32_t* tile_hcnt;   // [S][NT][G]   admitted blocks per head per tile
  uint64_t* tile_bits;  // [S][G][NT]   per-head admission bitmap words, a bit per screen lane (a
                        //              screen block; with 128-token blocks a page, both pages of a
                        //              block carrying its bit)
  float* tile_umax;     // [S][NT][G]   largest bound among complete blocks
  int32_t* tile_uarg;   // [S][NT][G]   its block index (lowest on ties)
  int32_t* tile_err;    // [S][NT]
  int32_t* seg_U;       // [S]          union entries (pages) per segment
  int32_t* seg_ub;      // [S]          screen blocks admitted by any head of the segment
  int32_t* seg_ntn;     // [S]          tiles of 64 blocks the segment uses
  int32_t* seg_err;     // [S]
  uint64_t* seg_done;   // [S]          arrivals (zeroed by finalize): bits 0-31 entries whose partial is
                        //              written, 32-47 the range holding the first entry, 48-63 the last
  int32_t* rng_stat;    // [kMaxAttendWgs][2] entries and duration (10 ns ticks) of each attend range
  int32_t* xcd_w;       // [kXcdClasses]  work weight of each die class (kWeightOne = 1)
  int32_t* st_head;     // [N*HQ]       admitted blocks per head
  int64_t* st_tokens;   // [N*HQ]
  int32_t* st_rescued;  // [N*HQ]
  // The arrays from tau to st_rescued lie in one block of scr_stride bytes,
  // followed by scr_copies more blocks of the same layout: the private copies
  // of the screen's results for the workgroups of the one-launch decode of
  // short segments (copy p at byte offset p * scr_stride from the first).
  int64_t scr_stride;
  int scr_copies;
  uint64_t* fused_done; // [S][kArrivalStride] arrivals of the one-launch decode (word 0 of each row):
                        //              bits 24-63 the call's tag, bits 0-23 the workgroups of the
                        //              segment whose partial is written
  float* part_ml;       // [(kMaxAttendWgs + S)][G][2]  split running max and sum
  float* part_acc;      // [(kMaxAttendWgs + S)][G][D]  split unnormalised outputs; the partial of
                        //              attend range k in segment s is slot k + s
};

size_t workspace_layout(const Dims& d, void* base, Ws* ws);  // base may be null (size only)

struct CacheView {
  int kv_dtype, D, HKV, num_pages;
  const void* k;
  const void* v;
  void* kw;   // writable views for append
  void* vw;
  uint16_t* mu;
  float* radius;
  uint16_t* sigma;  // may be null
  uint16_t* kmin;   // may be null (both or neither)
  uint16_t* kmax;
  uint8_t* mu8;     // may be null (with radius8): FP8 centroids
  float* radius8;
  int mu8_fmt;      // 0 E4M3, 1 E5M2
  int sub_rows;     // tokens per block of the other screen-block records (16, 32 or 128), 0 if none
  uint16_t* mu_sub;  // [pages][HKV][sub_slots(sub_rows)][D]; a 128-token block's record with its first page
  float* radius_sub;  // [pages][HKV][sub_slots(sub_rows)]
};

// Record slots per page for screen blocks of `rows` tokens: 64/rows for blocks
// inside a page, one (kept by the first page) for a block of two pages.
__host__ __device__ constexpr int sub_slots(int rows) { return rows < kBlock ? kBlock / rows : 1; }

struct SeqView {
  int N, MB;
  const int32_t* lens;
  const int32_t* bt;
};

struct DecodeParams {
  const void* q;
  int HQ, G, tau_mode;
  const float* w;
  const float* b;
  float a, beta, scale;
  int lwb;
  float* out;
  int deterministic;  // static work split and claims: bitwise-reproducible results
  int bound;          // 0 geometric, 1 dual (tightened by z deviations), 2 comparator box bound,
                      // 3 geometric over the FP8 records, 4 geometric over screen blocks of 16 or
                      // 32 tokens, 5 geometric over screen blocks of 128 tokens
  float z;
  int fixed_w[kXcdClasses];  // if fixed_w[0] > 0: per-die weights to use instead of measured ones
};

struct CalibParams {
  const void* q;  // [N][64 * MB][HQ][D]
  int HQ, num_bins;
  const float* w;    // [HQ][D] learned predictor, or null
  const float* b;    // [HQ]
  const float* rho;  // [HQ] target densities, or null
  float lo, hi;
  uint64_t* hist;   // [HQ][num_bins]
  uint64_t* above;  // [HQ]
  uint64_t* total;  // [HQ]
  float* c_out;     // [HQ]
  int* err;         // [1] device flag: an out-of-range page id was met
};

struct PrefillParams {
  const void* q;  // [N][64 * MB][HQ][D]
  int HQ, tau_mode;
  const float* w;  // [HQ][D] (learned)
  const float* b;  // [HQ]
  float a, beta;
  float* out;  // [N][64 * MB][HQ][D]
  int* err;    // [1] device flag: an out-of-range length or page id was met
};

// launchers (return hipError_t of the launch)
hipError_t launch_build_summaries(const CacheView& c, const SeqView& s, hipStream_t st);
hipError_t launch_append(const CacheView& c, const SeqView& s, const void* k_new, const void* v_new,
                         hipStream_t st);
// screen and finalize (in one launch for short segments with the geometric
// bound); also writes NaN rows for segments with no entries
hipError_t launch_screen_phase(const CacheView& c, const SeqView& s, const DecodeParams& p, const Dims& d,
                               const Ws& ws, hipStream_t st);
hipError_t launch_attend(const CacheView& c, const SeqView& s, const DecodeParams& p, const Dims& d,
                         const Ws& ws, int attend_wgs, hipStream_t st);
hipError_t launch_calibrate(const CacheView& c, const SeqView& s, const CalibParams& p, hipStream_t st);
hipError_t launch_prefill(const CacheView& c, const SeqView& s, const PrefillParams& p, hipStream_t st);
int attend_wgs_per_cu(int kv_dtype, int D, int G);  // occupancy of the attend kernel
// One launch for the whole decode step when every segment has at most
// kFusedTiles tiles and the bound is the geometric one on page blocks:
// wgs_per_segment workgroups per segment (at least 2, at most
// ws.scr_copies + 1), tag identifies the call in the arrival words.
hipError_t launch_decode_short(const CacheView& c, const SeqView& s, const DecodeParams& p, const Dims& d,
                               const Ws& ws, int wgs_per_segment, uint64_t tag, hipStream_t st);
bool decode_short_supported(int kv_dtype, int D, int G);

}  // namespace eta
