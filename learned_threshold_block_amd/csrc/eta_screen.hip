// Screen phase of one decode step: thresholds, O(1) bound test per block,
// compaction of admitted block ids, top-1 rescue and counts.
//
// "Elastic Threshold Attention" (paperpeel.com/paper/2609.20888):
//   threshold tau~ = w_h.q + b_h - a or c_h - a   (Sections 1, 4.7, D.1, G.1)
//   bound     s (q.mu^ + ||q|| R^) vs tau~ per block, without per-key products
//             (Section 3, 3.1, F.1); GQA: one record read serves the G heads of a
//             group, a block is loaded if any head admits it (Section 4.3, F.1)
//   forced    partial last block and the lwb most recent complete blocks (4.8)
//   rescue    block with the largest bound when a head admits nothing (3.2, F.4)
//   dual      optionally the bound is tightened to min(bound, s (q.mu^ + z ||q sigma^||))
//             with the per-block coordinate deviation sigma^ (Section 3.1, F.1)
//   box       or, as the comparator of Section 4.3, replaced by the best corner
//             s sum_i max(q_i kmax_i, q_i kmin_i) of the block's key box
//   fp8       or the geometric bound over the FP8 records (centroid mu8 in an
//             8-bit float, radius about it)
//   blocks    or the geometric bound on screen blocks of 16 or 32 tokens (2 or
//             4 per page, each with its own record; Appendix F.3's block size):
//             the block index j then counts those blocks, and the compacted
//             entries stay one per page, with a word of per-head block bits;
//             or on blocks of 128 tokens (two consecutive block-table entries,
//             the record kept with the first page): lanes stay pages, both
//             pages of a block take its bound and its bits, and the counts
//             count blocks
//   counts    per-head blocks, union blocks, attended tokens (F.4)
//
// k_screen: one wavefront per 64 consecutive blocks of one (sequence, KV head).
//   Lanes read the float16 centroids with 16-byte loads (16 lanes per row at
//   d = 128), form partial dot products with the G queries and finish them with
//   a transposing DPP reduction, so each lane ends up owning one block. Admitted
//   blocks are compacted in ascending order with a wavefront ballot + prefix.
// k_finalize: one workgroup per (sequence, KV head): per-head totals, rescue,
//   exclusive prefix over the tiles' compacted lists (the attend kernel reads
//   entries in place through it), the segment's union count and statistics.
//   The split of the total work over the attend grid needs only the union
//   counts; each attend and merge workgroup derives it from them itself, so no
//   workgroup has to wait for all the others here.
// k_screen_fin: both in one launch when every segment has at most eight tiles
//   (512 screen blocks) and the bound is the geometric one: one workgroup per
//   segment screens its tiles and then finalizes it, which saves a launch and
//   a dependent round at short lengths.
#include "eta_screen_dev.h"

namespace eta {
namespace {

// One wavefront per tile: grid ((NT + 3) / 4, S).
template <typename T, int D, int G, int MODE>
__global__ __launch_bounds__(256) void k_screen(ScreenArgs A) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) write_glob<D>(A);
  const int t = blockIdx.x * 4 + wave;
  if (t >= A.d.NT) return;
  screen_tile<T, D, G, MODE, 4>(A, blockIdx.y, t, wave, lane);
}

// One workgroup per segment, and one more for the per-die weights.
template <int G>
__global__ __launch_bounds__(256) void k_finalize(FinArgs A) {
  if ((int)blockIdx.x == A.d.S) {
    update_weights<4>(A);
    return;
  }
  finalize_segment<G, 4>(A, blockIdx.x);
}

// Short segments (at most kFusedTiles tiles) in one launch: a workgroup of
// kFusedTiles wavefronts screens one tile per wavefront, then finalizes its
// segment itself (the barrier publishes the tiles' results to the whole
// workgroup); one more workgroup updates the per-die weights.
template <typename T, int D, int G>
__global__ __launch_bounds__(64 * kFusedTiles) void k_screen_fin(ScreenArgs A, FinArgs F) {
  if ((int)blockIdx.x == A.d.S) {
    update_weights<kFusedTiles>(F);
    return;
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (blockIdx.x == 0 && threadIdx.x == 0) write_glob<D>(A);
  if (wave < A.d.NT) screen_tile<T, D, G, 0, kFusedTiles>(A, blockIdx.x, wave, wave, lane);
  __syncthreads();
  finalize_segment<G, kFusedTiles>(F, blockIdx.x);
}

template <typename T, int D, int G>
hipError_t screen_impl(const CacheView& c, const SeqView& s, const DecodeParams& p, const Dims& d,
                       const Ws& ws, hipStream_t st) {
  ScreenArgs a{c, s, p, d, ws};
  FinArgs f{c, s, d, ws, p.out, p.deterministic, {}};
  for (int x = 0; x < kXcdClasses; ++x) f.fixed_w[x] = p.fixed_w[x];
  if (p.bound == 0 && d.NT <= kFusedTiles) {
    hipLaunchKernelGGL((k_screen_fin<T, D, G>), dim3(d.S + 1), dim3(64 * kFusedTiles), 0, st, a, f);
    return hipGetLastError();
  }
  dim3 grid((d.NT + 3) / 4, d.S);
  if (p.bound == 1) hipLaunchKernelGGL((k_screen<T, D, G, 1>), grid, dim3(256), 0, st, a);
  else if (p.bound == 2) hipLaunchKernelGGL((k_screen<T, D, G, 2>), grid, dim3(256), 0, st, a);
  else if (p.bound == 3) hipLaunchKernelGGL((k_screen<T, D, G, 3>), grid, dim3(256), 0, st, a);
  else if (p.bound == 4) hipLaunchKernelGGL((k_screen<T, D, G, 4>), grid, dim3(256), 0, st, a);
  else if (p.bound == 5) hipLaunchKernelGGL((k_screen<T, D, G, 5>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((k_screen<T, D, G, 0>), grid, dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_finalize<G>), dim3(d.S + 1), dim3(256), 0, st, f);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t screen_g(const CacheView& c, const SeqView& s, const DecodeParams& p, const Dims& d,
                    const Ws& ws, hipStream_t st) {
  switch (d.G) {
    case 1: return screen_impl<T, D, 1>(c, s, p, d, ws, st);
    case 2: return screen_impl<T, D, 2>(c, s, p, d, ws, st);
    case 4: return screen_impl<T, D, 4>(c, s, p, d, ws, st);
    case 8: return screen_impl<T, D, 8>(c, s, p, d, ws, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_screen_phase(const CacheView& c, const SeqView& s, const DecodeParams& p, const Dims& d,
                              const Ws& ws, hipStream_t st) {
  if (c.kv_dtype == 1) return d.D == 128 ? screen_g<Bf16, 128>(c, s, p, d, ws, st) : screen_g<Bf16, 64>(c, s, p, d, ws, st);
  return d.D == 128 ? screen_g<F32, 128>(c, s, p, d, ws, st) : screen_g<F32, 64>(c, s, p, d, ws, st);
}

}  // namespace eta
