// Attend phase of one decode step: split flash-decode over the compacted lists
// of admitted blocks, and the associative merge of the splits.
//
// "Elastic Threshold Attention" (paperpeel.com/paper/2609.20888):
//   S = s q.k, S~ = S * sigmoid(beta (S - tau~)), o = sum e^{S~} v / sum e^{S~}
//   over the tokens of the admitted blocks (Sections 1, 2.2, E.3, G.1); a block
//   is read from HBM once for the G heads of its group and each head updates
//   only with the blocks it admitted (Section 4.3, F.1); partial last block
//   masked past the sequence end (F.4); the sequence split into parts merged by
//   an associative online-softmax reduction (Section 3.2, F.2, F.3).
//
// Work split: the screen produced, per (sequence, KV head) segment, a list of
// admitted blocks. Their concatenation (Utot entries) is cut into W' ranges,
// one per workgroup (W' = min(grid, ceil(Utot / 8)), grid = one workgroup per
// CU), so every workgroup streams about the same number of tiles whatever the
// density or the length mix. Range sizes follow per-die weights measured on
// the previous decode (dies differ in memory throughput). A range that spans
// several segments emits one partial per segment; the workgroup that
// completes a segment's entries (counted with one atomic per partial) merges
// the segment's partials into the output, so no separate merge launch waits
// for the slowest workgroup of all.
//
// Inside a workgroup the wavefronts claim kClaim entries at a time (one in the
// one-launch decode of short segments) from an LDS
// counter, so the wavefronts that run faster (older waves get issue priority on
// a SIMD) take more tiles. With ETA_DETERMINISTIC=1 in the environment the
// split uses equal weights and the claims are static (wavefront w takes claims
// w, w + NW, ...), so the result is bitwise reproducible; by default repeated
// calls agree to float32 rounding. A wavefront owns a whole tile: 16-byte
// loads of one 64 x d tile (lane (r, cb) holds rows RPI*i + r, 8 bf16
// columns), keys consumed by v_dot2 bf16 products into per-lane partial
// logits, finished by a transposing DPP reduction that leaves one token's logit
// per lane. The gate and the online softmax run per lane in float32 (running
// max per row of lanes); the weights go through LDS to the lanes holding the
// matching value rows. V of tile i streams while the logits of tile i are
// computed, K of tile i+1 while the values of tile i are accumulated. No float
// atomics anywhere.
#include "eta_screen_dev.h"

namespace eta {
namespace {

struct AttendArgs {
  CacheView c;
  SeqView s;
  DecodeParams p;
  Dims d;
  Ws ws;
  int fz_P;         // one-launch decode: workgroups per segment
  uint64_t fz_tag;  // one-launch decode: tag of this call in the arrival words (40 bits, not 0)
};

// Copy p of the screen's results (copy 0 is the one the statistics read).
__device__ __forceinline__ Ws screen_copy(Ws w, int p) {
  if (p == 0) return w;
  const int64_t off = (int64_t)p * w.scr_stride;
  auto sh = [off](auto* q) { return reinterpret_cast<decltype(q)>(reinterpret_cast<char*>(q) + off); };
  w.tau = sh(w.tau);
  w.tile_cnt = sh(w.tile_cnt);
  w.tile_ent = sh(w.tile_ent);
  w.tile_sub = sh(w.tile_sub);
  w.tile_off = sh(w.tile_off);
  w.tile_hcnt = sh(w.tile_hcnt);
  w.tile_bits = sh(w.tile_bits);
  w.tile_umax = sh(w.tile_umax);
  w.tile_uarg = sh(w.tile_uarg);
  w.tile_err = sh(w.tile_err);
  w.seg_U = sh(w.seg_U);
  w.seg_ub = sh(w.seg_ub);
  w.seg_ntn = sh(w.seg_ntn);
  w.seg_err = sh(w.seg_err);
  w.st_head = sh(w.st_head);
  w.st_tokens = sh(w.st_tokens);
  w.st_rescued = sh(w.st_rescued);
  return w;
}

// Entries [c, c + cnt) of the segment's compacted lists, one per lane
// (lane < cnt): the tile whose prefix covers the index is found by binary
// search over the prefix in LDS (index ntn is the rescue tile).
// With smaller screen blocks (tsub not null), *sw receives the entry's word of
// per-head block bits from the same position of the parallel list.
__device__ __forceinline__ int2 resolve_entries(const int* toff_lds, const int2* tents, int ntn, int NT,
                                                int c, int cnt, int lane, const uint32_t* tsub = nullptr,
                                                uint32_t* sw = nullptr) {
  int2 ev = make_int2(0, 0);
  if (lane < cnt) {
    const int x = c + lane;
    int lo_v = 0, hi_v = ntn;
    while (lo_v < hi_v) {
      const int mid = (lo_v + hi_v + 1) >> 1;
      if (toff_lds[mid] <= x) lo_v = mid;
      else hi_v = mid - 1;
    }
    const int phys = lo_v < ntn ? lo_v : NT;
    const int64_t at = (int64_t)phys * kTile + (x - toff_lds[lo_v]);
    ev = tents[at];
    if (tsub) *sw = tsub[at];
  }
  return ev;
}

// Claim of CL consecutive entries of the workgroup's current part. The first
// claim of every wavefront is static (entries e0 + wave CL ..), so no
// wavefront waits for the counter to be set up; later ones come from an LDS
// counter that starts at e0 + nw CL (the fastest wavefronts take the most
// entries), or, with `fixed`, follow the static pattern (claims wave,
// wave + nw, ... counted from e0), which makes the result independent of
// timing.
template <int CL>
__device__ __forceinline__ int claim_lds(int* ctr, int lane, bool fixed, int& nclaim, int wave, int nw, int e0) {
  const int c = nclaim++;
  if (fixed || c == 0) return e0 + (c * nw + wave) * CL;
  int v = 0;
  if (lane == 0) v = atomicAdd(ctr, CL);
  return __builtin_amdgcn_readfirstlane(v);
}

// Merge of one segment's partials into the output, by the workgroup that
// completed the segment: for each of its G heads,
// o = sum_p e^{m_p - M} acc_p / sum_p e^{m_p - M} l_p over the partial slots
// p = kf + s .. kl + s. NG threads take one segment: thread (group pg, head
// h, float4 column group cg) loads the partials pg, pg + PG, ...
// (kMergeBatch of them in flight: 48 partials in one round at 256 threads and 128 outputs) and folds them with an online maximum;
// the PG groups are then combined in a fixed order, so the result does not
// depend on timing. NaN when nothing was accumulated. The partials are read
// with device-coherent loads (they were written by workgroups on any die).
constexpr int kMergeBatch = 24;

template <int D, int G, int NG>
struct MergeLds {
  static constexpr int CG = D / 4;         // float4 column groups
  static constexpr int OUTS = G * CG;      // (head, column group) outputs
  static_assert(OUTS <= NG, "one thread per output at least");
  static constexpr int PG = NG / OUTS;     // thread groups splitting the partials
  float4 a[PG][OUTS];
  float2 ml[PG][OUTS];
};

// Part 1 (thread t < NG of the merge): fold this thread's share of the partials into M.a/M.ml.
template <int D, int G, int NG>
__device__ void merge_fold(const Ws& ws, MergeLds<D, G, NG>& M, int s, int kf, int kl, int t) {
  using ML = MergeLds<D, G, NG>;
  const int o = t % ML::OUTS, pg = t / ML::OUTS;
  if (pg >= ML::PG) return;
  const int h = o / ML::CG, cg = o % ML::CG;
  const int np = kl - kf + 1;
  const int64_t slot0 = (int64_t)kf + s;
  float Mx = -__builtin_inff(), l = 0.f;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int p0 = pg; p0 < np; p0 += kMergeBatch * ML::PG) {
    float4 v[kMergeBatch];
    float2 ml[kMergeBatch];
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const int p = p0 + j * ML::PG;
      const int64_t sl = slot0 + (p < np ? p : 0);
      v[j] = load_agent4(&ws.part_acc[(sl * G + h) * D + 4 * cg]);
      ml[j] = load_agent2(&ws.part_ml[(sl * G + h) * 2]);
      if (p >= np) ml[j].x = -__builtin_inff();
    }
    float Mb = Mx;
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) Mb = fmaxf(Mb, ml[j].x);
    if (Mb == -__builtin_inff()) continue;
    const float sc = Mx == -__builtin_inff() ? 0.f : fast_exp(Mx - Mb);
    l *= sc;
    a.x *= sc; a.y *= sc; a.z *= sc; a.w *= sc;
    Mx = Mb;
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const float wgt = ml[j].x == -__builtin_inff() ? 0.f : fast_exp(ml[j].x - Mx);
      l = fmaf(wgt, ml[j].y, l);
      a.x = fmaf(wgt, v[j].x, a.x);
      a.y = fmaf(wgt, v[j].y, a.y);
      a.z = fmaf(wgt, v[j].z, a.z);
      a.w = fmaf(wgt, v[j].w, a.w);
    }
  }
  M.a[pg][o] = a;
  M.ml[pg][o] = make_float2(Mx, l);
}

// Part 2 (after a workgroup barrier): combine the groups and write the output.
template <int D, int G, int NG>
__device__ void merge_write(const Ws& ws, const MergeLds<D, G, NG>& M, float* out, int s, int n, int g, int HQ,
                            int t) {
  using ML = MergeLds<D, G, NG>;
  const int o = t % ML::OUTS, pg = t / ML::OUTS;
  if (pg != 0) return;
  const int h = o / ML::CG, cg = o % ML::CG;
  float Mt = -__builtin_inff();
#pragma unroll
  for (int q = 0; q < ML::PG; ++q) Mt = fmaxf(Mt, M.ml[q][o].x);
  float4 tt = make_float4(0.f, 0.f, 0.f, 0.f);
  float lt = 0.f;
#pragma unroll
  for (int q = 0; q < ML::PG; ++q) {
    const float2 mq = M.ml[q][o];
    const float wq = mq.x == -__builtin_inff() ? 0.f : fast_exp(mq.x - Mt);
    const float4 u = M.a[q][o];
    lt = fmaf(wq, mq.y, lt);
    tt.x = fmaf(wq, u.x, tt.x);
    tt.y = fmaf(wq, u.y, tt.y);
    tt.z = fmaf(wq, u.z, tt.z);
    tt.w = fmaf(wq, u.w, tt.w);
  }
  float4 r;
  if (lt > 0.f) {
    r = make_float4(tt.x / lt, tt.y / lt, tt.z / lt, tt.w / lt);
  } else {
    const float nan = __builtin_nanf("");
    r = make_float4(nan, nan, nan, nan);
  }
  *(float4*)&out[((int64_t)n * HQ + g * G + h) * D + 4 * cg] = r;
  if (t == 0) __hip_atomic_store(&ws.seg_done[s], (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wavefronts per attend workgroup: eight (two per SIMD, one workgroup per CU)
// when a wavefront fits in 256 VGPRs, else four with the full register file.
template <typename T, int D, int G>
constexpr int attend_waves() {
  return (((T::kBytes == 2 || D == 64) && G <= 4) || (T::kBytes == 2 && D == 64)) ? 8 : 4;
}

// Bit q set when some head of the group admitted block q of the page (word
// of per-head block bits, bit q G + h).
template <int G>
__device__ __forceinline__ uint32_t block_union(uint32_t sw, int sb) {
  constexpr uint32_t full = (1u << G) - 1u;
  uint32_t u = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (q < sb && ((sw >> (q * G)) & full)) u |= 1u << q;
  return u;
}

// SUBB: screen blocks smaller than a page (2 or 4 per page, A.d.SB): each
// entry carries a word of per-head block bits (bit q G + h); a head attends
// only to the rows of its own blocks, and rows of blocks that no head of the
// group admitted are not loaded.
// ALL: every segment's tile prefix, used-tile count and union count fit in
// LDS (kSegLds ints); they are then read once in the first round.
constexpr int kSegLds = 12288;
// FUSED: the one-launch decode of short segments (at most kFusedTiles tiles of
// 64 blocks each, the geometric bound on page blocks): workgroup k belongs to
// segment k / fz_P as its member p = k % fz_P. It screens and finalizes the
// whole segment itself (a wavefront per tile) into copy p of the screen's
// results, so the segment's fz_P workgroups share nothing before their
// partials; each then attends to its share [p U / fz_P, (p + 1) U / fz_P) of
// the segment's U compacted entries. The screen's records of a segment are a
// few hundred KB, read by all its workgroups mostly from the dies' L2.
// Workgroup 0's copy is the one the statistics read. The last of a segment's
// workgroups to write its partial merges them; arrivals are counted in a
// word tagged with the call, so no earlier launch has to zero it.

template <typename T, int D, int G, bool SUBB, bool ALL, bool FUSED = false>
__global__ __launch_bounds__((64 * attend_waves<T, D, G>()))
__attribute__((amdgpu_waves_per_eu((attend_waves<T, D, G>() / 4), (attend_waves<T, D, G>() / 4))))
void k_attend(AttendArgs A) {
  static_assert(!FUSED || (!SUBB && !ALL && attend_waves<T, D, G>() == kFusedTiles),
                "the one-launch decode screens a tile per wavefront on page blocks");
  using L = TileLayout<T::kBytes, D>;
  constexpr int LPR = L::LPR, RPI = L::RPI, NI = L::NI, CPL = L::CPL, EPL = L::EPL, EPC = L::EPC;
  constexpr int NW = attend_waves<T, D, G>();  // wavefronts per workgroup
  constexpr int NTH = 64 * NW;
  // entries per claim: two on the long ranges of the two-launch path; one in
  // the one-launch decode, whose workgroups hold a dozen entries or so, where
  // the last claims' tail weighs more (both measured)
  constexpr int CL = FUSED ? 1 : kClaim;
  constexpr bool kBf16 = T::kBytes == 2;
  using St = typename T::Stored;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int r = lane / LPR, cb = lane % LPR;
  const uint64_t t_start = __builtin_amdgcn_s_memrealtime();
  const int HKV = A.d.HKV, HQ = A.d.HQ, S = A.d.S;
  const float scale = A.p.scale, beta = A.p.beta;

  __shared__ __attribute__((aligned(16))) float p_lds[NW][G][64];
  __shared__ float ml_lds[NW][G][2];
  __shared__ float acc_lds[NW][G][D];
  __shared__ int toff_lds[kMaxBlocksPerSeq / kTile + 2];
  __shared__ int ctr_lds;
  __shared__ int scan_lds[NW];
  __shared__ int pick_lds[3];
  const int NT = A.d.NT;

  // the screen's results this workgroup reads (its own copy in the one-launch decode)
  Ws W = A.ws;
  // queries of a group at this lane's columns, and its thresholds
  uint32_t qb[G][CPL * 4];  // packed bf16 pairs (bf16 path)
  float qf[G][EPL];         // float32 path
  float tau[G];
  const auto load_q_tau = [&](int n, int g) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const St* qrow = (const St*)A.p.q + ((int64_t)n * HQ + g * G + h) * D;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const uint4 v = *(const uint4*)(qrow + L::col(c, cb));
        if constexpr (kBf16) {
          qb[h][c * 4 + 0] = v.x; qb[h][c * 4 + 1] = v.y; qb[h][c * 4 + 2] = v.z; qb[h][c * 4 + 3] = v.w;
        } else {
          qf[h][c * 4 + 0] = __uint_as_float(v.x); qf[h][c * 4 + 1] = __uint_as_float(v.y);
          qf[h][c * 4 + 2] = __uint_as_float(v.z); qf[h][c * 4 + 3] = __uint_as_float(v.w);
        }
      }
      tau[h] = W.tau[(int64_t)n * HQ + g * G + h];
    }
  };
  __shared__ int fz_ntn;
  const int k = blockIdx.x;
  int s = 0, P = 0, Us = 0, Wp = 0, n_entries = 0;
  uint64_t arrival_seen = 0;  // one-launch decode, thread 0
  int64_t lo = 0, hi = 0;
  __shared__ int seg_lds[ALL ? kSegLds : 1];
  const int rowlen = NT + 2;
  constexpr bool all_lds = ALL;  // the host checked S (NT + 4) <= kSegLds
  if constexpr (FUSED) {
    const int fp = k % A.fz_P;
    s = k / A.fz_P;
    W = screen_copy(A.ws, fp);
    // the segment's arrival word as it is now (read long before it is needed)
    if (threadIdx.x == 0) arrival_seen = arrival_word(&A.ws.fused_done[(int64_t)s * kArrivalStride]);
    ScreenArgs sa{A.c, A.s, A.p, A.d, W};
    if (k == 0 && threadIdx.x == 0) write_glob<D>(sa);
    if (wave < NT) screen_tile<T, D, G, 0, NW>(sa, s, wave, wave, lane);
    __syncthreads();
    // the segment's queries and thresholds (the screen has written them) load
    // while the finalize runs; the finalize hands over the union count, the
    // used tiles and the tile prefix (in toff_lds) without a memory round trip
    load_q_tau(s / HKV, s % HKV);
    FinArgs fa{A.c, A.s, A.d, W, A.p.out, A.p.deterministic, {}};
    Us = __builtin_amdgcn_readfirstlane(finalize_segment<G, NW>(fa, s, toff_lds, &fz_ntn));
    lo = (int64_t)fp * Us / A.fz_P;
    hi = (int64_t)(fp + 1) * Us / A.fz_P;
    n_entries = (int)(hi - lo);
    if (threadIdx.x == 0) ctr_lds = (int)lo + NW * CL;
    __syncthreads();
  } else {
    // ---- round 1: the segments' union counts (the work split needs them all)
    //      and, when they fit in LDS, every segment's tile prefix, used-tile
    //      count and union count, so that the first segment's entries can be
    //      located without another round trip
    // (lane x of wavefront 0 loads the weight of die class x: a lane-dependent
    // load, which the compiler does not move to scalar registers at once, so
    // nothing waits for it before the other loads are issued)
    __shared__ int w_lds[kXcdClasses];
    const int v0 = (int)threadIdx.x < S ? A.ws.seg_U[threadIdx.x] : 0;
    const int wv = (int)threadIdx.x < kXcdClasses ? A.ws.xcd_w[threadIdx.x] : 0;
    if constexpr (ALL) {  // [S][NT + 2] tile prefixes, then [S] used tiles, then [S] union counts
      // loaded straight into LDS (lane l of a wavefront's 64-element chunk
      // writes element l): no registers, no wait until the scan's barrier, and
      // a short loop instead of a long unrolled one
      const int ntile = S * rowlen;
      for (int c = wave * 64; c < ntile; c += NTH)
        if (c + lane < ntile) __builtin_amdgcn_global_load_lds(A.ws.tile_off + c + lane, seg_lds + c, 4, 0, 0);
      for (int c = wave * 64; c < S; c += NTH)
        if (c + lane < S) {
          __builtin_amdgcn_global_load_lds(A.ws.seg_ntn + c + lane, seg_lds + ntile + c, 4, 0, 0);
          __builtin_amdgcn_global_load_lds(A.ws.seg_U + c + lane, seg_lds + ntile + S + c, 4, 0, 0);
        }
    }
    if ((int)threadIdx.x < kXcdClasses) w_lds[threadIdx.x] = clamp_weight(wv, A.p.deterministic);
    wait_stores();  // the loads into LDS above have landed before the scan's first barrier
    int tot0;
    const int incl0 = block_incl_scan<NW>(v0, &tot0, scan_lds);
    int Utot = tot0;
    if (S > NTH) {
      int rest = 0;
      for (int i = NTH + threadIdx.x; i < S; i += NTH) rest += A.ws.seg_U[i];
      int totr;
      block_incl_scan<NW>(rest, &totr, scan_lds);
      Utot += totr;
    }
    Utot = __builtin_amdgcn_readfirstlane(Utot);
    // at least 8 entries per range on average, so that no range is empty at any
    // weights in [1/2, 2]
    Wp = Utot < 8 * (int)gridDim.x ? (Utot + 7) / 8 : (int)gridDim.x;
    if (k >= Wp) return;
    {
      int wts[kXcdClasses];
#pragma unroll
      for (int x = 0; x < kXcdClasses; ++x) wts[x] = w_lds[x];  // written before the scan's barriers
      RangeSplit sp;
      sp.init(Utot, Wp, wts);
      lo = sp.B(k);
      hi = sp.B(k + 1);
    }
    n_entries = (int)(hi - lo);
    // the segment holding entry lo, its first entry and its count; the thread
    // that finds it also sets up the claim counter of that segment's part
    if (v0 > 0 && incl0 - v0 <= lo && lo < incl0) {
      pick_lds[0] = threadIdx.x;
      pick_lds[1] = incl0 - v0;
      pick_lds[2] = v0;
      ctr_lds = (int)(lo - (incl0 - v0)) + NW * CL;
    }
    if (lo < hi && lo >= tot0) {  // beyond the first NTH segments: scan the rest in chunks
      int carry = tot0;
      for (int c0 = NTH; c0 < S && carry <= lo; c0 += NTH) {
        const int i = c0 + threadIdx.x;
        const int v = i < S ? A.ws.seg_U[i] : 0;
        int tot;
        const int incl = carry + block_incl_scan<NW>(v, &tot, scan_lds);
        if (v > 0 && incl - v <= lo && lo < incl) {
          pick_lds[0] = i;
          pick_lds[1] = incl - v;
          pick_lds[2] = v;
          ctr_lds = (int)(lo - (incl - v)) + NW * CL;
        }
        carry += tot;
      }
    }
    __syncthreads();
    // (uniform values go through readfirstlane so that they live in scalar
    // registers: the streaming loop needs every vector register)
    s = __builtin_amdgcn_readfirstlane(lo < hi ? pick_lds[0] : 0);
    P = __builtin_amdgcn_readfirstlane(lo < hi ? pick_lds[1] : 0);
    Us = __builtin_amdgcn_readfirstlane(lo < hi ? pick_lds[2] : 0);
  }
  const int s_first = s, P_first = P, U_first = Us;
  const int64_t lo_first = lo;
  bool first_part = true;
  bool part_due = FUSED;  // the one-launch decode writes a partial even for an empty share

  // lane offset (elements) of load (i=0, c) inside a tile
  int loff[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) loff[c] = r * D + L::col(c, cb);
  const St* kbase = (const St*)A.c.k;
  const St* vbase = (const St*)A.c.v;
  // smaller screen blocks: log2 of their tokens, and the block of load i's rows
  const int lbs = SUBB ? (A.d.SB == 4 ? 4 : 5) : 6;

  while (lo < hi || part_due) {
    part_due = false;
    if constexpr (!FUSED) {
      while (lo >= (int64_t)P + Us) {  // next segment with entries
        P += Us;
        ++s;
        Us = all_lds ? seg_lds[S * rowlen + S + s] : A.ws.seg_U[s];
      }
    }
    const int e0 = (int)(lo - P);
    const int e1 = (int)((hi < (int64_t)P + Us ? hi : (int64_t)P + Us) - P);
    const int n = s / HKV, g = s % HKV;
    const int seq_len = A.s.lens[n];
    const int nfull = seq_len / kBlock;
    const int rem = seq_len - nfull * kBlock;

    if constexpr (!FUSED) load_q_tau(n, g);  // (the one-launch decode loaded them in its prologue)
    float m[G], l[G], acc[G][EPL];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = -__builtin_inff();
      l[h] = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
    }

    // the segment's tile prefix (to locate entries in the per-tile lists), and
    // the part's claim counter (for the first part, set up with the pick)
    const int* toffp = toff_lds;
    int ntn;
    if constexpr (ALL) {
      toffp = seg_lds + s * rowlen;
      ntn = seg_lds[S * rowlen + s];
      if (!first_part) {
        if (threadIdx.x == 0) ctr_lds = e0 + NW * CL;
        __syncthreads();
      }
    } else if constexpr (FUSED) {
      ntn = fz_ntn;  // toff_lds and the claim counter were set up in the prologue
    } else {
      ntn = W.seg_ntn[s];
      const int32_t* toff = W.tile_off + (int64_t)s * rowlen;  // the whole row: the loads do not wait for ntn
      for (int v = threadIdx.x; v < rowlen; v += NTH) toff_lds[v] = toff[v];
      if (threadIdx.x == 0) ctr_lds = e0 + NW * CL;
      __syncthreads();
    }
    first_part = false;
    const int2* tents = W.tile_ent + (int64_t)s * (NT + 1) * kTile;
    const uint32_t* tsubs = SUBB ? W.tile_sub + (int64_t)s * (NT + 1) * kTile : nullptr;

    // claims, two deep: the batch being streamed, the next one (resolved while
    // the current one streams) and the claim after it
    const bool fixed = A.p.deterministic != 0;
    int nclaim = 0;
    const int c0 = claim_lds<CL>(&ctr_lds, lane, fixed, nclaim, wave, NW, e0);
    int bc = c0 < e1 ? min(CL, e1 - c0) : 0;
    if (bc > 0) {
      uint32_t ews = 0, ewsn = 0;
      int2 ev = resolve_entries(toffp, tents, ntn, NT, c0, bc, lane, tsubs, &ews);
      int it = 0;
      int page_nx = __builtin_amdgcn_readlane(ev.x, 0);
      int jm_nx = __builtin_amdgcn_readlane(ev.y, 0);
      uint32_t sw_nx = SUBB ? (uint32_t)__builtin_amdgcn_readlane((int)ews, 0) : 0u;

      uint4 kr[NI][CPL], vr[NI][CPL];
      {
        const St* kt = kbase + ((int64_t)page_nx * HKV + g) * (kBlock * D);
        const uint32_t ub = SUBB ? block_union<G>(sw_nx, A.d.SB) : 0u;
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int c = 0; c < CPL; ++c)
            kr[i][c] = (!SUBB || ((ub >> ((RPI * i) >> lbs)) & 1u)) ? load_stream16(kt + loff[c] + i * RPI * D)
                                                                   : make_uint4(0, 0, 0, 0);
      }
      // the next claim is resolved while the first tile's keys are in flight
      const int c1 = claim_lds<CL>(&ctr_lds, lane, fixed, nclaim, wave, NW, e0);
      int bcn = c1 < e1 ? min(CL, e1 - c1) : 0;
      int2 evn = resolve_entries(toffp, tents, ntn, NT, c1, bcn, lane, tsubs, &ewsn);
      for (;;) {
        const int cur_page = page_nx, cur_jm = jm_nx;
        const uint32_t cur_sw = sw_nx;
        {
          const St* vt = vbase + ((int64_t)cur_page * HKV + g) * (kBlock * D);
          const uint32_t ub = SUBB ? block_union<G>(cur_sw, A.d.SB) : 0u;
#pragma unroll
          for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int c = 0; c < CPL; ++c)
              vr[i][c] = (!SUBB || ((ub >> ((RPI * i) >> lbs)) & 1u)) ? load_stream16(vt + loff[c] + i * RPI * D)
                                                                     : make_uint4(0, 0, 0, 0);
        }
        // next entry: from this batch, or the first of the next one
        bool has_next = true;
        if (++it >= bc) {
          ev = evn;
          ews = ewsn;
          bc = bcn;
          it = 0;
          if (bc > 0) {
            const int c2 = claim_lds<CL>(&ctr_lds, lane, fixed, nclaim, wave, NW, e0);
            bcn = c2 < e1 ? min(CL, e1 - c2) : 0;
            evn = resolve_entries(toffp, tents, ntn, NT, c2, bcn, lane, tsubs, &ewsn);
          } else {
            has_next = false;
          }
        }
        if (has_next) {
          page_nx = __builtin_amdgcn_readlane(ev.x, it);
          jm_nx = __builtin_amdgcn_readlane(ev.y, it);
          if (SUBB) sw_nx = (uint32_t)__builtin_amdgcn_readlane((int)ews, it);
        }
        const uint32_t hmask = (uint32_t)cur_jm & 0xffu;
        const int j = cur_jm >> 8;
        const bool tail = (j == nfull);  // only the partial last block has j == nfull
        const int tok = RPI * cb + r;     // token whose logit this lane finishes

        // ---- logits, gate, online softmax per admitted head
#pragma unroll
        for (int h = 0; h < G; ++h) {
          if (!(hmask & (1u << h))) continue;
          float pd[NI];
#pragma unroll
          for (int i = 0; i < NI; ++i) {
            float a = 0.f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
              const uint32_t kw[4] = {kr[i][c].x, kr[i][c].y, kr[i][c].z, kr[i][c].w};
#pragma unroll
              for (int w = 0; w < 4; ++w) {
                if constexpr (kBf16) {
                  a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qb[h][c * 4 + w]),
                                                      __builtin_bit_cast(bf16x2_t, kw[w]), a, false);
                } else {
                  a = fmaf(qf[h][c * 4 + w], __uint_as_float(kw[w]), a);
                }
              }
            }
            pd[i] = a;
          }
          transpose_reduce<LPR>(pd, lane);
          const float S_ = pd[0] * scale;
          const float x = beta * (S_ - tau[h]);
          const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * kLog2e));
          float sv = S_ * sg;
          if (tail && tok >= rem) sv = -__builtin_inff();
          if (SUBB && !((cur_sw >> ((tok >> lbs) * G + h)) & 1u)) sv = -__builtin_inff();  // not this head's block
          const float mt = group_max<LPR>(sv);
          const float mnew = fmaxf(m[h], mt);
          const float muse = mnew == -__builtin_inff() ? 0.f : mnew;
          const float alpha = fast_exp(m[h] - muse);
          const float p = fast_exp(sv - muse);
          l[h] = fmaf(l[h], alpha, p);
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
          m[h] = mnew;
          p_lds[wave][h][lane] = p;
        }

        // ---- K of the next tile streams while the values are accumulated
        if (has_next) {
          const St* kt = kbase + ((int64_t)page_nx * HKV + g) * (kBlock * D);
          const uint32_t ub = SUBB ? block_union<G>(sw_nx, A.d.SB) : 0u;
#pragma unroll
          for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int c = 0; c < CPL; ++c)
              kr[i][c] = (!SUBB || ((ub >> ((RPI * i) >> lbs)) & 1u)) ? load_stream16(kt + loff[c] + i * RPI * D)
                                                                     : make_uint4(0, 0, 0, 0);
        }
        if (tail) {  // junk rows past the end must not reach the sums (0 * NaN)
#pragma unroll
          for (int i = 0; i < NI; ++i)
            if (RPI * i + r >= rem)
#pragma unroll
              for (int c = 0; c < CPL; ++c) vr[i][c] = make_uint4(0, 0, 0, 0);
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();

        // ---- acc[h] += p_h(token) * v(token)
#pragma unroll
        for (int i4 = 0; i4 < NI / 4; ++i4) {
          float4 pw[G];
#pragma unroll
          for (int h = 0; h < G; ++h)
            if (hmask & (1u << h)) pw[h] = *(const float4*)&p_lds[wave][h][r * LPR + 4 * i4];
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int i = 4 * i4 + ii;
            float vf[EPL];
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
              const uint32_t vw[4] = {vr[i][c].x, vr[i][c].y, vr[i][c].z, vr[i][c].w};
              if constexpr (kBf16) {
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                  vf[c * 8 + 2 * w] = bf16_lo(vw[w]);
                  vf[c * 8 + 2 * w + 1] = bf16_hi(vw[w]);
                }
              } else {
#pragma unroll
                for (int w = 0; w < 4; ++w) vf[c * 4 + w] = __uint_as_float(vw[w]);
              }
            }
#pragma unroll
            for (int h = 0; h < G; ++h) {
              if (!(hmask & (1u << h))) continue;
              // smaller screen blocks: the RPI rows of load i lie in one block
              // (RPI <= 8 < 16 tokens); a head skips the rows of blocks it did
              // not admit, so their values never reach its sums (not even as
              // 0 * v, which a non-finite v would turn into NaN)
              if (SUBB && !((cur_sw >> (((RPI * i) >> lbs) * G + h)) & 1u)) continue;
              const float pv = ii == 0 ? pw[h].x : ii == 1 ? pw[h].y : ii == 2 ? pw[h].z : pw[h].w;
#pragma unroll
              for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pv, vf[e], acc[h][e]);
            }
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        if (!has_next) break;
      }
    }

    // ---- merge the rows of lanes, then the wavefronts, write one partial
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float lr = group_sum<LPR>(l[h]);
      float M = m[h];
#pragma unroll
      for (int o = LPR; o < 64; o <<= 1) M = fmaxf(M, shfl_xor_f(M, o));
      const float sc = m[h] == -__builtin_inff() ? 0.f : fast_exp(m[h] - M);
      float lw = sc * lr;
#pragma unroll
      for (int o = LPR; o < 64; o <<= 1) lw += shfl_xor_f(lw, o);
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        float a = sc * acc[h][e];
#pragma unroll
        for (int o = LPR; o < 64; o <<= 1) a += shfl_xor_f(a, o);
        acc[h][e] = a;
      }
      if (r == 0) {
#pragma unroll
        for (int c = 0; c < CPL; ++c)
#pragma unroll
          for (int e = 0; e < EPC; ++e) acc_lds[wave][h][L::col(c, cb) + e] = acc[h][c * EPC + e];
      }
      if (lane == 0) {
        ml_lds[wave][h][0] = M;
        ml_lds[wave][h][1] = lw;
      }
    }
    __syncthreads();
    const int64_t piece = FUSED ? (int64_t)k : (int64_t)k + s;
    for (int h = wave; h < G; h += NW) {
      float Mw[NW], M = -__builtin_inff();
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        Mw[w] = ml_lds[w][h][0];
        M = fmaxf(M, Mw[w]);
      }
      float sc[NW], Lsum = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        sc[w] = Mw[w] == -__builtin_inff() ? 0.f : fast_exp(Mw[w] - M);
        Lsum = fmaf(sc[w], ml_lds[w][h][1], Lsum);
      }
      float* pa = A.ws.part_acc + (piece * G + h) * D;
      for (int dd = lane; dd < D; dd += 64) {
        float a = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) a = fmaf(sc[w], acc_lds[w][h][dd], a);
        store_agent(pa + dd, a);
      }
      if (lane == 0) store_agent2(A.ws.part_ml + (piece * G + h) * 2, M, Lsum);
    }
    __syncthreads();
    lo = (int64_t)P + e1;
  }

  // ---- arrivals: for every segment the range touched, add its entries to the
  //      segment's count; the workgroup that completes a segment merges the
  //      segment's partials (slots kf + s .. kl + s) into the output. The
  //      partials were written with device-coherent stores; every wavefront
  //      waits for its stores to complete and the workgroup barrier orders
  //      that before thread 0's counts. A merging workgroup reads the
  //      partials with device-coherent loads after its count returned. No
  //      cache maintenance of the dies' L2s is needed.
  wait_stores();
  __syncthreads();
  if constexpr (FUSED) {
    // one arrival per workgroup in the segment's tagged arrival word
    __shared__ int last_lds;
    __shared__ MergeLds<D, G, NTH> mgf;
    if (threadIdx.x == 0)
      last_lds = arrive_tagged(&A.ws.fused_done[(int64_t)s * kArrivalStride], arrival_seen, A.fz_tag, A.fz_P) ? 1 : 0;
    __syncthreads();
    if (last_lds) {  // the segment's partials are slots s fz_P .. s fz_P + fz_P - 1
      merge_fold<D, G, NTH>(A.ws, mgf, s * A.fz_P, 0, A.fz_P - 1, threadIdx.x);
      __syncthreads();
      merge_write<D, G, NTH>(A.ws, mgf, A.p.out, s, s / HKV, s % HKV, HQ, threadIdx.x);
    }
    return;
  } else {
    // The segments this range touched, up to 64 at a time: wave 0's lane j
    // adds the entry count of the j-th of them with one 64-bit add, which
    // also carries, from the ranges holding the segment's first and last
    // entries, their indices. Every count is added before any merge starts,
    // so a merge here never delays another segment's completion; two
    // completed segments are merged side by side when the workgroup has the
    // threads for it.
    constexpr int NG2 = 2 * (G * D / 4) <= NTH ? NTH / 2 : NTH;  // threads per merge (one per output at least)
    constexpr int NPAR = NTH / NG2;                                               // merges side by side
    __shared__ MergeLds<D, G, NG2> mg[NPAR];
    __shared__ int done_s[64], done_kf[64], done_kl[64];
    __shared__ int ndone_lds;
    int s2 = s_first, P2 = P_first, U2 = U_first;
    int64_t x = lo_first;
    while (x < hi) {
      if (threadIdx.x == 0) ndone_lds = 0;
      __syncthreads();
      if (wave == 0) {
        int my_s = -1, my_c0 = 0, my_c1 = 0, my_u = 0;
        for (int j = 0; j < 64 && x < hi; ++j) {
          while (x >= (int64_t)P2 + U2) {
            P2 += U2;
            ++s2;
            U2 = all_lds ? seg_lds[S * rowlen + S + s2] : A.ws.seg_U[s2];
          }
          const int c0 = (int)(x - P2);
          const int c1 = (int)((hi < (int64_t)P2 + U2 ? hi : (int64_t)P2 + U2) - P2);
          if (lane == j) {
            my_s = s2;
            my_c0 = c0;
            my_c1 = c1;
            my_u = U2;
          }
          x = (int64_t)P2 + c1;
        }
        if (my_s >= 0) {
          const uint64_t add = (uint64_t)(my_c1 - my_c0) + (my_c0 == 0 ? (uint64_t)k << 32 : 0ull) +
                               (my_c1 == my_u ? (uint64_t)k << 48 : 0ull);
          const uint64_t tot =
              __hip_atomic_fetch_add(&A.ws.seg_done[my_s], add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + add;
          if ((uint32_t)tot == (uint32_t)my_u) {
            const int at = atomicAdd(&ndone_lds, 1);
            done_s[at] = my_s;
            done_kf[at] = (int)((tot >> 32) & 0xffffu);
            done_kl[at] = (int)(tot >> 48);
          }
        }
      } else {  // keep the other wavefronts' copy of the walk in step
        for (int j = 0; j < 64 && x < hi; ++j) {
          while (x >= (int64_t)P2 + U2) {
            P2 += U2;
            ++s2;
            U2 = all_lds ? seg_lds[S * rowlen + S + s2] : A.ws.seg_U[s2];
          }
          x = (int64_t)P2 + (int)((hi < (int64_t)P2 + U2 ? hi : (int64_t)P2 + U2) - P2);
        }
      }
      __syncthreads();
      const int nd = ndone_lds;
      for (int d0 = 0; d0 < nd; d0 += NPAR) {
        const int part = (int)threadIdx.x / NG2, t = (int)threadIdx.x % NG2;
        const int d = d0 + part;
        if (d < nd) merge_fold<D, G, NG2>(A.ws, mg[part], done_s[d], done_kf[d], done_kl[d], t);
        __syncthreads();
        if (d < nd) merge_write<D, G, NG2>(A.ws, mg[part], A.p.out, done_s[d], done_s[d] / HKV, done_s[d] % HKV, HQ, t);
        __syncthreads();
      }
    }
  }
  // entries and duration of this range, read by the next decode's weighting
  if (threadIdx.x == 0) {
    const uint64_t t_end = __builtin_amdgcn_s_memrealtime();
    A.ws.rng_stat[2 * k] = n_entries;
    A.ws.rng_stat[2 * k + 1] = (int)min<uint64_t>(t_end - t_start, 0x7fffffffu);
    if (k == 0) {
      A.ws.glob[kGlobStatMagic] = kStatMagic;
      A.ws.glob[kGlobStatW] = Wp;
    }
  }
}

template <typename T, int D, int G>
hipError_t attend_impl(const CacheView& c, const SeqView& s, const DecodeParams& p, const Dims& d,
                       const Ws& ws, int W, hipStream_t st) {
  AttendArgs a{c, s, p, d, ws};
  const dim3 grid(W), block(64 * attend_waves<T, D, G>());
  const bool all = (int64_t)d.S * (d.NT + 4) <= kSegLds;
  if (d.SB > 1) {
    if (all) hipLaunchKernelGGL((k_attend<T, D, G, true, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((k_attend<T, D, G, true, false>), grid, block, 0, st, a);
  } else {
    if (all) hipLaunchKernelGGL((k_attend<T, D, G, false, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((k_attend<T, D, G, false, false>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t attend_g(const CacheView& c, const SeqView& s, const DecodeParams& p, const Dims& d,
                    const Ws& ws, int W, hipStream_t st) {
  switch (d.G) {
    case 1: return attend_impl<T, D, 1>(c, s, p, d, ws, W, st);
    case 2: return attend_impl<T, D, 2>(c, s, p, d, ws, W, st);
    case 4: return attend_impl<T, D, 4>(c, s, p, d, ws, W, st);
    case 8: return attend_impl<T, D, 8>(c, s, p, d, ws, W, st);
  }
  return hipErrorInvalidValue;
}

// One-launch decode of short segments: fz_P workgroups per segment.
template <typename T, int D, int G>
hipError_t short_impl(const CacheView& c, const SeqView& s, const DecodeParams& p, const Dims& d,
                      const Ws& ws, int fz_P, uint64_t tag, hipStream_t st) {
  if constexpr (attend_waves<T, D, G>() != kFusedTiles) {
    return hipErrorNotSupported;
  } else {
    AttendArgs a{c, s, p, d, ws, fz_P, tag};
    hipLaunchKernelGGL((k_attend<T, D, G, false, false, true>), dim3(d.S * fz_P), dim3(64 * kFusedTiles), 0, st,
                       a);
    return hipGetLastError();
  }
}

template <typename T, int D>
hipError_t short_g(const CacheView& c, const SeqView& s, const DecodeParams& p, const Dims& d, const Ws& ws,
                   int fz_P, uint64_t tag, hipStream_t st) {
  switch (d.G) {
    case 1: return short_impl<T, D, 1>(c, s, p, d, ws, fz_P, tag, st);
    case 2: return short_impl<T, D, 2>(c, s, p, d, ws, fz_P, tag, st);
    case 4: return short_impl<T, D, 4>(c, s, p, d, ws, fz_P, tag, st);
    case 8: return short_impl<T, D, 8>(c, s, p, d, ws, fz_P, tag, st);
  }
  return hipErrorInvalidValue;
}

template <typename T, int D>
bool short_ok(int G) {
  switch (G) {
    case 1: return attend_waves<T, D, 1>() == kFusedTiles;
    case 2: return attend_waves<T, D, 2>() == kFusedTiles;
    case 4: return attend_waves<T, D, 4>() == kFusedTiles;
    case 8: return attend_waves<T, D, 8>() == kFusedTiles;
  }
  return false;
}

template <typename T, int D, int G>
int occupancy_impl() {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, reinterpret_cast<const void*>(&k_attend<T, D, G, false, true>),
                                                   64 * attend_waves<T, D, G>(), 0) != hipSuccess)
    return 1;
  return nb > 0 ? nb : 1;
}

template <typename T, int D>
int occupancy_g(int G) {
  switch (G) {
    case 1: return occupancy_impl<T, D, 1>();
    case 2: return occupancy_impl<T, D, 2>();
    case 4: return occupancy_impl<T, D, 4>();
    case 8: return occupancy_impl<T, D, 8>();
  }
  return 1;
}

}  // namespace

hipError_t launch_attend(const CacheView& c, const SeqView& s, const DecodeParams& p, const Dims& d,
                         const Ws& ws, int W, hipStream_t st) {
  if (c.kv_dtype == 1) return d.D == 128 ? attend_g<Bf16, 128>(c, s, p, d, ws, W, st) : attend_g<Bf16, 64>(c, s, p, d, ws, W, st);
  return d.D == 128 ? attend_g<F32, 128>(c, s, p, d, ws, W, st) : attend_g<F32, 64>(c, s, p, d, ws, W, st);
}

hipError_t launch_decode_short(const CacheView& c, const SeqView& s, const DecodeParams& p, const Dims& d,
                               const Ws& ws, int wgs_per_segment, uint64_t tag, hipStream_t st) {
  if (c.kv_dtype == 1)
    return d.D == 128 ? short_g<Bf16, 128>(c, s, p, d, ws, wgs_per_segment, tag, st)
                      : short_g<Bf16, 64>(c, s, p, d, ws, wgs_per_segment, tag, st);
  return d.D == 128 ? short_g<F32, 128>(c, s, p, d, ws, wgs_per_segment, tag, st)
                    : short_g<F32, 64>(c, s, p, d, ws, wgs_per_segment, tag, st);
}

bool decode_short_supported(int kv_dtype, int D, int G) {
  if (kv_dtype == 1) return D == 128 ? short_ok<Bf16, 128>(G) : short_ok<Bf16, 64>(G);
  return D == 128 ? short_ok<F32, 128>(G) : short_ok<F32, 64>(G);
}

int attend_wgs_per_cu(int kv_dtype, int D, int G) {
  if (kv_dtype == 1) return D == 128 ? occupancy_g<Bf16, 128>(G) : occupancy_g<Bf16, 64>(G);
  return D == 128 ? occupancy_g<F32, 128>(G) : occupancy_g<F32, 64>(G);
}

}  // namespace eta
