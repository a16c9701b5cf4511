// Device code of the screen phase shared by the screen kernels and the
// one-launch decode of short segments: the tile screen (thresholds, bound
// test, compaction of one tile of 64 blocks by one wavefront) and the
// finalize of a segment (totals, top-1 rescue, tile prefix, counts), with
// the arguments they read. Included by eta_screen.hip and eta_attend.hip;
// what each step computes, with its passages, is described at the top of
// eta_screen.hip.
#pragma once

#include <limits.h>

#include "eta_device.h"

namespace eta {
namespace {

struct ScreenArgs {
  CacheView c;
  SeqView s;
  DecodeParams p;
  Dims d;
  Ws ws;
};

template <typename T>
__device__ __forceinline__ void load8(const typename T::Stored* p, float (&out)[8]);
template <>
__device__ __forceinline__ void load8<Bf16>(const uint16_t* p, float (&out)[8]) {
  const uint4 v = *(const uint4*)p;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = bf16_lo(w[i]);
    out[2 * i + 1] = bf16_hi(w[i]);
  }
}
template <>
__device__ __forceinline__ void load8<F32>(const float* p, float (&out)[8]) {
  const float4 a = *(const float4*)p;
  const float4 b = *(const float4*)(p + 4);
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

// MODE: 0 geometric bound, 1 dual score, 2 comparator box bound, 3 geometric
// bound over the FP8 records, 4 geometric bound on smaller screen blocks
// (SB = A.d.SB of them per page), 5 geometric bound on 128-token blocks.
// The sizes this decode laid the workspace out for (the header).
template <int D>
__device__ __forceinline__ void write_glob(const ScreenArgs& A) {
  A.ws.glob[kGlobN] = A.d.N;
  A.ws.glob[kGlobMB] = A.d.MB;
  A.ws.glob[kGlobHQ] = A.d.HQ;
  A.ws.glob[kGlobHKV] = A.d.HKV;
  A.ws.glob[kGlobD] = D;
  A.ws.glob[kGlobSB] = A.d.SB;
  A.ws.glob[kGlobPB] = A.d.PB;
}

// Tile t (64 consecutive screen blocks) of segment s (sequence, KV head),
// screened by one wavefront.
template <typename T, int D, int G, int MODE, int NW>
__device__ __forceinline__ void screen_tile(const ScreenArgs& A, int s, int t, int wave, int lane) {
  constexpr bool DUAL = MODE == 1, BOX = MODE == 2, FP8 = MODE == 3, SUBB = MODE == 4, PAIR = MODE == 5;
  using L = TileLayout<2, D>;  // float16 centroid rows
  constexpr int LPR = L::LPR, RPI = L::RPI, NI = L::NI;
  static_assert(L::CPL == 1 && L::EPC == 8, "centroid rows are one 8-half chunk per lane");
  const int r = lane / LPR, cb = lane % LPR;
  const int HKV = A.d.HKV, MB = A.d.MB, NT = A.d.NT, HQ = A.d.HQ;
  const int n = s / HKV, g = s % HKV;
  const int64_t tix = (int64_t)s * NT + t;
  const int64_t tcx = (int64_t)s * (NT + 1) + t;  // index into tile_cnt / tile_ent
  const int j0 = t * kTile;

  // ---- every load that does not need another load's value is issued first:
  //      length, block-table entries (clamped to the row, whatever the length),
  //      queries and predictor weights; then centroids and radii
  const int seq_len = A.s.lens[n];
  const int32_t* bt = A.s.bt + (int64_t)n * MB;
  // screen blocks per page (1 unless SUBB) and its log2. A lane's unit j is a
  // screen block, or with 128-token blocks a page (block j / 2, whose record
  // lives with page j & ~1).
  const int SB = SUBB ? A.d.SB : 1, lsb = SUBB ? (A.d.SB == 4 ? 2 : 1) : 0;
  int pg[NI];  // pages holding the records
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int j = j0 + RPI * i + r;
    pg[i] = bt[min(PAIR ? (j & ~1) : j >> lsb, MB - 1)];
  }
  const int jl = j0 + RPI * cb + r;  // unit this lane owns after the reduction
  const int page_l = bt[min(jl >> lsb, MB - 1)];
  // 128-token blocks: the other page of the lane's block, and the page that
  // keeps the block's record (the first one)
  const int page_o = PAIR ? bt[min(jl ^ 1, MB - 1)] : page_l;
  const int page_r = PAIR && (jl & 1) ? page_o : page_l;

  float qf[G][8];
  const auto* qbase = (const typename T::Stored*)A.p.q;
#pragma unroll
  for (int h = 0; h < G; ++h) load8<T>(qbase + ((int64_t)n * HQ + g * G + h) * D + cb * 8, qf[h]);
  // predictor weights through a buffer of size 0 in calibrated mode (reads zeros)
  const auto w_rsrc = make_rsrc(A.p.w, A.p.tau_mode == 0 ? (uint32_t)(HQ * D * 4) : 0u);
  uint32_t wraw[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint32_t off = (uint32_t)(((g * G + h) * D + cb * 8) * 4);
    const auto w0 = __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, off, 0, 0);
    const auto w1 = __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, off + 16, 0, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      wraw[h][e] = w0[e];
      wraw[h][4 + e] = w1[e];
    }
  }

  const bool badT = seq_len < 1 || seq_len > kBlock * MB;
  const int bsz = PAIR ? 2 * kBlock : kBlock >> lsb;  // tokens per screen block
  const int nfull = badT ? 0 : seq_len / bsz;
  const int nblk = badT ? 0 : (seq_len + bsz - 1) / bsz;
  const int nunit = PAIR ? (badT ? 0 : (seq_len + kBlock - 1) / kBlock) : nblk;  // lanes' units in the sequence
  // A tile wholly past the sequence has nothing to screen, and the finalize
  // uses only the tiles below ceil(nunit / 64): it stops here, writing only
  // its zero head bitmaps (they are the per-head admitted sets the statistics
  // copy out whole). Tile 0 always runs (it writes the thresholds; with a bad
  // or zero length every block of it is invalid: no entries, zero bitmaps).
  if (t > 0 && j0 >= nunit) {
    if (lane < G) A.ws.tile_bits[((int64_t)s * G + lane) * NT + t] = 0;
    return;
  }
  const int jbl = PAIR ? jl >> 1 : jl;                                            // the lane's screen block
  const bool lvalid = jl < nunit && page_l >= 0 && page_l < A.c.num_pages;
  // a 128-token block is complete only when both of its pages are valid, so
  // that neither lane of it can be admitted, ranked or rescued otherwise
  const bool complete = jbl < nfull && lvalid && page_o >= 0 && page_o < A.c.num_pages;
  // records through buffer loads: an invalid block reads zeros, without a branch
  // (the box bound reads the key box's lower corner here and its upper one below;
  // a smaller screen block's record is block j mod SB of its page's records)
  const auto mu_rsrc = make_rsrc(BOX ? (const void*)A.c.kmin : (SUBB || PAIR) ? (const void*)A.c.mu_sub
                                                                              : (const void*)A.c.mu,
                                 (uint32_t)((int64_t)A.c.num_pages * HKV * SB * D * 2));
  const auto r_rsrc = make_rsrc((SUBB || PAIR) ? (const void*)A.c.radius_sub : (const void*)A.c.radius,
                                (uint32_t)((int64_t)A.c.num_pages * HKV * SB * 4));
  const auto mu8_rsrc = make_rsrc(A.c.mu8, FP8 ? (uint32_t)((int64_t)A.c.num_pages * HKV * D) : 0u);
  const auto r8_rsrc = make_rsrc(A.c.radius8, FP8 ? (uint32_t)((int64_t)A.c.num_pages * HKV * 4) : 0u);
  uint4 raw[NI];  // FP8: the lane's 8 bytes in .x/.y
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int j = j0 + RPI * i + r;
    const bool ok = (PAIR ? j >> 1 : j) < nfull && pg[i] >= 0 && pg[i] < A.c.num_pages;
    if constexpr (FP8) {
      const uint32_t off = ok ? (uint32_t)(((int64_t)pg[i] * HKV + g) * D + cb * 8) : kOutOfRange;
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(mu8_rsrc, off, 0, 0);
      raw[i] = make_uint4(v[0], v[1], 0u, 0u);
    } else {
      const int64_t rec = ((int64_t)pg[i] * HKV + g) * SB + (j & (SB - 1));
      const uint32_t off = ok ? (uint32_t)((rec * D + cb * 8) * 2) : kOutOfRange;
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(mu_rsrc, off, 0, 0);
      raw[i] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  }
  const uint32_t roff = complete ? (uint32_t)((((int64_t)page_r * HKV + g) * SB + (jl & (SB - 1))) * 4) : kOutOfRange;
  const float R = BOX ? 0.f
                      : __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(FP8 ? r8_rsrc : r_rsrc, roff, 0, 0));
  // dual screen: coordinate deviations; box bound: upper corners (both laid
  // out like the centroids)
  uint4 sraw[DUAL || BOX ? NI : 1];
  if constexpr (DUAL || BOX) {
    const auto s_rsrc = make_rsrc(BOX ? (const void*)A.c.kmax : (const void*)A.c.sigma,
                                  (uint32_t)((int64_t)A.c.num_pages * HKV * D * 2));
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int j = j0 + RPI * i + r;
      const bool ok = j < nfull && pg[i] >= 0 && pg[i] < A.c.num_pages;
      const uint32_t off = ok ? (uint32_t)((((int64_t)pg[i] * HKV + g) * D + cb * 8) * 2) : kOutOfRange;
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(s_rsrc, off, 0, 0);
      sraw[i] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  }

  // ---- thresholds and query norms (every row of lanes holds all D columns)
  float tau[G], qn[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float ssq = 0.f, dotw = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ssq = fmaf(qf[h][e], qf[h][e], ssq);
      dotw = fmaf(__uint_as_float(wraw[h][e]), qf[h][e], dotw);
    }
    const float dot = group_sum<LPR>(dotw);
    ssq = group_sum<LPR>(ssq);
    const float bh = A.p.b[g * G + h];
    tau[h] = (A.p.tau_mode == 0) ? (dot + bh) - A.p.a : bh - A.p.a;
    qn[h] = sqrtf(ssq);
  }
  if (t == 0 && lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) A.ws.tau[(int64_t)n * HQ + g * G + h] = tau[h];
  }

  // ---- q . mu^ (and, dual, sum of (q sigma^)^2): partial products per lane,
  //      transposing reduction over each row
  float pd[G][NI];
  float ps[DUAL ? G : 1][NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const uint32_t w4[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
    float mv[8];
    if constexpr (FP8) {
#pragma unroll
      for (int e = 0; e < 8; ++e) mv[e] = fp8_to_f32(w4[e >> 2] >> (8 * (e & 3)), A.c.mu8_fmt);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        mv[2 * e] = f16_bits_to_f32((uint16_t)(w4[e] & 0xffffu));
        mv[2 * e + 1] = f16_bits_to_f32((uint16_t)(w4[e] >> 16));
      }
    }
    if constexpr (BOX) {  // mv: lower corner; sum of max(q kmax, q kmin) per lane
      const uint32_t u4[4] = {sraw[i].x, sraw[i].y, sraw[i].z, sraw[i].w};
      float xv[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xv[2 * e] = f16_bits_to_f32((uint16_t)(u4[e] & 0xffffu));
        xv[2 * e + 1] = f16_bits_to_f32((uint16_t)(u4[e] >> 16));
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) a += fmaxf(qf[h][e] * xv[e], qf[h][e] * mv[e]);
        pd[h][i] = a;
      }
    } else {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) a = fmaf(qf[h][e], mv[e], a);
        pd[h][i] = a;
      }
    }
    if constexpr (DUAL) {
      const uint32_t s4[4] = {sraw[i].x, sraw[i].y, sraw[i].z, sraw[i].w};
      float sv[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sv[2 * e] = f16_bits_to_f32((uint16_t)(s4[e] & 0xffffu));
        sv[2 * e + 1] = f16_bits_to_f32((uint16_t)(s4[e] >> 16));
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float t = qf[h][e] * sv[e];
          a = fmaf(t, t, a);
        }
        ps[h][i] = a;
      }
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) transpose_reduce<LPR>(pd[h], lane);
  if constexpr (DUAL) {
#pragma unroll
    for (int h = 0; h < G; ++h) transpose_reduce<LPR>(ps[h], lane);
  }

  const uint32_t full = (1u << G) - 1u;
  uint32_t mask = 0;
  float ub[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    ub[h] = BOX ? A.p.scale * pd[h][0] : A.p.scale * (pd[h][0] + qn[h] * R);
    if constexpr (DUAL) {  // the smaller of the bound and the z-deviation estimate (a NaN side yields)
      const float est = A.p.scale * (pd[h][0] + A.p.z * sqrtf(ps[h][0]));
      ub[h] = fminf(ub[h], est);
    }
    // both pages of a 128-token block take the bound of its first page's lane
    // (unit j ^ 1 sits LPR lanes away), so they are admitted and ranked as one
    if constexpr (PAIR) ub[h] = __shfl(ub[h], lane & ~LPR, 64);
    if (complete && !(ub[h] < tau[h])) mask |= 1u << h;
  }
  if (complete && jbl >= nfull - A.p.lwb) mask = full;
  if (jbl == nfull && lvalid) mask = full;  // partial last block (exists iff nfull < nblk)

  // ---- back to block order (lane l then holds block j0 + l), the largest
  //      bound per head among complete blocks (lowest index on ties), and
  //      ballot compaction in ascending block order
  __shared__ uint32_t smask[NW][64];
  __shared__ int spage[NW][64];
  __shared__ float sub[NW][G][64];
  smask[wave][jl - j0] = mask | (complete ? 0x10000u : 0u);
  spage[wave][jl - j0] = page_l;
#pragma unroll
  for (int h = 0; h < G; ++h) sub[wave][h][jl - j0] = ub[h];
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  const uint32_t mfull = smask[wave][lane];
  const uint32_t mb = mfull & 0xffffu;
  const bool cpl = (mfull >> 16) != 0;
  const int pb = spage[wave][lane];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float u = cpl ? sub[wave][h][lane] : -__builtin_inff();
    const float mx = wave_max_f(u);
    const uint64_t at = __ballot(cpl && u == mx);
    if (lane == 0) {
      A.ws.tile_umax[tix * G + h] = at ? mx : -__builtin_inff();
      A.ws.tile_uarg[tix * G + h] = at ? j0 + (int)__builtin_ctzll(at) : INT_MAX;
    }
  }
  uint64_t ball;
  if constexpr (SUBB) {
    // one entry per page: the SB lanes of a page gather their head masks into
    // one word (bit q G + h: head h admitted block q of the page); the page's
    // first lane writes the entry with the union of the heads
    uint32_t sw = mb << ((lane & (SB - 1)) * G);
    sw |= (uint32_t)__shfl_xor((int)sw, 1, 64);
    if (SB == 4) sw |= (uint32_t)__shfl_xor((int)sw, 2, 64);
    uint32_t um = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (q < SB) um |= (sw >> (q * G)) & full;
    const bool lead = (lane & (SB - 1)) == 0 && um != 0;
    ball = __ballot(lead);
    const int pos = __popcll(ball & ((1ull << lane) - 1ull));
    if (lead) {
      A.ws.tile_ent[tcx * kTile + pos] = make_int2(pb, (((j0 + lane) >> lsb) << 8) | (int)um);
      A.ws.tile_sub[tcx * kTile + pos] = sw;
    }
  } else {
    ball = __ballot(mb != 0);
    const int pos = __popcll(ball & ((1ull << lane) - 1ull));
    if (mb) A.ws.tile_ent[tcx * kTile + pos] = make_int2(pb, ((j0 + lane) << 8) | (int)mb);
  }
  const bool bad_page = jl < nunit && !lvalid;
  const bool any_bad = __any(bad_page);
  if (lane == 0) {
    A.ws.tile_cnt[tcx] = __popcll(ball);
    A.ws.tile_err[tix] = any_bad ? 1 : 0;
  }
  // counts are in screen blocks: a 128-token block is counted on its first page
  const uint64_t cnt_lanes = PAIR ? 0x5555555555555555ull : ~0ull;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint64_t hb = __ballot((mb >> h) & 1u);
    if (lane == h) {
      A.ws.tile_bits[((int64_t)s * G + h) * NT + t] = hb;
      A.ws.tile_hcnt[tix * G + h] = __popcll(hb & cnt_lanes);
    }
  }
}


// ---------------------------------------------------------------- finalize
struct FinArgs {
  CacheView c;
  SeqView s;
  Dims d;
  Ws ws;
  float* out;
  int deterministic;
  int fixed_w[kXcdClasses];
};

// Arrival of one of a segment's `parts` workgroups in the segment's arrival
// word (bits 24-63 a call's tag, bits 0-23 the count), after everything the
// workgroup wrote for the others is at the device's coherence point. A word
// without this call's tag (another call's, or whatever the workspace held)
// counts as no arrival: it is replaced by (tag, 1) with one compare-and-swap
// against `seen`, the word as read when the workgroup started; once the word
// carries the tag, arrivals are additions. Returns true for the last arrival
// (thread 0 only).
__device__ __forceinline__ bool arrive_tagged(uint64_t* wp, uint64_t seen, uint64_t tag, int parts) {
  uint64_t old = seen, nw = 0;
  while ((old >> 24) != tag) {
    if (__hip_atomic_compare_exchange_strong(wp, &old, (tag << 24) + 1, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT)) {
      nw = (tag << 24) + 1;
      break;
    }
  }
  if (nw == 0) nw = __hip_atomic_fetch_add(wp, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1;
  return (int)(nw & 0xffffffu) == parts;
}
__device__ __forceinline__ uint64_t arrival_word(const uint64_t* wp) {
  return __hip_atomic_load(const_cast<uint64_t*>(wp), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Work weights of the attend ranges per die class (workgroup k of a launch runs
// on die k % 8; dies differ in memory throughput by several percent). The
// previous decode's attend kernel left entries and duration per range; a
// class's measured rate (entries per tick) relative to the mean rate, averaged
// with its previous weight, becomes its weight for this decode, clamped to
// [1/2, 2]. Equal weights when there is no valid record or in the
// deterministic mode. Runs as one extra workgroup of the finalize grid.
template <int NW>
__device__ void update_weights(const FinArgs& A) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (A.fixed_w[0] > 0 && !A.deterministic) {
    if (tid < kXcdClasses) A.ws.xcd_w[tid] = A.fixed_w[tid];
    return;
  }
  __shared__ int s_acc[NW][2 * kXcdClasses];
  const int magic = A.ws.glob[kGlobStatMagic];
  const int Wprev = A.ws.glob[kGlobStatW];
  const bool valid = !A.deterministic && magic == kStatMagic && Wprev >= 1 && Wprev <= kMaxAttendWgs;
  int e[kXcdClasses], t[kXcdClasses];
#pragma unroll
  for (int x = 0; x < kXcdClasses; ++x) e[x] = t[x] = 0;
  if (valid) {
    for (int k = tid; k < Wprev; k += 64 * NW) {
      const int ek = A.ws.rng_stat[2 * k], tk = min(A.ws.rng_stat[2 * k + 1], 1 << 22);
      if (ek > 0 && tk > 0) {
#pragma unroll
        for (int x = 0; x < kXcdClasses; ++x)
          if (k % kXcdClasses == x) {
            e[x] += ek;
            t[x] += tk;
          }
      }
    }
  }
#pragma unroll
  for (int x = 0; x < kXcdClasses; ++x) {
    const int es = wave_sum_i(e[x]), ts = wave_sum_i(t[x]);
    if (lane == 0) {
      s_acc[wave][x] = es;
      s_acc[wave][kXcdClasses + x] = ts;
    }
  }
  __syncthreads();
  if (tid != 0) return;
  float rate[kXcdClasses], mean = 0.f;
  int nr = 0;
#pragma unroll
  for (int x = 0; x < kXcdClasses; ++x) {
    int ei = 0, ti = 0;
    for (int w = 0; w < NW; ++w) {
      ei += s_acc[w][x];
      ti += s_acc[w][kXcdClasses + x];
    }
    const float es = (float)ei, ts = (float)ti;
    rate[x] = (es > 0.f && ts > 0.f) ? es / ts : 0.f;
    if (rate[x] > 0.f) {
      mean += rate[x];
      ++nr;
    }
  }
  mean = nr ? mean / nr : 0.f;
#pragma unroll
  for (int x = 0; x < kXcdClasses; ++x) {
    int w = kWeightOne;
    if (valid && rate[x] > 0.f && mean > 0.f) {
      const int old = A.ws.xcd_w[x];
      const float prev = (old >= kWeightOne / 2 && old <= 2 * kWeightOne) ? (float)old : (float)kWeightOne;
      const float meas = kWeightOne * rate[x] / mean;
      w = (int)(0.5f * (prev + meas) + 0.5f);
      w = w < kWeightOne / 2 ? kWeightOne / 2 : (w > 2 * kWeightOne ? 2 * kWeightOne : w);
    }
    A.ws.xcd_w[x] = w;
  }
}

// Segment s (sequence, KV head), by a workgroup of 256 threads once every
// tile of the segment is screened: totals, rescue, tile prefix, counts.
// Returns the segment's union entry count U (every thread). With `lds_toff`,
// the tile prefix is also written there (entries 0 .. ntn + 1, as in
// tile_off) and *lds_ntn receives the used-tile count, for a caller in the same
// workgroup that attends to the segment right after.
template <int G, int NW>
__device__ __forceinline__ int finalize_segment(const FinArgs& A, int s, int* lds_toff = nullptr,
                                                int* lds_ntn = nullptr) {
  constexpr int NTH = 64 * NW;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int HKV = A.d.HKV, MB = A.d.MB, NT = A.d.NT, HQ = A.d.HQ;
  const int n = s / HKV, g = s % HKV;
  const int seq_len = A.s.lens[n];
  const bool badT = seq_len < 1 || seq_len > kBlock * MB;
  const int SB = A.d.SB, lsb = SB == 4 ? 2 : SB == 2 ? 1 : 0;  // screen blocks per page
  const bool pair = A.d.PB == 2;                               // 128-token blocks, screen lanes are pages
  const bool blk_bits = SB > 1 || pair;                        // union counted from the bitmaps
  const int bsz = pair ? 2 * kBlock : kBlock >> lsb;           // tokens per screen block
  const int nfull = badT ? 0 : seq_len / bsz;
  const int nblk = badT ? 0 : (seq_len + bsz - 1) / bsz;
  const int nunit = pair ? (badT ? 0 : (seq_len + kBlock - 1) / kBlock) : nblk;  // screen lanes used
  const int ntn = (nunit + kTile - 1) / kTile;
  const uint64_t cnt_lanes = pair ? 0x5555555555555555ull : ~0ull;  // a block counts on its first lane
  const int64_t tix0 = (int64_t)s * NT;
  const int64_t tcx0 = (int64_t)s * (NT + 1);
  const int32_t* bt = A.s.bt + (int64_t)n * MB;
  int32_t* toff = A.ws.tile_off + (int64_t)s * (NT + 2);

  __shared__ int s_scan[NW];
  __shared__ int s_hcnt[NW][G];
  __shared__ float s_umax[NW][G];
  __shared__ int s_uarg[NW][G];
  __shared__ int s_err[NW];
  __shared__ int s_nres;
  __shared__ int s_res_j[2 * G];
  __shared__ int s_resc[G];
  __shared__ int s_ub[NW];

  // 1. per-head totals, largest bound, errors; exclusive prefix over tiles
  int hc[G];
  float um[G];
  int ua[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    hc[h] = 0;
    um[h] = -__builtin_inff();
    ua[h] = INT_MAX;
  }
  // the tile loads do not wait for the length: every tile of the segment's
  // row is read, and those past the sequence (which the screen skips, so
  // they hold an earlier decode's values) are masked afterwards
  int err = 0, carry = 0, ublk = 0;
  for (int t0 = 0; t0 < NT; t0 += NTH) {
    const int t = t0 + tid;
    int c = 0, e = 0, hcl[G], ual[G];
    uint64_t orb = 0;
    float uml[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      hcl[h] = 0;
      uml[h] = -__builtin_inff();
      ual[h] = INT_MAX;
    }
    if (t < NT) {
      c = A.ws.tile_cnt[tcx0 + t];
      e = A.ws.tile_err[tix0 + t];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        hcl[h] = A.ws.tile_hcnt[(tix0 + t) * G + h];
        uml[h] = A.ws.tile_umax[(tix0 + t) * G + h];
        ual[h] = A.ws.tile_uarg[(tix0 + t) * G + h];
        if (blk_bits) orb |= A.ws.tile_bits[((int64_t)s * G + h) * NT + t];
      }
    }
    const bool use = t < ntn;
    if (use) {
      err |= e;
      ublk += __popcll(orb & cnt_lanes);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        hc[h] += hcl[h];
        if (uml[h] > um[h] || (uml[h] == um[h] && ual[h] < ua[h])) {
          um[h] = uml[h];
          ua[h] = ual[h];
        }
      }
    } else {
      c = 0;
    }
    int tot;
    const int ex = block_incl_scan<NW>(c, &tot, s_scan) - c;
    if (use) {
      toff[t] = carry + ex;
      if (lds_toff) lds_toff[t] = carry + ex;
    }
    carry += tot;
  }
  const int ucnt = carry;
  const bool err_w = __any(err != 0);
  if (lane == 0) s_err[wave] = err_w ? 1 : 0;
  if (blk_bits) {
    const int ub_w = wave_sum_i(ublk);
    if (lane == 0) s_ub[wave] = ub_w;
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const int t_h = wave_sum_i(hc[h]);
    if (lane == 0) s_hcnt[wave][h] = t_h;
  }
  __syncthreads();
  // the block with the largest bound matters only to a head that admitted
  // nothing (the same decision in every thread)
  bool need_rescue = false;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    int tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) tot += s_hcnt[w][h];
    need_rescue |= tot == 0;
  }
  if (need_rescue) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        const float ov = __shfl_xor(um[h], m, 64);
        const int oj = __shfl_xor(ua[h], m, 64);
        if (ov > um[h] || (ov == um[h] && oj < ua[h])) {
          um[h] = ov;
          ua[h] = oj;
        }
      }
      if (lane == 0) {
        s_umax[wave][h] = um[h];
        s_uarg[wave][h] = ua[h];
      }
    }
    __syncthreads();
  }

  // 2. rescue (thread 0): a head with nothing admitted gets its best-bound
  //    block; if another head of the group loads it already, only the head's
  //    bit is added to that entry, otherwise it becomes a rescue-tile entry.
  //    The arg index is a screen lane: a block, or the first page of a
  //    128-token block (whose two pages both get the head's bit).
  if (tid == 0) {
    int nres = 0;
    int ub = 0;  // screen blocks admitted by any head
    if (blk_bits)
      for (int w = 0; w < NW; ++w) ub += s_ub[w];
    for (int h = 0; h < G; ++h) {
      int tot = 0;
      for (int w = 0; w < NW; ++w) tot += s_hcnt[w][h];
      float v = -__builtin_inff();
      int jb = INT_MAX;
      if (tot == 0) {  // the per-wave maxima exist only in this case
        for (int w = 0; w < NW; ++w) {
          if (s_umax[w][h] > v || (s_umax[w][h] == v && s_uarg[w][h] < jb)) {
            v = s_umax[w][h];
            jb = s_uarg[w][h];
          }
        }
      }
      s_resc[h] = -1;
      if (tot == 0 && jb >= 0 && (pair ? jb >> 1 : jb) < nfull) {
        s_resc[h] = jb;
        tot = 1;
        const int tt = jb / kTile;  // both pages of a 128-token block lie in one tile
        if (blk_bits) {             // a new block for the union unless another head admits it
          uint64_t any = 0;
          for (int h2 = 0; h2 < G; ++h2) any |= A.ws.tile_bits[((int64_t)s * G + h2) * NT + tt];
          if (!((any >> (jb % kTile)) & 1ull)) ++ub;
        }
        int2* ent = A.ws.tile_ent + (tcx0 + tt) * kTile;
        const int c = A.ws.tile_cnt[tcx0 + tt];
        for (int u = jb; u <= (pair ? jb + 1 : jb); ++u) {
          const int jp = u >> lsb;  // the unit's page
          // the screen ranks only blocks whose pages are all valid; a page id
          // out of range is never handed to the attend kernel
          if (bt[jp] < 0 || bt[jp] >= A.c.num_pages) continue;
          const uint32_t sbit = SB > 1 ? 1u << ((u & (SB - 1)) * G + h) : 0u;
          int found = -1;
          for (int k = 0; k < c; ++k)
            if ((ent[k].y >> 8) == jp) found = k;
          if (found >= 0) {
            ent[found].y |= 1 << h;
            if (SB > 1) A.ws.tile_sub[(tcx0 + tt) * kTile + found] |= sbit;
          } else {
            int q = 0;
            for (; q < nres; ++q)
              if (s_res_j[q] == jp) break;
            int2* rent = A.ws.tile_ent + (tcx0 + NT) * kTile;
            if (q == nres) {
              s_res_j[q] = jp;
              rent[q] = make_int2(bt[jp], jp << 8);
              if (SB > 1) A.ws.tile_sub[(tcx0 + NT) * kTile + q] = 0u;
              ++nres;
            }
            rent[q].y |= 1 << h;
            if (SB > 1) A.ws.tile_sub[(tcx0 + NT) * kTile + q] |= sbit;
          }
          A.ws.tile_bits[((int64_t)s * G + h) * NT + tt] |= 1ull << (u % kTile);
        }
      }
      s_hcnt[0][h] = tot;
    }
    s_nres = nres;
    s_ub[0] = ub;
    A.ws.tile_cnt[tcx0 + NT] = nres;
    toff[ntn] = ucnt;
    toff[ntn + 1] = ucnt + nres;
    if (lds_toff) {
      lds_toff[ntn] = ucnt;
      lds_toff[ntn + 1] = ucnt + nres;
      *lds_ntn = ntn;
    }
  }
  __syncthreads();
  const int U = badT ? 0 : ucnt + s_nres;

  // 3. statistics
  if (tid < G) {
    const int h = tid;
    const int64_t o = (int64_t)n * HQ + g * G + h;
    const int cnt = badT ? 0 : s_hcnt[0][h];
    const int tail_missing = (!badT && (seq_len % bsz)) ? bsz - seq_len % bsz : 0;
    A.ws.st_head[o] = cnt;
    A.ws.st_tokens[o] = cnt > 0 ? (int64_t)cnt * bsz - tail_missing : 0;
    A.ws.st_rescued[o] = s_resc[h] >= 0 ? 1 : 0;
  }
  if (tid == 0) {
    A.ws.seg_U[s] = U;
    A.ws.seg_ub[s] = blk_bits ? (badT ? 0 : s_ub[0]) : U;
    A.ws.seg_ntn[s] = ntn;
    int errs = 0;
    for (int w = 0; w < NW; ++w) errs |= s_err[w];
    A.ws.seg_err[s] = (badT || errs) ? 1 : 0;
    A.ws.seg_done[s] = 0;
  }
  // a segment without entries (invalid length) gets no attend work: its
  // heads' outputs are NaN, as for an empty softmax
  if (U == 0) {
    const int D = A.d.D;
    for (int i = tid; i < G * D; i += NTH)
      A.out[((int64_t)n * HQ + g * G) * D + i] = __builtin_nanf("");
  }
  return U;
}

}  // namespace
}  // namespace eta
