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
//   counts    per-head blocks, union blocks, attended tokens (F.4)
//
// k_screen: one wavefront per 64 consecutive blocks of one (sequence, KV head).
//   Lanes read the float16 centroids with 16-byte loads (16 lanes per row at
//   d = 128), form partial dot products with the G queries and finish them with
//   a transposing DPP reduction, so each lane ends up owning one block. Admitted
//   blocks are compacted in ascending order with a wavefront ballot + prefix.
// k_finalize: one workgroup per (sequence, KV head): per-head totals, rescue,
//   prefix over the tiles and copy into one contiguous list of (page, j|mask);
//   the last workgroup to finish (arrival counter) lays out the split of the
//   total work over the attend grid.
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

template <typename T, int D, int G>
__global__ __launch_bounds__(256) void k_screen(ScreenArgs A) {
  using L = TileLayout<2, D>;  // float16 centroid rows
  constexpr int LPR = L::LPR, RPI = L::RPI, NI = L::NI;
  static_assert(L::CPL == 1 && L::EPC == 8, "centroid rows are one 8-half chunk per lane");
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane / LPR, cb = lane % LPR;
  const int s = blockIdx.y;
  const int HKV = A.d.HKV, MB = A.d.MB, NT = A.d.NT, HQ = A.d.HQ;
  const int n = s / HKV, g = s % HKV;
  const int t = blockIdx.x * 4 + wave;

  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
    A.ws.glob[kGlobCounter] = 0;
    A.ws.glob[kGlobN] = A.d.N;
    A.ws.glob[kGlobMB] = MB;
    A.ws.glob[kGlobHQ] = HQ;
    A.ws.glob[kGlobHKV] = HKV;
    A.ws.glob[kGlobD] = D;
  }
  if (t >= NT) return;
  const int seq_len = A.s.lens[n];
  const bool badT = seq_len < 1 || seq_len > kBlock * MB;
  const int nfull = badT ? 0 : seq_len / kBlock;
  const int nblk = badT ? 0 : (seq_len + kBlock - 1) / kBlock;
  const int64_t tix = (int64_t)s * NT + t;
  const int j0 = t * kTile;

  if (j0 >= nblk) {
    if (lane == 0) {
      A.ws.tile_cnt[tix] = 0;
      A.ws.tile_err[tix] = 0;
    }
    if (lane < G) {
      A.ws.tile_hcnt[tix * G + lane] = 0;
      A.ws.tile_umax[tix * G + lane] = -__builtin_inff();
      A.ws.tile_uarg[tix * G + lane] = INT_MAX;
      A.ws.tile_bits[((int64_t)s * G + lane) * NT + t] = 0;
    }
    return;
  }

  // thresholds and query norms of the G heads (every row of lanes holds all D columns)
  float qf[G][8];
  float tau[G], qn[G];
  const auto* qbase = (const typename T::Stored*)A.p.q;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const int hq = g * G + h;
    load8<T>(qbase + ((int64_t)n * HQ + hq) * D + cb * 8, qf[h]);
    float ssq = 0.f, dot = 0.f;
    if (A.p.tau_mode == 0) {
      const float* wr = A.p.w + (int64_t)hq * D + cb * 8;
      const float4 w0 = *(const float4*)wr;
      const float4 w1 = *(const float4*)(wr + 4);
      const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) dot = fmaf(wv[e], qf[h][e], dot);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) ssq = fmaf(qf[h][e], qf[h][e], ssq);
    dot = group_sum<LPR>(dot);
    ssq = group_sum<LPR>(ssq);
    const float bh = A.p.b[hq];
    tau[h] = (A.p.tau_mode == 0) ? (dot + bh) - A.p.a : bh - A.p.a;
    qn[h] = sqrtf(ssq);
  }
  if (t == 0 && lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) A.ws.tau[(int64_t)n * HQ + g * G + h] = tau[h];
  }

  // partial dot products q . mu^ for the NI blocks this lane reads
  const int32_t* bt = A.s.bt + (int64_t)n * MB;
  float pd[G][NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int j = j0 + RPI * i + r;
    float mv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (j < nfull) {
      const int page = bt[j];
      if (page >= 0 && page < A.c.num_pages) {
        const uint4 raw = *(const uint4*)(A.c.mu + ((int64_t)page * HKV + g) * D + cb * 8);
        const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          mv[2 * e] = f16_bits_to_f32((uint16_t)(w4[e] & 0xffffu));
          mv[2 * e + 1] = f16_bits_to_f32((uint16_t)(w4[e] >> 16));
        }
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) a = fmaf(qf[h][e], mv[e], a);
      pd[h][i] = a;
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) transpose_reduce<LPR>(pd[h], lane);

  // this lane now owns block jl
  const int jl = j0 + RPI * cb + r;
  int page = -1;
  bool pvalid = false;
  if (jl < nblk) {
    page = bt[jl];
    pvalid = page >= 0 && page < A.c.num_pages;
  }
  const bool complete = jl < nfull && pvalid;
  const float R = complete ? A.c.radius[(int64_t)page * HKV + g] : 0.f;
  const uint32_t full = (1u << G) - 1u;
  uint32_t mask = 0;
  float ub[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    ub[h] = A.p.scale * (pd[h][0] + qn[h] * R);
    if (complete && !(ub[h] < tau[h])) mask |= 1u << h;
  }
  if (complete && jl >= nfull - A.p.lwb) mask = full;
  if (jl == nfull && jl < nblk && pvalid) mask = full;  // partial last block

  // largest bound per head among complete blocks (lowest index on ties)
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float v = complete ? ub[h] : -__builtin_inff();
    int jj = complete ? jl : INT_MAX;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const float ov = __shfl_xor(v, m, 64);
      const int oj = __shfl_xor(jj, m, 64);
      if (ov > v || (ov == v && oj < jj)) {
        v = ov;
        jj = oj;
      }
    }
    if (lane == 0) {
      A.ws.tile_umax[tix * G + h] = v;
      A.ws.tile_uarg[tix * G + h] = jj;
    }
  }

  // back to block order, then ballot compaction (ascending block index)
  __shared__ uint32_t smask[4][64];
  smask[wave][jl - j0] = mask;
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  const uint32_t mb = smask[wave][lane];
  const uint64_t ball = __ballot(mb != 0);
  const int pos = __popcll(ball & ((1ull << lane) - 1ull));
  if (mb) A.ws.tile_ent[tix * kTile + pos] = ((j0 + lane) << 8) | (int)mb;
  const bool bad_page = jl < nblk && !pvalid;
  const bool any_bad = __any(bad_page);
  if (lane == 0) {
    A.ws.tile_cnt[tix] = __popcll(ball);
    A.ws.tile_err[tix] = any_bad ? 1 : 0;
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint64_t hb = __ballot((mb >> h) & 1u);
    if (lane == h) {
      A.ws.tile_bits[((int64_t)s * G + h) * NT + t] = hb;
      A.ws.tile_hcnt[tix * G + h] = __popcll(hb);
    }
  }
}

// ---------------------------------------------------------------- finalize
struct FinArgs {
  CacheView c;
  SeqView s;
  Dims d;
  Ws ws;
  int W;  // attend grid size
};

// exclusive scan of one int per thread over a 256-thread workgroup
__device__ int block_excl_scan(int v, int* total, int* lds /*[8]*/) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) lds[wave] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int ws = lds[w];
    if (w < wave) base += ws;
    tot += ws;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

template <int G>
__global__ __launch_bounds__(256) void k_finalize(FinArgs A) {
  const int s = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int HKV = A.d.HKV, MB = A.d.MB, NT = A.d.NT, HQ = A.d.HQ;
  const int n = s / HKV, g = s % HKV;
  const int seq_len = A.s.lens[n];
  const bool badT = seq_len < 1 || seq_len > kBlock * MB;
  const int nfull = badT ? 0 : seq_len / kBlock;
  const int nblk = badT ? 0 : (seq_len + kBlock - 1) / kBlock;
  const int ntn = (nblk + kTile - 1) / kTile;
  const int64_t tix0 = (int64_t)s * NT;
  const int32_t* bt = A.s.bt + (int64_t)n * MB;

  __shared__ int s_scan[8];
  __shared__ int s_toff[kMaxBlocksPerSeq / kTile + 1];
  __shared__ int s_hcnt[4][G];
  __shared__ float s_umax[4][G];
  __shared__ int s_uarg[4][G];
  __shared__ int s_err[4];
  __shared__ int s_nres;
  __shared__ int s_res_j[G];
  __shared__ uint32_t s_res_bits[G];
  __shared__ int s_or_tile[G], s_or_pos[G];
  __shared__ uint32_t s_or_bits[G];
  __shared__ int s_nor;
  __shared__ int s_last;

  // 1. per-head totals, largest bound, errors; tile prefix
  int hc[G];
  float um[G];
  int ua[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    hc[h] = 0;
    um[h] = -__builtin_inff();
    ua[h] = INT_MAX;
  }
  int err = 0;
  int carry = 0;
  for (int t0 = 0; t0 < ntn; t0 += 256) {
    const int t = t0 + tid;
    int c = 0;
    if (t < ntn) {
      const int64_t tix = tix0 + t;
      c = A.ws.tile_cnt[tix];
      err |= A.ws.tile_err[tix];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        hc[h] += A.ws.tile_hcnt[tix * G + h];
        const float v = A.ws.tile_umax[tix * G + h];
        const int j = A.ws.tile_uarg[tix * G + h];
        if (v > um[h] || (v == um[h] && j < ua[h])) {
          um[h] = v;
          ua[h] = j;
        }
      }
    }
    int tot;
    const int ex = block_excl_scan(c, &tot, s_scan);
    if (t < ntn) s_toff[t] = carry + ex;
    carry += tot;
  }
  const int ucnt = carry;
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      hc[h] += __shfl_xor(hc[h], m, 64);
      const float ov = __shfl_xor(um[h], m, 64);
      const int oj = __shfl_xor(ua[h], m, 64);
      if (ov > um[h] || (ov == um[h] && oj < ua[h])) {
        um[h] = ov;
        ua[h] = oj;
      }
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) err |= __shfl_xor(err, m, 64);
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s_hcnt[wave][h] = hc[h];
      s_umax[wave][h] = um[h];
      s_uarg[wave][h] = ua[h];
    }
    s_err[wave] = err;
  }
  __syncthreads();

  // 2. rescue (thread 0): a head with nothing admitted gets its best-bound block
  if (tid == 0) {
    int nres = 0, nor = 0;
    for (int h = 0; h < G; ++h) {
      int tot = 0;
      float v = -__builtin_inff();
      int jb = INT_MAX;
      for (int w = 0; w < 4; ++w) {
        tot += s_hcnt[w][h];
        if (s_umax[w][h] > v || (s_umax[w][h] == v && s_uarg[w][h] < jb)) {
          v = s_umax[w][h];
          jb = s_uarg[w][h];
        }
      }
      s_hcnt[0][h] = tot;
      s_uarg[0][h] = -1;
      if (tot == 0 && jb >= 0 && jb < nfull) {
        s_uarg[0][h] = jb;
        s_hcnt[0][h] = 1;
        const int tt = jb / kTile;
        const int64_t tix = tix0 + tt;
        // already loaded for another head of the group?
        const int c = A.ws.tile_cnt[tix];
        int found = -1;
        for (int k = 0; k < c; ++k)
          if ((A.ws.tile_ent[tix * kTile + k] >> 8) == jb) found = k;
        if (found >= 0) {
          int q = 0;
          for (; q < nor; ++q)
            if (s_or_tile[q] == tt && s_or_pos[q] == found) break;
          if (q == nor) {
            s_or_tile[q] = tt;
            s_or_pos[q] = found;
            s_or_bits[q] = 0;
            ++nor;
          }
          s_or_bits[q] |= 1u << h;
        } else {
          int q = 0;
          for (; q < nres; ++q)
            if (s_res_j[q] == jb) break;
          if (q == nres) {
            s_res_j[q] = jb;
            s_res_bits[q] = 0;
            ++nres;
          }
          s_res_bits[q] |= 1u << h;
        }
        A.ws.tile_bits[((int64_t)s * G + h) * NT + tt] |= 1ull << (jb % kTile);
      }
    }
    s_nres = nres;
    s_nor = nor;
  }
  __syncthreads();

  // 3. contiguous list of (page, (j << 8) | mask)
  const int nres = s_nres, nor = s_nor;
  int2* list = A.ws.seg_list + (int64_t)s * MB;
  int perr = 0;
  for (int t = wave; t < ntn; t += 4) {
    const int64_t tix = tix0 + t;
    const int c = A.ws.tile_cnt[tix];
    if (lane < c) {
      int e = A.ws.tile_ent[tix * kTile + lane];
      for (int q = 0; q < nor; ++q)
        if (s_or_tile[q] == t && s_or_pos[q] == lane) e |= (int)s_or_bits[q];
      int page = bt[e >> 8];
      if (page < 0 || page >= A.c.num_pages) {
        page = 0;
        e &= ~0xff;
        perr = 1;
      }
      list[s_toff[t] + lane] = make_int2(page, e);
    }
  }
  if (tid < nres) {
    const int j = s_res_j[tid];
    list[ucnt + tid] = make_int2(bt[j], (j << 8) | (int)s_res_bits[tid]);
  }
  const int U = badT ? 0 : ucnt + nres;

  // 4. statistics
  if (tid < G) {
    const int h = tid;
    const int64_t o = (int64_t)n * HQ + g * G + h;
    const int cnt = badT ? 0 : s_hcnt[0][h];
    const int tail_missing = (!badT && (seq_len % kBlock)) ? kBlock - seq_len % kBlock : 0;
    A.ws.st_head[o] = cnt;
    A.ws.st_tokens[o] = cnt > 0 ? (int64_t)cnt * kBlock - tail_missing : 0;
    A.ws.st_rescued[o] = s_uarg[0][h] >= 0 ? 1 : 0;
  }
  const int any_perr = __syncthreads_or(perr);
  if (tid == 0) {
    A.ws.seg_U[s] = U;
    A.ws.seg_err[s] = (badT || s_err[0] || s_err[1] || s_err[2] || s_err[3] || any_perr) ? 1 : 0;
    __threadfence();
    const int old = atomicAdd(&A.ws.glob[kGlobCounter], 1);
    s_last = (old == A.d.S - 1) ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;

  // 5. last workgroup: prefix over segments and the attend work split
  __threadfence();
  const int S = A.d.S;
  int carry2 = 0, errs = 0;
  for (int s0 = 0; s0 < S; s0 += 256) {
    const int si = s0 + tid;
    const int u = si < S ? __atomic_load_n(&A.ws.seg_U[si], __ATOMIC_RELAXED) : 0;
    if (si < S) errs |= __atomic_load_n(&A.ws.seg_err[si], __ATOMIC_RELAXED);
    int tot;
    const int ex = block_excl_scan(u, &tot, s_scan);
    if (si < S) A.ws.seg_P[si] = carry2 + ex;
    carry2 += tot;
  }
  const int Utot = carry2;
  const int Wp = Utot < A.W ? Utot : A.W;
  errs = __syncthreads_or(errs);
  if (tid == 0) {
    A.ws.glob[kGlobUtot] = Utot;
    A.ws.glob[kGlobWeff] = Wp;
    A.ws.glob[kGlobErr] = errs;
    A.ws.glob[kGlobCounter] = 0;
  }
  if (Wp == 0) return;
  for (int si = tid; si < S; si += 256) {
    // recompute the prefix for this segment from the values written above
    const int u = __atomic_load_n(&A.ws.seg_U[si], __ATOMIC_RELAXED);
    const int P = A.ws.seg_P[si];
    if (u == 0) {
      A.ws.seg_plo[si] = 0;
      A.ws.seg_phi[si] = -1;
      continue;
    }
    const int64_t UU = Utot, WW = Wp;
    // attend workgroup k covers entries [floor(k U / W'), floor((k+1) U / W'))
    const int64_t k_lo = ((int64_t)P * WW + UU - 1) / UU;                 // first k starting in segment
    const int64_t k_hi = ((int64_t)(P + u) * WW + UU - 1) / UU - 1;       // last k starting in segment
    for (int64_t k = k_lo; k <= k_hi && k < WW; ++k) A.ws.wg_seg[k] = si;
    const int64_t kf = (((int64_t)P + 1) * WW - 1) / UU;                  // workgroup holding entry P
    const int64_t kl = (((int64_t)P + u) * WW - 1) / UU;                  // workgroup holding entry P+u-1
    A.ws.seg_plo[si] = (int)(kf + si);
    A.ws.seg_phi[si] = (int)(kl + si);
  }
}

template <typename T, int D, int G>
hipError_t screen_impl(const CacheView& c, const SeqView& s, const DecodeParams& p, const Dims& d,
                       const Ws& ws, hipStream_t st) {
  ScreenArgs a{c, s, p, d, ws};
  dim3 grid((d.NT + 3) / 4, d.S);
  hipLaunchKernelGGL((k_screen<T, D, G>), grid, dim3(256), 0, st, a);
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

template <int G>
hipError_t finalize_impl(const CacheView& c, const SeqView& s, const Dims& d, const Ws& ws, int W,
                         hipStream_t st) {
  FinArgs a{c, s, d, ws, W};
  hipLaunchKernelGGL((k_finalize<G>), dim3(d.S), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_screen(const CacheView& c, const SeqView& s, const DecodeParams& p, const Dims& d,
                         const Ws& ws, hipStream_t st) {
  if (c.kv_dtype == 1) return d.D == 128 ? screen_g<Bf16, 128>(c, s, p, d, ws, st) : screen_g<Bf16, 64>(c, s, p, d, ws, st);
  return d.D == 128 ? screen_g<F32, 128>(c, s, p, d, ws, st) : screen_g<F32, 64>(c, s, p, d, ws, st);
}

hipError_t launch_finalize(const CacheView& c, const SeqView& s, const Dims& d, const Ws& ws, int W,
                           hipStream_t st) {
  switch (d.G) {
    case 1: return finalize_impl<1>(c, s, d, ws, W, st);
    case 2: return finalize_impl<2>(c, s, d, ws, W, st);
    case 4: return finalize_impl<4>(c, s, d, ws, W, st);
    case 8: return finalize_impl<8>(c, s, d, ws, W, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace eta
