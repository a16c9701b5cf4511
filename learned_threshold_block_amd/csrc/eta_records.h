// Block record builder shared by the record kernels and the prompt pass:
// centroid mu^ (float16, nearest even) and radius R^ (float32, rounded up) of
// one complete key block (a 64-token page, or a screen block of 16, 32 or 128
// tokens), and optionally its coordinate deviation, its coordinate-wise key box
// (the comparator's record) and its FP8 record.
//
// "Elastic Threshold Attention" (paperpeel.com/paper/2609.20888), Section 3.2
// and Appendix F.1: the decode screen reads one compact record per block and
// KV head instead of the keys. The radius is measured about the stored
// (rounded) centroid, so that q.k <= q.mu^ + ||q|| R^ holds for every key of
// the block.
#pragma once

#include "eta_device.h"

namespace eta {

// float64 move across lanes by a DPP pattern (both halves).
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)u, CTRL, 0xf, 0xf, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), CTRL, 0xf, 0xf, false);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// float64 sum over each group of N (8 or 16) adjacent lanes: mirror, half
// mirror, xor 2, xor 1. Each step pairs lanes whose partial sums cover the
// same keys, so every lane of a group ends with the same bits.
template <int N>
__device__ __forceinline__ double group_sum_f64(double v) {
  if constexpr (N >= 16) v += dpp_d<kDppMirror>(v);
  if constexpr (N >= 8) v += dpp_d<kDppHalfMirror>(v);
  v += dpp_d<kDppXor2>(v);
  v += dpp_d<kDppXor1>(v);
  return v;
}

// A lane's EPL record values (EPC contiguous columns per chunk) stored with
// one access per chunk: 16 or 8 bytes of float16 bits, 8 or 4 bytes of FP8
// codes (partial-line stores of single elements cost a full write each).
template <int EPC, int CPL, int D>
__device__ __forceinline__ void store_u16(uint16_t* out, const uint16_t* v, int cb) {
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    uint16_t* p = out + c * (D / CPL) + cb * EPC;
    const uint16_t* w = v + c * EPC;
    if constexpr (EPC == 8) {
      *(uint4*)p = make_uint4(w[0] | (uint32_t)w[1] << 16, w[2] | (uint32_t)w[3] << 16, w[4] | (uint32_t)w[5] << 16,
                              w[6] | (uint32_t)w[7] << 16);
    } else {
      *(uint2*)p = make_uint2(w[0] | (uint32_t)w[1] << 16, w[2] | (uint32_t)w[3] << 16);
    }
  }
}
template <int EPC, int CPL, int D>
__device__ __forceinline__ void store_u8(uint8_t* out, const uint8_t* v, int cb) {
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    uint8_t* p = out + c * (D / CPL) + cb * EPC;
    const uint8_t* w = v + c * EPC;
    const uint32_t lo = w[0] | (uint32_t)w[1] << 8 | (uint32_t)w[2] << 16 | (uint32_t)w[3] << 24;
    if constexpr (EPC == 8) {
      *(uint2*)p = make_uint2(lo, w[4] | (uint32_t)w[5] << 8 | (uint32_t)w[6] << 16 | (uint32_t)w[7] << 24);
    } else {
      *(uint32_t*)p = lo;
    }
  }
}

// Element e (0 .. EPL-1) of a lane's row in the 16-byte-load layout: chunk
// e / EPC of the row, element e % EPC of that chunk.
template <typename T, int EPC>
__device__ __forceinline__ float chunk_elem(const uint4* ch, int e) {
  const uint4 w = ch[e / EPC];
  const int k = e % EPC;
  if constexpr (T::kBytes == 2) {
    const uint32_t u = (k >> 1) == 0 ? w.x : (k >> 1) == 1 ? w.y : (k >> 1) == 2 ? w.z : w.w;
    return (k & 1) ? bf16_hi(u) : bf16_lo(u);
  } else {
    return __uint_as_float(k == 0 ? w.x : k == 1 ? w.y : k == 2 ? w.z : w.w);
  }
}

// One wavefront. tile: [ROWS][D] keys of one block (a whole 64-token page, or
// a 16- or 32-token block of it); a 128-token block takes its first 64 rows
// from tile and the other 64 from tile_hi (its second page). If override_row
// is non-null, the last row is read from it instead.
//
// The rows are read with 16-byte loads in the tile layout (lane (r, cb) holds
// rows RPI i + r, EPL columns) and, where they fit in 128 registers, kept for
// the second pass. Column sums (float64, each lane over its rows in order,
// then a butterfly over the lanes sharing the columns, which leaves the same
// bits on all of them), per-row squared distances (float64, summed over the
// lanes of the row by DPP, same bits on all of them) and their maximum. Every builder calls this one
// function, so bulk, append and prompt-pass records are bit-identical.
//
// Writes the centroid and radius, the coordinate deviation if sig_out is not
// null, and the key box if kmin_out is not null: per coordinate the least key
// value rounded down and the greatest rounded up to float16 (Section 4.3, the
// comparator's per-block extrema; NaN for a block with a non-finite key), and
// the FP8 record if mu8_out is not null: the mean rounded to the FP8 format
// fmt8 (nearest even, saturating) and the radius about it, rounded up like R^
// (zero centroid and infinite radius for a block with a non-finite key).
template <typename T, int D, int ROWS = kBlock>
__device__ __forceinline__ void build_record(const typename T::Stored* tile, const typename T::Stored* override_row,
                             uint16_t* mu_out, float* r_out, uint16_t* sig_out, uint16_t* kmin_out,
                             uint16_t* kmax_out, uint8_t* mu8_out, float* r8_out, int fmt8, int lane,
                             const typename T::Stored* tile_hi = nullptr) {
  static_assert(ROWS == 16 || ROWS == 32 || ROWS == kBlock || ROWS == 2 * kBlock, "block of 16, 32, 64 or 128 keys");
  using L = TileLayout<T::kBytes, D>;
  using St = typename T::Stored;
  constexpr int LPR = L::LPR, RPI = L::RPI, CPL = L::CPL, EPC = L::EPC, EPL = L::EPL;
  constexpr int NR = ROWS / RPI;             // rows per lane
  constexpr bool KEEP = NR * CPL <= 32;      // rows stay in registers for the second pass
  static_assert(ROWS % RPI == 0, "whole load instructions");
  const int r = lane / LPR, cb = lane % LPR;

  uint4 raw[KEEP ? NR : 1][CPL];
  const auto row_ptr = [&](int i) -> const St* {
    const int row = RPI * i + r;
    if (override_row && row == ROWS - 1) return override_row;
    if (ROWS > kBlock && row >= kBlock) return tile_hi + (row - kBlock) * D;
    return tile + row * D;
  };
  const auto load_row = [&](int i, uint4 (&dst)[CPL]) {
    const St* rp = row_ptr(i);
#pragma unroll
    for (int c = 0; c < CPL; ++c) dst[c] = load_stream16(rp + L::col(c, cb));
  };
  if constexpr (KEEP) {
#pragma unroll
    for (int i = 0; i < NR; ++i) load_row(i, raw[i]);
  }

  // ---- pass 1: column sums, extrema, finiteness
  double sum[EPL];
  float cmin[EPL], cmax[EPL];
  bool finite = true;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    sum[e] = 0.0;
    cmin[e] = __builtin_inff();
    cmax[e] = -__builtin_inff();
  }
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    uint4 ld[CPL];
    if constexpr (!KEEP) load_row(i, ld);
    const uint4* ch = KEEP ? raw[i] : ld;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const float x = chunk_elem<T, EPC>(ch, e);
      finite = finite && (fabsf(x) <= 3.4028234663852886e38f);
      sum[e] += (double)x;
      cmin[e] = fminf(cmin[e], x);
      cmax[e] = fmaxf(cmax[e], x);
    }
    // rows in groups of four, so that the scheduler does not convert every
    // element to float64 at once (registers for two waves per SIMD)
    if ((i & 3) == 3) __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int m = LPR; m < 64; m <<= 1)
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      sum[e] += __shfl_xor(sum[e], m, 64);
      cmin[e] = fminf(cmin[e], __shfl_xor(cmin[e], m, 64));
      cmax[e] = fmaxf(cmax[e], __shfl_xor(cmax[e], m, 64));
    }
  // the float64 mean is sum * (1 / ROWS) (exact: ROWS is a power of two)
  uint16_t h[EPL];
  bool ok = finite;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    h[e] = f64_to_f16_rne(sum[e] * (1.0 / ROWS));
    ok = ok && ((h[e] & 0x7c00u) != 0x7c00u);
  }
  const bool all_ok = __all(ok);
  const bool all_finite = __all(finite);
  const bool writer = r == 0;  // one lane per column group stores
  float mu8[EPL];  // FP8 centroid values (exact in float32)
  if (mu8_out) {
    uint8_t b8[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      b8[e] = all_finite ? f64_to_fp8(sum[e] * (1.0 / ROWS), fmt8) : (uint8_t)0;
      mu8[e] = fp8_to_f32(b8[e], fmt8);
    }
    if (writer) store_u8<EPC, CPL, D>(mu8_out, b8, cb);
  }
  if (kmin_out && writer) {
    uint16_t lo[EPL], hi[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      lo[e] = all_finite ? f32_to_f16_dir(cmin[e], false) : (uint16_t)0x7e00u;
      hi[e] = all_finite ? f32_to_f16_dir(cmax[e], true) : (uint16_t)0x7e00u;
    }
    store_u16<EPC, CPL, D>(kmin_out, lo, cb);
    store_u16<EPC, CPL, D>(kmax_out, hi, cb);
  }
  float mu[EPL];  // stored centroid values (exact in float32)
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    if (!all_ok) h[e] = 0;
    mu[e] = f16_bits_to_f32(h[e]);
  }
  if (writer) store_u16<EPC, CPL, D>(mu_out, h, cb);

  // ---- pass 2: squared distances per row and their maximum (the radius);
  // then, only if asked for, the same about the FP8 centroid and the
  // deviations about the float64 mean, each in a loop of its own so that few
  // float64 values are live at a time. The empty asm keeps the compiler from
  // carrying pass 1's float64 conversions of every element over to here; the
  // rows are converted again from the kept 16-byte words.
  const auto fence_rows = [&]() {
    if constexpr (KEEP) {
#pragma unroll
      for (int i = 0; i < NR; ++i)
#pragma unroll
        for (int c = 0; c < CPL; ++c)
          asm volatile("" : "+v"(raw[i][c].x), "+v"(raw[i][c].y), "+v"(raw[i][c].z), "+v"(raw[i][c].w));
    }
  };
  // largest squared distance of a row to the centroid c (NaN propagates)
  const auto max_dist2 = [&](const float (&cen)[EPL]) {
    double rm = 0.0;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      uint4 ld[CPL];
      if constexpr (!KEEP) load_row(i, ld);
      const uint4* ch = KEEP ? raw[i] : ld;
      double part = 0.0;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const double dlt = (double)chunk_elem<T, EPC>(ch, e) - (double)cen[e];
        part += dlt * dlt;
      }
      part = group_sum_f64<LPR>(part);
      rm = (part > rm || part != part) ? part : rm;
      if ((i & 3) == 3) __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int m = LPR; m < 64; m <<= 1) {
      const double o = __shfl_xor(rm, m, 64);
      rm = (o > rm || o != o) ? o : rm;
    }
    return rm;
  };
  fence_rows();
  const double rmax = max_dist2(mu);
  double rmax8 = 0.0;
  if (mu8_out) {
    fence_rows();
    rmax8 = max_dist2(mu8);
  }
  // coordinate deviation (population) about the float64 mean, as float16
  if (sig_out) {
    fence_rows();
    double dev2[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) dev2[e] = 0.0;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      uint4 ld[CPL];
      if constexpr (!KEEP) load_row(i, ld);
      const uint4* ch = KEEP ? raw[i] : ld;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const double dm = (double)chunk_elem<T, EPC>(ch, e) - sum[e] * (1.0 / ROWS);
        dev2[e] += dm * dm;
      }
    }
#pragma unroll
    for (int m = LPR; m < 64; m <<= 1)
#pragma unroll
      for (int e = 0; e < EPL; ++e) dev2[e] += __shfl_xor(dev2[e], m, 64);
    if (writer) {
      uint16_t sg[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const double sd = sqrt(dev2[e] * (1.0 / ROWS));
        sg[e] = (sd < 1e300) ? f64_to_f16_rne(sd) : (uint16_t)0x7c00u;
      }
      store_u16<EPC, CPL, D>(sig_out, sg, cb);
    }
  }
  const bool any_bad = !all_finite;
  if (lane == 0) {
    float rr;
    if (any_bad || !(rmax < 1e300)) rr = __builtin_inff();
    else rr = f64_to_f32_up(sqrt(rmax) * (1.0 + 0x1p-40));
    *r_out = rr;
    if (mu8_out) *r8_out = (any_bad || !(rmax8 < 1e300)) ? __builtin_inff() : f64_to_f32_up(sqrt(rmax8) * (1.0 + 0x1p-40));
  }
}


}  // namespace eta
