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

template <typename T>
__device__ __forceinline__ float load_elem(const typename T::Stored* p);
template <>
__device__ __forceinline__ float load_elem<Bf16>(const uint16_t* p) {
  return __uint_as_float((uint32_t)(*p) << 16);
}
template <>
__device__ __forceinline__ float load_elem<F32>(const float* p) {
  return *p;
}

// One wavefront. tile: [ROWS][D] keys of one block (a whole 64-token page, or
// a 16- or 32-token block of it); a 128-token block takes its first 64 rows
// from tile and the other 64 from tile_hi (its second page). If override_row
// is non-null, the last row is read from it instead. Lanes own columns;
// the rows are read twice (sums, then distances and deviations), which keeps
// the register footprint small enough for eight wavefronts per SIMD. Writes
// the centroid and radius, the coordinate deviation if sig_out is not null,
// and the key box if kmin_out is not null: per coordinate the least key value
// rounded down and the greatest rounded up to float16 (Section 4.3, the
// comparator's per-block extrema; NaN for a block with a non-finite key), and
// the FP8 record if mu8_out is not null: the mean rounded to the FP8 format
// fmt8 (nearest even, saturating) and the radius about it, rounded up like R^
// (zero centroid and infinite radius for a block with a non-finite key).
template <typename T, int D, int ROWS = kBlock>
__device__ void build_record(const typename T::Stored* tile, const typename T::Stored* override_row,
                             uint16_t* mu_out, float* r_out, uint16_t* sig_out, uint16_t* kmin_out,
                             uint16_t* kmax_out, uint8_t* mu8_out, float* r8_out, int fmt8, int lane,
                             const typename T::Stored* tile_hi = nullptr) {
  static_assert(ROWS == 16 || ROWS == 32 || ROWS == kBlock || ROWS == 2 * kBlock, "block of 16, 32, 64 or 128 keys");
  constexpr int CPL = D / 64;  // columns per lane: 2 (D=128) or 1 (D=64)
  const auto row_at = [&](int r) -> const typename T::Stored* {
    if (r == ROWS - 1 && override_row) return override_row;
    if (ROWS > kBlock && r >= kBlock) return tile_hi + (r - kBlock) * D;
    return tile + r * D;
  };
  double sum[CPL];
  float cmin[CPL], cmax[CPL];
  bool finite = true;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    sum[c] = 0.0;
    cmin[c] = __builtin_inff();
    cmax[c] = -__builtin_inff();
  }
  for (int r = 0; r < ROWS; ++r) {
    const typename T::Stored* row = row_at(r);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const float x = load_elem<T>(row + lane * CPL + c);
      finite = finite && (fabsf(x) <= 3.4028234663852886e38f);
      sum[c] += (double)x;
      cmin[c] = fminf(cmin[c], x);
      cmax[c] = fmaxf(cmax[c], x);
    }
  }
  uint16_t h[CPL];
  double mu[CPL], mean[CPL], dev2[CPL], mu8[CPL];
  bool ok = finite;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    mean[c] = sum[c] * (1.0 / ROWS);
    dev2[c] = 0.0;
    h[c] = f64_to_f16_rne(mean[c]);
    ok = ok && ((h[c] & 0x7c00u) != 0x7c00u);
  }
  const bool all_ok = __all(ok);
  const bool all_finite = __all(finite);
  if (mu8_out) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const uint8_t b = all_finite ? f64_to_fp8(mean[c], fmt8) : (uint8_t)0;
      mu8[c] = (double)fp8_to_f32(b, fmt8);
      mu8_out[lane * CPL + c] = b;
    }
  }
  if (kmin_out) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      kmin_out[lane * CPL + c] = all_finite ? f32_to_f16_dir(cmin[c], false) : (uint16_t)0x7e00u;
      kmax_out[lane * CPL + c] = all_finite ? f32_to_f16_dir(cmax[c], true) : (uint16_t)0x7e00u;
    }
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    if (!all_ok) h[c] = 0;
    mu[c] = (double)f16_bits_to_f32(h[c]);
    mu_out[lane * CPL + c] = h[c];
  }
  double rmax = 0.0, rmax8 = 0.0;
  for (int r = 0; r < ROWS; ++r) {
    const typename T::Stored* row = row_at(r);
    double part = 0.0, part8 = 0.0;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const double x = (double)load_elem<T>(row + lane * CPL + c);
      const double dlt = x - mu[c];
      part += dlt * dlt;
      const double dm = x - mean[c];  // deviation about the float64 mean
      dev2[c] += dm * dm;
      if (mu8_out) {
        const double d8 = x - mu8[c];
        part8 += d8 * d8;
      }
    }
    const double tot = wave_sum_f64(part);
    rmax = (tot > rmax || tot != tot) ? tot : rmax;  // NaN propagates
    if (mu8_out) {
      const double tot8 = wave_sum_f64(part8);
      rmax8 = (tot8 > rmax8 || tot8 != tot8) ? tot8 : rmax8;
    }
  }
  // coordinate deviation (population) as float16
  if (sig_out) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const double sd = sqrt(dev2[c] * (1.0 / ROWS));
      sig_out[lane * CPL + c] = (sd < 1e300) ? f64_to_f16_rne(sd) : (uint16_t)0x7c00u;
    }
  }
  const bool any_bad = !all_finite;
  if (lane == 0) {
    float r;
    if (any_bad || !(rmax < 1e300)) r = __builtin_inff();
    else r = f64_to_f32_up(sqrt(rmax) * (1.0 + 0x1p-40));
    *r_out = r;
    if (mu8_out) *r8_out = (any_bad || !(rmax8 < 1e300)) ? __builtin_inff() : f64_to_f32_up(sqrt(rmax8) * (1.0 + 0x1p-40));
  }
}


}  // namespace eta
