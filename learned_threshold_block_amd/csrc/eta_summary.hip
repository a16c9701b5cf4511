// Block records: centroid mu^ (float16, nearest even) and radius R^ (float32,
// rounded up) of every complete 64-token key block, per KV head.
//
// "Elastic Threshold Attention" (paperpeel.com/paper/2609.20888), Section 3.2
// and Appendix F.1: the decode screen reads one compact record per block and KV
// head instead of the keys. The radius is measured about the stored (rounded)
// centroid, so that q.k <= q.mu^ + ||q|| R^ holds for every key of the block.
//
// Precision: the mean is accumulated in float64 (exact for 64 bfloat16 or
// float32 values of ordinary range) and rounded once to float16; squared
// distances are float64 and the radius is rounded up to float32 after a
// 2^-40 relative margin that covers the float64 summation error. With a
// deviation buffer, the coordinate standard deviation (population, about the
// float64 mean; Section F.1) is rounded once to float16. One wavefront builds
// one record; lanes own columns. The same device function serves the bulk
// builder and the append path, so both give identical bits.
#include "eta_device.h"

namespace eta {
namespace {

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

// One wavefront. tile: [64][D] keys of one (page, kv head). If override_row is
// non-null, row 63 is read from it instead of the tile. Lanes own columns;
// the rows are read twice (sums, then distances and deviations), which keeps
// the register footprint small enough for eight wavefronts per SIMD. Writes
// the centroid and radius, and the coordinate deviation if sig_out is not null.
template <typename T, int D>
__device__ void build_record(const typename T::Stored* tile, const typename T::Stored* override_row,
                             uint16_t* mu_out, float* r_out, uint16_t* sig_out, int lane) {
  constexpr int CPL = D / 64;  // columns per lane: 2 (D=128) or 1 (D=64)
  double sum[CPL];
  bool finite = true;
#pragma unroll
  for (int c = 0; c < CPL; ++c) sum[c] = 0.0;
  for (int r = 0; r < kBlock; ++r) {
    const typename T::Stored* row = (r == kBlock - 1 && override_row) ? override_row : tile + r * D;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const float x = load_elem<T>(row + lane * CPL + c);
      finite = finite && (fabsf(x) <= 3.4028234663852886e38f);
      sum[c] += (double)x;
    }
  }
  uint16_t h[CPL];
  double mu[CPL], mean[CPL], dev2[CPL];
  bool ok = finite;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    mean[c] = sum[c] * (1.0 / kBlock);
    dev2[c] = 0.0;
    h[c] = f64_to_f16_rne(mean[c]);
    ok = ok && ((h[c] & 0x7c00u) != 0x7c00u);
  }
  const bool all_ok = __all(ok);
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    if (!all_ok) h[c] = 0;
    mu[c] = (double)f16_bits_to_f32(h[c]);
    mu_out[lane * CPL + c] = h[c];
  }
  double rmax = 0.0;
  for (int r = 0; r < kBlock; ++r) {
    const typename T::Stored* row = (r == kBlock - 1 && override_row) ? override_row : tile + r * D;
    double part = 0.0;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const double x = (double)load_elem<T>(row + lane * CPL + c);
      const double dlt = x - mu[c];
      part += dlt * dlt;
      const double dm = x - mean[c];  // deviation about the float64 mean
      dev2[c] += dm * dm;
    }
    const double tot = wave_sum_f64(part);
    rmax = (tot > rmax || tot != tot) ? tot : rmax;  // NaN propagates
  }
  // coordinate deviation (population) as float16
  if (sig_out) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const double sd = sqrt(dev2[c] * (1.0 / kBlock));
      sig_out[lane * CPL + c] = (sd < 1e300) ? f64_to_f16_rne(sd) : (uint16_t)0x7c00u;
    }
  }
  const bool any_bad = __any(!finite);
  if (lane == 0) {
    float r;
    if (any_bad || !(rmax < 1e300)) r = __builtin_inff();
    else r = f64_to_f32_up(sqrt(rmax) * (1.0 + 0x1p-40));
    *r_out = r;
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void k_build(CacheView c, SeqView s) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t idx = (int64_t)blockIdx.x * 4 + wave;  // over N * MB * HKV
  const int64_t total = (int64_t)s.N * s.MB * c.HKV;
  if (idx >= total) return;
  const int g = (int)(idx % c.HKV);
  const int64_t nj = idx / c.HKV;
  const int j = (int)(nj % s.MB);
  const int n = (int)(nj / s.MB);
  const int len = s.lens[n];
  if (len < 1 || len > kBlock * s.MB) return;
  if (j >= len / kBlock) return;
  const int page = s.bt[(int64_t)n * s.MB + j];
  if (page < 0 || page >= c.num_pages) return;
  const int64_t rec = (int64_t)page * c.HKV + g;
  const auto* tile = (const typename T::Stored*)c.k + rec * kBlock * D;
  build_record<T, D>(tile, nullptr, c.mu + rec * D, c.radius + rec, c.sigma ? c.sigma + rec * D : nullptr, lane);
}

template <typename T, int D>
__global__ __launch_bounds__(64) void k_append(CacheView c, SeqView s, const void* k_new,
                                               const void* v_new) {
  const int lane = threadIdx.x;
  const int n = blockIdx.x / c.HKV, g = blockIdx.x % c.HKV;
  const int len = s.lens[n];
  if (len < 0 || len >= kBlock * s.MB) return;
  const int j = len / kBlock, row = len % kBlock;
  const int page = s.bt[(int64_t)n * s.MB + j];
  if (page < 0 || page >= c.num_pages) return;
  using St = typename T::Stored;
  const int64_t rec = (int64_t)page * c.HKV + g;
  const St* kn = (const St*)k_new + ((int64_t)n * c.HKV + g) * D;
  const St* vn = (const St*)v_new + ((int64_t)n * c.HKV + g) * D;
  St* kd = (St*)c.kw + (rec * kBlock + row) * D;
  St* vd = (St*)c.vw + (rec * kBlock + row) * D;
  for (int i = lane; i < D; i += 64) {
    kd[i] = kn[i];
    vd[i] = vn[i];
  }
  if (row == kBlock - 1) {
    const St* tile = (const St*)c.kw + rec * kBlock * D;
    build_record<T, D>(tile, kn, c.mu + rec * D, c.radius + rec, c.sigma ? c.sigma + rec * D : nullptr, lane);
  }
}

template <typename T, int D>
hipError_t build_impl(const CacheView& c, const SeqView& s, hipStream_t st) {
  const int64_t waves = (int64_t)s.N * s.MB * c.HKV;
  const int64_t grid = (waves + 3) / 4;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_build<T, D>), dim3((unsigned)grid), dim3(256), 0, st, c, s);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t append_impl(const CacheView& c, const SeqView& s, const void* kn, const void* vn,
                       hipStream_t st) {
  hipLaunchKernelGGL((k_append<T, D>), dim3(s.N * c.HKV), dim3(64), 0, st, c, s, kn, vn);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_build_summaries(const CacheView& c, const SeqView& s, hipStream_t st) {
  if (c.kv_dtype == 1) return c.D == 128 ? build_impl<Bf16, 128>(c, s, st) : build_impl<Bf16, 64>(c, s, st);
  return c.D == 128 ? build_impl<F32, 128>(c, s, st) : build_impl<F32, 64>(c, s, st);
}

hipError_t launch_append(const CacheView& c, const SeqView& s, const void* kn, const void* vn,
                         hipStream_t st) {
  if (c.kv_dtype == 1)
    return c.D == 128 ? append_impl<Bf16, 128>(c, s, kn, vn, st) : append_impl<Bf16, 64>(c, s, kn, vn, st);
  return c.D == 128 ? append_impl<F32, 128>(c, s, kn, vn, st) : append_impl<F32, 64>(c, s, kn, vn, st);
}

}  // namespace eta
