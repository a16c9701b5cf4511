// Block records: centroid mu^ (float16, nearest even) and radius R^ (float32,
// rounded up) of every complete key block, per KV head.
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
// one record from the block's keys read once in the 16-byte tile layout
// (build_record). The same device function serves the bulk builders, the
// append path and the prompt pass, so all give identical bits. Records of
// 16-, 32- and 128-token screen blocks (Appendix F.3's block size) follow the
// same rule over their keys.
#include "eta_records.h"

namespace eta {
namespace {

// One wavefront per (sequence, complete block, KV head). OPT: the cache
// carries optional records (deviation, key box or FP8); without them the
// record needs about half the registers, so that kernel runs four wavefronts
// per SIMD instead of two.
template <typename T, int D, bool OPT>
__device__ __forceinline__ void build_one(const CacheView& c, const SeqView& s) {
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
  if constexpr (OPT)
    build_record<T, D>(tile, nullptr, c.mu + rec * D, c.radius + rec, c.sigma ? c.sigma + rec * D : nullptr,
                       c.kmin ? c.kmin + rec * D : nullptr, c.kmax ? c.kmax + rec * D : nullptr,
                       c.mu8 ? c.mu8 + rec * D : nullptr, c.mu8 ? c.radius8 + rec : nullptr, c.mu8_fmt, lane);
  else
    build_record<T, D>(tile, nullptr, c.mu + rec * D, c.radius + rec, nullptr, nullptr, nullptr, nullptr, nullptr,
                       0, lane);
}

// wavefronts per SIMD of the lean kernel: four unless a row is 512 bytes
// (float32 at d = 128: the kept rows alone take 128 registers)
template <typename T, int D>
constexpr int build_waves() {
  return T::kBytes * D <= 256 ? 4 : 2;
}

template <typename T, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(build_waves<T, D>(), build_waves<T, D>())))
void k_build(CacheView c, SeqView s) {
  build_one<T, D, false>(c, s);
}

template <typename T, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_build_all(CacheView c, SeqView s) {
  build_one<T, D, true>(c, s);
}

// Records of the other screen blocks (ROWS = 16, 32 or 128 tokens): one
// wavefront per (sequence, block, KV head), complete blocks only. Block j of a
// sequence holds its tokens j ROWS .. j ROWS + ROWS - 1: with 16 or 32 tokens
// rows (j mod 64/ROWS) ROWS .. + ROWS - 1 of page block_table[n][j ROWS / 64],
// with 128 the pages block_table[n][2j] and [2j + 1], its record kept with
// the first of them.
template <typename T, int D, int ROWS>
__global__ __launch_bounds__(256) void k_build_sub(CacheView c, SeqView s) {
  constexpr int SB = sub_slots(ROWS);                      // record slots per page
  constexpr int PB = ROWS > kBlock ? ROWS / kBlock : 1;    // pages per block
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t nbs = ((int64_t)s.MB * SB + PB - 1) / PB;  // blocks per block-table row
  const int64_t idx = (int64_t)blockIdx.x * 4 + wave;      // over N * nbs * HKV
  const int64_t total = (int64_t)s.N * nbs * c.HKV;
  if (idx >= total) return;
  const int g = (int)(idx % c.HKV);
  const int64_t nj = idx / c.HKV;
  const int j = (int)(nj % nbs);
  const int n = (int)(nj / nbs);
  const int len = s.lens[n];
  if (len < 1 || len > kBlock * s.MB) return;
  if (j >= len / ROWS) return;
  const int p0 = (int)((int64_t)j * ROWS / kBlock);  // table entry of the block's first page
  const int page = s.bt[(int64_t)n * s.MB + p0];
  if (page < 0 || page >= c.num_pages) return;
  using St = typename T::Stored;
  const int64_t rec = ((int64_t)page * c.HKV + g) * SB + j % SB;
  const St* tile = (const St*)c.k + (((int64_t)page * c.HKV + g) * kBlock + (j % SB) * (kBlock / SB)) * D;
  const St* hi = nullptr;
  if constexpr (PB > 1) {  // p0 + 1 < ceil(len / 64) <= MB: the block is complete
    const int page1 = s.bt[(int64_t)n * s.MB + p0 + 1];
    if (page1 < 0 || page1 >= c.num_pages) return;
    hi = (const St*)c.k + ((int64_t)page1 * c.HKV + g) * kBlock * D;
  }
  build_record<T, D, ROWS>(tile, nullptr, c.mu_sub + rec * D, c.radius_sub + rec, nullptr, nullptr, nullptr,
                           nullptr, nullptr, 0, lane, hi);
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
    build_record<T, D>(tile, kn, c.mu + rec * D, c.radius + rec, c.sigma ? c.sigma + rec * D : nullptr,
                       c.kmin ? c.kmin + rec * D : nullptr, c.kmax ? c.kmax + rec * D : nullptr,
                     c.mu8 ? c.mu8 + rec * D : nullptr, c.mu8 ? c.radius8 + rec : nullptr, c.mu8_fmt, lane);
  }
  // the other screen block this token completes
  if (c.sub_rows == 32 && row % 32 == 31) {
    const int64_t srec = rec * 2 + row / 32;
    build_record<T, D, 32>((const St*)c.kw + srec * 32 * D, kn, c.mu_sub + srec * D, c.radius_sub + srec, nullptr,
                           nullptr, nullptr, nullptr, nullptr, 0, lane);
  } else if (c.sub_rows == 16 && row % 16 == 15) {
    const int64_t srec = rec * 4 + row / 16;
    build_record<T, D, 16>((const St*)c.kw + srec * 16 * D, kn, c.mu_sub + srec * D, c.radius_sub + srec, nullptr,
                           nullptr, nullptr, nullptr, nullptr, 0, lane);
  } else if (c.sub_rows == 128 && row == kBlock - 1 && (j & 1)) {
    // a 128-token block ends with this page: its record goes with the first page
    const int page0 = s.bt[(int64_t)n * s.MB + j - 1];
    if (page0 < 0 || page0 >= c.num_pages) return;
    const int64_t srec = (int64_t)page0 * c.HKV + g;
    build_record<T, D, 128>((const St*)c.kw + srec * kBlock * D, kn, c.mu_sub + srec * D, c.radius_sub + srec,
                            nullptr, nullptr, nullptr, nullptr, nullptr, 0, lane, (const St*)c.kw + rec * kBlock * D);
  }
}

template <typename T, int D>
hipError_t build_impl(const CacheView& c, const SeqView& s, hipStream_t st) {
  const int64_t waves = (int64_t)s.N * s.MB * c.HKV;
  const int64_t grid = (waves + 3) / 4;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (c.sigma || c.kmin || c.mu8) hipLaunchKernelGGL((k_build_all<T, D>), dim3((unsigned)grid), dim3(256), 0, st, c, s);
  else hipLaunchKernelGGL((k_build<T, D>), dim3((unsigned)grid), dim3(256), 0, st, c, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || c.sub_rows == 0) return e;
  const int64_t nbs = c.sub_rows > kBlock ? (s.MB + 1) / 2 : (int64_t)s.MB * (kBlock / c.sub_rows);
  const int64_t sgrid = ((int64_t)s.N * nbs * c.HKV + 3) / 4;
  if (sgrid > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 g3((unsigned)sgrid);
  if (c.sub_rows == 32) hipLaunchKernelGGL((k_build_sub<T, D, 32>), g3, dim3(256), 0, st, c, s);
  else if (c.sub_rows == 16) hipLaunchKernelGGL((k_build_sub<T, D, 16>), g3, dim3(256), 0, st, c, s);
  else hipLaunchKernelGGL((k_build_sub<T, D, 128>), g3, dim3(256), 0, st, c, s);
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
