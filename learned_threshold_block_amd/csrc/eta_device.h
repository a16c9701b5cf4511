// Device-side helpers for the gfx950 kernels: lane layouts, DPP butterflies,
// bf16 unpacking and exact float64 -> float16 rounding.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "eta_internal.h"

namespace eta {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- element types
struct Bf16 {
  using Stored = uint16_t;
  static constexpr int kBytes = 2;
};
struct F32 {
  using Stored = float;
  static constexpr int kBytes = 4;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 16-byte load marked non-temporal (the data is read once per call, so it
// should not displace other lines in the caches). On scattered 16 KB tiles
// this streams measurably faster from HBM than an ordinary load.
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 x = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(x[0], x[1], x[2], x[3]);
}

// Lane layout of a 64-row tile of D-element rows loaded with 16-byte accesses.
// Lane (r, cb), r = lane / LPR, cb = lane % LPR, holds for load i the row
// RPI*i + r, columns chunk(c) = c*(D/CPL) + cb*EPC .. +EPC for c < CPL. One load
// instruction covers RPI whole rows (contiguous when CPL == 1).
template <int EBYTES, int D>
struct TileLayout {
  static constexpr int EPC = 16 / EBYTES;            // elements per 16-byte chunk
  static constexpr int ROWB = D * EBYTES;            // bytes per row
  static constexpr int CPL = ROWB > 256 ? 2 : 1;     // chunks per lane per row
  static constexpr int LPR = ROWB / 16 / CPL;        // lanes per row (8 or 16)
  static constexpr int RPI = 64 / LPR;               // rows per load instruction
  static constexpr int NI = 64 / RPI;                // load instructions per tile (== LPR)
  static constexpr int EPL = EPC * CPL;              // elements per lane per row
  static constexpr int DPL = EPL * EBYTES / 4;       // dwords per lane per row
  static_assert(LPR == 8 || LPR == 16, "unsupported row width");
  static_assert(NI == LPR, "transpose reduction needs one value per lane of a row");
  __device__ static __forceinline__ int col(int c, int cb) { return c * (D / CPL) + cb * EPC; }
};

// ---------------------------------------------------------------- DPP
// quad_perm [1,0,3,2] and [2,3,0,1]; row_half_mirror; row_mirror.
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Partner for the butterfly step that splits lanes on bit log2(H) inside a
// group of 2H lanes: mirror (16), half mirror (8), quad xor 2 / xor 1.
template <int H>
__device__ __forceinline__ float bfly(float v) {
  if constexpr (H == 8) return dpp_f<kDppMirror>(v);
  else if constexpr (H == 4) return dpp_f<kDppHalfMirror>(v);
  else if constexpr (H == 2) return dpp_f<kDppXor2>(v);
  else return dpp_f<kDppXor1>(v);
}

// Transposing reduction inside groups of N lanes: lane j of a group starts with
// N values v[0..N) and ends with v[0] = sum over the group's lanes of v[j].
template <int N>
__device__ __forceinline__ void transpose_reduce(float* v, int lane) {
  if constexpr (N > 1) {
    constexpr int H = N / 2;
    const bool up = (lane & H) != 0;
#pragma unroll
    for (int k = 0; k < H; ++k) {
      const float keep = up ? v[k + H] : v[k];
      const float send = up ? v[k] : v[k + H];
      v[k] = keep + bfly<H>(send);
    }
    transpose_reduce<H>(v, lane);
  }
}

// All-reduce inside groups of N (8 or 16) lanes.
template <int N>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (N >= 16) v = fmaxf(v, dpp_f<kDppMirror>(v));
  if constexpr (N >= 8) v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  return v;
}
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 16) v += dpp_f<kDppMirror>(v);
  if constexpr (N >= 8) v += dpp_f<kDppHalfMirror>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppXor1>(v);
  return v;
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }
// Whole-wavefront maximum and integer sum without LDS traffic: DPP all-reduce
// inside each row of 16 lanes, then the four row results through readlane.
__device__ __forceinline__ float wave_max_f(float v) {
  v = group_max<16>(v);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ int wave_sum_i(int v) {
  v += dpp_i<kDppMirror>(v);
  v += dpp_i<kDppHalfMirror>(v);
  v += dpp_i<kDppXor2>(v);
  v += dpp_i<kDppXor1>(v);
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
         __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}


__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Inclusive scan of one int per thread over a workgroup of NW wavefronts;
// *total receives the workgroup's sum. lds: NW ints of scratch. Contains two
// workgroup barriers, so every thread of the workgroup must call it.
template <int NW>
__device__ __forceinline__ int block_incl_scan(int v, int* total, int* lds) {
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
  for (int w = 0; w < NW; ++w) {
    const int ws = lds[w];
    if (w < wave) base += ws;
    tot += ws;
  }
  __syncthreads();
  *total = tot;
  return base + x;
}

// Split of the Utot compacted entries over W attend ranges in proportion to
// per-die weights: range k has weight w[k % 8] (fixed point) and covers
// entries [B(k), B(k+1)), B(k) = floor(Utot C(k) / C(W)), C(k) = sum_{i<k} w[i % 8].
// Integer arithmetic, so every kernel that evaluates it gets the same ranges.
struct RangeSplit {
  int64_t utot, cw;
  int W, wsum;
  int w[kXcdClasses];
  __device__ void init(int64_t utot_, int W_, const int* w_) {
    utot = utot_;
    W = W_;
    wsum = 0;
#pragma unroll
    for (int x = 0; x < kXcdClasses; ++x) {
      w[x] = w_[x];
      wsum += w_[x];
    }
    cw = C(W);
  }
  // compile-time indices only, so the weights stay in registers
  __device__ int64_t C(int k) const {
    const int r = k % kXcdClasses;
    int part = 0;
#pragma unroll
    for (int x = 0; x < kXcdClasses; ++x) part += x < r ? w[x] : 0;
    return (int64_t)(k / kXcdClasses) * wsum + part;
  }
  __device__ int64_t B(int k) const { return utot * C(k) / cw; }
};

// A per-die weight as stored in the workspace, clamped to the range the
// weighting step writes (anything else reads as equal weights).
__device__ __forceinline__ int clamp_weight(int v, int deterministic) {
  return (!deterministic && v >= kWeightOne / 2 && v <= 2 * kWeightOne) ? v : kWeightOne;
}

// Raw buffer resource over [base, base + bytes): loads at offsets past the end
// return zeros instead of faulting (used for records of invalid pages).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
constexpr uint32_t kOutOfRange = 0x80000000u;

// Stores and loads coherent across the accelerator's dies (each die has its
// own L2): relaxed atomics at device scope are written through to, and read
// from, the device's coherence point, so data handed from one workgroup to
// another needs no L2 write-back or invalidation (which device-scope
// release and acquire fences perform on the whole L2 of a die). The writer
// waits for its stores to complete (wait_stores) before it signals.
__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store((uint32_t*)p, __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent2(float* p, float a, float b) {  // 8-byte aligned
  const uint64_t u = (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
  __hip_atomic_store((uint64_t*)p, u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 load_agent2(const float* p) {  // 8-byte aligned
  const uint64_t u = __hip_atomic_load((uint64_t*)const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((uint32_t)u), __uint_as_float((uint32_t)(u >> 32)));
}
__device__ __forceinline__ float4 load_agent4(const float* p) {  // 16-byte aligned
  const float2 a = load_agent2(p), b = load_agent2(p + 2);
  return make_float4(a.x, a.y, b.x, b.y);
}
// Wait until every vector memory access of this wavefront has completed (on
// gfx9 stores count in vmcnt too); the memory clobber keeps the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// exp(x) for the softmax weights: 2^(x log2 e) on the transcendental unit.
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

// ---------------------------------------------------------------- rounding
// float64 -> float16 bits, round to nearest even, in one rounding step
// (IEEE 754 binary16: 1 sign, 5 exponent, 10 fraction bits). Infinity and NaN
// map to infinity and a quiet NaN; overflow rounds to infinity.
__device__ __forceinline__ uint16_t f64_to_f16_rne(double x) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  const int bexp = (int)((b >> 52) & 0x7ff);
  const uint64_t frac = b & ((1ull << 52) - 1);
  if (bexp == 0x7ff) return sign | (frac ? 0x7e00 : 0x7c00);
  if (bexp == 0) return sign;  // float64 zero or subnormal: far below the float16 range
  const int e = bexp - 1023;
  if (e > 15) return sign | 0x7c00;
  const uint64_t m = (1ull << 52) | frac;   // 53 significant bits
  const int eu = e < -14 ? -14 : e;          // exponent of the result's leading place
  const int shift = 42 + (eu - e);           // bits of m below the result's last place
  if (shift >= 64) return sign;
  uint64_t q = m >> shift;
  const uint64_t rem = m & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) ++q;
  uint32_t bits = ((uint32_t)(eu + 14) << 10) + (uint32_t)q;
  if (bits >= 0x7c00u) bits = 0x7c00u;
  return sign | (uint16_t)bits;
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// float16 bits of the nearest value at or below (up = false) or at or above
// (up = true) a finite float32 x: round to nearest, then one step of the bit
// pattern if that landed on the wrong side (patterns of one sign order like
// their magnitudes; beyond the range: +-65504 or +-inf as the side requires).
__device__ __forceinline__ uint16_t f32_to_f16_dir(float x, bool up) {
  uint16_t h = f64_to_f16_rne((double)x);
  const float back = f16_bits_to_f32(h);
  if (up ? back < x : back > x) {
    if ((h & 0x7fffu) == 0) h = up ? 0x0001u : 0x8001u;
    else if (((h & 0x8000u) != 0) == up) h = (uint16_t)(h - 1u);
    else h = (uint16_t)(h + 1u);
  }
  return h;
}

// OCP 8-bit floats for the FP8 records: format 0 E4M3 (3 mantissa bits,
// exponent bias 7, largest 448, no infinities), format 1 E5M2 (2 mantissa bits,
// bias 15, largest 57344). Encoding rounds a finite float64 to nearest even
// and saturates at the largest finite magnitude.
template <int MBITS, int EMIN>
__device__ __forceinline__ uint8_t f64_to_fp8_sat(double x, double vmax, uint8_t maxcode) {
  const uint8_t sign = __double_as_longlong(x) < 0 ? 0x80u : 0u;
  const double a = fabs(x);
  if (a >= vmax) return sign | maxcode;
  if (a == 0.0) return sign;
  int e;
  (void)frexp(a, &e);
  e -= 1;  // floor(log2 a)
  if (e < EMIN) e = EMIN;
  const double r = rint(ldexp(a, MBITS - e));  // multiples of the binade's quantum
  if (ldexp(r, e - MBITS) >= vmax) return sign | maxcode;
  int m = (int)r;
  if (m == 0) return sign;
  if (m == (2 << MBITS)) {  // carried into the next binade
    e += 1;
    m = 1 << MBITS;
  }
  if (m < (1 << MBITS)) return sign | (uint8_t)m;  // subnormal: exponent field 0
  return sign | (uint8_t)(((e + 1 - EMIN) << MBITS) | (m - (1 << MBITS)));
}

__device__ __forceinline__ uint8_t f64_to_fp8(double x, int fmt) {
  return fmt == 0 ? f64_to_fp8_sat<3, -6>(x, 448.0, 0x7eu) : f64_to_fp8_sat<2, -14>(x, 57344.0, 0x7bu);
}

__device__ __forceinline__ float fp8_to_f32(uint32_t b, int fmt) {
  if (fmt != 0) return f16_bits_to_f32((uint16_t)((b & 0xffu) << 8));  // E5M2 is binary16's high byte
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  const float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
  return __uint_as_float(__float_as_uint(v) | ((b & 0x80u) << 24));
}

// Smallest float32 >= x (x >= 0), +inf for non-finite input.
__device__ __forceinline__ float f64_to_f32_up(double x) {
  if (!(x < 1e300)) return __builtin_inff();
  float f = (float)x;
  if ((double)f < x) f = __uint_as_float(__float_as_uint(f) + 1u);
  return f;
}

}  // namespace eta
