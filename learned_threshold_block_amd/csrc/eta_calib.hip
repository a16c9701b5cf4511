// Offline calibration of per-head constant thresholds: 1/t-weighted score
// histograms over calibration sequences and a search for each head's training
// density.
//
// "Elastic Threshold Attention" (paperpeel.com/paper/2609.20888), Section 4.7
// and Appendix D.2 (Algorithm 1; its body did not survive, the reading is):
//   * every position t (0-based) of a sequence is a query row over the keys
//     s <= t, scaled scores S = q_t . k_s / sqrt(d);
//   * each key of row t weighs floor(2^31 / (t + 1)) (integer, so every row
//     weighs about the same and the sums are exact and order-free);
//   * equal-width bins over [lo, hi), outside scores in the end bins;
//   * target: the weighted count of scores at or above the learned threshold
//     w_h . q_t + b_h (the head's training density), or floor(rho_h * total);
//   * c_h = the lowest bin edge whose weighted tail does not exceed the target.
//
// k_calib_mfma (bfloat16) and k_calib_hist (float32): one workgroup per
//   (sequence, KV head, tile of 64 query positions) walking the key tiles up to
//   the diagonal; scores on the matrix cores (bfloat16) or from the decode's
//   tile layout and transposing DPP reduction (float32); each lane bins its
//   scores into a per-workgroup LDS histogram with 64-bit integer atomics,
//   which is added to the global one at the end (non-empty bins only).
// k_calib_search: one wavefront per query head: suffix sums of the histogram
//   and the count of edges whose tail exceeds the target.
#include "eta_device.h"

namespace eta {
namespace {

struct CalibArgs {
  CacheView c;
  SeqView s;
  const void* q;       // [N][Lq][HQ][D]
  int Lq, HQ, B;
  const float* w;      // [HQ][D] or null
  const float* b;      // [HQ] or null
  const float* rho;    // [HQ] or null
  float lo, hi, bscale;  // bscale = B / (hi - lo)
  unsigned long long* hist;   // [HQ][B]
  unsigned long long* above;  // [HQ]
  unsigned long long* total;  // [HQ]
  float* c_out;               // [HQ]
  int* err;                   // [1] set on an out-of-range page id
};

__global__ void k_calib_zero(CalibArgs A) {
  const int64_t n = (int64_t)A.HQ * A.B;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    A.hist[i] = 0ull;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < A.HQ) {
    A.above[i] = 0ull;
    A.total[i] = 0ull;
  }
  if (i == 0) A.err[0] = 0;
}

// The learned threshold w_h . q_t + b_h of rows t0 + 16 wave .. + 15 (those
// below len) for every head of the group, into s_tau[t - t0][h]. Lanes in the
// tile layout: every row of lanes holds all D columns, so every lane has the
// same sum and lane 0 stores it.
template <typename T, int D, int G>
__device__ __forceinline__ void row_thresholds(const CalibArgs& A, int n, int g, int t0, int len, int wave, int lane,
                                               float (*s_tau)[kMaxGroup]) {
  using L = TileLayout<T::kBytes, D>;
  constexpr int LPR = L::LPR, CPL = L::CPL, EPL = L::EPL;
  constexpr bool kBf16 = T::kBytes == 2;
  using St = typename T::Stored;
  const int cb = lane % LPR;
  for (int i = 0; i < 16; ++i) {
    const int t = t0 + wave * 16 + i;
    if (t >= len) break;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const St* qrow = (const St*)A.q + (((int64_t)n * A.Lq + t) * A.HQ + g * G + h) * D;
      const float* wr = A.w + (int64_t)(g * G + h) * D;
      float pw = 0.f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const uint4 v = *(const uint4*)(qrow + L::col(c, cb));
        const uint32_t qw[4] = {v.x, v.y, v.z, v.w};
        const float4 w0 = *(const float4*)(wr + L::col(c, cb));
        const float4 w1 = EPL / CPL > 4 ? *(const float4*)(wr + L::col(c, cb) + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
        float qv[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (kBf16) {
            qv[2 * e] = bf16_lo(qw[e]);
            qv[2 * e + 1] = bf16_hi(qw[e]);
          } else {
            qv[e] = __uint_as_float(qw[e]);
            qv[4 + e] = 0.f;
          }
        }
        pw = fmaf(w0.x, qv[0], pw); pw = fmaf(w0.y, qv[1], pw);
        pw = fmaf(w0.z, qv[2], pw); pw = fmaf(w0.w, qv[3], pw);
        if constexpr (kBf16) {
          pw = fmaf(w1.x, qv[4], pw); pw = fmaf(w1.y, qv[5], pw);
          pw = fmaf(w1.z, qv[6], pw); pw = fmaf(w1.w, qv[7], pw);
        }
      }
      const float tau = group_sum<LPR>(pw) + A.b[g * G + h];
      if (lane == 0) s_tau[wave * 16 + i][h] = tau;
    }
  }
}

// Row totals of the tile's rows t0 .. t0 + 63 below len (one wavefront): row t
// has t + 1 keys of weight floor(2^31 / (t + 1)), the same for every head of
// the group; independent of the keys, so a skipped key tile leaves them whole.
template <int G>
__device__ __forceinline__ void row_totals(const CalibArgs& A, int g, int t0, int len, int lane) {
  const int t = t0 + lane;
  unsigned long long tw = t < len ? (unsigned long long)((1u << 31) / (unsigned)(t + 1)) * (unsigned)(t + 1) : 0ull;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) tw += __shfl_xor(tw, m, 64);
  if (lane < G) atomicAdd(&A.total[g * G + lane], tw);
}

// Workgroup -> (sequence, KV head, query tile). Consecutive workgroups are
// dispatched round-robin over the accelerator's eight dies, each with its own
// L2; the remap gives every die a contiguous run of (pair, tile) indices, so
// the tiles of one (sequence, KV head) pair, which all read the same key
// tiles, run on one die. The first 8 floor(n / 8) workgroups are permuted
// among themselves; the rest keep their index.
__device__ __forceinline__ void calib_tile(int MB, int HKV, int& n, int& g, int& qt) {
  const int total = gridDim.x, per = total / kXcdClasses, bid = blockIdx.x;
  const int L = bid < kXcdClasses * per ? (bid % kXcdClasses) * per + bid / kXcdClasses : bid;
  const int pair = L / MB;
  qt = L % MB;
  n = pair / HKV;
  g = pair % HKV;
}

template <typename T, int D, int G>
__global__ __launch_bounds__(256) void k_calib_hist(CalibArgs A) {
  using L = TileLayout<T::kBytes, D>;
  constexpr int LPR = L::LPR, RPI = L::RPI, NI = L::NI, CPL = L::CPL, EPL = L::EPL;
  constexpr bool kBf16 = T::kBytes == 2;
  using St = typename T::Stored;
  extern __shared__ unsigned long long lhist[];  // [G][B]
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int r = lane / LPR, cb = lane % LPR;
  const int HKV = A.c.HKV, MB = A.s.MB, B = A.B;
  int n, g, qt;
  calib_tile(MB, HKV, n, g, qt);
  const int len = A.s.lens[n];
  if (len < 1 || len > kBlock * MB || qt * kBlock >= len) return;
  for (int i = threadIdx.x; i < G * B; i += 256) lhist[i] = 0ull;
  __syncthreads();

  const float scale = 1.0f / sqrtf((float)D);
  const bool learned = A.w != nullptr;
  unsigned long long abv[G];
#pragma unroll
  for (int h = 0; h < G; ++h) abv[h] = 0ull;
  int loff[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) loff[c] = r * D + L::col(c, cb);
  const St* kbase = (const St*)A.c.k;
  const int tok = RPI * cb + r;  // key (within the tile) whose score this lane finishes

  // the learned threshold w_h . q_t + b_h of each of the wavefront's rows, once
  __shared__ float s_tau[kBlock][kMaxGroup];
  if (learned) {
    row_thresholds<T, D, G>(A, n, g, qt * kBlock, len, wave, lane, s_tau);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }
  if (wave == 0) row_totals<G>(A, g, qt * kBlock, len, lane);

  for (int j = 0; j <= qt; ++j) {
    const int page = A.s.bt[(int64_t)n * MB + j];
    if (page < 0 || page >= A.c.num_pages) {
      if (threadIdx.x == 0) A.err[0] = 1;
      continue;
    }
    uint4 kr[NI][CPL];
    const St* kt = kbase + ((int64_t)page * HKV + g) * (kBlock * D);
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int c = 0; c < CPL; ++c) kr[i][c] = *(const uint4*)(kt + loff[c] + i * RPI * D);
    const int s_key = j * kBlock + tok;
    for (int i = 0; i < 16; ++i) {
      const int t = qt * kBlock + wave * 16 + i;
      if (t >= len) break;
      const unsigned long long wt = (unsigned long long)((1u << 31) / (unsigned)(t + 1));
      const bool valid = s_key <= t;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const St* qrow = (const St*)A.q + (((int64_t)n * A.Lq + t) * A.HQ + g * G + h) * D;
        uint32_t qw[CPL * 4];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const uint4 v = *(const uint4*)(qrow + L::col(c, cb));
          qw[c * 4 + 0] = v.x; qw[c * 4 + 1] = v.y; qw[c * 4 + 2] = v.z; qw[c * 4 + 3] = v.w;
        }
        float pd[NI];
#pragma unroll
        for (int ii = 0; ii < NI; ++ii) {
          float a = 0.f;
#pragma unroll
          for (int c = 0; c < CPL; ++c) {
            const uint32_t kw[4] = {kr[ii][c].x, kr[ii][c].y, kr[ii][c].z, kr[ii][c].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if constexpr (kBf16) {
                a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qw[c * 4 + e]),
                                                    __builtin_bit_cast(bf16x2_t, kw[e]), a, false);
              } else {
                a = fmaf(__uint_as_float(qw[c * 4 + e]), __uint_as_float(kw[e]), a);
              }
            }
          }
          pd[ii] = a;
        }
        transpose_reduce<LPR>(pd, lane);
        const float S = pd[0] * scale;
        if (valid) {
          const float x = floorf((S - A.lo) * A.bscale);
          const int bin = !(x > 0.f) ? 0 : (x >= (float)(B - 1) ? B - 1 : (int)x);  // NaN: bin 0
          atomicAdd(&lhist[h * B + bin], wt);
        }
        if (learned && valid && S >= s_tau[wave * 16 + i][h]) abv[h] += wt;
      }
    }
  }
  // per-head sums of the wavefront, then the workgroup's bins into the totals
#pragma unroll
  for (int h = 0; h < G; ++h) {
    unsigned long long a = abv[h];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) a += __shfl_xor(a, m, 64);
    if (lane == 0 && learned && a) atomicAdd(&A.above[g * G + h], a);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < G * B; i += 256) {
    const unsigned long long v = lhist[i];
    if (v) atomicAdd(&A.hist[(int64_t)(g * G) * B + i], v);
  }
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// bfloat16 caches: the same histogram with the scores of each 64-query x
// 64-key tile pair on the matrix cores. Wavefront w takes the quadrant (query
// half w >> 1, key half w & 1) for every head of the group: S^T = K Q^T on
// v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 dims from an LDS key tile, B =
// 32 queries x 16 dims held in registers), so lane l holds query l % 32 of its
// half and, in element 4 i + j, key 8 i + 4 (l / 32) + j of its half. Rows
// past the sequence end and keys after the query are skipped. The workgroup
// order keeps the tiles of one (sequence, KV head) pair on one die.
template <int D, int G>
__global__ __launch_bounds__(256) void k_calib_mfma(CalibArgs A) {
  constexpr int KS = D / 16;  // 16-dim steps
  extern __shared__ unsigned long long lhist[];  // [G][B]
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int HKV = A.c.HKV, MB = A.s.MB, B = A.B;
  int n, g, qt;
  calib_tile(MB, HKV, n, g, qt);
  const int len = A.s.lens[n];
  if (len < 1 || len > kBlock * MB || qt * kBlock >= len) return;
  for (int i = threadIdx.x; i < G * B; i += 256) lhist[i] = 0ull;
  const bool learned = A.w != nullptr;
  if (wave == 0) row_totals<G>(A, g, qt * kBlock, len, lane);

  const int qh = wave >> 1, kh = wave & 1, nq = lane & 31, hi = lane >> 5;
  const int t = qt * kBlock + 32 * qh + nq;  // this lane's query (below 64 MB = Lq)
  const bool t_ok = t < len;
  const unsigned long long wt = t_ok ? (unsigned long long)((1u << 31) / (unsigned)(t + 1)) : 0ull;
  const float scale = 1.0f / sqrtf((float)D);
  // bin position of a product a (score a scale): (a scale - lo) B / (hi - lo)
  // as one fma; the threshold test compares a with tau / scale
  const float bmul = scale * A.bscale, badd = -A.lo * A.bscale, blast = (float)(B - 1);
  const uint16_t* qrow0 = (const uint16_t*)A.q + (((int64_t)n * A.Lq + t) * A.HQ + g * G) * D + 8 * hi;
  // The B operands (this lane's query, 16-byte rows of 8 dims) of up to four
  // heads stay in registers for a whole pass over the key tiles; eight heads
  // take two passes. Key tiles go through a double-buffered LDS area. Chunk c
  // (8 dims) of key row r sits at chunk c ^ swz(r) of its LDS row: a
  // wavefront's operand reads (consecutive lanes on consecutive rows, one
  // chunk) then spread over the banks.
  constexpr int HB = G < 4 ? G : 4;
  constexpr int CH = D / 8;              // 16-byte chunks per key row
  constexpr int TCH = kBlock * CH;       // chunks per tile
  static_assert(TCH % 256 == 0, "tile chunks");
  __shared__ __attribute__((aligned(16))) uint4 klds[2][TCH];
  const auto swz = [](int r) { return (r ^ (r / CH)) & (CH - 1); };
  const int tid = threadIdx.x;
  const auto valid_page = [&](int page) { return page >= 0 && page < A.c.num_pages ? page : -1; };
  const int* const bt_row = A.s.bt + (int64_t)n * MB;
  const int kr = 32 * kh + nq;  // this lane's key row of the A operand
  const auto mfma_head = [&](const uint4 (&ka)[KS], const uint4 (&qh_)[KS]) {
    f32x16_t acc = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, ka[ks]),
                                                    __builtin_bit_cast(bf16x8_t, qh_[ks]), acc, 0, 0, 0);
    return acc;
  };
  // Tile j + 1 is loaded into registers while tile j is scored and stored to
  // the other LDS buffer afterwards (loads straight into LDS would make every
  // histogram atomic wait for them).
  uint4* const kb = &klds[0][0];
  constexpr int CPT = TCH / 256;  // 16-byte chunks per thread per tile
  const auto load_tile = [&](int page, uint4 (&rg)[CPT]) {  // zeros for a missing page
    const uint16_t* kt = (const uint16_t*)A.c.k + ((int64_t)(page >= 0 ? page : 0) * HKV + g) * (kBlock * D);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int p = tid + 256 * i, r = p / CH;
      rg[i] = page >= 0 ? *(const uint4*)(kt + r * D + 8 * ((p % CH) ^ swz(r))) : make_uint4(0, 0, 0, 0);
    }
  };
  const auto store_tile = [&](const uint4 (&rg)[CPT], int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) kb[buf * TCH + tid + 256 * i] = rg[i];
  };
  // one product: its bin (the position clamped to [0, B - 1] by a median,
  // which is 0 for NaN; truncation is then the floor), the weighted count
  // into the workgroup's histogram, the threshold test
  const auto bin_score = [&](int h, float a, float taua, int& nabv) {
    const int bin = (int)__builtin_amdgcn_fmed3f(fmaf(a, bmul, badd), 0.f, blast);
    atomicAdd(&lhist[h * B + bin], wt);
    nabv += a >= taua ? 1 : 0;
  };
#pragma unroll 1
  for (int hb = 0; hb < G; hb += HB) {
    float taua[HB];
    int nabv[HB];  // products at or above the threshold: every score of a lane has its row's weight
    uint4 qr[HB][KS];
#pragma unroll
    for (int hh = 0; hh < HB; ++hh)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qr[hh][ks] = *(const uint4*)(qrow0 + (hb + hh) * D + 16 * ks);
    // the learned threshold w_h . q_t + b_h of this lane's row from the B
    // operands it holds (dims 16 ks + 8 hi .. + 7; the lane 32 apart holds the
    // other half), compared in product units
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
      float tau = __builtin_inff();
      if (learned) {
        const float* wr = A.w + (int64_t)(g * G + hb + hh) * D + 8 * hi;
        float pw = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const float4 w0 = *(const float4*)(wr + 16 * ks), w1 = *(const float4*)(wr + 16 * ks + 4);
          const uint4 v = qr[hh][ks];
          pw = fmaf(w0.x, bf16_lo(v.x), pw); pw = fmaf(w0.y, bf16_hi(v.x), pw);
          pw = fmaf(w0.z, bf16_lo(v.y), pw); pw = fmaf(w0.w, bf16_hi(v.y), pw);
          pw = fmaf(w1.x, bf16_lo(v.z), pw); pw = fmaf(w1.y, bf16_hi(v.z), pw);
          pw = fmaf(w1.z, bf16_lo(v.w), pw); pw = fmaf(w1.w, bf16_hi(v.w), pw);
        }
        pw += __shfl_xor(pw, 32, 64);
        tau = (pw + A.b[g * G + hb + hh]) / scale;
      }
      taua[hh] = tau;
      nabv[hh] = 0;
    }
    // lane l holds the block-table entry of tile 64 c + l of the current
    // chunk c of 64 tiles (a register read per tile, a load per chunk)
    int ents = lane <= qt ? bt_row[lane] : -1;
    int page = valid_page(__builtin_amdgcn_readlane(ents, 0));
    {
      uint4 rg[CPT];
      load_tile(page, rg);
      store_tile(rg, 0);
    }
    __syncthreads();
    for (int j = 0; j <= qt; ++j) {
      const bool cur_ok = page >= 0;
      if (!cur_ok && tid == 0) A.err[0] = 1;
      // the operand reads and the MFMA stay uniform over the workgroup: a
      // lane supplies a key row of the A operand for every lane's scores,
      // so only the binning is skipped for queries past the sequence end
      uint4 rg[CPT];
      const bool has_next = j < qt;
      int next_page = -1;
      if (has_next) {
        const int jn = j + 1;
        if ((jn & 63) == 0) ents = jn + lane <= qt ? bt_row[jn + lane] : -1;
        next_page = valid_page(__builtin_amdgcn_readlane(ents, jn & 63));
        load_tile(next_page, rg);
      }
      if (cur_ok) {
        uint4 ka[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) ka[ks] = kb[(j & 1) * TCH + kr * CH + ((2 * ks + hi) ^ swz(kr))];
        const int s0 = j * kBlock + 32 * kh + 4 * hi;  // key of element 0
#pragma unroll
        for (int hh = 0; hh < HB; ++hh) {
          const int h = hb + hh;
          const f32x16_t acc = mfma_head(ka, qr[hh]);
          if (t_ok) {
            if (j < qt) {  // every key of the tile precedes every query of this one
#pragma unroll
              for (int e = 0; e < 16; ++e) bin_score(h, acc[e], taua[hh], nabv[hh]);
            } else {  // the diagonal tile: keys after the query are skipped
#pragma unroll
              for (int e = 0; e < 16; ++e)
                if (s0 + 8 * (e >> 2) + (e & 3) <= t) bin_score(h, acc[e], taua[hh], nabv[hh]);
            }
          }
        }
      }
      if (has_next) store_tile(rg, (j + 1) & 1);
      __syncthreads();
      page = next_page;
    }
    if (learned) {
#pragma unroll
      for (int hh = 0; hh < HB; ++hh) {
        unsigned long long a = (unsigned long long)nabv[hh] * wt;
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) a += __shfl_xor(a, m, 64);
        if (lane == 0 && a) atomicAdd(&A.above[g * G + hb + hh], a);
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < G * B; i += 256) {
    const unsigned long long v = lhist[i];
    if (v) atomicAdd(&A.hist[(int64_t)(g * G) * B + i], v);
  }
}

// One wavefront per query head: tail(b) = sum of bins >= b is non-increasing,
// so the lowest edge with tail(b) <= target is the number of edges b < B whose
// tail exceeds it.
__global__ __launch_bounds__(64) void k_calib_search(CalibArgs A) {
  const int h = blockIdx.x, lane = threadIdx.x, B = A.B;
  const unsigned long long* hb = A.hist + (int64_t)h * B;
  unsigned long long target;
  if (A.rho) {
    target = (unsigned long long)floor((double)A.rho[h] * (double)A.total[h]);
  } else {
    target = A.above[h];
  }
  // lane l owns bins [l*per, (l+1)*per)
  const int per = (B + 63) / 64;
  const int b0 = lane * per, b1 = min(B, b0 + per);
  unsigned long long own = 0ull;
  for (int b = b0; b < b1; ++b) own += hb[b];
  // sum of the bins owned by higher lanes (inclusive suffix, minus own)
  unsigned long long suf = own;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned long long y = __shfl_down(suf, o, 64);
    if (lane + o < 64) suf += y;
  }
  unsigned long long tail = suf;  // tail(b0)
  int cnt = 0;
  for (int b = b0; b < b1; ++b) {
    if (tail > target) ++cnt;
    tail -= hb[b];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) cnt += __shfl_xor(cnt, o, 64);
  if (lane == 0) A.c_out[h] = (float)((double)A.lo + (double)cnt * ((double)A.hi - (double)A.lo) / (double)B);
}

template <typename T, int D, int G>
hipError_t calib_impl(const CalibArgs& a, int N, int MB, hipStream_t st) {
  const size_t lds = (size_t)G * a.B * sizeof(unsigned long long);
  if constexpr (T::kBytes == 2) hipLaunchKernelGGL((k_calib_mfma<D, G>), dim3(MB * N * a.c.HKV), dim3(256), lds, st, a);
  else hipLaunchKernelGGL((k_calib_hist<T, D, G>), dim3(MB * N * a.c.HKV), dim3(256), lds, st, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t calib_g(const CalibArgs& a, int G, int N, int MB, hipStream_t st) {
  switch (G) {
    case 1: return calib_impl<T, D, 1>(a, N, MB, st);
    case 2: return calib_impl<T, D, 2>(a, N, MB, st);
    case 4: return calib_impl<T, D, 4>(a, N, MB, st);
    case 8: return calib_impl<T, D, 8>(a, N, MB, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_calibrate(const CacheView& c, const SeqView& s, const CalibParams& p, hipStream_t st) {
  CalibArgs a;
  a.c = c;
  a.s = s;
  a.q = p.q;
  a.Lq = kBlock * s.MB;
  a.HQ = p.HQ;
  a.B = p.num_bins;
  a.w = p.w;
  a.b = p.b;
  a.rho = p.rho;
  a.lo = p.lo;
  a.hi = p.hi;
  a.bscale = (float)((double)p.num_bins / ((double)p.hi - (double)p.lo));
  a.hist = (unsigned long long*)p.hist;
  a.above = (unsigned long long*)p.above;
  a.total = (unsigned long long*)p.total;
  a.c_out = p.c_out;
  a.err = p.err;
  const int G = p.HQ / c.HKV;
  const int64_t nz = (int64_t)p.HQ * p.num_bins;
  const int zgrid = (int)((nz + 255) / 256 > 1024 ? 1024 : (nz + 255) / 256);
  hipLaunchKernelGGL(k_calib_zero, dim3(zgrid > 0 ? zgrid : 1), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (c.kv_dtype == 1) e = c.D == 128 ? calib_g<Bf16, 128>(a, G, s.N, s.MB, st) : calib_g<Bf16, 64>(a, G, s.N, s.MB, st);
  else e = c.D == 128 ? calib_g<F32, 128>(a, G, s.N, s.MB, st) : calib_g<F32, 64>(a, G, s.N, s.MB, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_calib_search, dim3(p.HQ), dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace eta
