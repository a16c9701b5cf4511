// Causal prompt pass: the gated attention rule at every prompt position, with
// the blocks' decode records built in the same launch.
//
// "Elastic Threshold Attention" (paperpeel.com/paper/2609.20888), Sections 2.2
// and 2.3 (the fused causal forward over query blocks and key blocks), E.1,
// E.3 and G.1 (the gate S~ = S sigmoid(beta (S - tau~)) inside the softmax),
// and 4.8 (records built while the prompt is processed). For position t of a
// sequence and query head h, over the keys s <= t:
//   S = q_t . k_s / sqrt(d),  S~ = S sigmoid(beta (S - tau~_t)),
//   o_t = sum_s exp(S~) v_s / sum_s exp(S~),
// tau~_t = w_h . q_t + b_h - a (learned) or c_h - a (calibrated). Nothing is
// pruned in the prompt pass; the gate alone filters.
//
// One workgroup of eight wavefronts takes one (sequence, KV head) and QT
// consecutive positions; wavefront w takes head w % G of the group and the 32
// positions (w / G) * 32 .. + 31. The workgroup walks the key blocks of 64
// tokens up to the diagonal; K (row-major) and V (transposed) of the next
// block stream into the other half of a double-buffered LDS area while the
// current one is used. Both products run on the matrix cores
// (v_mfma_f32_32x32x16_bf16, float32 accumulation):
//   S^T = K Q^T  (A = 32 keys x 16 dims from LDS, B = the wavefront's 32
//                 queries, held in registers for the whole pass): each lane
//                 ends with one query and 16 of the 32 keys, so the gate and
//                 the softmax are per-lane, with one exchange between the two
//                 half-waves for the row maximum and sum.
//   O^T += V^T P^T (A = 32 dims x 16 keys of V^T from LDS, B = the weights
//                 straight from the lane's registers): the keys of a step are
//                 taken in the order the lanes hold them, and V^T is read in the
//                 same order, so P needs no data movement.
// P enters the matrix cores as one float16 term (11 significant bits) against
// V converted to float16, which is exact when every value of V in the prompts
// lies within +-65280 (a range check over V before the pass decides, for the
// whole call); otherwise as two bfloat16 terms (its leading 8 mantissa bits
// and the rounded remainder, about 2^-16 relative) against V in bfloat16. One
// bfloat16 term would perturb outputs by a few 1e-3. The running maximum is
// only moved when a weight would exceed 2^8 (float32 and both forms are exact
// well beyond that), which spares most rescales of the accumulators.
//
// Records: the workgroup holding a complete block's last position builds the
// block's centroid, radius (and deviation, if the cache has a deviation
// buffer) with the same device function as the bulk builder, so the bits are
// the same as eta_build_block_summaries'.
#include "eta_records.h"

namespace eta {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Eight wavefronts per workgroup: with two per SIMD, K and V of a block are
// read from memory once for 8 x 32 (query, head) rows.
constexpr int kPfWaves = 8;
constexpr float kRescaleLog2 = 8.0f;  // weights stay <= 2^8 between rescales

struct PrefillArgs {
  CacheView c;
  SeqView s;
  const uint16_t* q;  // [N][Lq][HQ][D] bfloat16 bits
  int Lq, HQ, tau_mode;
  const float* w;  // [HQ][D] (learned)
  const float* b;  // [HQ] bias (learned) or constant (calibrated)
  float a, beta;
  float* out;  // [N][Lq][HQ][D]
  int* err;    // [1]
};

// err bit 0: invalid length or page id (reported); bit 1, internal: some V
// element of a sequence's prompt lies outside float16's exact range, so the
// two-term bfloat16 products run (cleared again by k_prefill_fin)
constexpr int kErrData = 1, kErrWideV = 2;

__global__ void k_prefill_zero(int* err) { *err = 0; }
__global__ void k_prefill_fin(int* err) {
  if (*err & kErrWideV) atomicAnd(err, kErrData);
}

// bfloat16 pair (two halves of w) -> float16 pair, toward zero: exact for
// every bfloat16 value the range test below admits (magnitudes up to 65280;
// below 2^-14 float16 keeps 2^-24 steps, far under the outputs' error bar)
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(bf16_lo(w), bf16_hi(w)));
}
// nonzero if either bfloat16 half of w is not finite or larger in magnitude
// than 65280, the largest bfloat16 value below float16's largest finite one
__device__ __forceinline__ uint32_t f16_unsafe(uint32_t w) {
  return ((w & 0x7fffu) > 0x477fu) | (((w >> 16) & 0x7fffu) > 0x477fu);
}

// One workgroup per (sequence, KV head, key block below the length): sets
// kErrWideV if a value of V in the prompt is not exact in float16.
template <int D>
__global__ __launch_bounds__(256) void k_prefill_vcheck(CacheView c, SeqView s, int* err) {
  const int j = blockIdx.x, n = blockIdx.y / c.HKV, g = blockIdx.y % c.HKV;
  const int T = s.lens[n];
  if (T < 1 || T > kBlock * s.MB || j * kBlock >= T) return;
  const int page = s.bt[(int64_t)n * s.MB + j];
  if (page < 0 || page >= c.num_pages) return;  // reported by the prompt pass
  const uint16_t* vt = (const uint16_t*)c.v + ((int64_t)page * c.HKV + g) * (kBlock * D);
  const int rows = min(kBlock, T - j * kBlock);
  uint32_t bad = 0;
  for (int ch = threadIdx.x; ch < rows * D / 8; ch += 256) {
    const uint4 v = *(const uint4*)(vt + ch * 8);
    bad |= f16_unsafe(v.x) | f16_unsafe(v.y) | f16_unsafe(v.z) | f16_unsafe(v.w);
  }
  if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(err, kErrWideV);
}

__device__ __forceinline__ uint32_t pack_f16_rne(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, _Float16 __attribute__((ext_vector_type(2)))));
}

__device__ __forceinline__ uint32_t pack_bf16_rne(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

template <int D>
struct PfLds {
  static constexpr int KS = D + 8;     // K row stride (elements): rows start 4 banks apart
  static constexpr int VS = 64 + 4;    // V^T row stride (elements): 8-byte reads of 32 rows hit 64 banks
  static constexpr int KE = 64 * KS;   // elements of one K buffer
  static constexpr int VE = D * VS;    // elements of one V^T buffer
  static constexpr int BUF = KE + VE;
};

template <int D, int NTH>
struct PfTileRegs {
  static constexpr int CPR = D / 8;              // 16-byte chunks per row
  static constexpr int KC = 64 * CPR / NTH;      // K chunks per thread
  static constexpr int VC = (32 * CPR + NTH - 1) / NTH;  // V (key pair, chunk) items per thread
  uint4 k[KC];
  uint4 v0[VC], v1[VC];  // rows 2 kp and 2 kp + 1 of V, 8 dims from 8 dc
};

// Loads key block kt of (n, g) into registers; rows at or past `rem` (the
// sequence's end inside this block) read as zeros, as does a block whose page
// id is out of range.
template <int D, int NTH>
__device__ __forceinline__ void pf_load(PfTileRegs<D, NTH>& R, const PrefillArgs& A, int page, bool valid, int rem,
                                        int g, int tid) {
  using TR = PfTileRegs<D, NTH>;
  constexpr int CPR = TR::CPR;
  const uint16_t* kt = (const uint16_t*)A.c.k + ((int64_t)page * A.c.HKV + g) * (kBlock * D);
  const uint16_t* vt = (const uint16_t*)A.c.v + ((int64_t)page * A.c.HKV + g) * (kBlock * D);
#pragma unroll
  for (int i = 0; i < TR::KC; ++i) {
    const int cidx = tid + i * NTH, row = cidx / CPR, col = (cidx % CPR) * 8;
    R.k[i] = (valid && row < rem) ? *(const uint4*)(kt + row * D + col) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < TR::VC; ++i) {
    const int it = tid + i * NTH, kp = it / CPR, dc = it % CPR;
    const bool own = it < 32 * CPR;
    R.v0[i] = (own && valid && 2 * kp < rem) ? *(const uint4*)(vt + (2 * kp) * D + dc * 8) : make_uint4(0, 0, 0, 0);
    R.v1[i] = (own && valid && 2 * kp + 1 < rem) ? *(const uint4*)(vt + (2 * kp + 1) * D + dc * 8)
                                                 : make_uint4(0, 0, 0, 0);
  }
}

// V^T goes to LDS as bfloat16 or, with F16, converted to float16.
template <int D, int NTH, bool F16>
__device__ __forceinline__ void pf_store(const PfTileRegs<D, NTH>& R, uint16_t* buf, int tid) {
  using L = PfLds<D>;
  using TR = PfTileRegs<D, NTH>;
  constexpr int CPR = TR::CPR;
  uint16_t* kl = buf;
  uint16_t* vl = buf + L::KE;
#pragma unroll
  for (int i = 0; i < TR::KC; ++i) {
    const int cidx = tid + i * NTH, row = cidx / CPR, col = (cidx % CPR) * 8;
    *(uint4*)(kl + row * L::KS + col) = R.k[i];
  }
#pragma unroll
  for (int i = 0; i < TR::VC; ++i) {
    const int it = tid + i * NTH, kp = it / CPR, dc = it % CPR;
    if (it < 32 * CPR) {
      const uint32_t a[4] = {R.v0[i].x, R.v0[i].y, R.v0[i].z, R.v0[i].w};
      const uint32_t b[4] = {R.v1[i].x, R.v1[i].y, R.v1[i].z, R.v1[i].w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        // dims 8 dc + 2u (low halves) and 8 dc + 2u + 1 (high halves): keys 2 kp, 2 kp + 1
        const uint32_t even = (a[u] & 0xffffu) | (b[u] << 16);
        const uint32_t odd = (a[u] >> 16) | (b[u] & 0xffff0000u);
        *(uint32_t*)(vl + (8 * dc + 2 * u) * L::VS + 2 * kp) = F16 ? bf16x2_to_f16x2(even) : even;
        *(uint32_t*)(vl + (8 * dc + 2 * u + 1) * L::VS + 2 * kp) = F16 ? bf16x2_to_f16x2(odd) : odd;
      }
    }
  }
}

// S^T of both 32-key halves of a block (keys 32 t + 8 i + 4 hh + j in acc
// element 4 i + j of s[t], query qi), then the gate in place,
// S -> S sigmoid(beta (S - tau~)) in the units of the accumulators, with keys
// past the lane's position set to -inf when MASK (lim: the largest key offset
// 32 t + 8 i + j the lane may see). The gate of the first half is issued
// between the products of the second half, so that vector work runs while the
// matrix cores are busy. Returns the lane's maximum.
template <bool MASK, int KSTEPS, int KSTR>
__device__ __forceinline__ float pf_scores_gated(f32x16_t (&s)[2], const uint16_t* kl, const uint4 (&qr)[KSTEPS],
                                                 int qi, int hh, float kb, float tb, int lim) {
  constexpr int PER = 16 / KSTEPS;  // first-half elements gated per product of the second half
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) s[t][e] = 0.f;
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    const bf16x8_t av = *(const bf16x8_t*)(kl + qi * KSTR + 16 * ks + 8 * hh);
    s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8_t, qr[ks]), s[0], 0, 0, 0);
  }
  float mx = -__builtin_inff();
  const auto gate = [&](int t, int e) {
    const float v = s[t][e];
    const float ex = __builtin_amdgcn_exp2f(fmaf(kb, v, tb));
    float y = v * __builtin_amdgcn_rcpf(1.0f + ex);
    if (MASK && 32 * t + 8 * (e >> 2) + (e & 3) > lim) y = -__builtin_inff();
    s[t][e] = y;
    mx = fmaxf(mx, y);
  };
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    const bf16x8_t av = *(const bf16x8_t*)(kl + (32 + qi) * KSTR + 16 * ks + 8 * hh);
    s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8_t, qr[ks]), s[1], 0, 0, 0);
#pragma unroll
    for (int u = 0; u < PER; ++u) gate(0, PER * ks + u);
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) gate(1, e);
  return mx;
}

// F16: the products O^T += V^T P^T take one float16 term (V exact in
// float16: the range check found no wider value); otherwise two bfloat16
// terms. Both instantiations are launched; the one that does not match the
// check's flag returns at once.
template <int D, int G, int NW, bool F16>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_prefill(PrefillArgs A) {
  if (F16 == ((*A.err & kErrWideV) != 0)) return;
  using L = PfLds<D>;
  constexpr int NTH = 64 * NW;
  constexpr int HW = G < NW ? G : NW;    // heads per workgroup
  constexpr int HC = G / HW;             // workgroups per (sequence, KV head, tile)
  constexpr int QT = 32 * (NW / HW);     // positions per workgroup
  constexpr int KSTEPS = D / 16;         // k-steps of S^T = K Q^T
  constexpr int DT = D / 32;             // 32-dim tiles of O^T
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * L::BUF];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int HKV = A.c.HKV, MB = A.s.MB, HQ = A.HQ, Lq = A.Lq;
  const int hc = blockIdx.y % HC, ng = blockIdx.y / HC;
  const int n = ng / HKV, g = ng % HKV;
  const int nqt = gridDim.x;
  const int P0 = (nqt - 1 - (int)blockIdx.x) * QT;  // longest rows first
  const int hl = hc * HW + wave % HW, hq = g * G + hl;
  const int pw0 = P0 + (wave / HW) * 32;  // first position of this wavefront
  const int qi = lane & 31, hh = lane >> 5;
  const int p = pw0 + qi;                // this lane's position
  int T = A.s.lens[n];
  if (T < 0 || T > kBlock * MB) {  // invalid length: flagged, every row NaN
    if (tid == 0) atomicOr(A.err, kErrData);
    T = 0;
  }
  const int64_t orow = (((int64_t)n * Lq + p) * HQ + hq) * D;

  if (P0 >= T) {  // no valid position in this tile
    if (p < Lq) {
      const float4 nan4 = make_float4(__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""));
#pragma unroll
      for (int m = 0; m < DT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) *(float4*)(A.out + orow + 32 * m + 8 * i + 4 * hh) = nan4;
    }
    return;
  }

  // ---- queries (B operand of S^T = K Q^T) and thresholds
  uint4 qr[KSTEPS];
  float dot = 0.f;
  const bool learned = A.tau_mode == 0;
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    const int d0 = 16 * ks + 8 * hh;
    qr[ks] = p < T ? *(const uint4*)(A.q + orow + d0) : make_uint4(0, 0, 0, 0);
    if (learned) {
      const float4 w0 = *(const float4*)(A.w + (int64_t)hq * D + d0);
      const float4 w1 = *(const float4*)(A.w + (int64_t)hq * D + d0 + 4);
      const uint32_t qw[4] = {qr[ks].x, qr[ks].y, qr[ks].z, qr[ks].w};
      dot = fmaf(w0.x, bf16_lo(qw[0]), dot);
      dot = fmaf(w0.y, bf16_hi(qw[0]), dot);
      dot = fmaf(w0.z, bf16_lo(qw[1]), dot);
      dot = fmaf(w0.w, bf16_hi(qw[1]), dot);
      dot = fmaf(w1.x, bf16_lo(qw[2]), dot);
      dot = fmaf(w1.y, bf16_hi(qw[2]), dot);
      dot = fmaf(w1.z, bf16_lo(qw[3]), dot);
      dot = fmaf(w1.w, bf16_hi(qw[3]), dot);
    }
  }
  dot += __shfl_xor(dot, 32, 64);
  const float bh = A.b[hq];
  const float tau = learned ? (dot + bh) - A.a : bh - A.a;
  const float scale = 1.0f / sqrtf((float)D);
  const float c2 = scale * kLog2e;                 // logits to log2 units
  const float kb = -A.beta * kLog2e * scale;       // exp2 argument of the gate: kb * acc + tb
  const float tb = A.beta * kLog2e * tau;
  const float thr = kRescaleLog2 / c2;             // headroom of the running maximum

  f32x16_t o[DT];
#pragma unroll
  for (int m = 0; m < DT; ++m)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[m][e] = 0.f;
  float mrun = -__builtin_inff(), lsum = 0.f;

  // ---- key blocks 0 .. last
  const int last = (min(P0 + QT, T) - 1) / kBlock;
  const int wlast = (min(pw0 + 31, T - 1)) / kBlock;  // last block this wavefront needs (pw0 < T or none)
  const bool wactive = pw0 < T;
  const int32_t* bt = A.s.bt + (int64_t)n * MB;
  // Two LDS slots: block kt + 1 is written into the other one while block kt
  // is used.
  PfTileRegs<D, NTH> R;
  {
    const int page = bt[0];
    const bool valid = page >= 0 && page < A.c.num_pages;
    if (!valid && tid == 0) atomicOr(A.err, kErrData);
    pf_load<D, NTH>(R, A, valid ? page : 0, valid, T, g, tid);
    pf_store<D, NTH, F16>(R, lds, tid);
  }
  __syncthreads();
  for (int kt = 0; kt <= last; ++kt) {
    const bool has_next = kt < last;
    if (has_next) {
      const int page = bt[kt + 1];
      const bool valid = page >= 0 && page < A.c.num_pages;
      if (!valid && tid == 0) atomicOr(A.err, kErrData);
      pf_load<D, NTH>(R, A, valid ? page : 0, valid, T - (kt + 1) * kBlock, g, tid);
    }
    const uint16_t* kl = lds + (kt & 1) * L::BUF;
    const uint16_t* vl = kl + L::KE;
    if (wactive && kt <= wlast) {
      // ---- S^T for keys 32 t + 8 i + 4 hh + j (acc element 4 i + j), query
      //      qi; gate, causal mask and running maximum
      f32x16_t s[2];
      float mx;
      if (kt * kBlock + kBlock - 1 > pw0)  // the diagonal block: some key may lie after some position
        mx = pf_scores_gated<true, KSTEPS, L::KS>(s, kl, qr, qi, hh, kb, tb, p - kt * kBlock - 4 * hh);
      else
        mx = pf_scores_gated<false, KSTEPS, L::KS>(s, kl, qr, qi, hh, kb, tb, 0);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const bool need = mx > mrun + thr;
      if (__any(need)) {
        const float mnew = need ? mx : mrun;
        const float alpha = need ? (mrun == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(c2 * (mrun - mnew))) : 1.f;
        lsum *= alpha;
#pragma unroll
        for (int m = 0; m < DT; ++m)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[m][e] *= alpha;
        mrun = mnew;
      }
      const float moff = mrun == -__builtin_inff() ? 0.f : -c2 * mrun;
      // ---- weights and O^T += V^T P^T: one float16 term (F16), or two
      //      bfloat16 terms, the leading 8 bits and the rounded remainder
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          uint32_t hb[4], lb[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(c2, s[t][8 * ks + 2 * u], moff));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(c2, s[t][8 * ks + 2 * u + 1], moff));
            lsum += p0 + p1;
            if constexpr (F16) {
              hb[u] = pack_f16_rne(p0, p1);
            } else {
              const uint32_t h0 = __float_as_uint(p0) & 0xffff0000u, h1 = __float_as_uint(p1) & 0xffff0000u;
              hb[u] = (h0 >> 16) | h1;
              lb[u] = pack_bf16_rne(p0 - __uint_as_float(h0), p1 - __uint_as_float(h1));
            }
          }
          const uint4 ph = make_uint4(hb[0], hb[1], hb[2], hb[3]);
          const int k0 = 32 * t + 16 * ks + 4 * hh;  // keys k0 .. k0+3 and k0+8 .. k0+11
#pragma unroll
          for (int m = 0; m < DT; ++m) {
            const uint16_t* vr = vl + (32 * m + qi) * L::VS;
            const uint2 x0 = *(const uint2*)(vr + k0);
            const uint2 x1 = *(const uint2*)(vr + k0 + 8);
            const uint4 va = make_uint4(x0.x, x0.y, x1.x, x1.y);
            if constexpr (F16) {
              o[m] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, va),
                                                            __builtin_bit_cast(f16x8_t, ph), o[m], 0, 0, 0);
            } else {
              const bf16x8_t av = __builtin_bit_cast(bf16x8_t, va);
              o[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8_t, ph), o[m], 0, 0, 0);
              o[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  av, __builtin_bit_cast(bf16x8_t, make_uint4(lb[0], lb[1], lb[2], lb[3])), o[m], 0, 0, 0);
            }
          }
        }
      }
    }
    if (has_next) pf_store<D, NTH, F16>(R, lds + ((kt + 1) & 1) * L::BUF, tid);
    __syncthreads();
  }

  // ---- outputs: O^T element 4 i + j of tile m is dim 32 m + 8 i + 4 hh + j of query qi
  if (p < Lq) {
    const float ltot = lsum + __shfl_xor(lsum, 32, 64);
    const bool ok = p < T;
    const float inv = 1.0f / ltot;
#pragma unroll
    for (int m = 0; m < DT; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float4 r;
        r.x = ok ? o[m][4 * i + 0] * inv : __builtin_nanf("");
        r.y = ok ? o[m][4 * i + 1] * inv : __builtin_nanf("");
        r.z = ok ? o[m][4 * i + 2] * inv : __builtin_nanf("");
        r.w = ok ? o[m][4 * i + 3] * inv : __builtin_nanf("");
        *(float4*)(A.out + orow + 32 * m + 8 * i + 4 * hh) = r;
      }
  }

  // ---- records of the complete blocks whose last position lies in this tile
  const int jb = P0 / kBlock + wave;
  if (hc == 0 && jb * kBlock + kBlock - 1 < P0 + QT && jb * kBlock + kBlock <= T) {
    const int page = bt[jb];
    if (page >= 0 && page < A.c.num_pages) {
      const int64_t rec = (int64_t)page * HKV + g;
      const uint16_t* tile = (const uint16_t*)A.c.k + rec * kBlock * D;
      build_record<Bf16, D>(tile, nullptr, A.c.mu + rec * D, A.c.radius + rec,
                            A.c.sigma ? A.c.sigma + rec * D : nullptr, A.c.kmin ? A.c.kmin + rec * D : nullptr,
                            A.c.kmax ? A.c.kmax + rec * D : nullptr, A.c.mu8 ? A.c.mu8 + rec * D : nullptr,
                            A.c.mu8 ? A.c.radius8 + rec : nullptr, A.c.mu8_fmt, lane);
    }
  }
  // records of the other screen blocks (16, 32 or 128 tokens) that end in this
  // tile: blocks js with P0 <= js rows + rows - 1 < P0 + QT
  if (hc == 0 && A.c.sub_rows) {
    const int rows = A.c.sub_rows, sb = sub_slots(rows);
    const int js_end = (P0 + QT) / rows;  // one past the last block ending in the tile
    for (int js = P0 / rows + wave; js < js_end; js += kPfWaves) {
      if (js * rows + rows > T) break;
      const int p0 = (int)((int64_t)js * rows / kBlock);  // table entry of the block's first page
      const int page = bt[p0];
      if (page < 0 || page >= A.c.num_pages) continue;
      const int64_t srec = ((int64_t)page * HKV + g) * sb + js % sb;
      const uint16_t* tile = (const uint16_t*)A.c.k + (((int64_t)page * HKV + g) * kBlock + (js % sb) * (kBlock / sb)) * D;
      if (rows == 16) {
        build_record<Bf16, D, 16>(tile, nullptr, A.c.mu_sub + srec * D, A.c.radius_sub + srec, nullptr, nullptr,
                                  nullptr, nullptr, nullptr, 0, lane);
      } else if (rows == 32) {
        build_record<Bf16, D, 32>(tile, nullptr, A.c.mu_sub + srec * D, A.c.radius_sub + srec, nullptr, nullptr,
                                  nullptr, nullptr, nullptr, 0, lane);
      } else {
        const int page1 = bt[p0 + 1];  // p0 + 1 < ceil(T / 64): the block is complete
        if (page1 < 0 || page1 >= A.c.num_pages) continue;
        build_record<Bf16, D, 128>(tile, nullptr, A.c.mu_sub + srec * D, A.c.radius_sub + srec, nullptr, nullptr,
                                   nullptr, nullptr, nullptr, 0, lane,
                                   (const uint16_t*)A.c.k + ((int64_t)page1 * HKV + g) * kBlock * D);
      }
    }
  }
}

// float32 caches: the same rule in float32 on the vector units. One
// workgroup of 256 threads takes one (sequence, query head) and 64 positions
// (one key block's worth, longest rows first); position P0 + i is handled by
// the four lanes 4 i .. 4 i + 3, lane part c owning dims c D/4 .. + D/4 - 1 of
// the query and of the output. Each key block of 64 tokens goes to LDS (K and
// V, float32); a position scores the keys up to it (keys after it are skipped,
// not weighted by 0, so a non-finite V reaches exactly the positions at or
// after its key), then the block's weights against the running maximum and
// the values. The workgroup of the group's first head that holds a complete
// block builds its records (the bulk builder's device function).
template <int D, int G>
__global__ __launch_bounds__(256) void k_prefill_f32(PrefillArgs A) {
  constexpr int DP = D / 4;  // dims per lane
  __shared__ __attribute__((aligned(16))) float ks[kBlock][D];
  __shared__ __attribute__((aligned(16))) float vs[kBlock][D];
  const int tid = threadIdx.x, lane = tid & 63, part = tid & 3, row = tid >> 2;
  const int HKV = A.c.HKV, MB = A.s.MB, HQ = A.HQ, Lq = A.Lq;
  const int n = blockIdx.y / HQ, hq = blockIdx.y % HQ, g = hq / G;
  const int P0 = ((int)gridDim.x - 1 - (int)blockIdx.x) * kBlock;
  const int p = P0 + row;
  int T = A.s.lens[n];
  if (T < 0 || T > kBlock * MB) {  // invalid length: flagged, every row NaN
    if (tid == 0) atomicOr(A.err, kErrData);
    T = 0;
  }
  float* orow = A.out + (((int64_t)n * Lq + p) * HQ + hq) * D + part * DP;
  if (P0 >= T) {
#pragma unroll
    for (int i = 0; i < DP; i += 4)
      *(float4*)(orow + i) = make_float4(__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""));
    return;
  }
  const bool pok = p < T;
  const float* qrow = (const float*)A.q + (((int64_t)n * Lq + p) * HQ + hq) * D + part * DP;
  float q[DP];
#pragma unroll
  for (int i = 0; i < DP; i += 4) {
    const float4 v = pok ? *(const float4*)(qrow + i) : make_float4(0.f, 0.f, 0.f, 0.f);
    q[i] = v.x; q[i + 1] = v.y; q[i + 2] = v.z; q[i + 3] = v.w;
  }
  float tau;
  if (A.tau_mode == 0) {
    const float* wr = A.w + (int64_t)hq * D + part * DP;
    float dw = 0.f;
#pragma unroll
    for (int i = 0; i < DP; ++i) dw = fmaf(wr[i], q[i], dw);
    dw += __shfl_xor(dw, 1, 64);
    dw += __shfl_xor(dw, 2, 64);
    tau = (dw + A.b[hq]) - A.a;
  } else {
    tau = A.b[hq] - A.a;
  }
  const float scale = 1.0f / sqrtf((float)D);
  float acc[DP];
#pragma unroll
  for (int i = 0; i < DP; ++i) acc[i] = 0.f;
  float m = -__builtin_inff(), l = 0.f;
  const int32_t* bt = A.s.bt + (int64_t)n * MB;
  const int last = (min(P0 + kBlock, T) - 1) / kBlock;  // the tile's own block
  for (int kt = 0; kt <= last; ++kt) {
    const int page = bt[kt];
    const bool valid = page >= 0 && page < A.c.num_pages;
    if (!valid && tid == 0) atomicOr(A.err, kErrData);
    const int rem = T - kt * kBlock;  // rows of the block inside the sequence
    const float* kt_p = (const float*)A.c.k + ((int64_t)(valid ? page : 0) * HKV + g) * (kBlock * D);
    const float* vt_p = (const float*)A.c.v + ((int64_t)(valid ? page : 0) * HKV + g) * (kBlock * D);
    __syncthreads();  // the previous block's reads are done
    for (int c = tid; c < kBlock * D / 4; c += 256) {
      const int r = c / (D / 4);
      const bool ok = valid && r < rem;
      *(float4*)(&ks[0][0] + 4 * c) = ok ? *(const float4*)(kt_p + 4 * c) : make_float4(0.f, 0.f, 0.f, 0.f);
      *(float4*)(&vs[0][0] + 4 * c) = ok ? *(const float4*)(vt_p + 4 * c) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();
    // keys kt 64 + s with s <= lim are at or before the position
    const int lim = pok ? min(kBlock - 1, p - kt * kBlock) : -1;
    float sc[kBlock];
    float mb = -__builtin_inff();
#pragma unroll
    for (int s2 = 0; s2 < kBlock; ++s2) {
      float d = 0.f;
#pragma unroll
      for (int i = 0; i < DP; ++i) d = fmaf(q[i], ks[s2][part * DP + i], d);
      d += __shfl_xor(d, 1, 64);
      d += __shfl_xor(d, 2, 64);
      const float S = d * scale;
      const float sg = __builtin_amdgcn_rcpf(1.0f + fast_exp(-A.beta * (S - tau)));
      const float y = S * sg;
      sc[s2] = y;
      if (s2 <= lim) mb = fmaxf(mb, y);
    }
    if (lim < 0) continue;
    const float mnew = fmaxf(m, mb);
    const float alpha = m == -__builtin_inff() ? 0.f : fast_exp(m - mnew);
    l *= alpha;
#pragma unroll
    for (int i = 0; i < DP; ++i) acc[i] *= alpha;
    m = mnew;
#pragma unroll
    for (int s2 = 0; s2 < kBlock; ++s2) {
      if (s2 > lim) continue;
      const float w = fast_exp(sc[s2] - m);
      l += w;
#pragma unroll
      for (int i = 0; i < DP; ++i) acc[i] = fmaf(w, vs[s2][part * DP + i], acc[i]);
    }
  }
  if (p < Lq) {
    const float inv = 1.0f / l;
#pragma unroll
    for (int i = 0; i < DP; i += 4) {
      float4 r4;
      r4.x = pok ? acc[i] * inv : __builtin_nanf("");
      r4.y = pok ? acc[i + 1] * inv : __builtin_nanf("");
      r4.z = pok ? acc[i + 2] * inv : __builtin_nanf("");
      r4.w = pok ? acc[i + 3] * inv : __builtin_nanf("");
      *(float4*)(orow + i) = r4;
    }
  }
  // ---- records of the tile's block (the group's first head only)
  if (hq % G != 0) return;
  const int wave = tid >> 6;
  const int jb = P0 / kBlock;
  if (wave == 0 && jb * kBlock + kBlock <= T) {
    const int page = bt[jb];
    if (page >= 0 && page < A.c.num_pages) {
      const int64_t rec = (int64_t)page * HKV + g;
      const float* tile = (const float*)A.c.k + rec * kBlock * D;
      build_record<F32, D>(tile, nullptr, A.c.mu + rec * D, A.c.radius + rec,
                           A.c.sigma ? A.c.sigma + rec * D : nullptr, A.c.kmin ? A.c.kmin + rec * D : nullptr,
                           A.c.kmax ? A.c.kmax + rec * D : nullptr, A.c.mu8 ? A.c.mu8 + rec * D : nullptr,
                           A.c.mu8 ? A.c.radius8 + rec : nullptr, A.c.mu8_fmt, lane);
    }
  }
  // records of the other screen blocks (16, 32 or 128 tokens) that end in this
  // tile, one wavefront each
  if (A.c.sub_rows) {
    const int rows = A.c.sub_rows, sb = sub_slots(rows);
    const int js_end = (P0 + kBlock) / rows;  // one past the last block ending in the tile
    for (int js = P0 / rows + wave; js < js_end; js += 4) {
      if (js * rows + rows > T) break;
      const int p0 = (int)((int64_t)js * rows / kBlock);  // table entry of the block's first page
      const int page = bt[p0];
      if (page < 0 || page >= A.c.num_pages) continue;
      const int64_t srec = ((int64_t)page * HKV + g) * sb + js % sb;
      const float* tile = (const float*)A.c.k + (((int64_t)page * HKV + g) * kBlock + (js % sb) * (kBlock / sb)) * D;
      if (rows == 16) {
        build_record<F32, D, 16>(tile, nullptr, A.c.mu_sub + srec * D, A.c.radius_sub + srec, nullptr, nullptr,
                                 nullptr, nullptr, nullptr, 0, lane);
      } else if (rows == 32) {
        build_record<F32, D, 32>(tile, nullptr, A.c.mu_sub + srec * D, A.c.radius_sub + srec, nullptr, nullptr,
                                 nullptr, nullptr, nullptr, 0, lane);
      } else {
        const int page1 = bt[p0 + 1];  // p0 + 1 < ceil(T / 64): the block is complete
        if (page1 < 0 || page1 >= A.c.num_pages) continue;
        build_record<F32, D, 128>(tile, nullptr, A.c.mu_sub + srec * D, A.c.radius_sub + srec, nullptr, nullptr,
                                  nullptr, nullptr, nullptr, 0, lane,
                                  (const float*)A.c.k + ((int64_t)page1 * HKV + g) * kBlock * D);
      }
    }
  }
}

template <int D>
hipError_t pf_f32_g(const PrefillArgs& a, int G, hipStream_t st) {
  const dim3 grid((a.Lq + kBlock - 1) / kBlock, a.s.N * a.HQ);
  switch (G) {
    case 1: hipLaunchKernelGGL((k_prefill_f32<D, 1>), grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((k_prefill_f32<D, 2>), grid, dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL((k_prefill_f32<D, 4>), grid, dim3(256), 0, st, a); break;
    case 8: hipLaunchKernelGGL((k_prefill_f32<D, 8>), grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D, int G>
hipError_t pf_launch(const PrefillArgs& a, hipStream_t st) {
  constexpr int NW = kPfWaves;
  constexpr int HW = G < NW ? G : NW;
  constexpr int QT = 32 * (NW / HW);
  const int nqt = (a.Lq + QT - 1) / QT;
  const dim3 grid(nqt, a.s.N * a.c.HKV * (G / HW));
  hipLaunchKernelGGL((k_prefill<D, G, NW, true>), grid, dim3(64 * NW), 0, st, a);
  hipLaunchKernelGGL((k_prefill<D, G, NW, false>), grid, dim3(64 * NW), 0, st, a);
  return hipGetLastError();
}

template <int D>
hipError_t pf_g(const PrefillArgs& a, int G, hipStream_t st) {
  switch (G) {
    case 1: return pf_launch<D, 1>(a, st);
    case 2: return pf_launch<D, 2>(a, st);
    case 4: return pf_launch<D, 4>(a, st);
    case 8: return pf_launch<D, 8>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_prefill(const CacheView& c, const SeqView& s, const PrefillParams& p, hipStream_t st) {
  PrefillArgs a;
  a.c = c;
  a.s = s;
  a.q = (const uint16_t*)p.q;
  a.Lq = kBlock * s.MB;
  a.HQ = p.HQ;
  a.tau_mode = p.tau_mode;
  a.w = p.w;
  a.b = p.b;
  a.a = p.a;
  a.beta = p.beta;
  a.out = p.out;
  a.err = p.err;
  hipLaunchKernelGGL(k_prefill_zero, dim3(1), dim3(1), 0, st, p.err);
  if (c.kv_dtype != 1) {  // float32 cache
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int G = p.HQ / c.HKV;
    return c.D == 128 ? pf_f32_g<128>(a, G, st) : pf_f32_g<64>(a, G, st);
  }
  const dim3 cgrid(s.MB, s.N * c.HKV);
  if (c.D == 128) hipLaunchKernelGGL((k_prefill_vcheck<128>), cgrid, dim3(256), 0, st, c, s, p.err);
  else hipLaunchKernelGGL((k_prefill_vcheck<64>), cgrid, dim3(256), 0, st, c, s, p.err);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int G = p.HQ / c.HKV;
  e = c.D == 128 ? pf_g<128>(a, G, st) : pf_g<64>(a, G, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_prefill_fin, dim3(1), dim3(1), 0, st, p.err);
  return hipGetLastError();
}

}  // namespace eta
