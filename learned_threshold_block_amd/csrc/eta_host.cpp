// Host side of the C ABI declared in include/eta.h: argument validation,
// workspace layout, launch geometry and statistics read-back.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "eta.h"
#include "eta_internal.h"

namespace eta {

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

size_t workspace_layout(const Dims& d, void* base, Ws* ws) {
  size_t off = 0;
  char* b = static_cast<char*>(base);
  auto take = [&](size_t bytes) -> void* {
    off = align_up(off, 256);
    void* p = b ? b + off : nullptr;
    off += bytes;
    return p;
  };
  const size_t S = (size_t)d.S, NT = (size_t)d.NT, G = (size_t)d.G;
  const size_t nq = (size_t)d.N * d.HQ;
  const size_t pieces = (size_t)kMaxAttendWgs + S;
  Ws w;
  w.glob = (int32_t*)take(sizeof(int32_t) * kGlobCount);
  // the screen's results, in one block that the one-launch decode of short
  // segments repeats once per workgroup of a segment (private copies)
  off = align_up(off, 256);
  const size_t scr0 = off;
  w.tau = (float*)take(sizeof(float) * nq);
  w.tile_cnt = (int32_t*)take(sizeof(int32_t) * S * (NT + 1));
  w.tile_ent = (int2*)take(sizeof(int2) * S * (NT + 1) * kTile);
  w.tile_sub = (uint32_t*)take(d.SB > 1 ? sizeof(uint32_t) * S * (NT + 1) * kTile : 0);
  w.tile_off = (int32_t*)take(sizeof(int32_t) * S * (NT + 2));
  w.tile_hcnt = (int32_t*)take(sizeof(int32_t) * S * NT * G);
  w.tile_bits = (uint64_t*)take(sizeof(uint64_t) * S * G * NT);
  w.tile_umax = (float*)take(sizeof(float) * S * NT * G);
  w.tile_uarg = (int32_t*)take(sizeof(int32_t) * S * NT * G);
  w.tile_err = (int32_t*)take(sizeof(int32_t) * S * NT);
  w.seg_U = (int32_t*)take(sizeof(int32_t) * S);
  w.seg_ub = (int32_t*)take(sizeof(int32_t) * S);
  w.seg_ntn = (int32_t*)take(sizeof(int32_t) * S);
  w.seg_err = (int32_t*)take(sizeof(int32_t) * S);
  w.st_head = (int32_t*)take(sizeof(int32_t) * nq);
  w.st_tokens = (int64_t*)take(sizeof(int64_t) * nq);
  w.st_rescued = (int32_t*)take(sizeof(int32_t) * nq);
  off = align_up(off, 256);
  w.scr_stride = (int64_t)(off - scr0);
  w.scr_copies = (d.NT <= kFusedTiles && S < (size_t)kFusedMaxWgs) ? (int)(kFusedMaxWgs / S) - 1 : 0;
  off += (size_t)w.scr_copies * (size_t)w.scr_stride;
  w.seg_done = (uint64_t*)take(sizeof(uint64_t) * S);
  w.fused_done = (uint64_t*)take(sizeof(uint64_t) * S * kArrivalStride);
  w.rng_stat = (int32_t*)take(sizeof(int32_t) * 2 * kMaxAttendWgs);
  w.xcd_w = (int32_t*)take(sizeof(int32_t) * kXcdClasses);
  w.part_ml = (float*)take(sizeof(float) * pieces * G * 2);
  w.part_acc = (float*)take(sizeof(float) * pieces * G * (size_t)d.D);
  if (ws) *ws = w;
  return align_up(off, 256);
}

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

eta_status check_cache(const eta_cache* c) {
  if (!c) return ETA_ERR_INVALID_ARGUMENT;
  if (c->kv_dtype != ETA_F32 && c->kv_dtype != ETA_BF16) return ETA_ERR_INVALID_ARGUMENT;
  if (c->num_kv_heads < 1 || c->num_pages < 1 || c->head_dim < 1 || c->block_size < 1)
    return ETA_ERR_INVALID_ARGUMENT;
  if (!c->k_pages || !c->v_pages || !c->mu || !c->radius) return ETA_ERR_INVALID_ARGUMENT;
  if (!aligned(c->k_pages, 16) || !aligned(c->v_pages, 16) || !aligned(c->mu, 16) ||
      !aligned(c->radius, 4) || !aligned(c->sigma, 16) || !aligned(c->kmin, 16) || !aligned(c->kmax, 16))
    return ETA_ERR_INVALID_ARGUMENT;
  if ((c->kmin == nullptr) != (c->kmax == nullptr)) return ETA_ERR_INVALID_ARGUMENT;
  if ((c->mu8 == nullptr) != (c->radius8 == nullptr) || !aligned(c->mu8, 16) || !aligned(c->radius8, 4))
    return ETA_ERR_INVALID_ARGUMENT;
  if (c->mu8 && c->mu8_format != ETA_FP8_E4M3 && c->mu8_format != ETA_FP8_E5M2) return ETA_ERR_INVALID_ARGUMENT;
  if ((c->mu_sub == nullptr) != (c->radius_sub == nullptr) || !aligned(c->mu_sub, 16) || !aligned(c->radius_sub, 4))
    return ETA_ERR_INVALID_ARGUMENT;
  if (c->mu_sub && c->sub_block != 16 && c->sub_block != 32 && c->sub_block != 2 * kBlock)
    return ETA_ERR_INVALID_ARGUMENT;
  if (c->head_dim != 64 && c->head_dim != 128) return ETA_ERR_UNSUPPORTED;
  if (c->block_size != kBlock) return ETA_ERR_UNSUPPORTED;
  if ((int64_t)c->num_pages * c->num_kv_heads > (int64_t)1 << 31) return ETA_ERR_UNSUPPORTED;
  return ETA_OK;
}

eta_status check_seqs(const eta_seqs* s) {
  if (!s || s->num_seqs < 1 || s->max_blocks_per_seq < 1) return ETA_ERR_INVALID_ARGUMENT;
  if (!s->seq_lens || !s->block_table) return ETA_ERR_INVALID_ARGUMENT;
  if (!aligned(s->seq_lens, 4) || !aligned(s->block_table, 4)) return ETA_ERR_INVALID_ARGUMENT;
  if (s->max_blocks_per_seq > kMaxBlocksPerSeq) return ETA_ERR_UNSUPPORTED;
  return ETA_OK;
}

CacheView view_of(const eta_cache* c) {
  CacheView v;
  v.kv_dtype = c->kv_dtype;
  v.D = c->head_dim;
  v.HKV = c->num_kv_heads;
  v.num_pages = c->num_pages;
  v.k = c->k_pages;
  v.v = c->v_pages;
  v.kw = c->k_pages;
  v.vw = c->v_pages;
  v.mu = c->mu;
  v.radius = c->radius;
  v.sigma = c->sigma;
  v.kmin = c->kmin;
  v.kmax = c->kmax;
  v.mu8 = c->mu8;
  v.radius8 = c->radius8;
  v.mu8_fmt = c->mu8_format == ETA_FP8_E5M2 ? 1 : 0;
  v.sub_rows = c->mu_sub ? c->sub_block : 0;
  v.mu_sub = c->mu_sub;
  v.radius_sub = c->radius_sub;
  return v;
}

SeqView view_of(const eta_seqs* s) {
  SeqView v;
  v.N = s->num_seqs;
  v.MB = s->max_blocks_per_seq;
  v.lens = s->seq_lens;
  v.bt = s->block_table;
  return v;
}

eta_status dims_of(const eta_cache* c, int N, int MB, int HQ, Dims* d, int SB = 1, int PB = 1) {
  if (N < 1 || MB < 1 || HQ < 1) return ETA_ERR_INVALID_ARGUMENT;
  if (HQ % c->num_kv_heads) return ETA_ERR_INVALID_ARGUMENT;
  const int G = HQ / c->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return ETA_ERR_UNSUPPORTED;
  if (MB > kMaxBlocksPerSeq) return ETA_ERR_UNSUPPORTED;
  const int64_t S = (int64_t)N * c->num_kv_heads;
  if (S > (1 << 24) || S * MB >= ((int64_t)1 << 31) / 64) return ETA_ERR_UNSUPPORTED;
  d->N = N;
  d->MB = MB;
  d->HQ = HQ;
  d->HKV = c->num_kv_heads;
  d->D = c->head_dim;
  d->G = G;
  d->S = (int)S;
  // smaller screen blocks multiply the blocks per sequence (the attend kernel
  // keeps a sequence's tile prefix in LDS, sized for kMaxBlocksPerSeq blocks)
  if ((int64_t)MB * SB > kMaxBlocksPerSeq || S * MB * SB >= ((int64_t)1 << 31) / 64) return ETA_ERR_UNSUPPORTED;
  d->SB = SB;
  d->PB = PB;
  d->NT = (MB * SB + kTile - 1) / kTile;
  return ETA_OK;
}

// Screen blocks per page of the cache's smaller-block records (1 if none or
// if they are 128-token blocks).
int sub_blocks(const eta_cache* c) { return c->mu_sub && c->sub_block < kBlock ? kBlock / c->sub_block : 1; }

// attend grid: one resident wave of workgroups over the whole device
std::mutex g_geom_mu;
struct Geom {
  int device = -1;
  int key = -1;
  int wgs = 0;
};
std::vector<Geom> g_geom;

int attend_grid(int kv_dtype, int D, int G) {
  if (const char* env = getenv("ETA_ATTEND_WGS")) {
    const int v = atoi(env);
    if (v >= 1) return v < kMaxAttendWgs ? v : kMaxAttendWgs;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  const int key = kv_dtype * 1000 + D * 10 + G;
  std::lock_guard<std::mutex> lk(g_geom_mu);
  for (const Geom& g : g_geom)
    if (g.device == dev && g.key == key) return g.wgs;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
  int per_cu = attend_wgs_per_cu(kv_dtype, D, G);
  int wgs = cus * per_cu;
  if (wgs > kMaxAttendWgs) wgs = kMaxAttendWgs;
  g_geom.push_back(Geom{dev, key, wgs});
  return wgs;
}

eta_status hip_status(hipError_t e) { return e == hipSuccess ? ETA_OK : ETA_ERR_HIP; }

struct Prepared {
  CacheView c;
  SeqView s;
  DecodeParams p;
  Dims d;
  Ws ws;
};

eta_status prepare(const eta_screen_opts* screen, const eta_cache* cache, const eta_seqs* seqs, const void* q,
                   int num_q_heads, int tau_mode, const float* w, const float* b_or_c, float a, float beta,
                   int lwb, int block_size, float* out, void* workspace, size_t ws_bytes, Prepared* P) {
  eta_status st = check_cache(cache);
  if (st != ETA_OK) return st;
  P->p.bound = 0;
  P->p.z = 0.f;
  if (screen) {
    if (screen->bound != ETA_BOUND_GEOMETRIC && screen->bound != ETA_BOUND_DUAL && screen->bound != ETA_BOUND_QUEST &&
        screen->bound != ETA_BOUND_GEOMETRIC_FP8 && screen->bound != ETA_BOUND_GEOMETRIC_SUB)
      return ETA_ERR_INVALID_ARGUMENT;
    if (screen->bound == ETA_BOUND_DUAL) {
      if (!cache->sigma || !isfinite(screen->z) || !(screen->z >= 0.f)) return ETA_ERR_INVALID_ARGUMENT;
      P->p.bound = 1;
      P->p.z = screen->z;
    }
    if (screen->bound == ETA_BOUND_QUEST) {
      if (!cache->kmin || !cache->kmax) return ETA_ERR_INVALID_ARGUMENT;
      P->p.bound = 2;
    }
    if (screen->bound == ETA_BOUND_GEOMETRIC_FP8) {
      if (!cache->mu8 || !cache->radius8) return ETA_ERR_INVALID_ARGUMENT;
      P->p.bound = 3;
    }
    if (screen->bound == ETA_BOUND_GEOMETRIC_SUB) {
      if (!cache->mu_sub) return ETA_ERR_INVALID_ARGUMENT;
      P->p.bound = cache->sub_block > kBlock ? 5 : 4;
    }
  }
  // the screen reads the records through buffer resources, whose size and
  // offsets are 32-bit: the largest record array it reads must stay below 4 GiB
  {
    const int slots = P->p.bound == 4 ? sub_blocks(cache) : 1;
    const int64_t elem = P->p.bound == 3 ? 1 : 2;  // FP8 codes or float16 values per coordinate
    const int64_t rec_bytes = (int64_t)cache->num_pages * cache->num_kv_heads * slots * cache->head_dim * elem;
    if (rec_bytes >= ((int64_t)1 << 32)) return ETA_ERR_UNSUPPORTED;
  }
  st = check_seqs(seqs);
  if (st != ETA_OK) return st;
  if (block_size != cache->block_size) return ETA_ERR_INVALID_ARGUMENT;
  if (!q || !aligned(q, 16) || !out || !aligned(out, 4) || !b_or_c || !aligned(b_or_c, 4))
    return ETA_ERR_INVALID_ARGUMENT;
  if (tau_mode != ETA_TAU_LEARNED && tau_mode != ETA_TAU_CALIBRATED) return ETA_ERR_INVALID_ARGUMENT;
  if (tau_mode == ETA_TAU_LEARNED && (!w || !aligned(w, 16))) return ETA_ERR_INVALID_ARGUMENT;
  if (!(beta > 0.f) || !isfinite(beta) || !isfinite(a) || lwb < 0) return ETA_ERR_INVALID_ARGUMENT;
  st = dims_of(cache, seqs->num_seqs, seqs->max_blocks_per_seq, num_q_heads, &P->d,
               P->p.bound == 4 ? sub_blocks(cache) : 1, P->p.bound == 5 ? 2 : 1);
  if (st != ETA_OK) return st;
  if (!workspace || !aligned(workspace, 256)) return ETA_ERR_INVALID_ARGUMENT;
  if (ws_bytes < workspace_layout(P->d, nullptr, nullptr)) return ETA_ERR_WORKSPACE_TOO_SMALL;
  workspace_layout(P->d, workspace, &P->ws);
  P->c = view_of(cache);
  P->s = view_of(seqs);
  P->p.q = q;
  P->p.HQ = num_q_heads;
  P->p.G = P->d.G;
  P->p.tau_mode = tau_mode;
  P->p.w = w;
  P->p.b = b_or_c;
  P->p.a = a;
  P->p.beta = beta;
  P->p.scale = (float)(1.0 / sqrt((double)cache->head_dim));
  P->p.lwb = lwb;
  P->p.out = out;
  const char* det = getenv("ETA_DETERMINISTIC");
  P->p.deterministic = (det != nullptr && det[0] == '1') ? 1 : 0;
  // ETA_RANGE_WEIGHTS="w0,...,w7" (each in [512, 2048], 1024 = 1): per-die
  // weights of the attend split instead of the measured ones (for testing)
  P->p.fixed_w[0] = 0;
  if (const char* env = getenv("ETA_RANGE_WEIGHTS")) {
    int v[kXcdClasses];
    int nread = 0;
    const char* c = env;
    while (nread < kXcdClasses && *c) {
      char* end = nullptr;
      const long x = strtol(c, &end, 10);
      if (end == c || x < kWeightOne / 2 || x > 2 * kWeightOne) break;
      v[nread++] = (int)x;
      c = *end == ',' ? end + 1 : end;
    }
    if (nread == kXcdClasses)
      for (int x = 0; x < kXcdClasses; ++x) P->p.fixed_w[x] = v[x];
  }
  return ETA_OK;
}

// Workgroups per segment of the one-launch decode of short segments for these
// sizes, or 0 when the step runs as the screen phase and the attend phase.
// ETA_FUSED=0 in the environment keeps the two phases (for testing).
int short_plan(const Prepared& P) {
  if (P.p.bound != 0 || P.d.SB != 1 || P.d.PB != 1 || P.d.NT > kFusedTiles) return 0;
  if (const char* env = getenv("ETA_FUSED"))
    if (env[0] == '0') return 0;
  if (!decode_short_supported(P.c.kv_dtype, P.d.D, P.d.G)) return 0;
  int grid = attend_grid(P.c.kv_dtype, P.d.D, P.d.G);
  if (grid > kFusedMaxWgs) grid = kFusedMaxWgs;
  const int per = grid / P.d.S;
  if (per < 2 || per - 1 > P.ws.scr_copies) return 0;
  return per;
}

// Tags of the one-launch decode's arrival words: 40 bits, never 0, a new one
// per call in this process.
std::atomic<uint64_t> g_call_tag{0};
uint64_t next_tag() {
  const uint64_t t = (g_call_tag.fetch_add(1, std::memory_order_relaxed) + 1) & ((1ull << 40) - 1);
  return t ? t : 1;
}

eta_status run_phase(int phase, const Prepared& P, hipStream_t st) {
  const int grid = attend_grid(P.c.kv_dtype, P.d.D, P.d.G);
  hipError_t e = hipSuccess;
  switch (phase) {
    case ETA_PHASE_SCREEN:
      e = launch_screen_phase(P.c, P.s, P.p, P.d, P.ws, st);
      break;
    case ETA_PHASE_ATTEND:
      e = launch_attend(P.c, P.s, P.p, P.d, P.ws, grid, st);
      break;
    case ETA_PHASE_MERGE:  // merged at the end of the attend phase
      break;
    default:
      return ETA_ERR_INVALID_ARGUMENT;
  }
  return hip_status(e);
}

}  // namespace
}  // namespace eta

using namespace eta;

extern "C" {

const char* eta_status_string(eta_status s) {
  switch (s) {
    case ETA_OK: return "ok";
    case ETA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case ETA_ERR_UNSUPPORTED: return "unsupported configuration";
    case ETA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case ETA_ERR_HIP: return "HIP runtime error";
    case ETA_ERR_DEVICE_DATA: return "invalid sequence length or page id in device data";
  }
  return "unknown status";
}

eta_status eta_build_block_summaries(const eta_cache* cache, const eta_seqs* seqs, eta_stream_t stream) {
  eta_status st = check_cache(cache);
  if (st != ETA_OK) return st;
  st = check_seqs(seqs);
  if (st != ETA_OK) return st;
  return hip_status(launch_build_summaries(view_of(cache), view_of(seqs), (hipStream_t)stream));
}

eta_status eta_append_kv(const eta_cache* cache, const eta_seqs* seqs, const void* k_new,
                         const void* v_new, eta_stream_t stream) {
  eta_status st = check_cache(cache);
  if (st != ETA_OK) return st;
  st = check_seqs(seqs);
  if (st != ETA_OK) return st;
  if (!k_new || !v_new || !aligned(k_new, 16) || !aligned(v_new, 16)) return ETA_ERR_INVALID_ARGUMENT;
  if ((int64_t)seqs->num_seqs * cache->num_kv_heads > 0x7fffffff) return ETA_ERR_UNSUPPORTED;
  return hip_status(launch_append(view_of(cache), view_of(seqs), k_new, v_new, (hipStream_t)stream));
}

size_t eta_decode_workspace_size(const eta_cache* cache, int num_seqs, int max_blocks_per_seq,
                                 int num_q_heads) {
  if (check_cache(cache) != ETA_OK) return 0;
  Dims d;
  if (dims_of(cache, num_seqs, max_blocks_per_seq, num_q_heads, &d) != ETA_OK) return 0;
  size_t need = workspace_layout(d, nullptr, nullptr);
  // large enough for a decode on the cache's smallest screen blocks as well
  // (more tiles; the page-block layout may still be the larger one, since it
  // carries the private copies of the one-launch decode when it has few tiles)
  if (sub_blocks(cache) > 1) {
    if (dims_of(cache, num_seqs, max_blocks_per_seq, num_q_heads, &d, sub_blocks(cache)) != ETA_OK) return 0;
    const size_t sub = workspace_layout(d, nullptr, nullptr);
    if (sub > need) need = sub;
  }
  return need;
}

eta_status eta_decode_ex(int phase, const eta_screen_opts* screen, const eta_cache* cache, const eta_seqs* seqs,
                         const void* q, int num_q_heads, int tau_mode, const float* w, const float* b_or_c,
                         float a, float beta, int lwb, int block_size, float* out, void* workspace,
                         size_t ws_bytes, eta_stream_t stream) {
  if (phase < ETA_PHASE_ALL || phase > ETA_PHASE_MERGE) return ETA_ERR_INVALID_ARGUMENT;
  Prepared P;
  eta_status st = prepare(screen, cache, seqs, q, num_q_heads, tau_mode, w, b_or_c, a, beta, lwb, block_size,
                          out, workspace, ws_bytes, &P);
  if (st != ETA_OK) return st;
  if (phase != ETA_PHASE_ALL) return run_phase(phase, P, (hipStream_t)stream);
  if (const int per = short_plan(P))
    return hip_status(launch_decode_short(P.c, P.s, P.p, P.d, P.ws, per, next_tag(), (hipStream_t)stream));
  for (int ph = ETA_PHASE_SCREEN; ph <= ETA_PHASE_MERGE; ++ph) {
    st = run_phase(ph, P, (hipStream_t)stream);
    if (st != ETA_OK) return st;
  }
  return ETA_OK;
}

int eta_decode_launches(const eta_screen_opts* screen, const eta_cache* cache, const eta_seqs* seqs,
                        int num_q_heads) {
  // the checks of prepare() that these arguments decide, with a host stand-in
  // for the query, output and workspace pointers (prepare only checks their
  // alignment and lays the workspace out; nothing is read or written there)
  alignas(256) static char stand_in[256];
  float one = 1.f;
  Prepared P;
  eta_status st = prepare(screen, cache, seqs, stand_in, num_q_heads, ETA_TAU_CALIBRATED, nullptr, &one, 0.f, 1.f,
                          0, cache ? cache->block_size : 0, reinterpret_cast<float*>(stand_in), stand_in,
                          (size_t)-1, &P);
  if (st != ETA_OK) return (int)st;
  return short_plan(P) ? 1 : 2;
}

eta_status eta_decode_phase(int phase, const eta_cache* cache, const eta_seqs* seqs, const void* q,
                            int num_q_heads, int tau_mode, const float* w, const float* b_or_c,
                            float a, float beta, int lwb, int block_size, float* out,
                            void* workspace, size_t ws_bytes, eta_stream_t stream) {
  if (phase < ETA_PHASE_SCREEN || phase > ETA_PHASE_MERGE) return ETA_ERR_INVALID_ARGUMENT;
  return eta_decode_ex(phase, nullptr, cache, seqs, q, num_q_heads, tau_mode, w, b_or_c, a, beta, lwb,
                       block_size, out, workspace, ws_bytes, stream);
}

eta_status eta_decode(const eta_cache* cache, const eta_seqs* seqs, const void* q, int num_q_heads,
                      int tau_mode, const float* w, const float* b_or_c, float a, float beta, int lwb,
                      int block_size, float* out, void* workspace, size_t ws_bytes,
                      eta_stream_t stream) {
  return eta_decode_ex(ETA_PHASE_ALL, nullptr, cache, seqs, q, num_q_heads, tau_mode, w, b_or_c, a, beta, lwb,
                       block_size, out, workspace, ws_bytes, stream);
}

eta_status eta_calibrate(const eta_cache* cache, const eta_seqs* seqs, const void* q, int num_q_heads,
                         const float* w, const float* b, const float* rho, const eta_calib_opts* opts,
                         uint64_t* hist, uint64_t* above, uint64_t* total, float* c_out, int32_t* err_flag,
                         eta_stream_t stream) {
  eta_status st = check_cache(cache);
  if (st != ETA_OK) return st;
  st = check_seqs(seqs);
  if (st != ETA_OK) return st;
  if (!opts || !q || !aligned(q, 16)) return ETA_ERR_INVALID_ARGUMENT;
  if (!hist || !above || !total || !c_out || !err_flag || !aligned(hist, 8) || !aligned(above, 8) ||
      !aligned(total, 8) || !aligned(c_out, 4) || !aligned(err_flag, 4))
    return ETA_ERR_INVALID_ARGUMENT;
  const bool learned = w != nullptr || b != nullptr;
  if (learned && (!w || !b || rho || !aligned(w, 16) || !aligned(b, 4))) return ETA_ERR_INVALID_ARGUMENT;
  if (!learned && (!rho || !aligned(rho, 4))) return ETA_ERR_INVALID_ARGUMENT;
  if (!(opts->lo < opts->hi) || !isfinite(opts->lo) || !isfinite(opts->hi) || opts->num_bins < 2)
    return ETA_ERR_INVALID_ARGUMENT;
  Dims d;
  st = dims_of(cache, seqs->num_seqs, seqs->max_blocks_per_seq, num_q_heads, &d);
  if (st != ETA_OK) return st;
  if ((int64_t)d.G * opts->num_bins > 8192) return ETA_ERR_UNSUPPORTED;
  if ((int64_t)seqs->num_seqs * d.HKV > 65535) return ETA_ERR_UNSUPPORTED;  // grid rows
  CalibParams p;
  p.q = q;
  p.HQ = num_q_heads;
  p.num_bins = opts->num_bins;
  p.w = w;
  p.b = b;
  p.rho = rho;
  p.lo = opts->lo;
  p.hi = opts->hi;
  p.hist = hist;
  p.above = above;
  p.total = total;
  p.c_out = c_out;
  p.err = err_flag;
  return hip_status(launch_calibrate(view_of(cache), view_of(seqs), p, (hipStream_t)stream));
}

eta_status eta_prefill(const eta_cache* cache, const eta_seqs* seqs, const void* q, int num_q_heads,
                       int tau_mode, const float* w, const float* b_or_c, float a, float beta, float* out,
                       int32_t* err_flag, eta_stream_t stream) {
  eta_status st = check_cache(cache);
  if (st != ETA_OK) return st;
  st = check_seqs(seqs);
  if (st != ETA_OK) return st;
  if (!q || !out || !b_or_c || !err_flag || !aligned(q, 16) || !aligned(out, 16) || !aligned(b_or_c, 4) ||
      !aligned(err_flag, 4))
    return ETA_ERR_INVALID_ARGUMENT;
  if (tau_mode != ETA_TAU_LEARNED && tau_mode != ETA_TAU_CALIBRATED) return ETA_ERR_INVALID_ARGUMENT;
  if (tau_mode == ETA_TAU_LEARNED && (!w || !aligned(w, 16))) return ETA_ERR_INVALID_ARGUMENT;
  if (!(beta > 0.f) || !isfinite(beta) || !isfinite(a)) return ETA_ERR_INVALID_ARGUMENT;
  Dims d;
  st = dims_of(cache, seqs->num_seqs, seqs->max_blocks_per_seq, num_q_heads, &d);
  if (st != ETA_OK) return st;
  if ((int64_t)seqs->num_seqs * num_q_heads > 65535) return ETA_ERR_UNSUPPORTED;  // grid rows
  PrefillParams p;
  p.q = q;
  p.HQ = num_q_heads;
  p.tau_mode = tau_mode == ETA_TAU_LEARNED ? 0 : 1;
  p.w = w;
  p.b = b_or_c;
  p.a = a;
  p.beta = beta;
  p.out = out;
  p.err = err_flag;
  return hip_status(launch_prefill(view_of(cache), view_of(seqs), p, (hipStream_t)stream));
}

eta_status eta_stats(const void* workspace, int num_seqs, int max_blocks_per_seq, int num_q_heads,
                     int num_kv_heads, int32_t* admitted_per_head, int32_t* union_per_kv,
                     int64_t* tokens_per_head, uint8_t* rescued, uint32_t* admitted_bitmap,
                     eta_stream_t stream) {
  if (!workspace || !aligned(workspace, 256) || !admitted_per_head || !union_per_kv)
    return ETA_ERR_INVALID_ARGUMENT;
  if (num_seqs < 1 || max_blocks_per_seq < 1 || num_kv_heads < 1 || num_q_heads < 1 ||
      num_q_heads % num_kv_heads)
    return ETA_ERR_INVALID_ARGUMENT;
  hipStream_t st = (hipStream_t)stream;
  if (hipStreamSynchronize(st) != hipSuccess) return ETA_ERR_HIP;
  int32_t glob[kGlobCount];  // the header region sits at the workspace's start whatever the sizes
  if (hipMemcpy(glob, workspace, sizeof(glob), hipMemcpyDeviceToHost) != hipSuccess) return ETA_ERR_HIP;
  if (glob[kGlobN] != num_seqs || glob[kGlobMB] != max_blocks_per_seq || glob[kGlobHQ] != num_q_heads ||
      glob[kGlobHKV] != num_kv_heads)
    return ETA_ERR_INVALID_ARGUMENT;
  Dims d;
  d.N = num_seqs;
  d.MB = max_blocks_per_seq;
  d.HQ = num_q_heads;
  d.HKV = num_kv_heads;
  d.G = num_q_heads / num_kv_heads;
  d.S = num_seqs * num_kv_heads;
  d.SB = (glob[kGlobSB] == 2 || glob[kGlobSB] == 4) ? glob[kGlobSB] : 1;
  d.PB = (d.SB == 1 && glob[kGlobPB] == 2) ? 2 : 1;
  d.NT = (max_blocks_per_seq * d.SB + kTile - 1) / kTile;
  d.D = 128;  // only the part_* sizes depend on D; they lie after everything read here
  Ws ws;
  workspace_layout(d, const_cast<void*>(workspace), &ws);
  const size_t nq = (size_t)num_seqs * num_q_heads;
  std::vector<int32_t> tmp(nq);
  if (hipMemcpy(admitted_per_head, ws.st_head, sizeof(int32_t) * nq, hipMemcpyDeviceToHost) != hipSuccess)
    return ETA_ERR_HIP;
  if (hipMemcpy(union_per_kv, ws.seg_ub, sizeof(int32_t) * d.S, hipMemcpyDeviceToHost) != hipSuccess)
    return ETA_ERR_HIP;
  if (tokens_per_head &&
      hipMemcpy(tokens_per_head, ws.st_tokens, sizeof(int64_t) * nq, hipMemcpyDeviceToHost) != hipSuccess)
    return ETA_ERR_HIP;
  if (rescued) {
    if (hipMemcpy(tmp.data(), ws.st_rescued, sizeof(int32_t) * nq, hipMemcpyDeviceToHost) != hipSuccess)
      return ETA_ERR_HIP;
    for (size_t i = 0; i < nq; ++i) rescued[i] = tmp[i] ? 1 : 0;
  }
  if (admitted_bitmap) {
    // tile_bits is [S][G][NT] == [N][HQ][NT] uint64 words, little-endian: the
    // same bit order as [N][HQ][2*NT] uint32 words. With 128-token blocks a
    // bit is a page and block m is bit 2m.
    const size_t nbits = d.PB == 2 ? (size_t)(max_blocks_per_seq + 1) / 2 : (size_t)max_blocks_per_seq * d.SB;
    const size_t words32 = (nbits + 31) / 32;
    std::vector<uint64_t> bits(nq * d.NT);
    if (hipMemcpy(bits.data(), ws.tile_bits, sizeof(uint64_t) * bits.size(), hipMemcpyDeviceToHost) != hipSuccess)
      return ETA_ERR_HIP;
    for (size_t i = 0; i < nq; ++i) {
      const uint64_t* row = bits.data() + i * d.NT;
      uint32_t* dst = admitted_bitmap + i * words32;
      if (d.PB == 2) {
        memset(dst, 0, sizeof(uint32_t) * words32);
        for (size_t m = 0; m < nbits; ++m)
          if ((row[(2 * m) / 64] >> ((2 * m) % 64)) & 1ull) dst[m / 32] |= 1u << (m % 32);
      } else {
        memcpy(dst, reinterpret_cast<const uint32_t*>(row), sizeof(uint32_t) * words32);
      }
    }
  }
  std::vector<int32_t> serr(d.S);
  if (hipMemcpy(serr.data(), ws.seg_err, sizeof(int32_t) * d.S, hipMemcpyDeviceToHost) != hipSuccess)
    return ETA_ERR_HIP;
  for (int32_t e : serr)
    if (e) return ETA_ERR_DEVICE_DATA;
  return ETA_OK;
}

}  // extern "C"
