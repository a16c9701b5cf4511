// eta_decode_noalloc: one decode step whose workspace is a fixed array in the
// library's own device memory, for callers that cannot allocate device memory
// (code under stream capture, tight serving loops, hosts that forbid it).
//
// The array `scratch` below holds what eta_decode keeps in the caller's
// workspace: the screen's compacted block lists and counts, the split
// partials, the arrival words of the merge and the per-die work weights. Each
// GPU the library runs on holds its own copy of it until the process ends. Its
// device address is looked up once per device (hipGetSymbolAddress, with that
// device current) and kept; the kernels receive that address, never the
// array's name, which in host code is only a stand-in.
//
// Contents carried from one call to the next are either rewritten by every
// call before they are read (lists, counts, partials; the two-phase decode's
// arrival words are zeroed by its screen phase, the one-launch decode's carry
// the call's tag and count as empty otherwise) or validated when read (the
// per-die weights and the previous call's range timings, which only steer
// the split of the work), so no clearing is needed between calls.
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "eta.h"
#include "eta_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)32 << 20;  // ETA_NOALLOC_WORKSPACE_BYTES in eta.h

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

struct DeviceScratch {
  int device;
  void* ptr;
};
std::mutex g_scratch_mu;
std::vector<DeviceScratch> g_scratch;  // one entry per device, filled on its first call

// Device address of the current device's copy of `scratch`.
eta_status scratch_on_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ETA_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  for (const DeviceScratch& e : g_scratch)
    if (e.device == dev) {
      *out = e.ptr;
      return ETA_OK;
    }
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return ETA_ERR_HIP;
  g_scratch.push_back(DeviceScratch{dev, p});
  *out = p;
  return ETA_OK;
}

}  // namespace

static_assert(kScratchBytes == ETA_NOALLOC_WORKSPACE_BYTES, "the header states the array's size");

extern "C" eta_status eta_decode_noalloc(const eta_cache* cache, const eta_seqs* seqs, const void* q,
                                         int num_q_heads, int tau_mode, const float* w, const float* b_or_c,
                                         float a, float beta, int lwb, int block_size, float* out,
                                         eta_stream_t stream) {
  void* ws = nullptr;
  const eta_status st = scratch_on_current_device(&ws);
  if (st != ETA_OK) return st;
  // eta_decode validates every argument first and refuses sizes whose
  // workspace exceeds the array (ETA_ERR_WORKSPACE_TOO_SMALL)
  return eta_decode(cache, seqs, q, num_q_heads, tau_mode, w, b_or_c, a, beta, lwb, block_size, out, ws,
                    kScratchBytes, stream);
}
