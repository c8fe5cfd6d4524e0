// Allocation-free entry points: variants of entry points whose kernels use a
// scratch buffer, for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid it).
//
// The scratch is one file-scope device array of kScratchBytes, held by every
// GPU the library runs on until the process ends.  In host code its name is
// only a stand-in for the symbol, not a device address, so the address is
// looked up once per device with hipGetSymbolAddress (with that device
// current: each GPU holds its own copy at its own address) and only that
// pointer is handed to kernels.  Every call on one GPU shares that GPU's
// array: calls that overlap in time on one GPU (different streams, or
// different host threads) race on it and must be serialised by the caller.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "tq_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;  // 16 MiB per device
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// the scratch's device address on `device`, looked up on first use; the
// device must be current
int scratch_on(int device, void** out) {
  if (device < 0 || device >= kMaxDevices) return TQ_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[device]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TQ_EHIP;
    g_scratch[device] = p;
  }
  *out = g_scratch[device];
  return TQ_OK;
}

}  // namespace

namespace tqdev {

int noalloc_prepare(int device) {
  void* p = nullptr;
  return scratch_on(device, &p);
}

}  // namespace tqdev

extern "C" {

size_t tq_noalloc_scratch_bytes(void) { return kScratchBytes; }

int tq_logits_noalloc(tq_handle h, const float* queries, int64_t groups, int64_t nq, const uint32_t* codes,
                      const uint32_t* signs, const float* norms, const float* rnorms, int64_t n, float* scores,
                      void* stream) {
  const int rc = tqdev::check_logits_args(h, queries, groups, nq, codes, signs, norms, rnorms, n, scores);
  if (rc != TQ_OK || groups == 0 || nq == 0 || n == 0) return rc;
  if (tq_logits_workspace_size(h, groups, nq) > kScratchBytes) return TQ_ESCRATCH;
  void* ws = nullptr;
  const int sr = scratch_on(h->device, &ws);
  if (sr != TQ_OK) return sr;
  // the query transform writes every workspace byte the scorers read before
  // they read it, so nothing needs clearing between calls
  return tqdev::run_logits(h, queries, groups, nq, codes, signs, norms, rnorms, n, scores, ws,
                           static_cast<hipStream_t>(stream));
}

}  // extern "C"
